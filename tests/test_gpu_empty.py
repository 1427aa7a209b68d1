"""Calls with nothing to do: zero tokens, zero pages or zero sequences.

Each entry point takes empty tensors (whose data pointers PyTorch may leave
NULL), returns WC_OK and leaves every cache array as it was; the outlier
selection over zero tokens sees all-zero energies and returns the m lowest
channels (ties go to the lower channel)."""
import pytest
import torch

from tests import helpers as H

pytestmark = pytest.mark.gpu


def _snapshot(cache):
    names = ["k_codes", "v_codes", "k_scale", "v_scale", "witness", "exact_slot", "exact_pool"]
    return {n: getattr(cache, n).clone() for n in names if getattr(cache, n) is not None}


def test_empty_calls_are_no_ops():
    L = H.need_gpu()
    print("empty calls", flush=True)
    dev = "cuda"
    cache = L.KVCache(L.WC_DITHER_INT8, 2, 8, 4, pool_capacity=4)
    cache.k_codes.fill_(7)
    cache.witness.fill_(0.5)
    before = _snapshot(cache)
    e_bf = torch.empty((0, 4, 128), dtype=torch.bfloat16, device=dev)
    e64 = torch.empty(0, dtype=torch.int64, device=dev)
    e32 = torch.empty(0, dtype=torch.int32, device=dev)

    L.wc_write_kv(cache, e_bf, e_bf, e64, e32, e64)
    L.wc_write_kv_pages(cache, e_bf, e_bf, e32, e32, e64)
    L.wc_witness(cache, e_bf, e_bf, e64)

    Hq, mp, ns = 28, 4, 16
    q = torch.empty((0, Hq, 128), dtype=torch.bfloat16, device=dev)
    tab = torch.empty((0, mp), dtype=torch.int32, device=dev)
    part = torch.empty(0, dtype=torch.float32, device=dev)
    assert L.wc_decode_workspace_bytes(0, Hq, ns) == 0
    L.wc_decode_attn_meter(cache, 0, q, tab, e32, e64, part, 0.088, 3, 1e-2, 1, 1, 1, ns)
    o = torch.empty((0, Hq, 128), device=dev)
    lse = torch.empty((0, Hq), device=dev)
    L.wc_lse_merge(part, 0, Hq, ns, o, lse)
    L.wc_lse_merge(part, 0, Hq, 40, o, lse)                 # the many-split merge

    risk = torch.empty((0, Hq, mp), device=dev)
    ws = torch.empty(0, dtype=torch.uint8, device=dev)
    pool_used = torch.zeros(1, dtype=torch.int64, device=dev)
    paged = torch.zeros(1, dtype=torch.int64, device=dev)
    L.wc_gate_pagein(cache, 0, risk, lse, tab, e32, 0.2, None, pool_used, paged, ws)
    L.wc_gate_pagein_tanh(cache, 0, risk, tab, e32, 0.2, None, pool_used, paged, ws)
    L.wc_dither_fill(1, 0, 0, 0, 0, torch.empty(0, dtype=torch.int16, device=dev))

    ch = torch.full((2, 4, 8), -1, dtype=torch.int32, device=dev)
    L.wc_outlier_select(torch.empty((2, 0, 4, 128), dtype=torch.bfloat16, device=dev), 8, ch)
    torch.cuda.synchronize()

    after = _snapshot(cache)
    for n, t in before.items():
        assert torch.equal(t, after[n]), n
    assert int(pool_used.item()) == 0 and int(paged.item()) == 0
    assert torch.equal(ch.cpu(), torch.arange(8, dtype=torch.int32).expand(2, 4, 8))


def test_empty_calls_still_check_their_other_arguments():
    L = H.need_gpu()
    print("empty calls, bad arguments", flush=True)
    dev = "cuda"
    cache = L.KVCache(L.WC_DITHER_INT8, 2, 8, 4)
    e_bf = torch.empty((0, 4, 128), dtype=torch.bfloat16, device=dev)
    e64 = torch.empty(0, dtype=torch.int64, device=dev)
    e32 = torch.empty(0, dtype=torch.int32, device=dev)
    with pytest.raises(L.WitcertError):
        L.wc_write_kv(cache, e_bf, e_bf, e64, e32, e64, layer0=2)          # layer out of range
    q = torch.empty((0, 27, 128), dtype=torch.bfloat16, device=dev)       # 27 heads over 4 KV heads
    tab = torch.empty((0, 4), dtype=torch.int32, device=dev)
    part = torch.empty(0, dtype=torch.float32, device=dev)
    with pytest.raises(L.WitcertError):
        L.wc_decode_attn_meter(cache, 0, q, tab, e32, e64, part, 0.088, 3, 1e-2, 1, 1, 1, 16)
    with pytest.raises(L.WitcertError):
        L.wc_lse_merge(part, 0, 28, 0, part, part)                        # no splits

"""A cache layer whose code arrays pass 4 GB: the write path and the decode
then address it with 64-bit offsets (below that size they use 32-bit offsets
from the layer's base).  The same tokens written into a small cache and into
one of 2^21 + 64 + P pages, with every odd page moved past the 4 GB line,
give the same code blocks, scales and witnesses, and the same decode, merge
and block risks, bit for bit."""
import numpy as np
import pytest
import torch

from certified_kv_cache_amd import inputs
from tests import helpers as H
from tests.scenario import Scenario

pytestmark = pytest.mark.gpu

SHIFT = (1 << 21) + 64        # pages of 2 KB: past it a block's offset within the layer exceeds 2^32 bytes


def _flush(msg):
    print(msg, flush=True)


def _decode(L, cache, q, tab, ctx, seed, n_split, mask, delta):
    B, Hq = q.shape[0], q.shape[1]
    part = torch.empty(L.wc_decode_workspace_bytes(B, Hq, n_split) // 4, dtype=torch.float32, device="cuda")
    br = torch.full((B, Hq, tab.shape[1]), float("nan"), device="cuda")
    L.wc_decode_attn_meter(cache, 0, q, tab, ctx, seed, part, H.SM, mask, delta[0], *delta[1:], n_split,
                           block_logrisk=br)
    o = torch.empty((B, Hq, 128), device="cuda")
    lse, ra, rb, ta, tb = (torch.empty((B, Hq), device="cuda") for _ in range(5))
    L.wc_lse_merge(part, B, Hq, n_split, o, lse, ra, rb, ta, tb)
    torch.cuda.synchronize()
    return {n: t.cpu().numpy() for n, t in dict(o=o, lse=lse, ra=ra, rb=rb, ta=ta, tb=tb, risk=br).items()}


@pytest.mark.parametrize("scheme,m", [("int8", 0), ("int8", 8), ("fp8", 0)])
def test_cache_past_4gb_matches_small_cache(scheme, m):
    L = H.need_gpu()
    _flush(f"large cache {scheme} m={m}")
    sch = L.WC_DITHER_INT8 if scheme == "int8" else L.WC_FP8_E4M3
    lens = [100, 37, 16, 1]
    n = int(sum(lens))
    d = inputs.layer(seed=21, S=n, Hq=7, Hkv=1, outliers=2)
    k, v = d["k"][:n], d["v"][:n]
    q = inputs.layer(seed=22, S=1, Hq=7, Hkv=1, batch=len(lens))["q"]
    sc = Scenario(sch, k, v, q, lens, "bf16", Hkv=1, layer=0, num_layers=1, num_outliers=m)
    tab_small = sc.tab
    tab_big = (tab_small + np.where(tab_small % 2 == 1, SHIFT, 0)).astype(np.int32)
    big = L.KVCache(sch, 1, SHIFT + sc.num_pages, 1, num_outliers=m)
    assert big.k_codes.numel() > (1 << 32)
    if m:
        big.outlier_ch[0] = torch.from_numpy(sc.bypass).cuda()
    slot, pos, seq = H.slots_for(tab_big, sc.ctx)
    L.wc_write_kv(big, H.dev_tensor(k, "bf16"), H.dev_tensor(v, "bf16"), torch.from_numpy(slot).cuda(),
                  torch.from_numpy(pos).cuda(), torch.from_numpy(sc.seeds[seq].view(np.int64)).cuda())
    torch.cuda.synchronize()
    # the blocks the tokens went to, small cache against big
    used = sorted({int(p) for b, S in enumerate(lens) for p in tab_small[b, :(S + 15) // 16]})
    pb = torch.tensor([p + (SHIFT if p % 2 else 0) for p in used], device="cuda")
    ps = torch.tensor(used, device="cuda")
    names = ["k_codes", "v_codes", "witness"] + (["k_scale", "v_scale"] if scheme == "int8" else []) + \
            (["k_outlier"] if m else [])
    for nm in names:
        a = getattr(sc.cache, nm)[0, ps].cpu().numpy()
        b = getattr(big, nm)[0, pb].cpu().numpy()
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), nm
    mask = 3 if scheme == "int8" else 1
    ctx = torch.from_numpy(sc.ctx.astype(np.int32)).cuda()
    seed = torch.from_numpy(sc.seeds.view(np.int64)).cuda()
    qd = H.dev_tensor(q, "bf16")
    small = _decode(L, sc.cache, qd, torch.from_numpy(tab_small).cuda(), ctx, seed, 3, mask, sc.delta)
    large = _decode(L, big, qd, torch.from_numpy(tab_big).cuda(), ctx, seed, 3, mask, sc.delta)
    for nm in small:
        assert np.array_equal(small[nm].view(np.uint32), large[nm].view(np.uint32)), nm
    del big
    torch.cuda.empty_cache()

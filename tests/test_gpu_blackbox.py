"""GPU parity of the black-box schemes: round-to-nearest INT8 (write bit-exact,
decode + Tier A), and the 16-bit store of an arbitrary scheme's output with
its witness from wc_witness (the one-tensor-function hook)."""
import numpy as np
import pytest
import torch

from certified_kv_cache_amd import inputs
from oracle import gate, quant
from tests import helpers as H
from tests.scenario import Scenario

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-3
MET_TOL = 1e-4


def _flush(msg):
    print(msg, flush=True)


def _layer(seed, lens, Hq=28, Hkv=4, outliers=2):
    n = int(sum(lens))
    d = inputs.layer(seed=seed, S=max(n, 1), Hq=Hq, Hkv=Hkv, outliers=outliers)
    q = inputs.layer(seed=seed + 100, S=1, Hq=Hq, Hkv=Hkv, batch=len(lens))["q"]
    return d["k"][:n], d["v"][:n], q


def _check(sc, out, repaired=None, exact_out=False):
    for b in range(sc.B):
        S = int(sc.ctx[b])
        for g in range(sc.Hkv):
            hs = slice(g * sc.G, (g + 1) * sc.G)
            if S == 0:
                assert np.all(out["o"][b, hs] == 0) and np.all(out["R_A"][b, hs] == 0)
                continue
            rep = None if repaired is None else repaired(b, g, S)
            _, r = sc.oracle(b, g, repaired=rep)
            err = H.rel_l2(out["o"][b, hs], r["o_exact"] if exact_out else r["o_tilde"])
            assert np.all(err <= OUT_TOL), (b, g, err.max())
            assert np.all(np.abs(out["lse"][b, hs] - r["lse"]) <= 1e-4 * np.maximum(1, np.abs(r["lse"]))), (b, g)
            for key in ("R_A", "T_A"):
                got = out[key][b, hs]
                slack = 1e-7 if key == "T_A" else 0.0
                assert np.all(np.abs(got - r[key]) <= MET_TOL * r[key] + slack), (key, b, g, got, r[key])
                assert np.all(got >= r["tv_true"] * (1 - 1e-6)), (key, b, g)
            assert np.all(out["R_B"][b, hs] == 0) and np.all(out["T_B"][b, hs] == 0)


# ---------------------------------------------------------------- RTN INT8
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rtn_write_bit_exact(dtype):
    L = H.need_gpu()
    _flush(f"rtn write {dtype}")
    lens = [37, 16, 130]
    if dtype == "bf16":
        k, v, q = _layer(80, lens)
    else:
        rng = np.random.default_rng(80)
        n = sum(lens)
        k = (rng.standard_normal((n, 4, 128)) * rng.uniform(0.01, 30, (n, 4, 1))).astype(np.float32)
        v = rng.standard_normal((n, 4, 128)).astype(np.float32)
        k[5, 1] = 0.0
        q = rng.standard_normal((3, 28, 128)).astype(np.float32)
    sc = Scenario(L.WC_RTN_INT8, k, v, q, lens, dtype, Hkv=4)
    torch.cuda.synchronize()
    kc, vc, wt = sc.cache.k_codes.cpu().numpy(), sc.cache.v_codes.cpu().numpy(), sc.cache.witness.cpu().numpy()
    ks, vs = sc.cache.k_scale.cpu().numpy(), sc.cache.v_scale.cpu().numpy()
    for b, S in enumerate(lens):
        for g in range(4):
            oc, _ = sc.oracle(b, g)
            gk = (H.gather_k_codes(kc, sc.layer, sc.tab[b], S, g).astype(np.int16) - 128).astype(np.int8)
            gv = (H.gather_v_codes(vc, sc.layer, sc.tab[b], S, g).astype(np.int16) - 128).astype(np.int8)
            assert np.array_equal(gk, oc["ck"]) and np.array_equal(gv, oc["cv"]), (b, g)
            assert np.array_equal(H.gather_rows(ks, sc.layer, sc.tab[b], S, g), oc["sk"])
            assert np.array_equal(H.gather_rows(vs, sc.layer, sc.tab[b], S, g), oc["sv"])
            w = H.gather_rows(wt, sc.layer, sc.tab[b], S, g)
            assert np.all(np.abs(w - oc["w"]) <= MET_TOL * oc["w"] + 1e-30) and np.all(w >= oc["w"]), (b, g)


@pytest.mark.parametrize("qdtype", ["bf16", "f32"])
def test_rtn_decode_parity(qdtype):
    L = H.need_gpu()
    _flush(f"rtn decode q={qdtype}")
    lens = [1, 17, 700, 0, 1500]
    k, v, q = _layer(81, lens)
    sc = Scenario(L.WC_RTN_INT8, k, v, q, lens, "bf16", Hkv=4)
    if qdtype == "f32":
        sc.dev["q"] = torch.from_numpy(H.to_f32(q, "bf16")).cuda()
    for n_split in (1, 6):
        _check(sc, sc.decode(n_split=n_split, mask=1, risk=True))
    with pytest.raises(L.WitcertError):                      # Tier B needs the dither
        sc.decode(n_split=2, mask=3)


def test_rtn_decode_large_group_and_risks():
    L = H.need_gpu()
    _flush("rtn decode G=12")
    lens = [300, 77]
    k, v, q = _layer(82, lens, Hq=24, Hkv=2, outliers=1)
    sc = Scenario(L.WC_RTN_INT8, k, v, q, lens, "bf16", Hkv=2)
    out = sc.decode(n_split=3, mask=1, risk=True)
    _check(sc, out)
    for b, S in enumerate(lens):
        P = -(-S // 16)
        for g in range(2):
            _, r = sc.oracle(b, g)
            hs = slice(g * 12, (g + 1) * 12)
            rho = np.exp(out["logrisk"][b, hs, :P].astype(np.float64) - out["lse"][b, hs, None])
            assert np.all(np.abs(rho - r["block_risk"]) <= 1e-4 * r["block_risk"] + 1e-30), (b, g)


# ---------------------------------------------------------------- 16-bit store + wc_witness
def _mantissa4(bits):
    """The scheme under test, as one tensor function: keep 4 of bf16's 8
    significant bits (round half up on the magnitude)."""
    b = bits.astype(np.uint32)
    return (((b + 0x4) & 0xFFF8) & 0xFFFF).astype(np.uint16)


@pytest.mark.parametrize("qdtype", ["bf16", "f32"])
def test_store_blackbox_write_witness_and_decode(qdtype):
    L = H.need_gpu()
    _flush(f"16-bit store q={qdtype}")
    lens = [1, 17, 700, 0, 1300]
    k, v, q = _layer(83, lens)
    kh, vh = _mantissa4(k), _mantissa4(v)
    sc = Scenario(L.WC_BF16_STORE, k, v, q, lens, "bf16", Hkv=4, khat=kh, vhat=vh)
    if qdtype == "f32":
        sc.dev["q"] = torch.from_numpy(H.to_f32(q, "bf16")).cuda()
    torch.cuda.synchronize()
    kc = sc.cache.k_codes.cpu().numpy().view(np.uint16)
    vc = sc.cache.v_codes.cpu().numpy().view(np.uint16)
    wt = sc.cache.witness.cpu().numpy()
    for b, S in enumerate(lens):
        s0 = sc.offsets[b]
        for g in range(4):
            assert np.array_equal(H.gather_k_bf16(kc, sc.layer, sc.tab[b], S, g), kh[s0:s0 + S, g])
            assert np.array_equal(H.gather_v_bf16(vc, sc.layer, sc.tab[b], S, g), vh[s0:s0 + S, g])
            if S == 0:
                continue
            oc, _ = sc.oracle(b, g)
            w = H.gather_rows(wt, sc.layer, sc.tab[b], S, g)
            assert np.all(np.abs(w - oc["w"]) <= MET_TOL * oc["w"] + 1e-30) and np.all(w >= oc["w"]), (b, g)
    for n_split in (1, 5):
        _check(sc, sc.decode(n_split=n_split, mask=1, risk=True))


def test_store_of_exact_keys_is_exact_attention():
    # x^ = x: the witness is 0, both bounds are 0 and the output is exact attention
    L = H.need_gpu()
    _flush("16-bit store, exact")
    lens = [250, 64]
    k, v, q = _layer(84, lens)
    sc = Scenario(L.WC_BF16_STORE, k, v, q, lens, "bf16", Hkv=4, khat=k, vhat=v)
    out = sc.decode(n_split=3, mask=1)
    assert np.all(out["R_A"] == 0) and np.all(out["T_A"] == 0)
    _check(sc, out, exact_out=True)
    # f32 witness hook on the same rows: x against itself gives zeros
    x = torch.from_numpy(H.to_f32(k, "bf16")).cuda()
    L.wc_witness(sc.cache, x, x.clone(), sc.dev["slot"], layer0=sc.layer)
    torch.cuda.synchronize()
    assert np.all(sc.cache.witness.cpu().numpy()[sc.layer] == 0)


def test_store_gate_then_decode():
    L = H.need_gpu()
    _flush("16-bit store gate")
    lens = [400, 129]
    k, v, q = _layer(85, lens)
    kh, vh = _mantissa4(k), _mantissa4(v)
    sc = Scenario(L.WC_BF16_STORE, k, v, q, lens, "bf16", Hkv=4, khat=kh, vhat=vh, pool_capacity=512)
    store = np.zeros((2, sc.num_pages, 4, 16, 128), dtype=np.uint16)
    for b, S in enumerate(lens):
        t = np.arange(S)
        store[sc.layer, sc.tab[b, t // 16], :, t % 16] = k[sc.offsets[b]:sc.offsets[b + 1]]
    host = torch.from_numpy(store.view(np.int16)).pin_memory()
    out = sc.decode(n_split=4, mask=1, risk=True)
    B, Hq, mp = sc.B, sc.Hq, sc.tab.shape[1]
    ws = torch.empty(L.wc_gate_workspace_bytes(B, 4, mp), dtype=torch.uint8, device="cuda")
    pool_used = torch.zeros(1, dtype=torch.int64, device="cuda")
    paged = torch.zeros(1, dtype=torch.int64, device="cuda")
    sel = torch.full((B, 4, mp + 1), -7, dtype=torch.int32, device="cuda")
    rho = torch.zeros((B, Hq, mp), dtype=torch.int64, device="cuda")
    tau = float(0.3 * np.median(out["R_A"]))
    L.wc_gate_pagein(sc.cache, sc.layer, torch.from_numpy(out["logrisk"]).cuda(),
                     torch.from_numpy(out["lse"]).cuda(), sc.dev["tab"], sc.dev["ctx"], tau, host, pool_used, paged,
                     ws, selected=sel, rho_fx=rho)
    torch.cuda.synchronize()
    sel, rho = sel.cpu().numpy(), rho.cpu().numpy().view(np.uint64)
    for b, S in enumerate(lens):
        P = -(-S // 16)
        for g in range(4):
            want = gate.select(rho[b, g * 7:(g + 1) * 7, :P], np.zeros(P, bool), gate.threshold_fx(tau))
            assert list(sel[b, g, 1:1 + sel[b, g, 0]]) == want, (b, g)
    slots = sc.cache.exact_slot.cpu().numpy()[sc.layer]
    nrep = int((slots >= 0).sum())
    assert 0 < nrep < sum(-(-S // 16) for S in lens) * 4

    def repaired(b, g, S):
        return slots[sc.tab[b, np.arange(S) // 16], g] >= 0

    _check(sc, sc.decode(n_split=4, mask=1), repaired=repaired)

"""GPU parity of the outlier bypass: channel selection bit-exact, the write
(codes, scales, exact side store) bit-exact, and decode + meter against the
oracle, including blocks repaired by the gate."""
import numpy as np
import pytest
import torch

from certified_kv_cache_amd import inputs
from oracle import gate, outlier
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


def test_outlier_select_bit_exact():
    L = H.need_gpu()
    _flush("outlier select")
    # three layers of bf16 keys with planted outlier channels, two budgets
    ks = [inputs.layer(seed=70 + i, S=1500, outliers=3)["k"] for i in range(3)]
    kb = np.stack(ks)                                      # [3, 1500, 4, 128] bf16 bits
    k32 = H.to_f32(kb, "bf16")
    for m in (8, 16, 1, 128):
        ch = torch.full((3, 4, m), -1, dtype=torch.int32, device="cuda")
        L.wc_outlier_select(H.dev_tensor(kb, "bf16"), m, ch)
        got = ch.cpu().numpy()
        for li in range(3):
            for g in range(4):
                assert np.array_equal(got[li, g], outlier.top_energy_channels(k32[li, :, g], m)), (m, li, g)
    # float32 input: ties (identical channels), a ragged token count, no tokens
    rng = np.random.default_rng(71)
    col = rng.standard_normal((37, 2, 1)).astype(np.float32)
    x = np.repeat(col, 128, axis=2) * rng.uniform(0.5, 2, (1, 1, 128)).astype(np.float32)
    x[:, 1, ::3] = col[:, 1]                               # head 1: every third channel ties
    for n_tok in (37, 0):
        xx = np.ascontiguousarray(x[:n_tok])
        ch = torch.full((1, 2, 8), -1, dtype=torch.int32, device="cuda")
        L.wc_outlier_select(torch.from_numpy(xx).cuda().reshape(n_tok, 2, 128), 8, ch)
        got = ch.cpu().numpy()[0]
        for g in range(2):
            assert np.array_equal(got[g], outlier.top_energy_channels(xx[:, g], 8)), (n_tok, g)


@pytest.mark.parametrize("m", [8, 16])
def test_bypass_write_bit_exact(m):
    L = H.need_gpu()
    _flush(f"bypass write m={m}")
    lens = [37, 16, 300]
    k, v, q = _layer(72, lens)
    sc = Scenario(L.WC_DITHER_INT8, k, v, q, lens, "bf16", Hkv=4, num_outliers=m)
    torch.cuda.synchronize()
    kc, vc = sc.cache.k_codes.cpu().numpy(), sc.cache.v_codes.cpu().numpy()
    wt = sc.cache.witness.cpu().numpy()
    ks, vs = sc.cache.k_scale.cpu().numpy(), sc.cache.v_scale.cpu().numpy()
    side = sc.cache.k_outlier.cpu().numpy().view(np.uint16)
    for b, S in enumerate(lens):
        for g in range(4):
            oc, _ = sc.oracle(b, g)
            gk = (H.gather_k_codes(kc, sc.layer, sc.tab[b], S, g).astype(np.int16) - 128).astype(np.int8)
            gv = (H.gather_v_codes(vc, sc.layer, sc.tab[b], S, g).astype(np.int16) - 128).astype(np.int8)
            assert np.array_equal(gk, oc["ck"]) and np.array_equal(gv, oc["cv"]), (b, g)
            assert np.array_equal(H.gather_rows(ks, sc.layer, sc.tab[b], S, g), oc["sk"]), (b, g)
            assert np.array_equal(H.gather_rows(vs, sc.layer, sc.tab[b], S, g), oc["sv"]), (b, g)
            s_got = H.to_f32(H.gather_rows(side, sc.layer, sc.tab[b], S, g), "bf16")
            assert np.array_equal(s_got, oc["side"]), (b, g)
            w = H.gather_rows(wt, sc.layer, sc.tab[b], S, g)
            assert np.all(np.abs(w - oc["w"]) <= MET_TOL * oc["w"] + 1e-30) and np.all(w >= oc["w"]), (b, g)
    # the planted x20 channels (and their RoPE partners) are among the selected ones
    assert sc.bypass.shape == (4, m)


def _check(sc, out, repaired=None):
    for b in range(sc.B):
        S = int(sc.ctx[b])
        for g in range(sc.Hkv):
            hs = slice(g * sc.G, (g + 1) * sc.G)
            if S == 0:
                assert np.all(out["o"][b, hs] == 0) and np.all(np.isneginf(out["lse"][b, hs]))
                assert np.all(out["R_A"][b, hs] == 0) and np.all(out["R_B"][b, hs] == 0)
                assert np.all(out["T_A"][b, hs] == 0) and np.all(out["T_B"][b, hs] == 0)
                continue
            rep = None if repaired is None else repaired(b, g, S)
            _, r = sc.oracle(b, g, repaired=rep)
            err = H.rel_l2(out["o"][b, hs], r["o_tilde"])
            assert np.all(err <= OUT_TOL), (b, g, err.max())
            assert np.all(np.abs(out["lse"][b, hs] - r["lse"]) <= 1e-4 * np.maximum(1, np.abs(r["lse"]))), (b, g)
            for key in ("R_A", "R_B", "T_A", "T_B"):
                got = out[key][b, hs]
                slack = 1e-7 if key[0] == "T" else 0.0
                assert np.all(np.abs(got - r[key]) <= MET_TOL * r[key] + slack), (key, b, g, got, r[key])
                assert np.all(got >= r["tv_true"] * (1 - 1e-6)), (key, b, g)


@pytest.mark.parametrize("m,qdtype", [(8, "bf16"), (16, "bf16"), (8, "f32"), (16, "f32")])
def test_bypass_decode_parity(m, qdtype):
    L = H.need_gpu()
    _flush(f"bypass decode m={m} q={qdtype}")
    lens = [1, 17, 700, 0, 1500]
    k, v, q = _layer(73, lens)
    sc = Scenario(L.WC_DITHER_INT8, k, v, q, lens, "bf16", Hkv=4, num_outliers=m)
    if qdtype == "f32":                                    # the same query values, fp32 operand path
        sc.dev["q"] = torch.from_numpy(H.to_f32(q, "bf16")).cuda()
    for n_split in (1, 6):
        out = sc.decode(n_split=n_split, mask=3, risk=True)
        _check(sc, out)
    # block risks: the gate tier (B) per block against the oracle
    for b in (2, 4):
        P = -(-lens[b] // 16)
        for g in range(4):
            _, r = sc.oracle(b, g)
            hs = slice(g * 7, (g + 1) * 7)
            rho = np.exp(out["logrisk"][b, hs, :P].astype(np.float64) - out["lse"][b, hs, None])
            assert np.all(np.abs(rho - r["block_risk"]) <= 1e-4 * r["block_risk"] + 1e-30), (b, g)
    # the bypass pays off on the x20-outlier keys: Tier B well below the plain cache's
    plain = Scenario(L.WC_DITHER_INT8, k, v, q, lens, "bf16", Hkv=4)
    pout = plain.decode(n_split=6, mask=3)
    live = np.repeat(np.asarray(lens) > 0, 28)
    assert np.all(out["R_B"].ravel()[live] < 0.5 * pout["R_B"].ravel()[live])


@pytest.mark.parametrize("m", [8, 16])
def test_bypass_decode_large_group(m):
    # 12 query heads per KV head: the uncompacted softmax path
    L = H.need_gpu()
    _flush(f"bypass decode G=12 m={m}")
    lens = [300, 77]
    k, v, q = _layer(74, lens, Hq=24, Hkv=2, outliers=1)
    sc = Scenario(L.WC_DITHER_INT8, k, v, q, lens, "bf16", Hkv=2, num_outliers=m)
    _check(sc, sc.decode(n_split=3, mask=3))


def test_bypass_gate_then_decode():
    # Repaired blocks use the exact pool for the channels off O and the side
    # store on O; both tiers are 0 there.
    L = H.need_gpu()
    _flush("bypass gate then decode")
    lens = [400, 129]
    k, v, q = _layer(75, lens)
    sc = Scenario(L.WC_DITHER_INT8, k, v, q, lens, "bf16", Hkv=4, pool_capacity=512, num_outliers=8)
    store = np.zeros((2, sc.num_pages, 4, 16, 128), dtype=np.uint16)
    for b, S in enumerate(lens):
        t = np.arange(S)
        store[sc.layer, sc.tab[b, t // 16], :, t % 16] = k[sc.offsets[b]:sc.offsets[b + 1]]
    host = torch.from_numpy(store.view(np.int16)).pin_memory()
    out = sc.decode(n_split=4, mask=3, risk=True)
    B, Hq, mp = sc.B, sc.Hq, sc.tab.shape[1]
    ws = torch.empty(L.wc_gate_workspace_bytes(B, 4, mp), dtype=torch.uint8, device="cuda")
    pool_used = torch.zeros(1, dtype=torch.int64, device="cuda")
    paged = torch.zeros(1, dtype=torch.int64, device="cuda")
    sel = torch.full((B, 4, mp + 1), -7, dtype=torch.int32, device="cuda")
    rho = torch.zeros((B, Hq, mp), dtype=torch.int64, device="cuda")
    tau = float(0.3 * np.median(out["R_B"]))               # a partial repair
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
    assert 0 < nrep < sum(-(-S // 16) for S in lens) * 4 and int(pool_used.item()) == nrep

    def repaired(b, g, S):
        return slots[sc.tab[b, np.arange(S) // 16], g] >= 0

    _check(sc, sc.decode(n_split=4, mask=3), repaired=repaired)

"""GPU parity of the gate: fixed-point risks, bit-exact block selection,
page-in from pinned host memory, witness zeroing, and decode on the
repaired cache, persistent repair across appended tokens, decisions on
independent risks, and sorts over many LDS tiles."""
import math

import numpy as np
import pytest
import torch

from certified_kv_cache_amd import inputs
from oracle import gate, meter
from tests import helpers as H
from tests.scenario import Scenario

pytestmark = pytest.mark.gpu

# fixed-point block risks against the oracle's: the meter's relative bar, plus
# one unit of the 2^-40 grid (the ceilings of the fp32 and float64 risks can
# fall on neighbouring integers)
RISK_TOL = 1e-4


def _setup(lens, seed=21, capacity=4096, scheme="fp8"):
    L = H.need_gpu()
    n = int(sum(lens))
    d = inputs.layer(seed=seed, S=n, Hq=28, Hkv=4, outliers=2)
    q = inputs.layer(seed=seed + 1, S=1, batch=len(lens))["q"]
    sch = L.WC_FP8_E4M3 if scheme == "fp8" else L.WC_DITHER_INT8
    sc = Scenario(sch, d["k"], d["v"], q, lens, "bf16", Hkv=4, pool_capacity=capacity)
    # pinned exact store [L][P][Hkv][16][128] bf16, filled through the page table
    store = np.zeros((2, sc.num_pages, 4, 16, 128), dtype=np.uint16)
    for b, S in enumerate(lens):
        t = np.arange(S)
        store[sc.layer, sc.tab[b, t // 16], :, t % 16] = d["k"][sc.offsets[b]:sc.offsets[b + 1]]
    host = torch.from_numpy(store.view(np.int16)).pin_memory()
    return L, sc, host


def _pool_bits(cache):
    """The exact pool as uint16 bf16 bit patterns [slot][16][128]."""
    return cache.exact_pool.view(torch.int16).cpu().numpy().view(np.uint16)


def _gate(L, sc, host, tau, budget=-1, mask=1):
    out = sc.decode(n_split=4, mask=mask, risk=True)
    B, Hq, mp = sc.B, sc.Hq, sc.tab.shape[1]
    ws = torch.empty(L.wc_gate_workspace_bytes(B, 4, mp), dtype=torch.uint8, device="cuda")
    pool_used = torch.zeros(1, dtype=torch.int64, device="cuda")
    paged = torch.zeros(1, dtype=torch.int64, device="cuda")
    sel = torch.full((B, 4, mp + 1), -7, dtype=torch.int32, device="cuda")
    rho = torch.zeros((B, Hq, mp), dtype=torch.int64, device="cuda")
    L.wc_gate_pagein(sc.cache, sc.layer, torch.from_numpy(out["logrisk"]).cuda(),
                     torch.from_numpy(out["lse"]).cuda(), sc.dev["tab"], sc.dev["ctx"], tau, host, pool_used, paged,
                     ws, budget_blocks=budget, selected=sel, rho_fx=rho)
    torch.cuda.synchronize()
    return out, sel.cpu().numpy(), rho.cpu().numpy().view(np.uint64), int(pool_used.item()), int(paged.item())


@pytest.mark.parametrize("tau", [0.05, 0.2, 1.0])
def test_gate_selection_bit_exact_and_pagein(tau):
    lens = [300, 1000, 64]
    L, sc, host = _setup(lens)
    print(f"gate tau={tau}", flush=True)
    rep0 = sc.cache.exact_slot.cpu().numpy()[sc.layer].copy()
    out, sel, rho, used, paged = _gate(L, sc, host, tau)
    T = gate.threshold_fx(tau)
    total = 0
    for b, S in enumerate(lens):
        P = -(-S // 16)
        for g in range(4):
            fx = rho[b, g * 7:(g + 1) * 7, :P]
            repaired = rep0[sc.tab[b, :P], g] >= 0
            want = gate.select(fx, repaired, T)
            got = list(sel[b, g, 1:1 + sel[b, g, 0]])
            assert got == want, (b, g)
            total += len(want)
            # fixed-point risks follow the oracle's float64 risks
            _, r = sc.oracle(b, g)
            ref = gate.rho_to_fx(r["block_risk"]).astype(np.float64)
            dev = np.abs(fx.astype(np.float64) - ref)
            assert np.all(dev <= RISK_TOL * ref + 1), (b, g, (dev - 1).max())
    assert used == total and paged == 4096 * total
    # repaired blocks: exact bf16 keys in the pool (bit for bit), witness
    # zeroed, slot recorded
    slots = sc.cache.exact_slot.cpu().numpy()[sc.layer]
    pool = _pool_bits(sc.cache)
    wit = sc.cache.witness.cpu().numpy()[sc.layer]
    store = host.numpy().view(np.uint16)[sc.layer]
    for b in range(len(lens)):
        for g in range(4):
            for j in sel[b, g, 1:1 + sel[b, g, 0]]:
                p = sc.tab[b, j]
                s = slots[p, g]
                assert s >= 0
                assert np.array_equal(pool[s], store[p, g])
                assert np.all(wit[p, g] == 0)


def test_gate_then_decode_matches_oracle_on_repaired_cache():
    lens = [400, 129]
    L, sc, host = _setup(lens, seed=31)
    print("gate then decode", flush=True)
    _gate(L, sc, host, 0.05)
    out2 = sc.decode(n_split=3, mask=1)
    slots = sc.cache.exact_slot.cpu().numpy()[sc.layer]
    nrep = 0
    for b, S in enumerate(lens):
        for g in range(4):
            t = np.arange(S)
            rep = slots[sc.tab[b, t // 16], g] >= 0
            nrep += rep.sum()
            _, r = sc.oracle(b, g, repaired=rep)
            hs = slice(g * 7, (g + 1) * 7)
            assert np.all(H.rel_l2(out2["o"][b, hs], r["o_tilde"]) <= 2e-3)
            assert np.all(np.abs(out2["R_A"][b, hs] - r["R_A"]) <= 1e-4 * r["R_A"] + 1e-30)
            assert np.all(out2["R_A"][b, hs] >= r["tv_true"])
    assert nrep > 0


def test_gate_full_repair_and_no_trigger():
    lens = [200, 50]
    L, sc, host = _setup(lens, seed=41)
    print("gate full repair", flush=True)
    _, sel, _, used, _ = _gate(L, sc, host, 1000.0)
    assert used == 0 and np.all(sel[:, :, 0] == 0)
    _gate(L, sc, host, 0.0)
    out = sc.decode(n_split=2, mask=1)
    assert np.all(out["R_A"] == 0)
    for b, S in enumerate(lens):
        for g in range(4):
            _, r = sc.oracle(b, g, repaired=np.ones(S, bool))
            hs = slice(g * 7, (g + 1) * 7)
            # keys are exact, values stay quantized: the compressed output with
            # exact attention weights, and zero true TV
            assert np.all(H.rel_l2(out["o"][b, hs], r["o_tilde"]) <= 2e-3)
            assert np.all(r["tv_true"] < 1e-15)


def test_gate_on_a_131072_token_sequence():
    """One sequence of 131072 tokens: 8192 blocks per (sequence, KV head), two
    LDS tiles merged in the workspace.  Decisions bit-exact for the certificate
    gate and the tanh gate, risks within 1e-4 relative plus one unit of the
    2^-40 grid."""
    lens = [131072]
    L, sc, host = _setup(lens, seed=41, capacity=32768)
    assert sc.tab.shape[1] == 8192
    print("gate at 8192 pages", flush=True)
    rep0 = sc.cache.exact_slot.cpu().numpy()[sc.layer].copy()
    out, sel, rho, used, paged = _gate(L, sc, host, 0.2)
    T = gate.threshold_fx(0.2)
    total = 0
    for g in range(4):
        fx = rho[0, g * 7:(g + 1) * 7, :8192]
        want = gate.select(fx, rep0[sc.tab[0], g] >= 0, T)
        got = list(sel[0, g, 1:1 + sel[0, g, 0]])
        assert got == want, g
        total += len(want)
        _, r = sc.oracle(0, g)
        ref = gate.rho_to_fx(r["block_risk"]).astype(np.float64)
        dev = np.abs(fx.astype(np.float64) - ref)
        assert np.all(dev <= RISK_TOL * ref + 1), (g, (dev - 1).max())
    assert used == total and paged == 4096 * total
    print(f"selected {total} blocks", flush=True)
    # the tanh gate ranks the same 8192 pages (a fresh cache of the same input)
    L, sc, host = _setup(lens, seed=41, capacity=32768)
    out = sc.decode(n_split=4, mask=1, cmax=True)
    cm = out["cmax"]
    tau = float(np.median(out["T_A"]))
    rep0 = sc.cache.exact_slot.cpu().numpy()[sc.layer].copy()
    sel, used, paged = _tanh_gate(L, sc, host, cm, tau)
    total = 0
    for g in range(4):
        want = gate.select_tanh(cm[0, g * 7:(g + 1) * 7, :8192], rep0[sc.tab[0], g] >= 0, tau)
        assert list(sel[0, g, 1:1 + sel[0, g, 0]]) == want, g
        total += len(want)
    assert used == total and paged == 4096 * total
    print(f"tanh gate selected {total} blocks", flush=True)


@pytest.mark.parametrize("n_pages", [4096 * 3 + 100, 4097])
def test_gate_sort_across_tiles_with_ties(n_pages):
    """The selection's sort on synthetic block risks (no decode): one sequence
    of n_pages blocks, one KV head of 7 query heads, log-risks on a coarse grid
    so that many blocks tie (ties go to the lower block index).  The ranking
    of 3 or 4 LDS tiles merged in the workspace must equal the oracle's, for
    the certificate gate (checked on its exported fixed-point risks) and the
    tanh gate; the pool capacity bounds what is paged in."""
    L = H.need_gpu()
    print(f"gate sort, {n_pages} blocks", flush=True)
    rng = np.random.default_rng(n_pages)
    G, cap = 7, 3000
    cache = L.KVCache(L.WC_FP8_E4M3, 1, n_pages, 1, pool_capacity=cap)
    tab = torch.from_numpy(rng.permutation(n_pages).astype(np.int32)[None]).cuda()
    ctx = torch.tensor([16 * n_pages], dtype=torch.int32, device="cuda")
    logrisk = np.round(rng.uniform(-14.0, -6.0, (1, G, n_pages)) * 4.0) / 4.0   # 33 distinct values
    logrisk[0, :, rng.random(n_pages) < 0.05] = -np.inf                          # riskless blocks
    lse = np.zeros((1, G), dtype=np.float32)
    host = torch.zeros((1, n_pages, 1, 16, 128), dtype=torch.bfloat16).pin_memory()
    ws = torch.empty(L.wc_gate_workspace_bytes(1, 1, n_pages), dtype=torch.uint8, device="cuda")
    for tau in (0.0, 0.02):
        pool_used = torch.zeros(1, dtype=torch.int64, device="cuda")
        paged = torch.zeros(1, dtype=torch.int64, device="cuda")
        sel = torch.full((1, 1, n_pages + 1), -7, dtype=torch.int32, device="cuda")
        rho = torch.zeros((1, G, n_pages), dtype=torch.int64, device="cuda")
        cache.exact_slot.fill_(-1)
        L.wc_gate_pagein(cache, 0, torch.from_numpy(logrisk.astype(np.float32)).cuda(), torch.from_numpy(lse).cuda(),
                         tab, ctx, tau, host, pool_used, paged, ws, selected=sel, rho_fx=rho)
        torch.cuda.synchronize()
        fx = rho.cpu().numpy().view(np.uint64)[0]
        want = gate.select(fx, np.zeros(n_pages, bool), gate.threshold_fx(tau))
        got = list(sel.cpu().numpy()[0, 0, 1:1 + sel.cpu().numpy()[0, 0, 0]])
        assert len(want) > cap and got == want[:cap], tau
        assert int(pool_used.item()) == cap
    cmax = np.round(rng.uniform(0.0, 3.0, (1, G, n_pages)) * 8.0) / 8.0
    for tau in (0.3, 0.9):
        cache.exact_slot.fill_(-1)
        pool_used = torch.zeros(1, dtype=torch.int64, device="cuda")
        paged = torch.zeros(1, dtype=torch.int64, device="cuda")
        sel = torch.full((1, 1, n_pages + 1), -7, dtype=torch.int32, device="cuda")
        L.wc_gate_pagein_tanh(cache, 0, torch.from_numpy(cmax.astype(np.float32)).cuda(), tab, ctx, tau, host,
                              pool_used, paged, ws, selected=sel)
        torch.cuda.synchronize()
        want = gate.select_tanh(cmax.astype(np.float32)[0], np.zeros(n_pages, bool), tau)
        got = list(sel.cpu().numpy()[0, 0, 1:1 + sel.cpu().numpy()[0, 0, 0]])
        assert got == want[:cap], tau


def test_gate_budget_and_pool_capacity():
    lens = [300, 300]
    L, sc, host = _setup(lens, seed=51, capacity=5)
    print("gate capacity", flush=True)
    out, sel, rho, used, paged = _gate(L, sc, host, 0.0, budget=2)
    assert used <= 5 and paged == 4096 * used
    counts = sel[:, :, 0].ravel()
    assert np.all(counts <= 2) and counts.sum() == used
    T = gate.threshold_fx(0.0)
    left = 5
    for b in range(2):
        for g in range(4):
            want = gate.select(rho[b, g * 7:(g + 1) * 7, :19], np.zeros(19, bool), T, budget=2)
            take = min(len(want), left)
            left -= take
            assert list(sel[b, g, 1:1 + sel[b, g, 0]]) == want[:take]


def _tanh_gate(L, sc, host, cmax, tau, budget=-1):
    B, Hq, mp = sc.B, sc.Hq, sc.tab.shape[1]
    ws = torch.empty(L.wc_gate_workspace_bytes(B, 4, mp), dtype=torch.uint8, device="cuda")
    pool_used = torch.zeros(1, dtype=torch.int64, device="cuda")
    paged = torch.zeros(1, dtype=torch.int64, device="cuda")
    sel = torch.full((B, 4, mp + 1), -7, dtype=torch.int32, device="cuda")
    L.wc_gate_pagein_tanh(sc.cache, sc.layer, torch.from_numpy(cmax).cuda(), sc.dev["tab"], sc.dev["ctx"], tau, host,
                          pool_used, paged, ws, budget_blocks=budget, selected=sel)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), int(pool_used.item()), int(paged.item())


@pytest.mark.parametrize("scheme", ["fp8", "int8"])
def test_tanh_gate_bit_exact_and_bound_met(scheme):
    lens = [300, 1000, 64]
    L, sc, host = _setup(lens, seed=61, scheme=scheme)
    print(f"tanh gate {scheme}", flush=True)
    mask = 1 if scheme == "fp8" else 3
    out = sc.decode(n_split=4, mask=mask, cmax=True)
    tkey = "T_A" if scheme == "fp8" else "T_B"
    cm = out["cmax"]
    for b, S in enumerate(lens):
        P = -(-S // 16)
        for g in range(4):
            _, r = sc.oracle(b, g)
            hs = slice(g * 7, (g + 1) * 7)
            got = cm[b, hs, :P].astype(np.float64)
            assert np.all(np.abs(got - r["block_cmax"]) <= 1e-4 * r["block_cmax"] + 1e-30), (b, g)
            # the merged tanh bound is the tanh of the largest block value
            assert np.allclose(out[tkey][b, hs], np.tanh(0.5 * got.max(-1)), rtol=1e-5, atol=0)
    # a threshold that repairs part of the blocks
    tau = float(np.median(out[tkey]))
    rep0 = sc.cache.exact_slot.cpu().numpy()[sc.layer].copy()
    sel, used, paged = _tanh_gate(L, sc, host, cm, tau)
    total = 0
    for b, S in enumerate(lens):
        P = -(-S // 16)
        for g in range(4):
            want = gate.select_tanh(cm[b, g * 7:(g + 1) * 7, :P], rep0[sc.tab[b, :P], g] >= 0, tau)
            assert list(sel[b, g, 1:1 + sel[b, g, 0]]) == want, (b, g)
            total += len(want)
    assert 0 < total and used == total and paged == 4096 * total
    # the repaired cache meets the bound: every head's tanh bound is now <= tau
    after = sc.decode(n_split=4, mask=mask)
    assert np.all(after[tkey] <= tau * (1 + 1e-6)), (after[tkey].max(), tau)
    # witness zeroed and exact keys in place for what was paged in
    slots = sc.cache.exact_slot.cpu().numpy()[sc.layer]
    wit = sc.cache.witness.cpu().numpy()[sc.layer]
    for b in range(len(lens)):
        for g in range(4):
            for j in sel[b, g, 1:1 + sel[b, g, 0]]:
                assert slots[sc.tab[b, j], g] >= 0 and np.all(wit[sc.tab[b, j], g] == 0)


def test_tanh_gate_budget_and_no_trigger():
    lens = [300, 200]
    L, sc, host = _setup(lens, seed=62)
    print("tanh gate budget", flush=True)
    out = sc.decode(n_split=2, mask=1, cmax=True)
    sel, used, _ = _tanh_gate(L, sc, host, out["cmax"], 1.0)       # tanh < 1: never triggers
    assert used == 0 and np.all(sel[:, :, 0] == 0)
    sel, used, _ = _tanh_gate(L, sc, host, out["cmax"], 0.0, budget=3)
    for b, S in enumerate(lens):
        P = -(-S // 16)
        for g in range(4):
            want = gate.select_tanh(out["cmax"][b, g * 7:(g + 1) * 7, :P], np.zeros(P, bool), 0.0, budget=3)
            assert list(sel[b, g, 1:1 + sel[b, g, 0]]) == want
    assert used == int(sel[:, :, 0].sum())


def _gate_meter(L, sc, host, out, tau, meter):
    B, Hq, mp = sc.B, sc.Hq, sc.tab.shape[1]
    ws = torch.empty(L.wc_gate_workspace_bytes(B, 4, mp), dtype=torch.uint8, device="cuda")
    pool_used = torch.zeros(1, dtype=torch.int64, device="cuda")
    paged = torch.zeros(1, dtype=torch.int64, device="cuda")
    sel = torch.full((B, 4, mp + 1), -7, dtype=torch.int32, device="cuda")
    L.wc_gate_pagein(sc.cache, sc.layer, torch.from_numpy(out["logrisk"]).cuda(),
                     torch.from_numpy(out["lse"]).cuda(), sc.dev["tab"], sc.dev["ctx"], tau, host, pool_used, paged,
                     ws, selected=sel, meter=None if meter is None else torch.from_numpy(meter).cuda())
    torch.cuda.synchronize()
    return sel.cpu().numpy(), int(pool_used.item()), int(paged.item())


@pytest.mark.parametrize("scheme,mask,tier", [("fp8", 1, "R_A"), ("int8", 3, "R_B")])
def test_meter_fast_path_same_decisions(scheme, mask, tier):
    """With the merged meter given, quiet (sequence, KV head) pairs skip the
    block pass; every decision, pool slot and page-in count must equal the
    exact pass's, at thresholds where all, some and no pairs trigger."""
    lens = [300, 1000, 64, 700, 17]
    L, sc0, _ = _setup(lens, seed=31, scheme=scheme)
    out0 = sc0.decode(n_split=4, mask=mask, risk=True)
    R = out0[tier]
    per_pair = R.reshape(len(lens), 4, 7).max(axis=2)
    taus = [float(np.min(per_pair)) * 0.5, float(np.median(per_pair)), float(np.max(per_pair)) * 1.5]
    mixed = None
    for tau in taus:
        print(f"gate fast path {scheme} tau={tau:.4g}", flush=True)
        got = []
        for meter in (None, R):
            L, sc, host = _setup(lens, seed=31, scheme=scheme)
            out = sc.decode(n_split=4, mask=mask, risk=True)
            assert np.array_equal(out[tier], R)
            got.append(_gate_meter(L, sc, host, out, tau, meter))
        (s0, u0, p0), (s1, u1, p1) = got
        assert u0 == u1 and p0 == p1, (tau, u0, u1)
        for b in range(len(lens)):
            for g in range(4):
                n = s0[b, g, 0]
                assert s1[b, g, 0] == n, (tau, b, g)
                assert np.array_equal(s0[b, g, 1:1 + n], s1[b, g, 1:1 + n]), (tau, b, g)
        if tau == taus[1]:
            mixed = s0[:, :, 0]
    # the middle threshold leaves some pairs quiet and triggers others
    assert np.any(mixed > 0) and np.any(mixed == 0), mixed


# ---------------------------------------------------------------- persistent repair across appends
def _decode_flow(L, cache, layer, q_d, tab_d, ctx, seeds_d, mask, risk, mp, n_split=4):
    B, Hq = q_d.shape[0], q_d.shape[1]
    ctx_d = torch.from_numpy(np.asarray(ctx, dtype=np.int32)).cuda()
    part = torch.empty(L.wc_decode_workspace_bytes(B, Hq, n_split) // 4, device="cuda")
    br = torch.full((B, Hq, mp), float("nan"), device="cuda") if risk else None
    L.wc_decode_attn_meter(cache, layer, q_d, tab_d, ctx_d, seeds_d, part, H.SM, mask, 1e-2, 28, 28, 256, n_split,
                           block_logrisk=br)
    o = torch.empty((B, Hq, 128), device="cuda")
    lse = torch.empty((B, Hq), device="cuda")
    ra, rb = torch.empty((B, Hq), device="cuda"), torch.empty((B, Hq), device="cuda")
    L.wc_lse_merge(part, B, Hq, n_split, o, lse, ra, rb)
    torch.cuda.synchronize()
    return ctx_d, br, o, lse, ra, rb


@pytest.mark.parametrize("scheme,tau", [("fp8", 0.0), ("int8", 0.0), ("int8", 0.02)])
def test_repair_persists_across_appends(scheme, tau):
    """Gate a ragged batch whose last pages are partly filled, with a host
    store that holds only the tokens written so far (every other row of it
    holds unrelated keys), then append 1-17 tokens per sequence in two calls
    and decode: the appended tokens that land in repaired blocks must be
    decoded with their exact keys and c = 0 (their pool rows written by the
    write path, their witnesses 0), the others from the quantized cache."""
    L = H.need_gpu()
    print(f"repair across appends {scheme} tau={tau}", flush=True)
    lens0 = np.array([300, 1000, 64, 700, 17, 33])
    adds = np.array([1, 17, 5, 4, 15, 16])
    full = lens0 + adds
    B, G, layer = len(full), 7, 1
    offs = np.concatenate([[0], np.cumsum(full)])
    d = inputs.layer(seed=71, S=int(full.sum()), Hq=28, Hkv=4, outliers=2)
    q = inputs.layer(seed=72, S=1, batch=B)["q"]
    tab, npages = inputs.page_table(71, full, extra_pages=3)
    seeds = inputs.seeds(B, base=1071)
    sch = L.WC_FP8_E4M3 if scheme == "fp8" else L.WC_DITHER_INT8
    mask = 1 if scheme == "fp8" else 3
    cache = L.KVCache(sch, 2, npages, 4, pool_capacity=npages * 4)

    def write(t0s, t1s):
        rows, slot, pos, sd = [], [], [], []
        for b in range(B):
            t = np.arange(t0s[b], t1s[b])
            rows.append(offs[b] + t)
            slot.append(tab[b, t // 16].astype(np.int64) * 16 + t % 16)
            pos.append(t.astype(np.int32))
            sd.append(np.full(len(t), seeds[b]))
        rows = np.concatenate(rows)
        L.wc_write_kv(cache, H.dev_tensor(d["k"][rows], "bf16"), H.dev_tensor(d["v"][rows], "bf16"),
                      torch.from_numpy(np.concatenate(slot)).cuda(), torch.from_numpy(np.concatenate(pos)).cuda(),
                      torch.from_numpy(np.concatenate(sd).astype(np.uint64).view(np.int64)).cuda(), layer0=layer)

    write(np.zeros(B, int), lens0)
    rng = np.random.default_rng(5)
    store = inputs.f32_to_bf16_bits(rng.standard_normal((2, npages, 4, 16, 128)).astype(np.float32) * 3)
    for b in range(B):
        t = np.arange(lens0[b])
        store[layer, tab[b, t // 16], :, t % 16] = d["k"][offs[b] + t]
    host = torch.from_numpy(store.view(np.int16)).pin_memory()
    q_d = H.dev_tensor(q, "bf16")
    tab_d = torch.from_numpy(tab).cuda()
    seeds_d = torch.from_numpy(seeds.view(np.int64)).cuda()
    mp = tab.shape[1]
    ctx_d, br, _, lse, ra, rb = _decode_flow(L, cache, layer, q_d, tab_d, lens0, seeds_d, mask, True, mp)
    ws = torch.empty(L.wc_gate_workspace_bytes(B, 4, mp), dtype=torch.uint8, device="cuda")
    pool_used = torch.zeros(1, dtype=torch.int64, device="cuda")
    paged = torch.zeros(1, dtype=torch.int64, device="cuda")
    L.wc_gate_pagein(cache, layer, br, lse, tab_d, ctx_d, tau, host, pool_used, paged, ws)
    torch.cuda.synchronize()
    slots = cache.exact_slot.cpu().numpy()[layer]
    partial_rep = [(b, g) for b in range(B) for g in range(4)
                   if lens0[b] % 16 and slots[tab[b, (lens0[b] - 1) // 16], g] >= 0]
    assert partial_rep, "no partially filled page was repaired"
    # append in two calls (the first token, then the rest)
    write(lens0, lens0 + 1)
    write(lens0 + 1, full)
    _, _, o, lse2, ra2, rb2 = _decode_flow(L, cache, layer, q_d, tab_d, full, seeds_d, mask, False, mp)
    o, ra2, rb2 = o.cpu().numpy(), ra2.cpu().numpy(), rb2.cpu().numpy()
    pool = _pool_bits(cache)
    wit = cache.witness.cpu().numpy()[layer]
    n_app_rep = 0
    for b in range(B):
        t = np.arange(full[b])
        for g in range(4):
            rep = slots[tab[b, t // 16], g] >= 0
            # appended tokens in repaired blocks: exact key in the pool, witness 0
            for tt in range(lens0[b], full[b]):
                s = slots[tab[b, tt // 16], g]
                if s >= 0:
                    n_app_rep += 1
                    assert np.array_equal(pool[s, tt % 16], d["k"][offs[b] + tt, g]), (b, g, tt)
                    assert np.all(wit[tab[b, tt // 16], g, tt % 16] == 0)
            k32 = H.to_f32(d["k"][offs[b]:offs[b + 1], g], "bf16")
            v32 = H.to_f32(d["v"][offs[b]:offs[b + 1], g], "bf16")
            qg = H.to_f32(q[b, g * G:(g + 1) * G], "bf16").astype(np.float64)
            S = int(full[b])
            if scheme == "int8":
                oc = H.oracle_int8_cache(k32, v32, int(seeds[b]), layer, g, S)
                lt = math.log(2 * S / meter.delta_loc(1e-2, 28, 28, 256))
                r = meter.decode_group(qg, k32, oc["khat"], v32, oc["vhat"], oc["w"], H.SM, k_scale=oc["sk"],
                                       log_term=lt, repaired=rep)
            else:
                oc = H.oracle_fp8_cache(k32, v32)
                r = meter.decode_group(qg, k32, oc["khat"], v32, oc["vhat"], oc["w"], H.SM, repaired=rep)
            hs = slice(g * G, (g + 1) * G)
            assert np.all(H.rel_l2(o[b, hs], r["o_tilde"]) <= 2e-3), (b, g)
            assert np.all(np.abs(ra2[b, hs] - r["R_A"]) <= 1e-4 * r["R_A"] + 1e-30), (b, g)
            assert np.all(ra2[b, hs] >= r["tv_true"]), (b, g)
            if scheme == "int8":
                assert np.all(np.abs(rb2[b, hs] - r["R_B"]) <= 1e-4 * r["R_B"] + 1e-30), (b, g)
    print(f"  {len(partial_rep)} partial pages repaired, {n_app_rep} appended (token, head) rows in repaired blocks",
          flush=True)
    assert n_app_rep > 0


# ---------------------------------------------------------------- decisions from independent risks
def _divergence_explained(fx_o, got, want, T, band=1e-4, rank_band=2e-4):
    """Whether the first place where the kernel's selection `got` and the
    oracle's `want` (both from oracle.gate.select's rule, on the kernel's fp32
    and the oracle's float64 risks) part is a near tie of the oracle's own
    numbers: a remaining sum within `band` of the threshold where one stops
    and the other goes on, or two blocks whose ranking risks are within
    `rank_band` of each other."""
    rho = [[int(x) for x in row] for row in fx_o]
    X = [sum(row) for row in rho]
    k = 0
    while k < min(len(got), len(want)) and got[k] == want[k]:
        k += 1
    if k < min(len(got), len(want)):                  # different blocks at rank k
        kg = max(rho[h][got[k]] for h in range(len(rho)))
        kw = max(rho[h][want[k]] for h in range(len(rho)))
        return abs(kg - kw) <= rank_band * max(kg, kw) + 2
    rem = [X[h] - sum(rho[h][j] for j in want[:k]) for h in range(len(rho))]
    return any(abs(r - T) <= band * max(T, X[h]) + 2 for h, r in enumerate(rem))


@pytest.mark.parametrize("scheme", ["fp8", "int8"])
def test_gate_decisions_from_independent_risks(scheme):
    """End to end: the oracle's selection on its own float64 block risks
    against the kernel's.  Decisions may part only at near ties of the fixed
    point sums (|X - T| within 1e-4 T) or of the ranking risks; the count of
    (sequence, KV head) pairs where they part is reported."""
    lens = [300, 1000, 64, 700, 17, 2000, 513, 129]
    mask = 1 if scheme == "fp8" else 3
    total = parted = 0
    for tau in (0.02, 0.05, 0.2, 1.0):
        L, sc, host = _setup(lens, seed=81, scheme=scheme)
        print(f"independent risks {scheme} tau={tau}", flush=True)
        out, sel, rho, used, paged = _gate(L, sc, host, tau, mask=mask)
        T = gate.threshold_fx(tau)
        for b, S in enumerate(lens):
            P = -(-S // 16)
            for g in range(4):
                _, r = sc.oracle(b, g)
                fx_o = gate.rho_to_fx(r["block_risk"])
                want = gate.select(fx_o, np.zeros(P, bool), T)
                got = [int(x) for x in sel[b, g, 1:1 + sel[b, g, 0]]]
                total += 1
                if got != want:
                    parted += 1
                    assert _divergence_explained(fx_o, got, want, T), (tau, b, g, got[:8], want[:8])
    print(f"  {scheme}: decisions part on {parted} of {total} (sequence, KV head, tau) cases", flush=True)
    assert parted <= total // 10

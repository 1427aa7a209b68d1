"""GPU parity of the gate: fixed-point risks, bit-exact block selection,
page-in from pinned host memory, witness zeroing, and decode on the
repaired cache."""
import numpy as np
import pytest
import torch

from certified_kv_cache_amd import inputs
from oracle import gate
from tests import helpers as H
from tests.scenario import Scenario

pytestmark = pytest.mark.gpu


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
            # (2e-4 relative, plus one unit of the 2^-40 grid: the ceiling of
            # the fp32 risk and that of the float64 one can differ by a step)
            ref = gate.rho_to_fx(r["block_risk"]).astype(np.float64)
            dev = np.abs(fx.astype(np.float64) - ref)
            assert np.all(dev <= 2e-4 * ref + 1), (b, g, (dev - 1).max())
    assert used == total and paged == 4096 * total
    # repaired blocks: exact keys in the pool, witness zeroed, slot recorded
    slots = sc.cache.exact_slot.cpu().numpy()[sc.layer]
    pool = sc.cache.exact_pool.cpu().numpy().astype(np.float64)
    scale = sc.cache.exact_scale.cpu().numpy().astype(np.float64)
    wit = sc.cache.witness.cpu().numpy()[sc.layer]
    store = host.numpy().view(np.uint16)[sc.layer]
    for b in range(len(lens)):
        for g in range(4):
            for j in sel[b, g, 1:1 + sel[b, g, 0]]:
                p = sc.tab[b, j]
                s = slots[p, g]
                assert s >= 0
                exact = inputs.bf16_bits_to_f32(store[p, g]).astype(np.float64)
                assert np.array_equal(pool[s] * scale[s][:, None], exact)
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


def test_gate_at_the_sort_capacity():
    """One sequence of 65536 tokens: 4096 pages, the most blocks the selection
    ranks in one workgroup.  Decisions bit-exact, risks within 2e-4 relative
    plus one unit of the 2^-40 grid."""
    lens = [65536]
    L, sc, host = _setup(lens, seed=41, capacity=16384)
    assert sc.tab.shape[1] == 4096
    print("gate at 4096 pages", flush=True)
    rep0 = sc.cache.exact_slot.cpu().numpy()[sc.layer].copy()
    out, sel, rho, used, paged = _gate(L, sc, host, 0.2)
    T = gate.threshold_fx(0.2)
    total = 0
    for g in range(4):
        fx = rho[0, g * 7:(g + 1) * 7, :4096]
        want = gate.select(fx, rep0[sc.tab[0], g] >= 0, T)
        got = list(sel[0, g, 1:1 + sel[0, g, 0]])
        assert got == want, g
        total += len(want)
        _, r = sc.oracle(0, g)
        ref = gate.rho_to_fx(r["block_risk"]).astype(np.float64)
        dev = np.abs(fx.astype(np.float64) - ref)
        assert np.all(dev <= 2e-4 * ref + 1), (g, (dev - 1).max())
    assert used == total and paged == 4096 * total
    print(f"selected {total} blocks", flush=True)
    # the tanh gate ranks the same 4096 pages (a fresh cache of the same input)
    L, sc, host = _setup(lens, seed=41, capacity=16384)
    out = sc.decode(n_split=4, mask=1, cmax=True)
    cm = out["cmax"]
    tau = float(np.median(out["T_A"]))
    rep0 = sc.cache.exact_slot.cpu().numpy()[sc.layer].copy()
    sel, used, paged = _tanh_gate(L, sc, host, cm, tau)
    total = 0
    for g in range(4):
        want = gate.select_tanh(cm[0, g * 7:(g + 1) * 7, :4096], rep0[sc.tab[0], g] >= 0, tau)
        assert list(sel[0, g, 1:1 + sel[0, g, 0]]) == want, g
        total += len(want)
    assert used == total and paged == 4096 * total
    print(f"tanh gate selected {total} blocks", flush=True)


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

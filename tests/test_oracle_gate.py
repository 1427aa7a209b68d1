"""Pins of the oracle's gate: invariants the pages fix for meter-driven repair
(nothing repaired above threshold, full repair removes all risk, a lower
threshold repairs a superset, the repaired state meets the threshold)."""
import math

import numpy as np

from oracle import gate, meter


def _risks(G=7, P=40, seed=0):
    rng = np.random.default_rng(seed)
    base = rng.exponential(1.0, P) * rng.uniform(0, 1, P) ** 4
    rho = base[None, :] * rng.uniform(0.5, 1.5, (G, P)) * 0.05
    return rho


def test_threshold_matches_meter_form():
    for tau in [0.0, 0.05, 0.2, 1.0, 7.5]:
        E = gate.e_tau(tau)
        assert abs(E * (1 + E / 2) - tau) < 1e-12
        T = gate.threshold_fx(tau)
        assert T <= E * 2 ** 40 < T + 1


def test_fixed_point_rounds_up_and_caps():
    fx = gate.rho_to_fx(np.array([0.0, 2.0 ** -40, 1e-9, 1.0, 1e9, np.inf]))
    assert fx[0] == 0 and fx[1] == 1 and fx[2] == math.ceil(1e-9 * 2 ** 40)
    assert fx[3] == 2 ** 40 and fx[4] == gate.FX_CAP and fx[5] == gate.FX_CAP


def test_infinite_tau_selects_nothing():
    rho = gate.rho_to_fx(_risks())
    assert gate.select(rho, np.zeros(40, bool), 1 << 62) == []


def test_prefix_property_and_post_repair_condition():
    rho = gate.rho_to_fx(_risks(seed=1))
    rep = np.zeros(40, bool)
    prev = None
    for tau in [5.0, 1.0, 0.2, 0.05, 0.01, 0.0]:
        T = gate.threshold_fx(tau)
        sel = gate.select(rho, rep, T)
        rem = rho.astype(object).sum(axis=1) - rho[:, sel].astype(object).sum(axis=1) if sel else rho.astype(object).sum(axis=1)
        assert all(r <= T for r in rem)
        # shortest prefix: dropping the last block breaks the condition
        if sel:
            rem2 = rem + rho[:, sel[-1]].astype(object)
            assert any(r > T for r in rem2)
        if prev is not None:
            assert set(prev) <= set(sel) and sel[:len(prev)] == prev
        prev = sel


def test_rank_order_and_ties():
    rho = np.zeros((2, 6), dtype=np.uint64)
    rho[0] = [5, 9, 9, 1, 0, 3]
    rho[1] = [6, 2, 9, 1, 0, 3]
    sel = gate.select(rho, np.zeros(6, bool), 0)
    assert sel == [1, 2, 0, 5, 3]


def test_repaired_blocks_skipped_and_budget():
    rho = gate.rho_to_fx(_risks(seed=2))
    rep = np.zeros(40, bool)
    full = gate.select(rho, rep, 0)
    rep[full[0]] = True
    rho2 = rho.copy()
    rho2[:, full[0]] = 0
    sel = gate.select(rho2, rep, 0)
    assert full[0] not in sel
    assert gate.select(rho, np.zeros(40, bool), 0, budget=3) == full[:3]


def test_full_repair_zeroes_meter():
    # End to end on the oracle: repairing every selected block at tau = 0
    # leaves zero risk, hence R = 0 on the repaired cache.
    from oracle import dither, quant
    rng = np.random.default_rng(3)
    S = 96
    k = rng.standard_normal((S, 128)).astype(np.float32)
    v = rng.standard_normal((S, 128)).astype(np.float32)
    code, val = quant.fp8_e4m3(k)
    w = quant.witness(k, val)
    q = rng.standard_normal((7, 128))
    sm = 1 / math.sqrt(128)
    out = meter.decode_group(q, k, val, v, v, w, sm)
    rho = gate.rho_to_fx(out["block_risk"])
    sel = gate.select(rho, np.zeros(6, bool), 0)
    rep = np.zeros(S, bool)
    for j in sel:
        rep[16 * j:16 * j + 16] = True
    out2 = meter.decode_group(q, k, val, v, v, w, sm, repaired=rep)
    assert np.all(out2["R_A"] == 0) and np.all(out2["tv_true"] < 1e-15)

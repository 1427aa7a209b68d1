"""Pins of the oracle's deterministic tanh bound and of the tanh gate."""
import math

import numpy as np
import pytest

from oracle import gate, meter


def test_two_token_supremum_is_tanh_of_half_bound():
    # Two tokens, |eps_t| <= c: TV = |p1 - p~1| is largest when the two
    # logits move by +c and -c and p1 = 1 / (1 + e^c); its value tanh(c/2)
    # is found here by brute force over the logit gap, independently of
    # meter.tanh_bound.
    for c in (0.01, 0.3, 1.0, 3.0):
        gaps = np.linspace(-12, 12, 240001)
        p1 = 1 / (1 + np.exp(-gaps))
        q1 = 1 / (1 + np.exp(-(gaps + 2 * c)))
        best = np.max(np.abs(q1 - p1))
        assert abs(best - meter.tanh_bound(np.array([c, c]))) < 1e-9
        assert best <= math.tanh(c / 2) + 1e-15


def test_tanh_bound_sound_on_random_perturbations():
    rng = np.random.default_rng(20)
    for _ in range(400):
        S = int(rng.integers(1, 12))
        lt = rng.standard_normal(S) * rng.uniform(0.1, 5)
        c = rng.uniform(0, 2, S) * (rng.uniform(size=S) < 0.7)
        pt = meter.softmax(lt)
        T = meter.tanh_bound(c)
        for _ in range(10):
            sgn = rng.choice([-1.0, 1.0], S)
            dl = sgn * c if rng.uniform() < 0.5 else rng.uniform(-1, 1, S) * c
            assert meter.tv(meter.softmax(lt + dl), pt) <= T + 1e-12


def test_tanh_bound_closed_forms_and_comparison_with_certificate():
    pt = meter.softmax(np.random.default_rng(21).standard_normal(50))
    assert meter.tanh_bound(np.zeros(50)) == 0.0
    assert meter.tanh_bound(np.zeros(0)) == 0.0
    x = 0.4
    assert abs(meter.tanh_bound(np.full(50, x)) - math.tanh(x / 2)) < 1e-15
    # a uniform bound: the certificate (e^{2x} - 1)/2 is the looser one;
    # a bound on one unlikely token only: the certificate is far tighter
    _, R, _ = meter.meter_from(pt, np.full(50, x))
    assert R > meter.tanh_bound(np.full(50, x))
    c = np.zeros(50)
    j = int(np.argmin(pt))
    c[j] = 3.0
    _, R1, _ = meter.meter_from(pt, c)
    assert abs(R1 - (pt[j] * math.expm1(3.0)) * (1 + pt[j] * math.expm1(3.0) / 2)) < 1e-15
    assert R1 < 0.1 * meter.tanh_bound(c)


@pytest.mark.parametrize("n_split", [1, 3, 8])
def test_split_merge_tanh_invariance(n_split):
    rng = np.random.default_rng(22)
    S, G = 100, 3
    q = rng.standard_normal((G, 128))
    kh = rng.standard_normal((S, 128))
    vh = rng.standard_normal((S, 128))
    ca = rng.uniform(0, 0.5, (G, S))
    cb = rng.uniform(0, 0.2, (G, S))
    res = meter.lse_merge(meter.split_partials(q, kh, vh, ca, cb, 0.1, n_split))
    assert np.allclose(res["T_A"], np.tanh(0.5 * ca.max(-1)), rtol=0, atol=1e-15)
    assert np.allclose(res["T_B"], np.tanh(0.5 * cb.max(-1)), rtol=0, atol=1e-15)


def test_tanh_gate_brings_every_head_under_tau_with_no_extra_block():
    rng = np.random.default_rng(23)
    for _ in range(200):
        G, P = int(rng.integers(1, 8)), int(rng.integers(1, 40))
        cmax = (rng.exponential(0.3, (G, P)) * (rng.uniform(size=(G, P)) < 0.8)).astype(np.float32)
        rep = rng.uniform(size=P) < 0.2
        tau = float(rng.choice([0.0, 0.05, 0.2, 0.6, 1.0, 3.0]))
        sel = gate.select_tanh(cmax, rep, tau)
        done = rep.copy()
        done[sel] = True
        left = np.where(done[None, :], 0.0, cmax.astype(np.float64))
        # every head's tanh bound over the unrepaired blocks is at most tau
        # (up to the float32 rounding of the threshold)
        assert np.all(np.tanh(0.5 * left.max(-1, initial=0.0)) <= tau * (1 + 1e-6) + 1e-12)
        # and every repaired block was needed: some head's bound there exceeded tau
        for j in sel:
            assert not rep[j] and math.tanh(0.5 * float(cmax[:, j].max())) > tau * (1 - 1e-6)
        # rank order: descending block maximum, ties to the lower block
        keys = [(-float(cmax[:, j].max()), j) for j in sel]
        assert keys == sorted(keys)
        if tau >= 1.0:
            assert sel == []
    # budget caps the ranking
    cmax = np.array([[0.5, 2.0, 1.0, 2.0]], dtype=np.float32)
    assert gate.select_tanh(cmax, np.zeros(4, bool), 0.0) == [1, 3, 2, 0]
    assert gate.select_tanh(cmax, np.zeros(4, bool), 0.0, budget=2) == [1, 3]

"""Pins of the oracle's outlier bypass: channel selection, the bypassed
quantizer, and Tier B with the bypassed channels removed."""
import math

import numpy as np
import pytest

from oracle import dither, meter, outlier, quant
from certified_kv_cache_amd import inputs

SM = 1.0 / math.sqrt(128)


def _bf16_exact(x):
    """float32 values rounded to bf16 and back."""
    return inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def test_planted_outlier_channels_are_selected():
    # Channels scaled x20 carry ~400x the energy of the others: the selection
    # must return exactly the planted set, whatever m is up to its size.
    rng = np.random.default_rng(0)
    x = rng.standard_normal((512, 128)).astype(np.float32)
    planted = np.array([3, 17, 40, 64, 77, 90, 101, 127])
    gains = np.linspace(20, 27, planted.size)
    x[:, planted] *= gains
    x = _bf16_exact(x)
    np.testing.assert_array_equal(outlier.top_energy_channels(x, 8), planted)
    # the 4 largest gains are the last 4 planted channels
    np.testing.assert_array_equal(outlier.top_energy_channels(x, 4), planted[4:])
    assert outlier.top_energy_channels(x, 0).size == 0


def test_energy_exact_on_small_integers():
    # Small integers: every square and partial sum is exact in float32, so the
    # token-order float32 sum equals the integer sum of squares.
    rng = np.random.default_rng(1)
    xi = rng.integers(-30, 31, size=(300, 128))
    e = outlier.channel_energy(xi.astype(np.float32))
    np.testing.assert_array_equal(e.astype(np.int64), (xi ** 2).sum(0))


def test_energy_is_float32_in_token_order():
    # One large term first, then many small ones: a token-order float32 sum
    # absorbs each small square (below half an ulp of 2^24) and stays at 2^24;
    # an exact or pairwise sum would not.
    x = np.zeros((1 + 1000, 1), dtype=np.float32)
    x[0, 0] = np.float32(4096.0)                # square 2^24
    x[1:, 0] = np.float32(1.0)                  # squares 1 = half an ulp at 2^24: ties to even
    assert outlier.channel_energy(x)[0] == np.float32(2 ** 24)


def test_ties_go_to_the_lower_channel():
    rng = np.random.default_rng(2)
    col = rng.standard_normal(64).astype(np.float32)
    x = np.tile(col[:, None], (1, 128))         # every channel has the same energy
    np.testing.assert_array_equal(outlier.top_energy_channels(x, 8), np.arange(8))
    x[:, 100] *= 2
    np.testing.assert_array_equal(outlier.top_energy_channels(x, 8), np.r_[np.arange(7), 100])


def test_selection_agrees_with_float64_when_gaps_are_wide():
    # Brute force against float64 energies on inputs whose top-m gap exceeds
    # any float32 accumulation error.
    rng = np.random.default_rng(3)
    checked = 0
    for trial in range(20):
        x = rng.standard_normal((256, 128)).astype(np.float32) * rng.uniform(0.5, 3, 128).astype(np.float32)
        x = _bf16_exact(x)
        e64 = (x.astype(np.float64) ** 2).sum(0)
        srt = np.sort(e64)[::-1]
        m = 8
        if srt[m - 1] - srt[m] < 1e-3 * srt[0]:
            continue
        ref = np.sort(np.argsort(-e64, kind="stable")[:m])
        np.testing.assert_array_equal(outlier.top_energy_channels(x, m), ref)
        checked += 1
    assert checked >= 5


def test_bypass_with_no_channels_is_the_plain_quantizer():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    xi = dither.dither_rows(7, 0, 0, np.arange(64))
    c0, s0, i0 = quant.dither_int8(x, xi)
    c1, s1, i1, side = outlier.dither_int8_bypass(x, xi, [])
    np.testing.assert_array_equal(c0, c1)
    np.testing.assert_array_equal(s0, s1)
    assert side.shape == (64, 0)


def test_bypass_scale_ignores_outliers_and_reconstruction_is_exact_on_them():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((200, 128)).astype(np.float32)
    O = np.array([5, 6, 70, 71, 100, 101, 120, 127])
    x[:, O] *= 1000.0                          # would dominate the absmax without the bypass
    x = _bf16_exact(x)
    xi = dither.dither_rows(8, 2, 1, np.arange(200))
    code, s, inv, side = outlier.dither_int8_bypass(x, xi, O)
    keep = np.setdiff1d(np.arange(128), O)
    am = np.max(np.abs(x[:, keep]), axis=1)
    np.testing.assert_array_equal(s, (am / np.float32(127)).astype(np.float32))
    assert np.all(code[:, O] == 0)
    khat = outlier.dequant_bypass(code, s, xi, side, O)
    np.testing.assert_array_equal(khat[:, O], x[:, O].astype(np.float64))
    err = np.abs(khat[:, keep] - x[:, keep])
    assert np.all(err <= s[:, None] * (0.5 + 1e-5))
    w = quant.witness(x, khat)
    # the witness of the bypassed cache is far below that of the plain one
    cp, sp, _ = quant.dither_int8(x, xi)
    wp = quant.witness(x, quant.dequant_dither_int8(cp, sp, xi))
    assert np.median(w.sum(1) / wp.sum(1)) < 0.01


def test_tier_b_variance_with_bypass_by_monte_carlo():
    # With O exact, eps_t = sm q . r_t sums independent uniform residuals over
    # the channels off O only: Var = sm^2 s_t^2 sum_{c not in O} q_c^2 / 12.
    # The query is large on O, so keeping those channels in the proxy fails.
    rng = np.random.default_rng(6)
    S, R = 6, 1200
    k = _bf16_exact(rng.standard_normal((S, 128)).astype(np.float32))
    O = np.array([1, 9, 33, 65, 73, 97, 110, 126])
    q = rng.standard_normal((2, 128))
    q[:, O] *= 10.0
    errs, s = [], None
    for seed in range(R):
        xi = dither.dither_rows(90_000 + seed, 0, 0, np.arange(S))
        code, s, _, side = outlier.dither_int8_bypass(k, xi, O)
        khat = outlier.dequant_bypass(code, s, xi, side, O)
        errs.append(SM * q @ (khat - k).T)
    errs = np.array(errs)
    var = meter.tier_b_sigma2(q, s, SM, bypass=O)
    ratio = errs.var(axis=0) / var
    assert np.all(np.abs(ratio - 1) < 5 * math.sqrt(2 / R))
    full = meter.tier_b_sigma2(q, s, SM)
    assert np.all(full > 3 * var)


def test_bypass_meter_sound_and_tighter_on_outlier_keys():
    # The layer workload's keys (x20 outlier channels): with the bypass over
    # the top-8 energy channels both tiers stay above the true TV and Tier B
    # shrinks well below the plain cache's.
    lay = inputs.layer(11, S=1024)
    k32 = inputs.bf16_bits_to_f32(lay["k"])[:, 0]
    v32 = inputs.bf16_bits_to_f32(lay["v"])[:, 0]
    qf = inputs.bf16_bits_to_f32(lay["q"])[0, :7].astype(np.float64)
    S = k32.shape[0]
    O = outlier.top_energy_channels(k32, 8)
    xi = dither.dither_rows(21, 0, 0, np.arange(S))
    lt = math.log(2 * S / meter.delta_loc(1e-2, 28, 28, 256))
    code, s, _, side = outlier.dither_int8_bypass(k32, xi, O)
    khat = outlier.dequant_bypass(code, s, xi, side, O)
    cv, sv, _ = quant.dither_int8(v32, xi)
    vhat = quant.dequant_dither_int8(cv, sv, xi)
    res = meter.decode_group(qf, k32, khat, v32, vhat, quant.witness(k32, khat), SM, k_scale=s, log_term=lt,
                             bypass=O)
    assert np.all(res["R_A"] >= res["tv_true"])
    assert np.all(res["R_B"] >= res["tv_true"])
    cp, sp, _ = quant.dither_int8(k32, xi)
    kp = quant.dequant_dither_int8(cp, sp, xi)
    plain = meter.decode_group(qf, k32, kp, v32, vhat, quant.witness(k32, kp), SM, k_scale=sp, log_term=lt)
    assert np.all(res["R_B"] < 0.2 * plain["R_B"])

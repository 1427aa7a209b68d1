"""Pins of the oracle's value-side certificate E_V = sum_t p~_t ||v^_t - v_t||
and of the joint output bound it gives with the key side's TV."""
import math

import numpy as np
import pytest

from oracle import dither, meter, quant

SM = 1.0 / math.sqrt(128)


def _quantized(S, seed, scheme):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((S, 128)).astype(np.float32)
    v = (rng.standard_normal((S, 128)) * rng.uniform(0.2, 3, (S, 1))).astype(np.float32)
    if scheme == "dither":
        xi = dither.dither_rows(seed, 0, 0, np.arange(S))
        ck, sk, _ = quant.dither_int8(k, xi)
        cv, sv, _ = quant.dither_int8(v, xi)
        kh, vh = quant.dequant_dither_int8(ck, sk, xi), quant.dequant_dither_int8(cv, sv, xi)
    elif scheme == "rtn":
        ck, sk, _ = quant.rtn_int8(k)
        cv, sv, _ = quant.rtn_int8(v)
        kh, vh = quant.dequant_rtn_int8(ck, sk), quant.dequant_rtn_int8(cv, sv)
    else:
        _, kh = quant.fp8_e4m3(k)
        _, vh = quant.fp8_e4m3(v)
    return k, v, kh, vh


@pytest.mark.parametrize("scheme", ["dither", "rtn", "fp8"])
def test_v_certificate_bounds_the_value_error_and_the_output(scheme):
    k, v, kh, vh = _quantized(300, 40, scheme)
    q = np.random.default_rng(41).standard_normal((5, 128)) * 2
    w = quant.witness(k, kh)
    wv = quant.witness_v(v, vh)
    out = meter.decode_group(q, k, kh, v, vh, w, SM, wv=wv)
    # the value part of the output error, computed directly
    pt = out["p_tilde"]
    dv = np.linalg.norm(pt @ (vh.astype(np.float64) - v), axis=-1)
    assert np.allclose(dv, out["dv_true"], rtol=1e-12)
    assert np.all(dv <= out["E_V"] * (1 + 1e-12))
    # joint: the whole output error is within E_V + 2 TV max ||v||, also with
    # the Tier A meter in place of the true TV
    err = np.linalg.norm(out["o_tilde"] - out["o_exact"], axis=-1)
    vmax = np.max(np.linalg.norm(v.astype(np.float64), axis=-1))
    assert np.all(err <= out["E_V"] + 2 * out["tv_true"] * vmax + 1e-12)
    assert np.all(err <= out["E_V"] + 2 * np.minimum(1, out["R_A"]) * vmax + 1e-12)


def test_v_certificate_equality_and_zero_cases():
    rng = np.random.default_rng(42)
    S = 50
    v = rng.standard_normal((S, 128))
    u = rng.standard_normal(128)
    u /= np.linalg.norm(u)
    alpha = rng.uniform(0, 0.3, S)
    vh = v + alpha[:, None] * u[None, :]               # parallel residuals: the triangle inequality is tight
    pt = meter.softmax(rng.standard_normal((3, S)))
    E = meter.v_certificate(pt, quant.witness_v(v, vh))
    assert np.allclose(E, np.linalg.norm(pt @ (vh - v), axis=-1), rtol=1e-12)
    assert np.allclose(E, pt @ alpha, rtol=1e-12)
    assert np.all(meter.v_certificate(pt, quant.witness_v(v, v)) == 0)
    # the witness is the Euclidean norm of the residual
    assert np.allclose(quant.witness_v(v, vh), alpha, rtol=1e-12)


@pytest.mark.parametrize("n_split", [1, 4, 9])
def test_v_certificate_split_merge_invariance(n_split):
    rng = np.random.default_rng(43)
    S, G = 200, 3
    q = rng.standard_normal((G, 128))
    kh = rng.standard_normal((S, 128))
    vh = rng.standard_normal((S, 128))
    wv = rng.uniform(0, 1, S)
    ca = np.zeros((G, S))
    res = meter.lse_merge(meter.split_partials(q, kh, vh, ca, ca, 0.1, n_split, wv=wv))
    pt = meter.softmax(0.1 * q @ kh.T)
    assert np.allclose(res["E_V"], pt @ wv, rtol=1e-12)

"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Bars: codes, dither draws and gate decisions bit-exact; witness, meters and
block risks within 1e-4 relative; attention output within 2e-3 relative L2;
and the GPU meter never below the oracle's true TV.
"""
import math

import numpy as np
import pytest
import torch

from certified_kv_cache_amd import inputs
from oracle import dither, quant
from tests import helpers as H
from tests.scenario import Scenario

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-3
MET_TOL = 1e-4


def _flush(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------- dither
def test_dither_fill_bit_exact():
    L = H.need_gpu()
    for seed, layer, head, pos0, n in [(1, 0, 0, 0, 300), (2 ** 40 + 77, 27, 3, 12345, 257), (9, 5, 1, 2 ** 25, 64)]:
        out = torch.empty((n, 128), dtype=torch.int16, device="cuda")
        L.wc_dither_fill(seed, layer, head, pos0, n, out)
        got = out.cpu().numpy().view(np.uint16)
        want = dither.dither_k16(seed, layer, head, np.arange(pos0, pos0 + n)[:, None], np.arange(128)[None, :])
        assert np.array_equal(got, want)


# ---------------------------------------------------------------- write path
def _ragged_layer(seed, lens, Hkv=4, dtype="bf16", outliers=2):
    n = int(sum(lens))
    d = inputs.layer(seed=seed, S=max(n, 1), Hq=Hkv * 7, Hkv=Hkv, outliers=outliers)
    q = inputs.layer(seed=seed + 100, S=1, Hq=Hkv * 7, Hkv=Hkv, batch=len(lens))["q"]
    return d["k"][:n], d["v"][:n], q


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("scheme", ["int8", "fp8"])
def test_write_codes_bit_exact_and_witness(scheme, dtype):
    L = H.need_gpu()
    _flush(f"write {scheme} {dtype}")
    lens = [37, 16, 130]
    if dtype == "bf16":
        k, v, q = _ragged_layer(3, lens)
    else:
        rng = np.random.default_rng(3)
        n = sum(lens)
        k = (rng.standard_normal((n, 4, 128)) * rng.uniform(0.01, 30, (n, 4, 1))).astype(np.float32)
        v = rng.standard_normal((n, 4, 128)).astype(np.float32)
        k[5, 1] = 0.0                              # an all-zero row
        q = rng.standard_normal((3, 28, 128)).astype(np.float32)
    sch = L.WC_DITHER_INT8 if scheme == "int8" else L.WC_FP8_E4M3
    sc = Scenario(sch, k, v, q, lens, dtype, Hkv=4)
    torch.cuda.synchronize()
    kc = sc.cache.k_codes.cpu().numpy()
    vc = sc.cache.v_codes.cpu().numpy()
    wt = sc.cache.witness.cpu().numpy()
    for b in range(3):
        S = lens[b]
        for g in range(4):
            k32, v32, _ = sc.seq_inputs(b, g)
            oc = (H.oracle_int8_cache(k32, v32, int(sc.seeds[b]), sc.layer, g, S) if scheme == "int8"
                  else H.oracle_fp8_cache(k32, v32))
            gk = H.gather_k_codes(kc, sc.layer, sc.tab[b], S, g)
            gv = H.gather_v_codes(vc, sc.layer, sc.tab[b], S, g)
            if scheme == "int8":                   # offset binary in HBM
                gk, gv = (gk.astype(np.int16) - 128).astype(np.int8), (gv.astype(np.int16) - 128).astype(np.int8)
            assert np.array_equal(gk.view(oc["ck"].dtype), oc["ck"]), (b, g)
            assert np.array_equal(gv.view(oc["cv"].dtype), oc["cv"]), (b, g)
            w = H.gather_rows(wt, sc.layer, sc.tab[b], S, g)
            assert np.all(np.abs(w - oc["w"]) <= MET_TOL * oc["w"] + 1e-30), (b, g)
            assert np.all(w >= oc["w"])           # rounding guard keeps the witness sound
            if scheme == "int8":
                ks = H.gather_rows(sc.cache.k_scale.cpu().numpy(), sc.layer, sc.tab[b], S, g)
                vs = H.gather_rows(sc.cache.v_scale.cpu().numpy(), sc.layer, sc.tab[b], S, g)
                assert np.array_equal(ks, oc["sk"]) and np.array_equal(vs, oc["sv"])
    # the same cache decoded with the query in the input dtype (fp32 queries
    # take the kernels' hi/lo split operand)
    for n_split in (1, 3):
        out = sc.decode(n_split=n_split, mask=3 if scheme == "int8" else 1)
        _check_decode(sc, out)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_write_kivi2_bit_exact(dtype):
    L = H.need_gpu()
    _flush(f"write kivi2 {dtype}")
    rng = np.random.default_rng(4)
    n, Hkv = 96, 2
    k = (rng.standard_normal((n, Hkv, 128)) * rng.uniform(0.1, 5, (1, Hkv, 128))).astype(np.float32)
    v = rng.standard_normal((n, Hkv, 128)).astype(np.float32)
    k[32:64, 0, 7] = 1.5                            # a constant key group
    if dtype == "bf16":
        kb, vb = inputs.f32_to_bf16_bits(k), inputs.f32_to_bf16_bits(v)
        k, v = inputs.bf16_bits_to_f32(kb), inputs.bf16_bits_to_f32(vb)
        kd, vd = H.dev_tensor(kb, "bf16"), H.dev_tensor(vb, "bf16")
    else:
        kd, vd = H.dev_tensor(k, "f32"), H.dev_tensor(v, "f32")
    pages = np.array([4, 0, 2])
    cache = L.KVCache(L.WC_KIVI2, 1, 5, Hkv)
    slot = torch.from_numpy((pages[np.arange(n) // 32] * 32 + np.arange(n) % 32).astype(np.int64)).cuda()
    pos = torch.arange(n, dtype=torch.int32, device="cuda")
    sd = torch.zeros(n, dtype=torch.int64, device="cuda")
    L.wc_write_kv(cache, kd, vd, slot, pos, sd)
    torch.cuda.synchronize()
    kc, vc = cache.k_codes.cpu().numpy()[0], cache.v_codes.cpu().numpy()[0]
    ka, va = cache.k_aux.cpu().numpy()[0], cache.v_aux.cpu().numpy()[0]
    wt = cache.witness.cpu().numpy()[0]
    for g in range(Hkv):
        code, scale, mn, xhat = quant.kivi2_keys(k[:, g])
        vcode, vscale, vmn, vxhat = quant.kivi2_values(v[:, g])
        w = quant.witness(k[:, g], xhat)
        for gi, p in enumerate(pages):
            packed = kc[p, g]                                      # [128][8]
            got = (packed[:, np.arange(32) // 4] >> (2 * (np.arange(32) % 4))) & 3   # [128][32]
            assert np.array_equal(got.T, code[32 * gi:32 * gi + 32])
            assert np.array_equal(ka[p, g, :, 0], scale[gi]) and np.array_equal(ka[p, g, :, 1], mn[gi])
            vp = vc[p, g]                                          # [32][32]
            vgot = (vp[:, np.arange(128) // 4] >> (2 * (np.arange(128) % 4))) & 3
            assert np.array_equal(vgot, vcode[32 * gi:32 * gi + 32])
            assert np.array_equal(va[p, g, :, :, 0], vscale[32 * gi:32 * gi + 32])
            assert np.array_equal(va[p, g, :, :, 1], vmn[32 * gi:32 * gi + 32])
            ww = wt[p, g]
            ref = w[32 * gi:32 * gi + 32]
            assert np.all(np.abs(ww - ref) <= MET_TOL * ref + 1e-30) and np.all(ww >= ref)


# ---------------------------------------------------------------- decode + meter
def _check_decode(sc, out, n_check=None):
    for b in range(sc.B):
        S = int(sc.ctx[b])
        for g in range(sc.Hkv):
            hs = slice(g * sc.G, (g + 1) * sc.G)
            if S == 0:
                assert np.all(out["o"][b, hs] == 0) and np.all(np.isneginf(out["lse"][b, hs]))
                assert np.all(out["R_A"][b, hs] == 0)
                continue
            _, r = sc.oracle(b, g)
            err = H.rel_l2(out["o"][b, hs], r["o_tilde"])
            assert np.all(err <= OUT_TOL), (b, g, err.max())
            assert np.all(np.abs(out["lse"][b, hs] - r["lse"]) <= 1e-4 * np.maximum(1, np.abs(r["lse"]))), (b, g)
            ra = out["R_A"][b, hs]
            # The stored witness is the band norm rounded up by 1 + 2^-20 (the
            # write path's soundness guard): every Tier A bound c_t rises by at
            # most that fraction, which e^c turns into at most
            # 2 (e^{c_max 2^-20} - 1) relative in R = E (1 + E/2) -- 2.2e-5 at
            # the largest c_max of these cases (11.3, fp32 keys scaled up to 30
            # under fp8, R ~ 1e8), so the plain 1e-4 bar holds for saturated
            # meters too.
            assert np.all(np.abs(ra - r["R_A"]) <= MET_TOL * r["R_A"]), (b, g, ra, r["R_A"])
            assert np.all(ra >= r["R_A"] * (1 - MET_TOL)), (b, g)
            assert np.all(ra >= r["tv_true"]), (b, g)
            # the tanh bound of Tier A: deterministic, sound
            ta = out["T_A"][b, hs]
            assert np.all(np.abs(ta - r["T_A"]) <= MET_TOL * r["T_A"] + 1e-7), (b, g, ta, r["T_A"])
            assert np.all(ta >= r["tv_true"] * (1 - 1e-6)), (b, g)
            if sc.scheme == sc.L.WC_DITHER_INT8:
                rb = out["R_B"][b, hs]
                assert np.all(np.abs(rb - r["R_B"]) <= MET_TOL * r["R_B"]), (b, g, rb, r["R_B"])
                tb = out["T_B"][b, hs]
                assert np.all(np.abs(tb - r["T_B"]) <= MET_TOL * r["T_B"] + 1e-7), (b, g, tb, r["T_B"])
            else:
                assert np.all(out["T_B"][b, hs] == 0)


def test_decode_tiny_fp32():
    L = H.need_gpu()
    _flush("decode tiny fp32")
    d = inputs.tiny(seed=1)
    for n_split in (1, 3):
        sc = Scenario(L.WC_DITHER_INT8, d["k"], d["v"], d["q"], [256], "f32", Hkv=1, delta=(1e-2, 1, 1, 1))
        out = sc.decode(n_split=n_split)
        _check_decode(sc, out)


@pytest.mark.parametrize("n_split", [1, 16])
def test_decode_layer_outliers(n_split):
    L = H.need_gpu()
    _flush(f"decode layer n_split={n_split}")
    d = inputs.layer(seed=2)
    sc = Scenario(L.WC_DITHER_INT8, d["k"], d["v"], d["q"], [4096], "bf16", Hkv=4)
    out = sc.decode(n_split=n_split)
    _check_decode(sc, out)


@pytest.mark.parametrize("scheme", ["int8", "fp8"])
def test_decode_ragged_batch(scheme):
    L = H.need_gpu()
    _flush(f"decode ragged {scheme}")
    lens = [1, 15, 16, 17, 300, 0, 1000, 33]
    k, v, _ = _ragged_layer(6, lens)
    q = inputs.layer(seed=7, S=1, Hq=28, Hkv=4, batch=len(lens))["q"]
    sch = L.WC_DITHER_INT8 if scheme == "int8" else L.WC_FP8_E4M3
    sc = Scenario(sch, k, v, q, lens, "bf16", Hkv=4)
    for n_split in (1, 5, 70):
        out = sc.decode(n_split=n_split, mask=3 if scheme == "int8" else 1)
        _check_decode(sc, out)


def test_meter_off_is_bit_identical_and_split_invariant():
    L = H.need_gpu()
    _flush("meter on/off")
    lens = [700, 129]
    k, v, _ = _ragged_layer(8, lens)
    q = inputs.layer(seed=9, S=1, batch=2)["q"]
    sc = Scenario(L.WC_DITHER_INT8, k, v, q, lens, "bf16", Hkv=4)
    on = sc.decode(n_split=4, mask=3, risk=True)
    off = sc.decode(n_split=4, mask=0)
    a_only = sc.decode(n_split=4, mask=1)
    assert np.array_equal(on["o"].view(np.uint32), off["o"].view(np.uint32))
    assert np.array_equal(on["lse"].view(np.uint32), off["lse"].view(np.uint32))
    assert np.array_equal(on["o"].view(np.uint32), a_only["o"].view(np.uint32))
    again = sc.decode(n_split=4, mask=3, risk=True)
    for key in ("o", "lse", "R_A", "R_B", "logrisk"):
        assert np.array_equal(on[key].view(np.uint32), again[key].view(np.uint32)), key
    one = sc.decode(n_split=1)
    # the split changes the running max, hence the fp16 rounding of the
    # attention weights fed to the PV product: invariant to half the output bar
    assert np.all(H.rel_l2(one["o"], on["o"]) < OUT_TOL / 2)
    assert np.allclose(one["R_A"], on["R_A"], rtol=1e-5) and np.allclose(one["R_B"], on["R_B"], rtol=1e-5)


@pytest.mark.parametrize("scheme", ["int8", "fp8"])
def test_block_risk_matches_oracle(scheme):
    L = H.need_gpu()
    _flush(f"block risk {scheme}")
    lens = [513, 64]
    k, v, _ = _ragged_layer(10, lens)
    q = inputs.layer(seed=11, S=1, batch=2)["q"]
    sch = L.WC_DITHER_INT8 if scheme == "int8" else L.WC_FP8_E4M3
    sc = Scenario(sch, k, v, q, lens, "bf16", Hkv=4)
    out = sc.decode(n_split=3, mask=3 if scheme == "int8" else 1, risk=True)
    for b in range(2):
        P = -(-lens[b] // 16)
        for g in range(4):
            _, r = sc.oracle(b, g)
            hs = slice(g * sc.G, (g + 1) * sc.G)
            rho = np.exp(out["logrisk"][b, hs, :P].astype(np.float64) - out["lse"][b, hs, None])
            ref = r["block_risk"]
            assert np.all(np.abs(rho - ref) <= 1e-4 * ref + 1e-30), (b, g)


@pytest.mark.parametrize("scheme", ["int8", "fp8", "rtn"])
def test_decode_fp32_query_ragged(scheme):
    """fp32 keys, values and queries (the query's hi/lo operand split on a
    ragged grouped batch, 2 waves per SIMD) with block risks, one to many
    splits."""
    L = H.need_gpu()
    _flush(f"decode fp32 query {scheme}")
    lens = [1, 17, 700, 0, 129]
    n = sum(lens)
    rng = np.random.default_rng(31)
    k = (rng.standard_normal((n, 4, 128)) * rng.uniform(0.05, 5.0, (n, 4, 1))).astype(np.float32)
    v = (rng.standard_normal((n, 4, 128)) * rng.uniform(0.1, 3.0, (n, 4, 1))).astype(np.float32)
    q = rng.standard_normal((len(lens), 28, 128)).astype(np.float32)
    sch = {"int8": L.WC_DITHER_INT8, "fp8": L.WC_FP8_E4M3, "rtn": L.WC_RTN_INT8}[scheme]
    sc = Scenario(sch, k, v, q, lens, "f32", Hkv=4)
    for n_split in (1, 4, 9):
        out = sc.decode(n_split=n_split, mask=3 if scheme == "int8" else 1, risk=True)
        _check_decode(sc, out)
        for b, S in enumerate(lens):
            P = -(-S // 16)
            for g in range(4):
                if S == 0:
                    continue
                _, r = sc.oracle(b, g)
                hs = slice(g * 7, (g + 1) * 7)
                rho = np.exp(out["logrisk"][b, hs, :P].astype(np.float64) - out["lse"][b, hs, None])
                assert np.all(np.abs(rho - r["block_risk"]) <= 1e-4 * r["block_risk"] + 1e-30), (n_split, b, g)


@pytest.mark.parametrize("Hq,Hkv", [(32, 2), (9, 1), (8, 1), (4, 4), (8, 4), (16, 4), (15, 3), (12, 1)])
def test_decode_group_sizes(Hq, Hkv):
    # groups of more than 8 query heads take the uncompacted softmax path;
    # the block outputs leave in runs of up to 4 heads x 16 pages, so groups
    # of 1 to 16 heads take one to four rounds
    L = H.need_gpu()
    _flush(f"decode group {Hq}/{Hkv}")
    lens = [300, 77]
    n = sum(lens)
    d = inputs.layer(seed=12, S=n, Hq=Hq, Hkv=Hkv, outliers=1)
    q = inputs.layer(seed=13, S=1, Hq=Hq, Hkv=Hkv, batch=2)["q"]
    sc = Scenario(L.WC_DITHER_INT8, d["k"], d["v"], q, lens, "bf16", Hkv=Hkv)
    out = sc.decode(n_split=3, mask=3, risk=True)
    _check_decode(sc, out)
    cm = sc.decode(n_split=3, mask=3, cmax=True)["cmax"]
    for b, S in enumerate(lens):
        P = -(-S // 16)
        for g in range(Hkv):
            _, r = sc.oracle(b, g)
            hs = slice(g * sc.G, (g + 1) * sc.G)
            rho = np.exp(out["logrisk"][b, hs, :P].astype(np.float64) - out["lse"][b, hs, None])
            assert np.all(np.abs(rho - r["block_risk"]) <= 1e-4 * r["block_risk"] + 1e-30), (b, g)
            got = cm[b, hs, :P].astype(np.float64)
            assert np.all(np.abs(got - r["block_cmax"]) <= 1e-4 * r["block_cmax"] + 1e-30), (b, g)
            # entries past the sequence's pages are left as they were
            assert np.all(np.isnan(out["logrisk"][b, hs, P:])) and np.all(np.isnan(cm[b, hs, P:])), (b, g)


@pytest.mark.parametrize("scheme", ["int8", "rtn"])
@pytest.mark.parametrize("scales", ["small", "large", "mixed"])
def test_decode_small_and_large_value_scales(scheme, scales):
    """Value rows whose absmax spans [1e-3, 1e-2] (small), about 1e4 (large),
    or [1e-3, 1e4] within one sequence (mixed): the attention weights times the
    value scales, fed to the fp16 PV operand, must stay in fp16's range (the
    kernel offsets its running max by a power of two chosen from the largest
    value scale), so the output keeps the 2e-3 bar."""
    L = H.need_gpu()
    _flush(f"value scales {scales} {scheme}")
    lens = [700, 129, 33]
    n = sum(lens)
    k, v, _ = _ragged_layer(21, lens)
    q = inputs.layer(seed=22, S=1, batch=len(lens))["q"]
    rng = np.random.default_rng(23)
    lo, hi = {"small": (1e-3, 1e-2), "large": (5e3, 2e4), "mixed": (1e-3, 1e4)}[scales]
    target = np.exp(rng.uniform(np.log(lo), np.log(hi), (n, 4, 1)))
    v32 = inputs.bf16_bits_to_f32(v).astype(np.float64)
    v32 = v32 / np.max(np.abs(v32), axis=-1, keepdims=True) * target
    vb = inputs.f32_to_bf16_bits(v32.astype(np.float32))
    sch = L.WC_DITHER_INT8 if scheme == "int8" else L.WC_RTN_INT8
    sc = Scenario(sch, k, vb, q, lens, "bf16", Hkv=4)
    for n_split in (1, 3):
        out = sc.decode(n_split=n_split, mask=3 if scheme == "int8" else 1)
        for b in range(len(lens)):
            for g in range(4):
                _, r = sc.oracle(b, g)
                hs = slice(g * sc.G, (g + 1) * sc.G)
                err = H.rel_l2(out["o"][b, hs], r["o_tilde"])
                assert np.all(err <= OUT_TOL), (scales, n_split, b, g, err.max())
                assert np.all(np.abs(out["R_A"][b, hs] - r["R_A"]) <= MET_TOL * r["R_A"]), (b, g)

"""GPU parity of the value-side certificate: the value witness written by
every scheme (and by the black-box hook), and E_V from the decode against the
oracle, never below the value error it bounds."""
import numpy as np
import pytest
import torch

from certified_kv_cache_amd import inputs
from oracle import quant
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


def _mantissa4(bits):
    b = bits.astype(np.uint32)
    return (((b + 0x4) & 0xFFF8) & 0xFFFF).astype(np.uint16)


SCHEMES = ["int8", "fp8", "rtn", "store16", "int8-bypass"]


def _scenario(L, scheme, k, v, q, lens, **kw):
    if scheme == "store16":
        return Scenario(L.WC_BF16_STORE, k, v, q, lens, "bf16", Hkv=4, khat=_mantissa4(k), vhat=_mantissa4(v),
                        v_witness=True, **kw)
    sch = {"int8": L.WC_DITHER_INT8, "fp8": L.WC_FP8_E4M3, "rtn": L.WC_RTN_INT8,
           "int8-bypass": L.WC_DITHER_INT8}[scheme]
    return Scenario(sch, k, v, q, lens, "bf16", Hkv=4, v_witness=True,
                    num_outliers=8 if scheme == "int8-bypass" else 0, **kw)


@pytest.mark.parametrize("scheme", SCHEMES)
def test_value_witness_and_certificate(scheme):
    L = H.need_gpu()
    _flush(f"value certificate {scheme}")
    lens = [1, 17, 600, 0, 1100]
    k, v, q = _layer(90, lens)
    sc = _scenario(L, scheme, k, v, q, lens)
    torch.cuda.synchronize()
    wv_all = sc.cache.v_witness.cpu().numpy()
    mask = 3 if scheme.startswith("int8") else 1
    outs = [sc.decode(n_split=ns, mask=mask, vcert=True, risk=True) for ns in (1, 6)]
    plain = sc.decode(n_split=6, mask=mask)
    for b, S in enumerate(lens):
        for g in range(4):
            hs = slice(g * 7, (g + 1) * 7)
            if S == 0:
                assert all(np.all(o["E_V"][b, hs] == 0) for o in outs)
                continue
            oc, r = sc.oracle(b, g)
            v32 = H.to_f32(v[sc.offsets[b]:sc.offsets[b + 1], g], "bf16")
            want = quant.witness_v(v32, oc["vhat"])
            got = H.gather_rows(wv_all, sc.layer, sc.tab[b], S, g)
            assert np.all(np.abs(got - want) <= MET_TOL * want + 1e-30) and np.all(got >= want), (b, g)
            for o in outs:
                ev = o["E_V"][b, hs]
                assert np.all(np.abs(ev - r["E_V"]) <= MET_TOL * r["E_V"]), (b, g, ev, r["E_V"])
                assert np.all(ev >= r["dv_true"]), (b, g)
                assert np.all(H.rel_l2(o["o"][b, hs], r["o_tilde"]) <= OUT_TOL), (b, g)
    # the value certificate changes nothing else: output and key meters bit-identical
    for key in ("o", "lse", "R_A", "R_B"):
        assert np.array_equal(outs[1][key].view(np.uint32), plain[key].view(np.uint32)), key
    assert np.all(plain["E_V"] == 0)


def test_value_witness_kivi2_write():
    L = H.need_gpu()
    _flush("value witness kivi2")
    rng = np.random.default_rng(91)
    n, Hkv = 96, 2
    k = rng.standard_normal((n, Hkv, 128)).astype(np.float32)
    v = (rng.standard_normal((n, Hkv, 128)) * rng.uniform(0.1, 4, (n, Hkv, 1))).astype(np.float32)
    pages = np.array([2, 0, 1])
    cache = L.KVCache(L.WC_KIVI2, 1, 3, Hkv, v_witness=True)
    slot = torch.from_numpy((pages[np.arange(n) // 32] * 32 + np.arange(n) % 32).astype(np.int64)).cuda()
    pos = torch.arange(n, dtype=torch.int32, device="cuda")
    L.wc_write_kv(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), slot, pos,
                  torch.zeros(n, dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    wv = cache.v_witness.cpu().numpy()[0]
    for g in range(Hkv):
        _, _, _, vxhat = quant.kivi2_values(v[:, g])
        want = quant.witness_v(v[:, g], vxhat)
        for gi, p in enumerate(pages):
            got = wv[p, g]
            ref = want[32 * gi:32 * gi + 32]
            assert np.all(np.abs(got - ref) <= MET_TOL * ref + 1e-30) and np.all(got >= ref)


@pytest.mark.parametrize("scheme", ["fp8", "int8"])
def test_joint_output_bound_on_the_gpu_meters(scheme):
    # ||o~ - o|| <= E_V + 2 min(1, R_A) max ||v||: the value certificate and the
    # key meter from the decode bound the whole error of the output the GPU
    # returns.  For dithered INT8 that output takes each value draw's low byte
    # at its mean, which moves a token's v^ by at most 2^-9 sqrt(128) s_t.
    L = H.need_gpu()
    _flush(f"joint bound {scheme}")
    lens = [800, 300]
    k, v, q = _layer(92, lens)
    sc = _scenario(L, scheme, k, v, q, lens)
    out = sc.decode(n_split=4, mask=1, vcert=True)
    for b, S in enumerate(lens):
        for g in range(4):
            hs = slice(g * 7, (g + 1) * 7)
            oc, r = sc.oracle(b, g)
            low = 2.0 ** -9 * np.sqrt(128) * float(np.max(oc["sv"])) if scheme == "int8" else 0.0
            v32 = H.to_f32(v[sc.offsets[b]:sc.offsets[b + 1], g], "bf16").astype(np.float64)
            vmax = np.max(np.linalg.norm(v32, axis=-1))
            err = np.linalg.norm(out["o"][b, hs] - r["o_exact"], axis=-1)
            bound = out["E_V"][b, hs] + low + 2 * np.minimum(1, out["R_A"][b, hs]) * vmax
            assert np.all(err <= bound), (b, g, err, bound)
            # the value part alone: the GPU output against the oracle's p~ on
            # the exact v, within E_V plus the low-byte term
            ev_err = np.linalg.norm(out["o"][b, hs] - r["p_tilde"] @ v32, axis=-1)
            assert np.all(ev_err <= out["E_V"][b, hs] + low + OUT_TOL * np.linalg.norm(r["o_tilde"], axis=-1)), (b, g)

"""GPU parity of the whole-page write (wc_write_kv_pages): against the oracle
on every page, and bit-identical to the per-token write of the same tokens,
both in page order (each workgroup of the per-token write then holds one whole
page and stores it as whole lines) and shuffled (each row stores its own
bytes)."""
import numpy as np
import pytest
import torch

from certified_kv_cache_amd import inputs
from oracle import outlier, quant
from tests import helpers as H

pytestmark = pytest.mark.gpu

MET_TOL = 1e-4
NL, NP, HKV = 3, 9, 4                       # layers, pages, KV heads


def _flush(msg):
    print(msg, flush=True)


def _inputs(dtype, seed=95):
    rng = np.random.default_rng(seed)
    n = NP * 16
    k = (rng.standard_normal((NL, n, HKV, 128)) * rng.uniform(0.05, 8, (NL, 1, HKV, 128))).astype(np.float32)
    v = rng.standard_normal((NL, n, HKV, 128)).astype(np.float32)
    k[1, 5, 2] = 0.0                                                    # an all-zero row
    k[:, :, :, 7] *= 30.0                                               # an outlier channel
    if dtype == "bf16":
        return inputs.f32_to_bf16_bits(k), inputs.f32_to_bf16_bits(v)
    return k, v


@pytest.mark.parametrize("scheme,dtype,m", [("int8", "bf16", 0), ("int8", "f32", 0), ("int8", "bf16", 8),
                                            ("fp8", "bf16", 0), ("rtn", "f32", 0), ("rtn", "bf16", 0)])
def test_write_pages_matches_oracle_and_row_write(scheme, dtype, m):
    L = H.need_gpu()
    _flush(f"write pages {scheme} {dtype} m={m}")
    sch = {"int8": L.WC_DITHER_INT8, "fp8": L.WC_FP8_E4M3, "rtn": L.WC_RTN_INT8}[scheme]
    kb, vb = _inputs(dtype)
    k32, v32 = H.to_f32(kb, dtype), H.to_f32(vb, dtype)
    rng = np.random.default_rng(96)
    P = NP + 4
    pages = rng.permutation(P)[:NP].astype(np.int32)
    pos0 = (16 * rng.integers(0, 1000, NP)).astype(np.int32)
    seeds = rng.integers(0, 2 ** 62, NP).astype(np.int64)
    caches = [L.KVCache(sch, NL + 1, P, HKV, num_outliers=m, v_witness=True) for _ in range(3)]
    O = None
    if m:
        O = np.stack([np.stack([outlier.top_energy_channels(k32[l, :, g], m) for g in range(HKV)])
                      for l in range(NL)])
        for c in caches:
            c.outlier_ch[1:] = torch.from_numpy(O).cuda()
    kd, vd = H.dev_tensor(kb, dtype), H.dev_tensor(vb, dtype)
    L.wc_write_kv_pages(caches[0], kd, vd, torch.from_numpy(pages).cuda(), torch.from_numpy(pos0).cuda(),
                        torch.from_numpy(seeds).cuda(), layer0=1)
    t = np.arange(NP * 16)
    slot = torch.from_numpy(pages[t // 16].astype(np.int64) * 16 + t % 16).cuda()
    pos = torch.from_numpy((pos0[t // 16] + t % 16).astype(np.int32)).cuda()
    tseed = torch.from_numpy(seeds[t // 16]).cuda()
    L.wc_write_kv(caches[1], kd, vd, slot, pos, tseed, layer0=1)
    sh = torch.from_numpy(rng.permutation(NP * 16)).cuda()              # no workgroup holds a whole page
    L.wc_write_kv(caches[2], kd[:, sh].contiguous(), vd[:, sh].contiguous(), slot[sh], pos[sh], tseed[sh], layer0=1)
    torch.cuda.synchronize()
    names = ["k_codes", "v_codes", "witness", "v_witness"] + (["k_scale", "v_scale"] if scheme != "fp8" else []) + \
            (["k_outlier"] if m else [])
    for nm in names:                                 # the three writes agree bit for bit
        a = getattr(caches[0], nm).cpu().numpy()
        for j in (1, 2):
            b = getattr(caches[j], nm).cpu().numpy()
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (nm, j)
    c = caches[0]
    kc, vc, wt, wv = (getattr(c, nm).cpu().numpy() for nm in ("k_codes", "v_codes", "witness", "v_witness"))
    for l in range(NL):
        for g in range(HKV):
            row = pages.astype(np.int64)                 # page i of the input
            x, y = k32[l, :, g], v32[l, :, g]
            if scheme == "int8":
                from oracle import dither
                xi = np.concatenate([dither.dither_rows(int(seeds[i]), l + 1, g, pos0[i] + np.arange(16))
                                     for i in range(NP)])
                if m:
                    ck, sk, _, side = outlier.dither_int8_bypass(x, xi, O[l, g])
                    kh = outlier.dequant_bypass(ck, sk, xi, side, O[l, g])
                else:
                    ck, sk, _ = quant.dither_int8(x, xi)
                    kh = quant.dequant_dither_int8(ck, sk, xi)
                cv, sv, _ = quant.dither_int8(y, xi)
                vh = quant.dequant_dither_int8(cv, sv, xi)
            elif scheme == "rtn":
                ck, sk, _ = quant.rtn_int8(x)
                cv, sv, _ = quant.rtn_int8(y)
                kh, vh = quant.dequant_rtn_int8(ck, sk), quant.dequant_rtn_int8(cv, sv)
            else:
                ck, kh = quant.fp8_e4m3(x)
                cv, vh = quant.fp8_e4m3(y)
            gk = H.gather_k_codes(kc, l + 1, row, NP * 16, g)
            gv = H.gather_v_codes(vc, l + 1, row, NP * 16, g)
            if scheme != "fp8":
                gk = (gk.astype(np.int16) - 128).astype(np.int8)
                gv = (gv.astype(np.int16) - 128).astype(np.int8)
                assert np.array_equal(H.gather_rows(c.k_scale.cpu().numpy(), l + 1, row, NP * 16, g), sk)
                assert np.array_equal(H.gather_rows(c.v_scale.cpu().numpy(), l + 1, row, NP * 16, g), sv)
            assert np.array_equal(gk.view(ck.dtype), ck) and np.array_equal(gv.view(cv.dtype), cv), (l, g)
            w_ref = quant.witness(x, kh)
            w = H.gather_rows(wt, l + 1, row, NP * 16, g)
            assert np.all(np.abs(w - w_ref) <= MET_TOL * w_ref + 1e-30) and np.all(w >= w_ref), (l, g)
            wv_ref = quant.witness_v(y, vh)
            wvg = H.gather_rows(wv, l + 1, row, NP * 16, g)
            assert np.all(np.abs(wvg - wv_ref) <= MET_TOL * wv_ref + 1e-30) and np.all(wvg >= wv_ref), (l, g)

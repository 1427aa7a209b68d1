"""GPU parity at the full sizes of the benchmark workloads.

* decode: batch 32 x 32768 tokens, 28 query / 4 KV heads, 16 KV splits, block
  risks on -- the launch configuration bench.py times -- for the dithered INT8
  cache (Tier A + B), the fp8 raw-cast cache (Tier A), and the variants bench.py
  reports beside them (outlier bypass m = 8, RTN INT8, the 16-bit store of a
  4-bit-mantissa scheme, the value certificate); codes, scales, witnesses,
  outputs, meters, tanh bounds and block risks of sampled (sequence, KV head)
  pairs against the oracle, and size-independent properties on every head;
* write: the 28-layer prefill (4096 tokens, 4 KV heads, per-channel variance
  log-uniform in [0.1, 10]) for all three schemes, sampled (layer, head) rows
  bit-exact against the oracle;
* gate: a 64-sequence ragged batch (contexts uniform in [1024, 32768]) on an
  fp8 cache at tau in {0.05, 0.2, 1.0}: selections bit-exact for every
  (sequence, KV head), risks and repaired blocks checked on samples, and the
  repaired cache's outputs and meters against the oracle on samples.
"""
import math

import numpy as np
import pytest
import torch

from certified_kv_cache_amd import inputs
from oracle import gate, meter, outlier, quant
from tests import helpers as H

pytestmark = pytest.mark.gpu

B, S, HQ, HKV, G, NSPLIT = 32, 32768, 28, 4, 7, 16
DELTA = (1e-2, 28, 28, 256)
OUT_TOL, MET_TOL = 2e-3, 1e-4


def _flush(msg):
    print(msg, flush=True)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _codes_of(cache, layer, pages, g):
    """[S_pages*16, 128] key and value codes of one KV head over `pages`, in
    page order (re-indexing of the documented layouts only)."""
    idx = torch.from_numpy(np.asarray(pages, dtype=np.int64)).cuda()
    kc = cache.k_codes[layer, idx, g].cpu().numpy()[None, :, None]      # [1][P][1][2][4][16][16]
    vc = cache.v_codes[layer, idx, g].cpu().numpy()[None, :, None]
    n = 16 * len(pages)
    row = np.arange(len(pages))
    return H.gather_k_codes(kc, 0, row, n, 0), H.gather_v_codes(vc, 0, row, n, 0)


def _rows_of(arr, layer, pages, g):
    idx = torch.from_numpy(np.asarray(pages, dtype=np.int64)).cuda()
    return arr[layer, idx, g].cpu().numpy().reshape((16 * len(pages),) + tuple(arr.shape[4:]))


# ---------------------------------------------------------------- decode, bench configuration
def _mantissa4_t(x):
    """The 16-bit store's scheme under test (torch, on the device): bf16 with 4
    of its 8 significant bits, rounded half up on the magnitude."""
    b = x.view(torch.int16).to(torch.int32) & 0xFFFF
    return (((b + 4) & 0xFFF8) & 0xFFFF).to(torch.int16).view(torch.bfloat16)


def _decode_full(scheme_name, seed=3):
    L = H.need_gpu()
    scheme = {"int8": L.WC_DITHER_INT8, "fp8": L.WC_FP8_E4M3, "int8-bypass8": L.WC_DITHER_INT8,
              "rtn": L.WC_RTN_INT8, "store16": L.WC_BF16_STORE, "int8-vcert": L.WC_DITHER_INT8}[scheme_name]
    mask = 3 if scheme_name.startswith("int8") else 1
    vcert = scheme_name == "int8-vcert"
    k, v = inputs.decode_kv_torch(seed, B, S, Hkv=HKV)
    q = inputs.query_torch(seed, B, Hq=HQ)
    ctx = np.full(B, S)
    tab, npages = inputs.page_table(seed, ctx)
    seeds = inputs.seeds(B, base=1000 + seed)
    cache = L.KVCache(scheme, 1, npages, HKV, num_outliers=8 if scheme_name == "int8-bypass8" else 0,
                      v_witness=vcert)
    if scheme_name == "int8-bypass8":                 # calibration: the first 4096 cached tokens
        L.wc_outlier_select(k[:4096].contiguous(), 8, cache.outlier_ch)
    tab_d = torch.from_numpy(tab).cuda()
    t = torch.arange(S, device="cuda")
    slot = (tab_d[:, t // 16].long() * 16 + (t % 16)[None]).reshape(-1)
    pos = t.int().repeat(B)
    sd = torch.from_numpy(seeds.view(np.int64)).cuda()
    if scheme_name == "store16":
        kh, vh = _mantissa4_t(k), _mantissa4_t(v)
        L.wc_write_kv(cache, kh, vh, slot, pos, sd.repeat_interleave(S))
        L.wc_witness(cache, k, kh, slot)
        del kh, vh
    else:
        L.wc_write_kv(cache, k, v, slot, pos, sd.repeat_interleave(S))
    part = torch.empty(L.wc_decode_workspace_bytes(B, HQ, NSPLIT) // 4, device="cuda")
    risk = torch.full((B, HQ, tab.shape[1]), float("nan"), device="cuda")
    ctx_d = torch.full((B,), S, dtype=torch.int32, device="cuda")
    L.wc_decode_attn_meter(cache, 0, q, tab_d, ctx_d, sd, part, H.SM, mask | (L.WC_METER_V if vcert else 0),
                           DELTA[0], *DELTA[1:], NSPLIT, block_logrisk=risk)
    o = torch.empty((B, HQ, 128), device="cuda")
    lse = torch.empty((B, HQ), device="cuda")
    ra, rb, ta, tb, ev = (torch.empty((B, HQ), device="cuda") for _ in range(5))
    L.wc_lse_merge(part, B, HQ, NSPLIT, o, lse, ra, rb, ta, tb, ev)
    torch.cuda.synchronize()
    out = dict(o=o.cpu().numpy(), lse=lse.cpu().numpy(), R_A=ra.cpu().numpy(), R_B=rb.cpu().numpy(),
               T_A=ta.cpu().numpy(), T_B=tb.cpu().numpy(), E_V=ev.cpu().numpy(), logrisk=risk.cpu().numpy())
    return L, cache, k, v, q, tab, seeds, out


@pytest.mark.parametrize("scheme", ["int8", "fp8", "int8-bypass8", "rtn", "store16", "int8-vcert"])
def test_decode_bench_size_sampled_against_oracle(scheme):
    _flush(f"full-size decode {scheme}: B={B} S={S} splits={NSPLIT}")
    L, cache, k, v, q, tab, seeds, out = _decode_full(scheme)
    P = S // 16
    dither = scheme.startswith("int8")
    O = None
    if scheme == "int8-bypass8":                     # the selection, bit-exact, from the oracle's energies
        calib = k[:4096].float().cpu().numpy()
        O = np.stack([outlier.top_energy_channels(calib[:, g], 8) for g in range(HKV)])
        assert np.array_equal(cache.outlier_ch[0].cpu().numpy(), O)
    # every head: finite outputs, nonnegative meters, and the block risks sum
    # to the gate tier's E (R = E (1 + E/2)) -- properties of any size
    assert np.all(np.isfinite(out["o"])) and np.all(np.isfinite(out["lse"]))
    assert np.all(out["R_A"] >= 0)
    r_gate = out["R_B"] if dither else out["R_A"]
    e_gate = np.sqrt(1.0 + 2.0 * r_gate.astype(np.float64)) - 1.0
    rho_sum = np.exp(out["logrisk"][:, :, :P].astype(np.float64) - out["lse"][:, :, None]).sum(-1)
    assert np.all(np.abs(rho_sum - e_gate) <= 1e-4 * e_gate + 1e-30)
    rng = np.random.default_rng(11)
    pairs = [(0, 0), (B - 1, HKV - 1)] + [(int(rng.integers(B)), int(rng.integers(HKV))) for _ in range(2)]
    lt = math.log(2 * S / meter.delta_loc(*DELTA))
    for b, g in pairs:
        _flush(f"  oracle pair b={b} g={g}")
        k32 = k[b * S:(b + 1) * S, g].float().cpu().numpy()
        v32 = v[b * S:(b + 1) * S, g].float().cpu().numpy()
        qg = q[b, g * G:(g + 1) * G].float().cpu().numpy().astype(np.float64)
        wt = _rows_of(cache.witness, 0, tab[b, :P], g)
        if dither:
            oc = H.oracle_int8_cache(k32, v32, int(seeds[b]), 0, g, S, bypass=None if O is None else O[g])
            r = meter.decode_group(qg, k32, oc["khat"], v32, oc["vhat"], oc["w"], H.SM, k_scale=oc["sk"],
                                   log_term=lt, bypass=None if O is None else O[g])
        elif scheme == "rtn":
            oc = H.oracle_rtn_cache(k32, v32)
            r = meter.decode_group(qg, k32, oc["khat"], v32, oc["vhat"], oc["w"], H.SM)
        elif scheme == "store16":
            kh = _mantissa4_t(k[b * S:(b + 1) * S, g]).float().cpu().numpy()
            vh = _mantissa4_t(v[b * S:(b + 1) * S, g]).float().cpu().numpy()
            oc = dict(khat=kh, vhat=vh, w=quant.witness(k32, kh))
            r = meter.decode_group(qg, k32, kh, v32, vh, oc["w"], H.SM)
        else:
            oc = H.oracle_fp8_cache(k32, v32)
            r = meter.decode_group(qg, k32, oc["khat"], v32, oc["vhat"], oc["w"], H.SM)
        if scheme != "store16":
            gk, gv = _codes_of(cache, 0, tab[b, :P], g)
            if scheme != "fp8":                          # offset binary in HBM
                gk = (gk.astype(np.int16) - 128).astype(np.int8)
                gv = (gv.astype(np.int16) - 128).astype(np.int8)
                assert np.array_equal(_rows_of(cache.k_scale, 0, tab[b, :P], g), oc["sk"])
                assert np.array_equal(_rows_of(cache.v_scale, 0, tab[b, :P], g), oc["sv"])
            assert np.array_equal(gk.view(oc["ck"].dtype), oc["ck"]), (b, g)
            assert np.array_equal(gv.view(oc["cv"].dtype), oc["cv"]), (b, g)
        if O is not None:
            side = _rows_of(cache.k_outlier, 0, tab[b, :P], g).view(np.uint16)
            assert np.array_equal(inputs.bf16_bits_to_f32(side), oc["side"]), (b, g)
        assert np.all(np.abs(wt - oc["w"]) <= MET_TOL * oc["w"] + 1e-30) and np.all(wt >= oc["w"])
        hs = slice(g * G, (g + 1) * G)
        assert np.all(H.rel_l2(out["o"][b, hs], r["o_tilde"]) <= OUT_TOL), (b, g)
        assert np.all(np.abs(out["lse"][b, hs] - r["lse"]) <= 1e-4 * np.maximum(1, np.abs(r["lse"])))
        assert np.all(np.abs(out["R_A"][b, hs] - r["R_A"]) <= MET_TOL * r["R_A"]), (b, g)
        assert np.all(out["R_A"][b, hs] >= r["tv_true"])
        assert np.all(np.abs(out["T_A"][b, hs] - r["T_A"]) <= MET_TOL * r["T_A"] + 1e-7), (b, g)
        assert np.all(out["T_A"][b, hs] >= r["tv_true"] * (1 - 1e-6))
        if dither:
            assert np.all(np.abs(out["R_B"][b, hs] - r["R_B"]) <= MET_TOL * r["R_B"]), (b, g)
            assert np.all(np.abs(out["T_B"][b, hs] - r["T_B"]) <= MET_TOL * r["T_B"] + 1e-7), (b, g)
        if scheme == "int8-vcert":
            wv = _rows_of(cache.v_witness, 0, tab[b, :P], g)
            want = quant.witness_v(v32, oc["vhat"])
            assert np.all(np.abs(wv - want) <= MET_TOL * want + 1e-30) and np.all(wv >= want)
            assert np.all(np.abs(out["E_V"][b, hs] - r["E_V"]) <= MET_TOL * r["E_V"]), (b, g)
            assert np.all(out["E_V"][b, hs] >= r["dv_true"])
        rho = np.exp(out["logrisk"][b, hs, :P].astype(np.float64) - out["lse"][b, hs, None])
        assert np.all(np.abs(rho - r["block_risk"]) <= 1e-4 * r["block_risk"] + 1e-30), (b, g)
    del cache, k, v
    _free()


# ---------------------------------------------------------------- prefill write, 28 layers
@pytest.mark.parametrize("scheme", ["int8", "fp8", "kivi2"])
def test_write_prefill_28_layers_sampled(scheme):
    L = H.need_gpu()
    _flush(f"full-size write {scheme}: 28 layers x 4096 tokens x 4 heads")
    NL, NT, seed = 28, 4096, 9
    k, v = inputs.prefill_kv_torch(seed, layers=NL, n_tok=NT, Hkv=HKV)
    sch = {"int8": L.WC_DITHER_INT8, "fp8": L.WC_FP8_E4M3, "kivi2": L.WC_KIVI2}[scheme]
    ps = 32 if scheme == "kivi2" else 16
    tab, npages = inputs.page_table(seed, [NT], page_size=ps)
    cache = L.KVCache(sch, NL, npages, HKV)
    t = np.arange(NT)
    slot = torch.from_numpy(tab[0, t // ps].astype(np.int64) * ps + t % ps).cuda()
    pos = torch.arange(NT, dtype=torch.int32, device="cuda")
    dseed = 777
    sd = torch.full((NT,), dseed, dtype=torch.int64, device="cuda")
    L.wc_write_kv(cache, k, v, slot, pos, sd)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    picks = [(0, 0), (NL - 1, HKV - 1)] + [(int(rng.integers(NL)), int(rng.integers(HKV))) for _ in range(2)]
    pages = tab[0, :NT // ps]
    for layer, g in picks:
        _flush(f"  oracle layer={layer} g={g}")
        k32 = k[layer, :, g].float().cpu().numpy()
        v32 = v[layer, :, g].float().cpu().numpy()
        idx = torch.from_numpy(pages.astype(np.int64)).cuda()
        if scheme == "kivi2":
            code, scale, mn, xhat = quant.kivi2_keys(k32)
            vcode, vscale, vmn, _ = quant.kivi2_values(v32)
            w = quant.witness(k32, xhat)
            kc = cache.k_codes[layer, idx, g].cpu().numpy()          # [P][128][8]
            vc = cache.v_codes[layer, idx, g].cpu().numpy()          # [P][32][32]
            ka = cache.k_aux[layer, idx, g].cpu().numpy()
            va = cache.v_aux[layer, idx, g].cpu().numpy()
            wt = cache.witness[layer, idx, g].cpu().numpy()
            got = (kc[:, :, np.arange(32) // 4] >> (2 * (np.arange(32) % 4))) & 3   # [P][128][32]
            assert np.array_equal(got.transpose(0, 2, 1).reshape(NT, 128), code)
            assert np.array_equal(ka[:, :, 0], scale) and np.array_equal(ka[:, :, 1], mn)
            vgot = (vc[:, :, np.arange(128) // 4] >> (2 * (np.arange(128) % 4))) & 3
            assert np.array_equal(vgot.reshape(NT, 128), vcode)
            assert np.array_equal(va[..., 0].reshape(NT, 4), vscale) and np.array_equal(va[..., 1].reshape(NT, 4), vmn)
            wt = wt.reshape(NT, 8)
        else:
            if scheme == "int8":
                oc = H.oracle_int8_cache(k32, v32, dseed, layer, g, NT)
            else:
                oc = H.oracle_fp8_cache(k32, v32)
            gk, gv = _codes_of(cache, layer, pages, g)
            if scheme == "int8":
                gk = (gk.astype(np.int16) - 128).astype(np.int8)
                gv = (gv.astype(np.int16) - 128).astype(np.int8)
                assert np.array_equal(_rows_of(cache.k_scale, layer, pages, g), oc["sk"])
                assert np.array_equal(_rows_of(cache.v_scale, layer, pages, g), oc["sv"])
            assert np.array_equal(gk.view(oc["ck"].dtype), oc["ck"]), (layer, g)
            assert np.array_equal(gv.view(oc["cv"].dtype), oc["cv"]), (layer, g)
            w = oc["w"]
            wt = _rows_of(cache.witness, layer, pages, g)
        assert np.all(np.abs(wt - w) <= MET_TOL * w + 1e-30) and np.all(wt >= w)
    del cache, k, v
    _free()


# ---------------------------------------------------------------- gate flow, ragged batch of 64
def test_gate_flow_64_ragged_fp8():
    L = H.need_gpu()
    seed, NB = 13, 64
    lens = np.random.default_rng(seed).integers(1024, 32769, NB)
    _flush(f"gate flow: {NB} sequences, {int(lens.sum())} tokens, fp8")
    k, v = inputs.ragged_kv_torch(seed, lens, Hkv=HKV)
    q = inputs.query_torch(seed, NB, Hq=HQ)
    tab, npages = inputs.page_table(seed, lens)
    mp = tab.shape[1]
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    slot_np = np.concatenate([tab[b, np.arange(S_) // 16].astype(np.int64) * 16 + np.arange(S_) % 16
                              for b, S_ in enumerate(lens)])
    slot = torch.from_numpy(slot_np).cuda()
    pos = torch.from_numpy(np.concatenate([np.arange(S_) for S_ in lens]).astype(np.int32)).cuda()
    sd = torch.zeros(int(lens.sum()), dtype=torch.int64, device="cuda")
    # exact keys in pinned host memory, paged like the cache: [1][P][Hkv][16][128]
    store = torch.zeros((1, npages, HKV, 16, 128), dtype=torch.bfloat16, device="cuda")
    store[0, slot // 16, :, slot % 16, :] = k
    host = torch.empty(store.shape, dtype=torch.bfloat16, pin_memory=True)
    host.copy_(store)
    del store
    tab_d = torch.from_numpy(tab).cuda()
    ctx_d = torch.from_numpy(lens.astype(np.int32)).cuda()
    seeds_d = torch.zeros(NB, dtype=torch.int64, device="cuda")
    rng = np.random.default_rng(3)
    samples = [(0, 0), (NB - 1, 3)] + [(int(rng.integers(NB)), int(rng.integers(HKV))) for _ in range(3)]
    ref = {}
    for b, g in samples:                      # oracle block risks of the quantized cache
        k32 = k[starts[b]:starts[b] + lens[b], g].float().cpu().numpy()
        v32 = v[starts[b]:starts[b] + lens[b], g].float().cpu().numpy()
        qg = q[b, g * G:(g + 1) * G].float().cpu().numpy().astype(np.float64)
        oc = H.oracle_fp8_cache(k32, v32)
        ref[(b, g)] = (k32, v32, qg, oc, meter.decode_group(qg, k32, oc["khat"], v32, oc["vhat"], oc["w"], H.SM))

    def decode(cache):
        part = torch.empty(L.wc_decode_workspace_bytes(NB, HQ, NSPLIT) // 4, device="cuda")
        risk = torch.empty((NB, HQ, mp), device="cuda")
        L.wc_decode_attn_meter(cache, 0, q, tab_d, ctx_d, seeds_d, part, H.SM, 1, DELTA[0], *DELTA[1:], NSPLIT,
                               block_logrisk=risk)
        o = torch.empty((NB, HQ, 128), device="cuda")
        lse = torch.empty((NB, HQ), device="cuda")
        ra = torch.empty((NB, HQ), device="cuda")
        L.wc_lse_merge(part, NB, HQ, NSPLIT, o, lse, ra)
        return risk, lse, ra, o

    for tau in (1.0, 0.2, 0.05):
        _flush(f"  tau={tau}")
        cache = L.KVCache(L.WC_FP8_E4M3, 1, npages, HKV, pool_capacity=int(npages) * HKV)   # never runs out
        L.wc_write_kv(cache, k, v, slot, pos, sd)
        risk, lse, ra, _ = decode(cache)
        ws = torch.empty(L.wc_gate_workspace_bytes(NB, HKV, mp), dtype=torch.uint8, device="cuda")
        pool_used = torch.zeros(1, dtype=torch.int64, device="cuda")
        paged = torch.zeros(1, dtype=torch.int64, device="cuda")
        sel = torch.full((NB, HKV, mp + 1), -7, dtype=torch.int32, device="cuda")
        rho = torch.zeros((NB, HQ, mp), dtype=torch.int64, device="cuda")
        L.wc_gate_pagein(cache, 0, risk, lse, tab_d, ctx_d, tau, host, pool_used, paged, ws, selected=sel,
                         rho_fx=rho)
        torch.cuda.synchronize()
        sel_np, rho_np = sel.cpu().numpy(), rho.cpu().numpy().view(np.uint64)
        lse_np = lse.cpu().numpy()
        T = gate.threshold_fx(tau)
        total = 0
        for b in range(NB):                     # every (sequence, KV head): bit-exact selection
            P = -(-int(lens[b]) // 16)
            for g in range(HKV):
                want = gate.select(rho_np[b, g * G:(g + 1) * G, :P], np.zeros(P, bool), T)
                got = list(sel_np[b, g, 1:1 + sel_np[b, g, 0]])
                assert got == want, (tau, b, g)
                total += len(want)
        assert int(pool_used.item()) == total and int(paged.item()) == 4096 * total
        for (b, g), (k32, v32, qg, oc, r) in ref.items():
            P = -(-int(lens[b]) // 16)
            fx_ref = gate.rho_to_fx(r["block_risk"])
            got = rho_np[b, g * G:(g + 1) * G, :P].astype(np.float64)
            assert np.all(np.abs(got - fx_ref) <= 1e-4 * fx_ref.astype(np.float64) + 1), (tau, b, g)
        # the repaired cache: exact keys in the pool, witnesses zeroed, and the
        # sampled heads' outputs and meters against the oracle on the repaired
        # cache (repairs move the softmax too, so the new meter is re-measured,
        # not inferred from the gate's arithmetic)
        risk2, lse2, ra2, o2 = decode(cache)
        torch.cuda.synchronize()
        ra2_np = ra2.cpu().numpy()
        _flush(f"    {total} blocks repaired; max meter {float(ra.cpu().numpy().max()):.4g} -> {float(ra2_np.max()):.4g}")
        # untriggered heads already had R <= tau; repaired ones should land at
        # about tau (not a theorem: a repair also renormalizes the softmax)
        assert float(ra2_np.max()) <= tau * 1.05 + 1e-12
        slots = cache.exact_slot.cpu().numpy()[0]
        for (b, g), (k32, v32, qg, oc, r) in ref.items():
            S_ = int(lens[b])
            t = np.arange(S_)
            rep = slots[tab[b, t // 16], g] >= 0
            r2 = meter.decode_group(qg, k32, oc["khat"], v32, oc["vhat"], oc["w"], H.SM, repaired=rep)
            hs = slice(g * G, (g + 1) * G)
            assert np.all(np.abs(ra2_np[b, hs] - r2["R_A"]) <= MET_TOL * r2["R_A"] + 1e-30), (tau, b, g)
            assert np.all(ra2_np[b, hs] >= r2["tv_true"])
            assert np.all(H.rel_l2(o2.cpu().numpy()[b, hs], r2["o_tilde"]) <= OUT_TOL)
            for j in sel_np[b, g, 1:1 + sel_np[b, g, 0]][:4]:
                p = tab[b, j]
                s = slots[p, g]
                exact = k[starts[b] + 16 * j:starts[b] + 16 * j + 16, g].view(torch.int16).cpu().numpy()
                pool = cache.exact_pool[s].view(torch.int16).cpu().numpy()
                rows = min(16, S_ - 16 * j)
                assert np.array_equal(pool[:rows], exact[:rows])         # bf16 bit for bit
                assert np.all(cache.witness[0, p, g].cpu().numpy() == 0)
        del cache
        _free()
    del k, v, host
    _free()

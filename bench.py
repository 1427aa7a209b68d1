"""Benchmark of the WitCert hot path on one MI355X.

Default workload: decode batch 32, 32768 cached tokens
per sequence, Qwen2.5-7B attention shape (28 query / 4 KV heads, d = 128),
dithered INT8 cache paged at 16 tokens with a random page permutation,
16 KV splits, Tier A + Tier B meter (delta_req 1e-2 over L = 28, H = 28,
T = 256).  Inputs are synthetic and seeded (bf16 N(0,1), RoPE on K).

One step = append one token per sequence (wc_write_kv), fused decode +
meter with block risks (wc_decode_attn_meter), LSE merge (wc_lse_merge) and
the gate at tau = 0.2 (wc_gate_pagein).  The cache is resident in HBM before
the timed region.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HQ, HKV, D, NSPLIT = 28, 4, 128, 16
G_ = HQ // HKV
DELTA = (1e-2, 28, 28, 256)
TAU = 0.2
PEAK_GBS = 8000.0
METRIC = "fused INT8 decode attn+meter: achieved HBM GB/s (% peak), overhead vs no meter"
COUNTERS = os.path.join(ROOT, "profiles", "decode_int8_b32_s32k_counters.json")


def decode_source_sha():
    h = hashlib.sha256()
    for f in ("decode.hip", "wc_common.h"):
        h.update(open(os.path.join(ROOT, "certified_kv_cache_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def decode_bytes(B, S, meter, scales=True):
    """Algorithmic HBM bytes of one decode launch: cache, page table, query.
    (scales=False: the fp8 raw-cast cache, which stores none.)"""
    per_tok = 128 + 128 + (8 if scales else 0) + (32 if meter else 0)   # K, V codes, K, V scales, witness
    P = -(-S // 16)
    return B * S * HKV * per_tok + B * P * 4 + B * HQ * D * 2 + B * 4 + B * 8


def step_bytes(B, S):
    """Algorithmic bytes of one whole step (decode + append + merge + gate)."""
    P = -(-S // 16)
    write = B * HKV * (2 * D * 2 + 2 * D + 2 * 4 + 32) + B * (8 + 4 + 8)
    merge_out = B * HQ * (D * 4 + 3 * 4)
    risk = 2 * B * HQ * P * 4                         # block risks written by decode, read by the gate
    return decode_bytes(B, S, True) + write + merge_out + risk


def setup(B, S, seed=3):
    import numpy as np
    import torch

    from certified_kv_cache_amd import _lib as L
    from certified_kv_cache_amd import inputs

    k, v = inputs.decode_kv_torch(seed, B, S, Hkv=HKV)
    q = inputs.query_torch(seed, B, Hq=HQ)
    ctx = np.full(B, S)
    tab, npages = inputs.page_table(seed, ctx)
    seeds = inputs.seeds(B, base=1000 + seed)
    cache = L.KVCache(L.WC_DITHER_INT8, 1, npages, HKV, pool_capacity=4096)
    dev = torch.device("cuda")
    tab_d = torch.from_numpy(tab).to(dev)
    t = torch.arange(S, device=dev)
    slot = (tab_d[:, t // 16].long() * 16 + (t % 16)[None]).reshape(-1)
    pos = t.int().repeat(B)
    sd = torch.from_numpy(seeds.view(np.int64)).to(dev)
    L.wc_write_kv(cache, k, v, slot, pos, sd.repeat_interleave(S))
    last = torch.arange(B, device=dev) * S + (S - 1)
    new = dict(k=k[last].contiguous(), v=v[last].contiguous(), slot=slot[last].contiguous(),
               pos=pos[last].contiguous(), seed=sd.clone())
    # exact backing store in pinned host memory, paged like the cache
    store = torch.empty((1, npages, HKV, 16, D), dtype=torch.bfloat16, device=dev)
    store[0, slot // 16, :, slot % 16, :] = k
    host = torch.empty(store.shape, dtype=torch.bfloat16, pin_memory=True)
    host.copy_(store)
    del store
    torch.cuda.synchronize()
    return dict(L=L, cache=cache, k=k, v=v, q=q, tab=tab_d, ctx=torch.full((B,), S, dtype=torch.int32, device=dev),
                seed=sd, new=new, host=host, npages=npages, tab_np=tab, seeds=seeds, slot=slot, pos=pos)


def fp8_variant(w, B, S, iters):
    """The same workload on the fp8 raw-cast cache (Tier A only)."""
    import torch
    L = w["L"]
    cache = L.KVCache(L.WC_FP8_E4M3, 1, w["npages"], HKV)
    L.wc_write_kv(cache, w["k"], w["v"], w["slot"], w["pos"], torch.zeros_like(w["pos"], dtype=torch.int64))
    mp = w["tab"].shape[1]
    part = torch.empty(L.wc_decode_workspace_bytes(B, HQ, NSPLIT) // 4, device="cuda")
    risk = torch.empty((B, HQ, mp), device="cuda")
    sm = 1.0 / math.sqrt(D)

    def decode(mask=1, with_risk=True):
        L.wc_decode_attn_meter(cache, 0, w["q"], w["tab"], w["ctx"], w["seed"], part, sm, mask, DELTA[0],
                               *DELTA[1:], NSPLIT, block_logrisk=risk if with_risk else None)

    floor = make_floor(w, B, cache)

    def run(mask=1, with_risk=True, fl=False):
        if fl:
            floor(mask=mask)
        else:
            decode(mask, with_risk)

    t = time_modes(run, iters, {"risk": dict(mask=1, with_risk=True), "on": dict(mask=1, with_risk=False),
                                "off": dict(mask=0, with_risk=False), "floor": dict(mask=1, fl=True)}, warm=60)
    t_risk, t_on, t_off = t["risk"], t["on"], t["off"]
    nb = decode_bytes(B, S, True, scales=False)
    del cache
    return {"decode_us": round(t_risk, 2), "decode_meter_on_us": round(t_on, 2), "decode_meter_off_us": round(t_off, 2),
            "meter_overhead": round(t_on / t_off - 1, 4), "decode_bytes": nb, "load_floor_us": round(t["floor"], 2),
            "achieved_GBps": round(nb / (t_risk * 1e-6) / 1e9, 1), "frac": round(nb / (t_risk * 1e-6) / 1e9 / PEAK_GBS, 4)}


def scheme_variant(w, B, S, iters, scheme):
    """The same workload on a black-box scheme with Tier A: RTN INT8, or the
    16-bit store (x^ = x here; its witness comes from wc_witness)."""
    import torch
    L = w["L"]
    sch = {"rtn": L.WC_RTN_INT8, "store16": L.WC_BF16_STORE}[scheme]
    cache = L.KVCache(sch, 1, w["npages"], HKV)
    L.wc_write_kv(cache, w["k"], w["v"], w["slot"], w["pos"], w["seed"].repeat_interleave(S))
    if scheme == "store16":
        L.wc_witness(cache, w["k"], w["k"], w["slot"])
    mp = w["tab"].shape[1]
    part = torch.empty(L.wc_decode_workspace_bytes(B, HQ, NSPLIT) // 4, device="cuda")
    risk = torch.empty((B, HQ, mp), device="cuda")
    sm = 1.0 / math.sqrt(D)

    def decode(mask=1, with_risk=True):
        L.wc_decode_attn_meter(cache, 0, w["q"], w["tab"], w["ctx"], w["seed"], part, sm, mask, DELTA[0],
                               *DELTA[1:], NSPLIT, block_logrisk=risk if with_risk else None)

    t = time_modes(decode, iters, {"risk": dict(mask=1, with_risk=True), "on": dict(mask=1, with_risk=False),
                                   "off": dict(mask=0, with_risk=False)}, warm=60)
    t_risk, t_on, t_off = t["risk"], t["on"], t["off"]
    if scheme == "store16":
        nb = B * S * HKV * (2 * 2 * D + 32) + B * (-(-S // 16)) * 4 + B * HQ * D * 2 + B * 12
    else:
        nb = decode_bytes(B, S, True)
    del cache
    return {"decode_us": round(t_risk, 2), "decode_meter_on_us": round(t_on, 2), "decode_meter_off_us": round(t_off, 2),
            "meter_overhead": round(t_on / t_off - 1, 4), "decode_bytes": nb,
            "achieved_GBps": round(nb / (t_risk * 1e-6) / 1e9, 1), "frac": round(nb / (t_risk * 1e-6) / 1e9 / PEAK_GBS, 4)}


def vcert_variant(w, B, S, iters):
    """The 32 x 32768 INT8 decode with the value certificate added (value witness
    stored at write time, E_V in the same pass)."""
    import torch
    L = w["L"]
    cache = L.KVCache(L.WC_DITHER_INT8, 1, w["npages"], HKV, v_witness=True)
    L.wc_write_kv(cache, w["k"], w["v"], w["slot"], w["pos"], w["seed"].repeat_interleave(S))
    mp = w["tab"].shape[1]
    part = torch.empty(L.wc_decode_workspace_bytes(B, HQ, NSPLIT) // 4, device="cuda")
    risk = torch.empty((B, HQ, mp), device="cuda")
    sm = 1.0 / math.sqrt(D)

    def decode(mask=3, with_risk=True):
        L.wc_decode_attn_meter(cache, 0, w["q"], w["tab"], w["ctx"], w["seed"], part, sm, mask, DELTA[0],
                               *DELTA[1:], NSPLIT, block_logrisk=risk if with_risk else None)

    t = time_modes(decode, iters, {"v": dict(mask=3 | L.WC_METER_V), "kv": dict(mask=3)}, warm=60)
    t_v, t_kv = t["v"], t["kv"]
    nb = decode_bytes(B, S, True) + B * S * HKV * 4
    del cache
    return {"decode_us": round(t_v, 2), "decode_without_v_us": round(t_kv, 2),
            "v_overhead": round(t_v / t_kv - 1, 4), "decode_bytes": nb,
            "achieved_GBps": round(nb / (t_v * 1e-6) / 1e9, 1), "frac": round(nb / (t_v * 1e-6) / 1e9 / PEAK_GBS, 4)}


def needle_variant(w, B, S, iters, outs):
    """The structured stand-in for concentrated attention: the same workload
    with a sink key at position 0 (+8 on the mean query's logit) and 4 seeded
    needle keys (+6) per (sequence, KV head).  Decode time, and the meters of
    both workloads side by side (median over heads)."""
    import numpy as np
    import torch
    from certified_kv_cache_amd import inputs
    L = w["L"]
    kn = inputs.plant_needles_torch(w["k"], w["q"], B, S, Hkv=HKV, seed=3)
    cache = L.KVCache(L.WC_DITHER_INT8, 1, w["npages"], HKV)
    L.wc_write_kv(cache, kn, w["v"], w["slot"], w["pos"], w["seed"].repeat_interleave(S))
    del kn
    mp = w["tab"].shape[1]
    part = torch.empty(L.wc_decode_workspace_bytes(B, HQ, NSPLIT) // 4, device="cuda")
    risk = torch.empty((B, HQ, mp), device="cuda")
    sm = 1.0 / math.sqrt(D)

    def decode(mask=3, with_risk=True):
        L.wc_decode_attn_meter(cache, 0, w["q"], w["tab"], w["ctx"], w["seed"], part, sm, mask, DELTA[0],
                               *DELTA[1:], NSPLIT, block_logrisk=risk if with_risk else None)

    t = min(time_decode(decode, iters, warm=100), time_decode(decode, iters))
    decode()
    o = torch.empty((B, HQ, D), device="cuda")
    lse = torch.empty((B, HQ), device="cuda")
    ra, rb, ta = (torch.empty((B, HQ), device="cuda") for _ in range(3))
    L.wc_lse_merge(part, B, HQ, NSPLIT, o, lse, ra, rb, ta)
    torch.cuda.synchronize()
    med = lambda x: float(np.median(x.cpu().numpy()))
    res = {"decode_us": round(t, 2), "R_A_median": med(ra), "R_B_median": med(rb), "tanh_A_median": med(ta),
           "uniform_R_A_median": med(outs["ra"]), "uniform_R_B_median": med(outs["rb"])}
    del cache
    return res


def outlier_variant(w, B, S, iters, m):
    """The same workload with the outlier bypass of the keys (m exact bf16
    channels per KV head, chosen by key energy over the first 4096 cached
    tokens), Tier A+B with block risks."""
    import torch
    L = w["L"]
    cache = L.KVCache(L.WC_DITHER_INT8, 1, w["npages"], HKV, num_outliers=m)
    L.wc_outlier_select(w["k"][:4096].contiguous(), m, cache.outlier_ch)
    L.wc_write_kv(cache, w["k"], w["v"], w["slot"], w["pos"], w["seed"].repeat_interleave(S))
    mp = w["tab"].shape[1]
    part = torch.empty(L.wc_decode_workspace_bytes(B, HQ, NSPLIT) // 4, device="cuda")
    risk = torch.empty((B, HQ, mp), device="cuda")
    sm = 1.0 / math.sqrt(D)

    def decode(mask=3, with_risk=True):
        L.wc_decode_attn_meter(cache, 0, w["q"], w["tab"], w["ctx"], w["seed"], part, sm, mask, DELTA[0],
                               *DELTA[1:], NSPLIT, block_logrisk=risk if with_risk else None)

    t = time_modes(decode, iters, {"risk": dict(mask=3, with_risk=True), "off": dict(mask=0, with_risk=False)}, warm=60)
    t_risk, t_off = t["risk"], t["off"]
    nb = decode_bytes(B, S, True) + B * S * HKV * 2 * m
    del cache
    return {"m": m, "decode_us": round(t_risk, 2), "decode_meter_off_us": round(t_off, 2), "decode_bytes": nb,
            "achieved_GBps": round(nb / (t_risk * 1e-6) / 1e9, 1), "frac": round(nb / (t_risk * 1e-6) / 1e9 / PEAK_GBS, 4)}


def make_step(w, B, S):
    import torch
    L = w["L"]
    mp = w["tab"].shape[1]
    part = torch.empty(L.wc_decode_workspace_bytes(B, HQ, NSPLIT) // 4, device="cuda")
    risk = torch.empty((B, HQ, mp), device="cuda")
    o = torch.empty((B, HQ, D), device="cuda")
    lse = torch.empty((B, HQ), device="cuda")
    ra = torch.empty((B, HQ), device="cuda")
    rb = torch.empty((B, HQ), device="cuda")
    gws = torch.empty(L.wc_gate_workspace_bytes(B, HKV, mp), dtype=torch.uint8, device="cuda")
    pool_used = torch.zeros(1, dtype=torch.int64, device="cuda")
    paged = torch.zeros(1, dtype=torch.int64, device="cuda")
    sm = 1.0 / math.sqrt(D)
    n = w["new"]

    def decode(mask=3, with_risk=True):
        L.wc_decode_attn_meter(w["cache"], 0, w["q"], w["tab"], w["ctx"], w["seed"], part, sm, mask, DELTA[0],
                               *DELTA[1:], NSPLIT, block_logrisk=risk if with_risk else None)

    def step(ev=None):
        # ev: a pair of HIP events recorded around the decode on its stream
        L.wc_write_kv(w["cache"], n["k"], n["v"], n["slot"], n["pos"], n["seed"])
        if ev is not None:
            ev[0].record()
        decode()
        if ev is not None:
            ev[1].record()
        L.wc_lse_merge(part, B, HQ, NSPLIT, o, lse, ra, rb)
        L.wc_gate_pagein(w["cache"], 0, risk, lse, w["tab"], w["ctx"], TAU, w["host"], pool_used, paged, gws,
                         meter=rb)

    return step, decode, dict(o=o, lse=lse, ra=ra, rb=rb, paged=paged)


def make_floor(w, B, cache):
    """Launcher of the decode's load floor on `cache` (same page table and
    splits as the decode)."""
    import torch
    L = w["L"]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def floor(mask=3, match=True):
        L.wc_decode_load_floor(cache, 0, HQ, w["tab"], w["ctx"], NSPLIT, mask, sink, match_residency=match)

    return floor


def time_modes(decode, iters, modes, rounds=3, warm=20):
    """Median loop time (us) of each decode mode in `modes` (name -> keyword
    arguments of `decode`), the modes' loops taken in turn for `rounds`
    rounds after `warm` launches of each."""
    import numpy as np
    for kw in modes.values():
        for _ in range(warm):
            decode(**kw)
    got = {m: [] for m in modes}
    for _ in range(rounds):
        for m, kw in modes.items():
            got[m].append(time_decode(decode, iters, **kw))
    return {m: float(np.median(v)) for m, v in got.items()}


def time_decode(decode, iters, warm=1, **kw):
    """Mean duration (us) of one decode launch: `iters` back-to-back launches
    between one pair of HIP events on the launch stream, after `warm` untimed
    launches."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(warm):
        decode(**kw)
    a.record()
    for _ in range(iters):
        decode(**kw)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / iters * 1e3


def cpu_baseline(w, B, S, budget_s=12.0):
    """The float64 oracle's read path (dither regeneration, dequantization,
    attention, Tier A/B, TV meter) on (sequence, KV head) pairs of the same
    workload, one thread, taken in a seeded random order until about
    `budget_s` seconds of timed work; scaled to GB/s of the same algorithmic
    bytes.  The cache the read path consumes (codes, scales, witness) is made
    by the oracle's write path outside the timed region."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import dither, meter, quant
    sm = 1.0 / math.sqrt(D)
    lt = math.log(2 * S / meter.delta_loc(*DELTA))
    order = np.random.default_rng(0).permutation(B * HKV)
    total, done = 0.0, 0
    with threadpool_limits(limits=1):
        for idx in order:
            b, g = int(idx) // HKV, int(idx) % HKV
            k32 = w["k"][b * S:(b + 1) * S, g].float().cpu().numpy()
            v32 = w["v"][b * S:(b + 1) * S, g].float().cpu().numpy()
            q = w["q"][b, g * G_:(g + 1) * G_].float().cpu().numpy().astype(np.float64)
            seed = int(w["seeds"][b])
            pos = np.arange(S)
            xi0 = dither.dither_rows(seed, 0, g, pos)
            ck, sk, _ = quant.dither_int8(k32, xi0)
            cv, sv, _ = quant.dither_int8(v32, xi0)
            wt = quant.witness(k32, quant.dequant_dither_int8(ck, sk, xi0))
            t0 = time.perf_counter()
            xi = dither.dither_rows(seed, 0, g, pos)
            khat = quant.dequant_dither_int8(ck, sk, xi)
            vhat = quant.dequant_dither_int8(cv, sv, xi)
            meter.decode_group(q, k32, khat, v32, vhat, wt, sm, k_scale=sk, log_term=lt)
            total += time.perf_counter() - t0
            done += 1
            if total >= budget_s:
                break
    sample_bytes = done * decode_bytes(B, S, True) / (B * HKV)
    from threadpoolctl import threadpool_info
    blas = sorted({i.get("internal_api", "?") + ":" + str(i.get("num_threads")) for i in threadpool_info()})
    return dict(value=round(sample_bytes / total / 1e9, 4), unit="GB/s", cores=1, kind="oracle",
                host_cores=len(os.sched_getaffinity(0)), blas_threads_default=blas,
                sample=f"{done} of {B * HKV} (sequence, KV head) pairs, all {S} tokens each, "
                       f"{total:.1f} s single-threaded float64 numpy")


def prefill_write(iters, seed=4, NL=28, NT=4096):
    """Write path at prefill scale: 28 layers x 4 KV heads x 4096 tokens, bf16
    K/V with per-(layer, head, channel) variance log-uniform in [0.1, 10]; one
    call per scheme writes all layers, per token (wc_write_kv) and in whole
    pages (wc_write_kv_pages, suffix _pages)."""
    import numpy as np
    import torch

    from certified_kv_cache_amd import _lib as L
    from certified_kv_cache_amd import inputs
    k, v = inputs.prefill_kv_torch(seed, layers=NL, n_tok=NT, Hkv=HKV)
    in_bytes = 2 * k.numel() * 2
    out = {"metric": "write path throughput: GB/s written and total GB/s (% of HBM peak)", "unit": "GB/s",
           "data": "synthetic", "config": {"workload": f"prefill write {NL} layers x {HKV} KV heads x {NT} tokens, bf16"},
           "schemes": {}}
    for name, sch in (("int8", L.WC_DITHER_INT8), ("fp8", L.WC_FP8_E4M3), ("kivi2", L.WC_KIVI2)):
        ps = 32 if sch == L.WC_KIVI2 else 16
        tab, npages = inputs.page_table(seed, [NT], page_size=ps)
        cache = L.KVCache(sch, NL, npages, HKV)
        t = np.arange(NT)
        slot = torch.from_numpy(tab[0, t // ps].astype(np.int64) * ps + t % ps).cuda()
        pos = torch.arange(NT, dtype=torch.int32, device="cuda")
        sd = torch.full((NT,), 777, dtype=torch.int64, device="cuda")
        n_tok_heads = NL * NT * HKV
        if sch == L.WC_DITHER_INT8:
            written = n_tok_heads * (2 * D + 2 * 4 + 32)
        elif sch == L.WC_FP8_E4M3:
            written = n_tok_heads * (2 * D + 32)
        else:                                   # 2-bit codes (2 x d/4 B per token-head), group params, witness
            written = n_tok_heads * (2 * D // 4 + 32) + NL * HKV * (NT // 32) * (D * 2 * 4 + 32 * 4 * 2 * 4)
        calls = [("", lambda: L.wc_write_kv(cache, k, v, slot, pos, sd))]
        if sch != L.WC_KIVI2:                   # whole pages: one workgroup per page-head block
            pg = torch.from_numpy(tab[0, :NT // 16].astype(np.int32)).cuda()
            p0 = torch.arange(0, NT, 16, dtype=torch.int32, device="cuda")
            psd = torch.full((NT // 16,), 777, dtype=torch.int64, device="cuda")
            calls.append(("_pages", lambda: L.wc_write_kv_pages(cache, k, v, pg, p0, psd)))
        for suffix, call in calls:
            # 400 untimed calls first (the shader clock that the power limit
            # leaves takes tens of milliseconds of back-to-back work to
            # settle), then the median of three timed loops
            us = float(np.median([time_decode(call, iters, warm=400 if r == 0 else 0) for r in range(3)]))
            tot = in_bytes + written
            out["schemes"][name + suffix] = {"us": round(us, 2), "bytes_written": written, "bytes_total": tot,
                                             "written_GBps": round(written / (us * 1e-6) / 1e9, 1),
                                             "total_GBps": round(tot / (us * 1e-6) / 1e9, 1),
                                             "pct_peak": round(100 * tot / (us * 1e-6) / 1e9 / PEAK_GBS, 2)}
        del cache
    return out


# gate variants: (label, meter_mask, gate) -- "cert" is the certificate gate on
# the block risks of the gate tier (B when the mask has it, else A), "tanh" the
# tanh gate on the blocks' largest bound of Tier A (deterministic, delta = 0)
GATE_VARIANTS = {
    "fp8": [("certificate_A", 1, "cert")],
    "int8": [("certificate_B", 3, "cert"), ("certificate_A", 1, "cert"), ("tanh_A", 1, "tanh")],
}


def gate_flow(n_layers, n_steps, seed=5, NB=64, taus=(1.0, 0.2, 0.05), scheme="fp8"):
    """Ragged decode with the gate: 64 sequences, contexts uniform in
    [1024, 32768], fp8 raw-cast (or dithered INT8) cache on `n_layers`
    resident layers, exact keys in pinned host memory.  Each step appends one
    token per sequence and layer, then per layer decodes (block risks or block
    maxima), merges and gates at tau.  Reports page-in bytes of the cold first
    step and the mean of the rest, per gate variant."""
    import numpy as np
    import torch

    from certified_kv_cache_amd import _lib as L
    from certified_kv_cache_amd import inputs
    dev = torch.device("cuda")
    lens0 = np.random.default_rng(seed).integers(1024, 32769, NB)
    cap = lens0 + n_steps                              # room for the appended tokens
    tab, npages = inputs.page_table(seed, cap)
    mp = tab.shape[1]
    tab_d = torch.from_numpy(tab).to(dev)
    q = inputs.query_torch(seed, NB, Hq=HQ)
    seeds_d = torch.arange(1000, 1000 + NB, dtype=torch.int64, device=dev)
    sch = L.WC_FP8_E4M3 if scheme == "fp8" else L.WC_DITHER_INT8
    n0 = int(lens0.sum())
    slot0 = torch.from_numpy(np.concatenate([tab[b, np.arange(S_) // 16].astype(np.int64) * 16 + np.arange(S_) % 16
                                             for b, S_ in enumerate(lens0)])).to(dev)
    pos0 = torch.from_numpy(np.concatenate([np.arange(S_) for S_ in lens0]).astype(np.int32)).to(dev)
    tseed0 = seeds_d.repeat_interleave(torch.from_numpy(lens0).to(dev))
    # the exact host store holds the keys of the tokens written so far: the
    # prefix now, each appended token when it is written (a repair copies the
    # rows of its block that exist; the write path keeps the pool rows of
    # tokens appended later)
    host = torch.zeros((n_layers, npages, HKV, 16, D), dtype=torch.bfloat16, pin_memory=True)
    layer_kv = []
    for layer in range(n_layers):                      # per-layer K/V, the prefix's exact keys to the host store
        k, v = inputs.ragged_kv_torch(seed * 100 + layer, cap, Hkv=HKV)
        starts = np.concatenate([[0], np.cumsum(cap)[:-1]])
        first = torch.from_numpy(np.concatenate([starts[b] + np.arange(S_) for b, S_ in enumerate(lens0)])).to(dev)
        store = torch.zeros((npages, HKV, 16, D), dtype=torch.bfloat16, device=dev)
        store[slot0 // 16, :, slot0 % 16, :] = k[first]
        host[layer].copy_(store)
        del store
        later = [torch.from_numpy(starts + lens0 + s).to(dev) for s in range(n_steps)]
        layer_kv.append((k[first].contiguous(), v[first].contiguous(),
                         [(k[i].contiguous(), v[i].contiguous()) for i in later]))
        del k, v
    torch.cuda.synchronize()
    sm = 1.0 / math.sqrt(D)
    part = torch.empty(L.wc_decode_workspace_bytes(NB, HQ, NSPLIT) // 4, device=dev)
    risk = torch.empty((NB, HQ, mp), device=dev)
    o = torch.empty((NB, HQ, D), device=dev)
    lse = torch.empty((NB, HQ), device=dev)
    ra = torch.empty((NB, HQ), device=dev)
    rb = torch.empty((NB, HQ), device=dev)
    gws = torch.empty(L.wc_gate_workspace_bytes(NB, HKV, mp), dtype=torch.uint8, device=dev)
    # the appended keys' copies for the host store, made before the steps: a
    # step then runs its 28 layers back to back, with no device-to-host copy
    # (and so no wait) between them
    kn_host = [[kn.cpu() for kn, _ in layer_kv[layer][2]] for layer in range(n_layers)]
    cname = "fp8 raw-cast" if scheme == "fp8" else "dithered INT8"
    res = {"metric": "gated ragged decode: page-in bytes per step and attention throughput", "data": "synthetic",
           "config": {"workload": f"{NB} sequences, contexts U[1024, 32768], {n_layers} resident layers, {cname}, "
                                  f"{n_steps} steps, exact keys in pinned host memory", "layers": n_layers,
                      "steps": n_steps, "tokens": n0, "scheme": scheme}, "tau": {}}
    for tau, (label, mask, kind) in [(t, v) for t in taus for v in GATE_VARIANTS[scheme]]:
        cache = L.KVCache(sch, n_layers, npages, HKV, pool_capacity=int(npages) * HKV * n_layers)
        for layer in range(n_layers):
            kf, vf, _ = layer_kv[layer]
            L.wc_write_kv(cache, kf, vf, slot0, pos0, tseed0, layer0=layer)
        for s in range(n_steps):                       # the appended tokens are not in the host store yet
            t_ = lens0 + s
            sl = torch.from_numpy(tab[np.arange(NB), t_ // 16].astype(np.int64) * 16 + t_ % 16)
            host[:, sl // 16, :, sl % 16, :] = 0
        pool_used = torch.zeros(1, dtype=torch.int64, device=dev)
        paged = torch.zeros(1, dtype=torch.int64, device=dev)
        per_step, dec_us = [], []
        for s in range(n_steps):
            lens = lens0 + s + 1
            ctx = torch.from_numpy(lens.astype(np.int32)).to(dev)
            pos = torch.from_numpy((lens - 1).astype(np.int32)).to(dev)
            slot = torch.from_numpy(tab[np.arange(NB), (lens - 1) // 16].astype(np.int64) * 16 + (lens - 1) % 16).to(dev)
            before = int(paged.item())
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(n_layers)]
            slot_h = slot.cpu()
            for layer in range(n_layers):
                kn, vn = layer_kv[layer][2][s]
                L.wc_write_kv(cache, kn, vn, slot, pos, seeds_d, layer0=layer)
                host[layer][slot_h // 16, :, slot_h % 16, :] = kn_host[layer][s]
                a, b = evs[layer]
                a.record()
                L.wc_decode_attn_meter(cache, layer, q, tab_d, ctx, seeds_d, part, sm,
                                       mask | (L.WC_BLOCK_CMAX if kind == "tanh" else 0), DELTA[0], *DELTA[1:],
                                       NSPLIT, block_logrisk=risk)
                b.record()
                L.wc_lse_merge(part, NB, HQ, NSPLIT, o, lse, ra, rb)
                if kind == "tanh":
                    L.wc_gate_pagein_tanh(cache, layer, risk, tab_d, ctx, tau, host, pool_used, paged, gws)
                else:
                    L.wc_gate_pagein(cache, layer, risk, lse, tab_d, ctx, tau, host, pool_used, paged, gws,
                                     meter=rb if mask & 2 else ra)
            torch.cuda.synchronize()
            t_dec = sum(a.elapsed_time(b) for a, b in evs) * 1e3
            per_step.append(int(paged.item()) - before)
            dec_us.append(t_dec)
        nbytes = decode_bytes_ragged(lens0 + n_steps, scales=scheme == "int8") * n_layers
        res["tau"].setdefault(str(tau), {})[label] = {
            "pagein_bytes_step1": per_step[0],
            "pagein_bytes_later_mean": round(float(np.mean(per_step[1:])), 1),
            "decode_us_per_step": round(float(np.mean(dec_us[1:])), 1),
            "attention_GBps": round(nbytes / (float(np.mean(dec_us[1:])) * 1e-6) / 1e9, 1)}
        del cache
        torch.cuda.empty_cache()
    for tau, r in res["tau"].items():                 # the certificate's page-in saving over the tanh gate
        if "tanh_A" in r:
            tb = r["tanh_A"]["pagein_bytes_step1"]
            for lab in ("certificate_B", "certificate_A"):
                if tb > 0:
                    r[lab]["pagein_reduction_vs_tanh"] = round(1.0 - r[lab]["pagein_bytes_step1"] / tb, 4)
    return res


def decode_bounds(B, S, iters=20):
    """What bounds the decode: the 32 x 32768 launch (dithered INT8 with block
    risks, and meter off; fp8 raw cast the same) with its random page table,
    and again with every page-table entry folded into 64 physical pages, so
    that the cache the launch reads stays in L2 and the time is the kernel's
    compute alone."""
    import torch
    w = setup(B, S)
    L = w["L"]
    mp = w["tab"].shape[1]
    part = torch.empty(L.wc_decode_workspace_bytes(B, HQ, NSPLIT) // 4, device="cuda")
    risk = torch.empty((B, HQ, mp), device="cuda")
    c8 = L.KVCache(L.WC_FP8_E4M3, 1, w["npages"], HKV)
    L.wc_write_kv(c8, w["k"], w["v"], w["slot"], w["pos"], torch.zeros_like(w["pos"], dtype=torch.int64))
    folded = (w["tab"] % 64).contiguous()
    sm = 1.0 / math.sqrt(D)
    res = {"metric": "decode time with the cache in HBM and with it L2-resident (compute alone)", "unit": "us",
           "data": "synthetic", "config": {"workload": f"decode B={B} S={S} Hq={HQ} Hkv={HKV} d={D}, {NSPLIT} splits"},
           "hbm": {}, "l2_resident": {}}
    for tname, tab in (("hbm", w["tab"]), ("l2_resident", folded)):
        modes = {}
        for name, cache, mask, r in (("int8_risk", w["cache"], 3, True), ("int8_off", w["cache"], 0, False),
                                     ("fp8_risk", c8, 1, True), ("fp8_off", c8, 0, False)):
            modes[name] = (cache, mask, r)

        def decode(name):
            cache, mask, r = modes[name]
            L.wc_decode_attn_meter(cache, 0, w["q"], tab, w["ctx"], w["seed"], part, sm, mask, DELTA[0], *DELTA[1:],
                                   NSPLIT, block_logrisk=risk if r else None)

        t = time_modes(decode, iters, {n: dict(name=n) for n in modes}, warm=60)
        res[tname] = {n: round(v, 2) for n, v in t.items()}
        # board power and shader clock while each mode runs back to back for
        # about four seconds (amd-smi sampled once in the middle): the clock
        # the power limit leaves differs between the two tables
        res.setdefault("power_clock", {})[tname] = {n: power_clock(lambda: decode(n)) for n in modes}
    # the decode's loads alone (INT8 cache, meter on, same grid and residency)
    floor = make_floor(w, B, w["cache"])
    res["hbm"]["int8_load_floor"] = round(time_modes(lambda: floor(), iters, {"f": {}}, warm=60)["f"], 2)
    res["power_clock"]["hbm"]["int8_load_floor"] = power_clock(lambda: floor())
    return res


def power_clock(launch, seconds=4.0):
    """Socket power (W) and current shader clock (MHz) read by amd-smi while
    `launch` runs back to back on the device; None where amd-smi is absent."""
    import shutil
    import subprocess
    import threading
    import torch
    smi = shutil.which("amd-smi") or ("/opt/rocm/bin/amd-smi" if os.path.exists("/opt/rocm/bin/amd-smi") else None)
    if smi is None:
        return None
    stop = [False]

    def run():
        while not stop[0]:
            for _ in range(20):
                launch()
            torch.cuda.synchronize()

    th = threading.Thread(target=run)
    th.start()
    time.sleep(seconds / 2)
    try:
        out = subprocess.run([smi, "metric", "-g", "0", "-p", "-c", "--json"], capture_output=True, text=True,
                             timeout=30).stdout
    except (OSError, subprocess.SubprocessError):
        out = ""
    time.sleep(seconds / 2)
    stop[0] = True
    th.join()
    try:
        d = json.loads(out)
        g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        clk = g["clock"]
        gfx = [v["clk"]["value"] for k, v in clk.items() if k.startswith("gfx_") and isinstance(v, dict)]
        out = {"socket_power_W": g["power"]["socket_power"]["value"],
               "gfx_clock_MHz_mean": round(sum(gfx) / len(gfx), 1), "gfx_clock_MHz_min": min(gfx),
               "gfx_clock_MHz_max": max(gfx)}
        if isinstance(clk.get("mem_0"), dict):
            out["mem_clock_MHz"] = clk["mem_0"]["clk"]["value"]
        return out
    except (ValueError, KeyError, IndexError, TypeError):
        return None


def latency(iters=200):
    """Decode + merge latency of the two parity-size workloads: one head with
    256 fp32 tokens (dithered INT8, Tier A+B), and one layer of 28 q / 4 KV
    heads with 4096 bf16 tokens (x20 outlier channels), 4 splits."""
    import numpy as np
    import torch

    from certified_kv_cache_amd import _lib as L
    from certified_kv_cache_amd import inputs
    res = {"metric": "decode + merge latency at the parity sizes", "unit": "us", "data": "synthetic", "configs": {}}
    for name, d, hkv, n_split, delta in (("tiny S=256 1q/1kv fp32", inputs.tiny(seed=1), 1, 1, (1e-2, 1, 1, 1)),
                                         ("layer S=4096 28q/4kv bf16", inputs.layer(seed=2), 4, 4, DELTA)):
        dt = torch.float32 if d["dtype"] == "f32" else torch.bfloat16
        conv = (lambda a: torch.from_numpy(a).cuda()) if dt == torch.float32 else \
            (lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16))
        k, v, q = conv(d["k"]), conv(d["v"]), conv(d["q"])
        S = k.shape[0]
        tab, npages = inputs.page_table(1, [S])
        cache = L.KVCache(L.WC_DITHER_INT8, 1, npages, hkv)
        t = np.arange(S)
        slot = torch.from_numpy(tab[0, t // 16].astype(np.int64) * 16 + t % 16).cuda()
        L.wc_write_kv(cache, k, v, slot, torch.arange(S, dtype=torch.int32, device="cuda"),
                      torch.full((S,), 5, dtype=torch.int64, device="cuda"))
        Hq = q.shape[1]
        part = torch.empty(L.wc_decode_workspace_bytes(1, Hq, n_split) // 4, device="cuda")
        o = torch.empty((1, Hq, D), device="cuda")
        lse, ra, rb = (torch.empty((1, Hq), device="cuda") for _ in range(3))
        tab_d = torch.from_numpy(tab).cuda()
        ctx = torch.tensor([S], dtype=torch.int32, device="cuda")
        sd = torch.tensor([5], dtype=torch.int64, device="cuda")

        def call():
            L.wc_decode_attn_meter(cache, 0, q, tab_d, ctx, sd, part, 1.0 / math.sqrt(D), 3, delta[0], *delta[1:],
                                   n_split)
            L.wc_lse_merge(part, 1, Hq, n_split, o, lse, ra, rb)

        for _ in range(20):
            call()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(iters):
            call()
        b.record()
        torch.cuda.synchronize()
        res["configs"][name] = {"us_per_decode_and_merge": round(a.elapsed_time(b) / iters * 1e3, 2),
                                "n_split": n_split}
    return res


def decode_bytes_ragged(lens, scales=True):
    """Algorithmic decode bytes of one layer over a ragged batch (meter on)."""
    per_tok = 128 + 128 + (8 if scales else 0) + 32
    return int(sum(int(S_) * HKV * per_tok + (-(-int(S_) // 16)) * 4 for S_ in lens)) + len(lens) * (HQ * D * 2 + 12)


HEADLINE_KERNEL = "decode_kernel<0, false, true, true, 0, false, 2>"
FLOOR_KERNEL = "decode_floor_kernel<0, true>"


def _counter_rows(d):
    """(kernel name, grid size, dispatch id, counter, value) of every row of
    the rocprofv3 counter_collection CSVs under directory d."""
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                k = {c.lower(): c for c in r}
                rows.append((r[k["kernel_name"]], int(r[k["grid_size"]]), int(r[k["dispatch_id"]]),
                             r[k["counter_name"]], float(r[k["counter_value"]])))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return rows


def reduce_counters(fetch_dir, write_dir, launches, B, S, floor_launches=0):
    """HBM bytes per launch of the headline decode from two rocprofv3 --pmc
    runs of bench.py (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each
    scaled by what the same counter reads for the three 1 GiB device copies
    that --copy-ref adds at the end of the run (1 GiB read and 1 GiB written
    per copy).  The decode's
    figure is the mean over its first `launches` dispatches (the warm-up and
    timed steps); the load floor's over its first `floor_launches`
    dispatches (the loops taken with the decode's, meter on)."""
    import numpy as np
    out = {"source_sha": decode_source_sha(), "batch": B, "ctx": S, "launches": launches}
    total = 0.0
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _counter_rows(d) if r[3] == name]
        # the 1 GiB copies of --copy-ref are the run's last three device copies
        copies = sorted((r for r in rows if "copyBuffer" in r[0]), key=lambda r: r[2])[-3:]
        if len(copies) < 3:
            raise SystemExit(f"{name}: no device copy dispatches (run bench.py with --copy-ref)")
        ref_kib = float(np.median([r[4] for r in copies]))
        factor = (1 << 20) / ref_kib                    # KiB that 1 GiB moves
        dec = sorted((r for r in rows if HEADLINE_KERNEL in r[0]), key=lambda r: r[2])[:launches]
        flo = sorted((r for r in rows if FLOOR_KERNEL in r[0]), key=lambda r: r[2])[:floor_launches]
        if len(dec) < launches:
            raise SystemExit(f"{name}: {len(dec)} headline decode dispatches, expected {launches}")
        kib = float(np.mean([r[4] for r in dec]))
        key = name.split("_")[0].lower()
        out[f"{key}_factor"] = factor
        out[f"{key}_copy_ref_KiB"] = ref_kib
        out[f"{key}_KiB_per_launch"] = kib
        out[f"{key}_bytes_per_launch"] = int(round(kib * 1024 * factor))
        if flo:
            out[f"floor_{key}_bytes_per_launch"] = int(round(float(np.mean([r[4] for r in flo])) * 1024 * factor))
        total += kib * 1024 * factor
    out["hbm_bytes_per_launch"] = int(round(total))
    out["algorithmic_bytes_per_launch"] = decode_bytes(B, S, True)
    return out


def trace_phases(kt_dir, warmup, steps, loops=10, iters=20):
    """Per-phase durations of the headline decode from a rocprofv3
    --kernel-trace run of the default bench line (same --warmup and
    --steps): its dispatches in order are the warm-up and timed steps, then
    `loops` rounds of one untimed and `iters` timed launches with block
    risks and the same without (the meter-off launches are another
    instance).  Returns the step mean and, per mode, the median of the loop
    means (us), next to the rocprofv3 statistics of every kernel."""
    import csv
    import glob
    import numpy as np
    rows = []
    for f in sorted(glob.glob(os.path.join(kt_dir, "**", "*kernel_trace.csv"), recursive=True)):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                rows.append((r["Kernel_Name"], int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    if not rows:
        raise SystemExit(f"no kernel_trace.csv under {kt_dir}")
    dec = sorted((r for r in rows if HEADLINE_KERNEL in r[0]), key=lambda r: r[1])
    us = [(r[2] - r[1]) / 1e3 for r in dec]
    n0 = warmup + steps
    out = {"headline_dispatches": len(dec), "steps_mean_us": round(float(np.mean(us[warmup:n0])), 2)}
    per = 2 * (iters + 1)
    risk = [float(np.mean(us[n0 + k * per + 1:n0 + k * per + 1 + iters])) for k in range(loops)]
    on = [float(np.mean(us[n0 + k * per + iters + 2:n0 + (k + 1) * per])) for k in range(loops)]
    out["risk_loops_median_us"] = round(float(np.median(risk)), 2)
    out["on_loops_median_us"] = round(float(np.median(on)), 2)
    flo = sorted((r for r in rows if FLOOR_KERNEL in r[0]), key=lambda r: r[1])
    if flo:
        fus = [(r[2] - r[1]) / 1e3 for r in flo]
        out["floor_first_loops_median_us"] = round(float(np.median(
            [np.mean(fus[k * (iters + 1) + 1:(k + 1) * (iters + 1)]) for k in range(loops)])), 2)
    stats = {}
    for f in sorted(glob.glob(os.path.join(kt_dir, "**", "*kernel_stats.csv"), recursive=True)):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                try:
                    stats[r["Name"]] = {"calls": int(r["Calls"]), "avg_us": round(float(r["AverageNs"]) / 1e3, 2),
                                        "min_us": round(float(r["MinNs"]) / 1e3, 2),
                                        "max_us": round(float(r["MaxNs"]) / 1e3, 2),
                                        "pct": round(float(r["Percentage"]), 2)}
                except (KeyError, ValueError):
                    continue
    out["kernel_stats"] = stats
    return out


def counter_means(dirs, launches, kernels=None):
    """Mean per dispatch of every counter in rocprofv3 --pmc runs (the
    directories given): over the first `launches` dispatches of the dithered
    INT8 and fp8 headline decode instances, or, with `kernels` (name
    substrings), over every dispatch of each kernel whose name holds one."""
    import numpy as np
    out = {}
    rows_all = [row for d in dirs for row in _counter_rows(d)]
    if kernels:
        names = sorted({r[0].split("(")[0] for r in rows_all if any(k in r[0] for k in kernels)})
    else:
        names = [HEADLINE_KERNEL, HEADLINE_KERNEL.replace("<0,", "<1,")]
    for name in names:
        acc = {}
        for d in dirs:
            rows = [r for r in _counter_rows(d) if name in r[0]]
            ids = sorted({r[2] for r in rows})
            if not kernels:
                ids = ids[:launches]
            for c in sorted({r[3] for r in rows}):
                per = {}
                for r in rows:
                    if r[3] == c:
                        per[r[2]] = per.get(r[2], 0.0) + r[4]
                acc[c] = float(np.mean([per[i] for i in ids if i in per]))
        out[name] = acc
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the decode reaches its steady rate after ~100-200 back-to-back launches
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--batch", type=int, default=32)
    ap.add_argument("--ctx", type=int, default=32768)
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the CPU baseline and the amd-smi power reading (the profiler runs)")
    ap.add_argument("--copy-ref", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill-write", "gate-flow", "gate-compare", "latency", "decode-bounds"],
                    help="decode: the 32 x 32768 decode step line (default); prefill-write: the 28-layer write path per scheme; "
                         "gate-flow: a ragged 64-sequence fp8 decode with the gate over several steps; "
                         "gate-compare: the same on the dithered INT8 cache, certificate gates against the tanh gate; "
                         "latency: decode + merge latency at the two parity sizes; "
                         "decode-bounds: the decode with its cache in HBM and L2-resident (compute alone)")
    ap.add_argument("--layers", type=int, default=28, help="gate-flow, gate-compare: resident layers")
    ap.add_argument("--reduce-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: turn the rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs of "
                         "`bench.py --steps K --warmup W --no-cpu --copy-ref` (same K, W, --batch, --ctx given here) "
                         "into the headline decode's HBM bytes per launch, written to " + COUNTERS)
    ap.add_argument("--trace-phases", metavar="KT_DIR",
                    help="no GPU: the headline decode's per-phase durations from a rocprofv3 --kernel-trace --stats "
                         "run of the default line (same --steps, --warmup)")
    ap.add_argument("--counter-means", nargs="+", metavar="DIR",
                    help="no GPU: per-dispatch means of the counters of rocprofv3 --pmc runs of "
                         "`bench.py --steps K --warmup W --no-cpu` for the INT8 and fp8 decode instances")
    ap.add_argument("--kernels", default=None,
                    help="--counter-means: comma-separated kernel name substrings (every dispatch of each)")
    args = ap.parse_args()
    if args.trace_phases:
        print(json.dumps(trace_phases(args.trace_phases, args.warmup, args.steps)), flush=True)
        return
    if args.counter_means:
        print(json.dumps(counter_means(args.counter_means, args.warmup + args.steps,
                                       args.kernels.split(",") if args.kernels else None)), flush=True)
        return
    if args.reduce_counters:
        res = reduce_counters(*args.reduce_counters, args.warmup + args.steps, args.batch, args.ctx,
                              floor_launches=10 * (max(args.steps, 10) + 1))
        with open(COUNTERS, "w") as fh:
            json.dump(res, fh, indent=1)
        print(json.dumps(res), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: runs on one GPU (sequences and KV heads shard without communication), "
              "so --gpus must be 1", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    if args.workload == "prefill-write":
        print(json.dumps(prefill_write(args.steps)), flush=True)
        return
    if args.workload == "gate-flow":
        print(json.dumps(gate_flow(args.layers, max(2, min(args.steps, 8)))), flush=True)
        return
    if args.workload == "latency":
        print(json.dumps(latency()), flush=True)
        return
    if args.workload == "decode-bounds":
        print(json.dumps(decode_bounds(args.batch, args.ctx)), flush=True)
        return
    if args.workload == "gate-compare":
        print(json.dumps(gate_flow(args.layers, max(2, min(args.steps, 8)), taus=(0.1, 0.05, 0.02), scheme="int8")),
              flush=True)
        return
    B, S = args.batch, args.ctx
    w = setup(B, S)
    step, decode, outs = make_step(w, B, S)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # each timed step's decode between a pair of HIP events on its stream (the
    # roofline's launch duration); recording them adds no synchronization
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3
    in_step = [e0.elapsed_time(e1) * 1e3 for e0, e1 in evs]
    t_in_step = float(np.mean(in_step))
    # the step's decode (meter on, block risks), the same kernel without block
    # risks, and with the meter off, each timed as 10 loops of back-to-back
    # launches taken in turn (risk, on, off, risk, ...) so that a drift of the
    # GPU's clocks over the run falls on all three alike; median and p10-p90
    # of the loop means
    iters = max(args.steps, 10)
    floor = make_floor(w, B, w["cache"])
    loops, on_loops, off_loops, floor_loops = [], [], [], []
    for _ in range(10):
        loops.append(time_decode(decode, iters, mask=3, with_risk=True))
        on_loops.append(time_decode(decode, iters, mask=3, with_risk=False))
        off_loops.append(time_decode(decode, iters, mask=0, with_risk=False))
        floor_loops.append(time_decode(floor, iters, mask=3, match=True))
    loops.sort()
    t_risk = float(np.median(loops))
    t_on = float(np.median(on_loops))
    t_off = float(np.median(off_loops))
    t_floor = float(np.median(floor_loops))
    fl = time_modes(floor, iters, {"free": dict(mask=3, match=False), "off": dict(mask=0, match=True)}, warm=20)
    dec_step_us = t_risk
    bytes_on = decode_bytes(B, S, True)
    ach = bytes_on / (dec_step_us * 1e-6) / 1e9             # back-to-back loops
    ach_step = bytes_on / (t_in_step * 1e-6) / 1e9          # inside the timed steps
    traffic = None
    if os.path.exists(COUNTERS):
        cnt = json.load(open(COUNTERS))
        if cnt.get("source_sha") == decode_source_sha() and cnt.get("batch") == B and cnt.get("ctx") == S:
            traffic = cnt.get("hbm_bytes_per_launch")
    value = step_bytes(B, S) / (ms_step * 1e-3) / 1e9
    props = torch.cuda.get_device_properties(0)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": f"decode B={B} S={S} Hq={HQ} Hkv={HKV} d={D} dithered-int8 Tier A+B, "
                               f"{NSPLIT} KV splits, 16-token pages (random permutation), append+decode+merge+gate",
                   "batch": B, "ctx": S, "n_split": NSPLIT, "tau": TAU},
        "roofline": {"bound": "hbm", "achieved": round(ach_step, 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach_step / PEAK_GBS, 4), "traffic": traffic},
        "decode_us_in_steps": round(t_in_step, 2),
        "decode_in_steps": f"the decode of each of the {args.steps} timed steps between HIP events on its stream, "
                           f"mean (the roofline's launch duration); decode_us and pct_peak time the same kernel "
                           f"back to back, where the board stays at its power limit throughout",
        "decode_us": round(dec_step_us, 2), "decode_us_p10": round(loops[1], 2), "decode_us_p90": round(loops[8], 2),
        "decode_loops": f"10 rounds of three loops of {iters} back-to-back launches (block risks, meter on, meter "
                        f"off, in turn); median, and p10, p90 of the loop means with block risks",
        "decode_meter_on_us": round(t_on, 2),
        "decode_meter_off_us": round(t_off, 2), "meter_overhead": round(t_on / t_off - 1, 4),
        "meter_overhead_with_risks": round(t_risk / t_off - 1, 4),
        "pct_peak": round(100 * ach / PEAK_GBS, 2),
        "kv_tokens_per_s": round(B * S / (dec_step_us * 1e-6), 1),
        "decode_steps_per_s_per_layer": round(1e6 / dec_step_us, 1),
        "load_floor": {"us": round(t_floor, 2), "GBps": round(bytes_on / (t_floor * 1e-6) / 1e9, 1),
                       "decode_pct_of_floor": round(100 * t_floor / dec_step_us, 2),
                       "us_without_lds_reservation": round(fl["free"], 2), "meter_off_us": round(fl["off"], 2),
                       "what": "wc_decode_load_floor: the decode's page loads (codes, scales, witness, page "
                               "table) on the same grid, no arithmetic; 10 loops taken in turn with the "
                               "decode's, median"},
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                   "compute_units": props.multi_processor_count},
        "decode_bytes": bytes_on, "step_bytes": step_bytes(B, S),
        "pages_paged_in": int(outs["paged"].item()) // 4096,
    }
    if not args.no_cpu:
        # board power and shader clock while the step's decode, then its load
        # floor, run back to back (amd-smi read once in the middle of about
        # four seconds of each): the INT8 decode runs at the board's power limit
        out["power_clock"] = {"decode_block_risks": power_clock(lambda: decode(mask=3, with_risk=True)),
                              "load_floor": power_clock(lambda: floor(mask=3, match=True))}
    out["fp8_variant"] = fp8_variant(w, B, S, iters)
    out["outlier_variant"] = [outlier_variant(w, B, S, iters, m) for m in (8, 16)]
    out["rtn_variant"] = scheme_variant(w, B, S, iters, "rtn")
    out["store16_variant"] = scheme_variant(w, B, S, iters, "store16")
    out["vcert_variant"] = vcert_variant(w, B, S, iters)
    out["needle_variant"] = needle_variant(w, B, S, iters, outs)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, B, S)
    if args.copy_ref:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_ref_bytes"] = 2 * src.numel() * 4
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Host logic of bench.py (no GPU): the algorithmic byte counts behind the
roofline, checked against the cache the binding allocates, and the one-GPU
exit."""
import os
import subprocess
import sys

import bench
from certified_kv_cache_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bytes_per_token(cache, names):
    """HBM bytes one (token, KV head) occupies in the arrays named, from the
    allocation itself (one layer, one page, one KV head)."""
    tot = sum(getattr(cache, n).numel() * getattr(cache, n).element_size() for n in names)
    return tot // cache.page_size


def test_decode_bytes_follow_the_cache_layout():
    c8 = L.KVCache(L.WC_DITHER_INT8, 1, 1, 1, device="cpu")
    f8 = L.KVCache(L.WC_FP8_E4M3, 1, 1, 1, device="cpu")
    on = _bytes_per_token(c8, ["k_codes", "v_codes", "k_scale", "v_scale", "witness"])
    off = _bytes_per_token(c8, ["k_codes", "v_codes", "k_scale", "v_scale"])
    fp8 = _bytes_per_token(f8, ["k_codes", "v_codes", "witness"])
    assert (on, off, fp8) == (296, 264, 288)
    B, S = 32, 32768
    per_launch = B * (S // 16) * 4 + B * bench.HQ * bench.D * 2 + B * 4 + B * 8   # table, q, lengths, seeds
    assert bench.decode_bytes(B, S, True) == B * S * bench.HKV * on + per_launch == 1242005888
    assert bench.decode_bytes(B, S, False) == B * S * bench.HKV * off + per_launch
    assert bench.decode_bytes(B, S, True, scales=False) == B * S * bench.HKV * fp8 + per_launch
    # a ragged last page counts its page-table entry once
    assert bench.decode_bytes(1, 17, True) - bench.decode_bytes(1, 16, True) == bench.HKV * on + 4


def test_more_than_one_gpu_exits_with_a_message():
    for args, env in [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})]:
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT, capture_output=True,
                           text=True, timeout=120, env={**os.environ, **env})
        assert r.returncode == 2, (args, env, r.returncode)
        assert "one GPU" in r.stderr and r.stdout == ""


def _counter_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    head = ("Correlation_Id,Dispatch_Id,Agent_Id,Queue_Id,Process_Id,Thread_Id,Grid_Size,Kernel_Id,Kernel_Name,"
            "Workgroup_Size,LDS_Block_Size,Scratch_Size,VGPR_Count,Accum_VGPR_Count,SGPR_Count,Counter_Name,"
            "Counter_Value,Start_Timestamp,End_Timestamp\n")
    with open(path, "w") as fh:
        fh.write(head)
        for i, (name, grid, counter, value) in enumerate(rows):
            fh.write(f'{i},{i + 1},1,1,1,1,{grid},7,"{name}",256,0,0,64,0,32,{counter},{value},0,1\n')


def test_counter_reducer(tmp_path):
    # two passes as rocprofv3 writes them: the decode's step dispatches come
    # first, timing loops after; the 1 GiB copies calibrate each counter
    dec = "void wc::" + bench.HEADLINE_KERNEL + "(wc_cache, wc::DecodeArgs)"
    other = "void wc::decode_kernel<0, false, true, true, 0, false, 1>(wc_cache, wc::DecodeArgs)"
    copy = "__amd_rocclr_copyBuffer"
    flo = "void wc::" + bench.FLOOR_KERNEL + "(wc_cache, wc::FloorArgs)"
    fetch = [(copy, 1 << 26, "FETCH_SIZE", 4108.0)]           # an earlier copy (a larger grid)
    fetch += [(dec, 100, "FETCH_SIZE", 600000 + i) for i in range(4)] + [(dec, 100, "FETCH_SIZE", 9e9),
                                                                          (other, 100, "FETCH_SIZE", 1.0),
                                                                          (copy, 64, "FETCH_SIZE", 5.0),
                                                                          (flo, 100, "FETCH_SIZE", 610000)]
    fetch += [(copy, 4096, "FETCH_SIZE", 524288)] * 3
    write = [(dec, 100, "WRITE_SIZE", 30000)] * 4 + [(copy, 4096, "WRITE_SIZE", 1048576)] * 3
    _counter_csv(str(tmp_path / "f" / "host" / "1_counter_collection.csv"), fetch)
    _counter_csv(str(tmp_path / "w" / "host" / "1_counter_collection.csv"), write)
    r = bench.reduce_counters(str(tmp_path / "f"), str(tmp_path / "w"), 4, 32, 32768, floor_launches=1)
    assert r["fetch_factor"] == 2.0 and r["write_factor"] == 1.0
    assert r["fetch_bytes_per_launch"] == round(600001.5 * 1024 * 2)
    assert r["write_bytes_per_launch"] == 30000 * 1024
    assert r["hbm_bytes_per_launch"] == r["fetch_bytes_per_launch"] + r["write_bytes_per_launch"]
    assert r["floor_fetch_bytes_per_launch"] == 610000 * 1024 * 2
    assert r["source_sha"] == bench.decode_source_sha() and r["algorithmic_bytes_per_launch"] == 1242005888


def test_trace_phases(tmp_path):
    # the headline instance's dispatches in bench order: 3 warm-up and 2 timed
    # steps, then rounds of (1 + 4) block-risk and (1 + 4) meter-on launches
    dec = "void wc::" + bench.HEADLINE_KERNEL + "(wc_cache, wc::DecodeArgs)"
    durs = [900, 900, 900, 250, 252]
    for k in range(3):
        durs += [999] + [240 + k] * 4 + [999] + [230 + k] * 4
    os.makedirs(tmp_path / "kt" / "host")
    with open(tmp_path / "kt" / "host" / "kt_kernel_trace.csv", "w") as fh:
        fh.write("Kernel_Name,Start_Timestamp,End_Timestamp\n")
        t = 0
        for d in durs:
            fh.write(f'"{dec}",{t},{t + d * 1000}\n')
            fh.write(f'"other",{t + 1},{t + 2}\n')
            t += 10 ** 7
    with open(tmp_path / "kt" / "host" / "kt_kernel_stats.csv", "w") as fh:
        fh.write("Name,Calls,TotalDurationNs,AverageNs,Percentage,MinNs,MaxNs,StdDev\n")
        fh.write(f'"{dec}",35,0,300000.0,90.5,230000,999000,1\n')
    r = bench.trace_phases(str(tmp_path / "kt"), 3, 2, loops=3, iters=4)
    assert r["headline_dispatches"] == 35 and r["steps_mean_us"] == 251.0
    assert r["risk_loops_median_us"] == 241.0 and r["on_loops_median_us"] == 231.0
    assert r["kernel_stats"][dec]["avg_us"] == 300.0 and r["kernel_stats"][dec]["calls"] == 35


def test_counter_means(tmp_path):
    dec = "void wc::" + bench.HEADLINE_KERNEL + "(wc_cache, wc::DecodeArgs)"
    wr = "void wc::write_rows_kernel<unsigned short, 0, false>(wc_cache, unsigned short const*)"
    rows = [(dec, 100, "SQ_INSTS_VALU", 10.0 * (i + 1)) for i in range(6)] + \
           [(wr, 100, "FETCH_SIZE", 5.0), (wr, 100, "FETCH_SIZE", 7.0)]
    _counter_csv(str(tmp_path / "s" / "h" / "1_counter_collection.csv"), rows)
    r = bench.counter_means([str(tmp_path / "s")], 4)
    assert r[bench.HEADLINE_KERNEL]["SQ_INSTS_VALU"] == 25.0      # the first four dispatches
    r = bench.counter_means([str(tmp_path / "s")], 4, kernels=["wc::write"])
    assert list(r) == ["void wc::write_rows_kernel<unsigned short, 0, false>"]
    assert r["void wc::write_rows_kernel<unsigned short, 0, false>"]["FETCH_SIZE"] == 6.0

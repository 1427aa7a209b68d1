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

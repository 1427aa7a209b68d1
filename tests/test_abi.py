"""CPU checks of the C ABI: the library loads, exports every function that
include/witcert.h declares, and rejects bad arguments on the host before
any launch (these calls never reach the device)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from certified_kv_cache_amd import _lib
    return _lib


def _declared():
    txt = open(os.path.join(ROOT, "include", "witcert.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(wc_[a-z_0-9]+)\s*\(", txt)))


def test_header_declares_the_four_entry_points():
    names = _declared()
    for fn in ["wc_write_kv", "wc_decode_attn_meter", "wc_lse_merge", "wc_gate_pagein"]:
        assert fn in names


def test_library_exports_every_declared_symbol():
    L = _lib()
    raw = ctypes.CDLL(L.LIB_PATH)
    for name in _declared():
        assert hasattr(raw, name), name
    assert set(_declared()) == set(L.EXPORTS)


def test_version_and_workspace_sizes():
    L = _lib()
    assert L.lib.wc_version().startswith(b"witcert")
    assert L.wc_decode_workspace_bytes(32, 28, 16) == 32 * 28 * 16 * 136 * 4
    assert L.wc_decode_workspace_bytes(-1, 28, 16) == 0
    assert L.wc_gate_workspace_bytes(2, 4, 10) > 0


def _cache(L, **kw):
    """A descriptor with fake non-NULL array pointers (never dereferenced on
    the host) and no exact pool unless asked for."""
    c = L.WcCache(L.WC_DITHER_INT8, 128, 4, 8, 16, 2, 10, *([1] * 9), 0)
    c.exact_slot = None
    c.exact_pool = None
    for k, v in kw.items():
        setattr(c, k, v)
    return c


POOL = dict(exact_slot=16, exact_pool=16, pool_capacity=4)


def test_write_rejects_bad_arguments():
    L = _lib()
    f = L.lib.wc_write_kv
    p = ctypes.c_void_p(16)
    ok = _cache(L)
    assert f(None, 0, 1, p, p, 1, 4, 0, p, p, p, None) == L.WC_EINVAL
    assert f(ctypes.byref(_cache(L, head_dim=64)), 0, 1, p, p, 1, 4, 0, p, p, p, None) == L.WC_EUNSUPPORTED
    assert f(ctypes.byref(ok), 1, 2, p, p, 1, 4, 0, p, p, p, None) == L.WC_EINVAL      # layer range
    assert f(ctypes.byref(ok), 0, 1, p, p, 7, 4, 0, p, p, p, None) == L.WC_EUNSUPPORTED  # dtype
    assert f(ctypes.byref(ok), 0, 2, p, p, 1, 4, 10, p, p, p, None) == L.WC_EINVAL     # layer stride
    assert f(ctypes.byref(_cache(L, page_size=32)), 0, 1, p, p, 1, 4, 0, p, p, p, None) == L.WC_EUNSUPPORTED
    assert f(ctypes.byref(_cache(L, scheme=2)), 0, 1, p, p, 1, 31, 0, p, p, p, None) == L.WC_EUNSUPPORTED
    assert f(ctypes.byref(_cache(L, scheme=9)), 0, 1, p, p, 1, 4, 0, p, p, p, None) == L.WC_EUNSUPPORTED
    assert f(ctypes.byref(_cache(L, k_scale=None)), 0, 1, p, p, 1, 4, 0, p, p, p, None) == L.WC_EINVAL
    assert f(ctypes.byref(ok), 0, 1, p, p, 1, 0, 0, p, p, p, None) == L.WC_OK         # nothing to do
    assert b"wc_write_kv" in L.lib.wc_last_error()


def test_decode_rejects_bad_arguments():
    L = _lib()
    f = L.lib.wc_decode_attn_meter
    p = ctypes.c_void_p(16)
    c = ctypes.byref(_cache(L))
    ws = L.wc_decode_workspace_bytes(2, 28, 4)

    def call(cache=c, layer=0, qd=1, B=2, Hq=28, mp=8, mask=3, dr=1e-2, ns=4, wsb=ws, br=None, seed=p):
        return f(cache, layer, p, qd, B, Hq, p, mp, p, seed, 0.088, mask, dr, 28, 28, 256, ns, p, wsb, br, None)

    assert call(wsb=ws - 1) == L.WC_EWORKSPACE
    assert call(Hq=30) == L.WC_EINVAL                 # not a multiple of Hkv
    assert call(Hq=4 * 17) == L.WC_EINVAL             # group larger than 16
    assert call(ns=0) == L.WC_EINVAL
    assert call(layer=2) == L.WC_EINVAL
    assert call(qd=5) == L.WC_EUNSUPPORTED
    assert call(mask=2) == L.WC_EINVAL                # Tier B without Tier A
    assert call(mask=8) == L.WC_EINVAL
    assert call(mask=0, br=p) == L.WC_EINVAL          # block risk needs the meter
    assert call(dr=0.0) == L.WC_EINVAL
    assert call(seed=None) == L.WC_EINVAL
    assert call(cache=ctypes.byref(_cache(L, scheme=1)), mask=3) == L.WC_EINVAL   # Tier B needs INT8
    assert call(cache=ctypes.byref(_cache(L, scheme=2))) == L.WC_EUNSUPPORTED
    assert call(cache=ctypes.byref(_cache(L, num_pages=0))) == L.WC_EUNSUPPORTED   # no physical page
    assert call(B=0) == L.WC_OK


def test_merge_and_gate_reject_bad_arguments():
    L = _lib()
    p = ctypes.c_void_p(16)
    assert L.lib.wc_lse_merge(None, 1, 1, 1, p, p, None, None, None, None, None, None) == L.WC_EINVAL
    assert L.lib.wc_lse_merge(p, 1, 1, 0, p, p, None, None, None, None, None, None) == L.WC_EINVAL
    g = L.lib.wc_gate_pagein
    c = ctypes.byref(_cache(L, scheme=1, **POOL))
    wsb = L.wc_gate_workspace_bytes(2, 4, 8)

    def call(cache=c, tau=0.2, mp=8, wsb=wsb, host=p):
        return g(cache, 0, p, p, None, 2, 28, p, mp, p, tau, -1, host, p, p, None, None, p, wsb, None)

    assert call(host=None) == L.WC_EINVAL
    assert call(tau=-1.0) == L.WC_EINVAL
    assert call(tau=1e6) == L.WC_EINVAL
    assert call(mp=65537) == L.WC_EINVAL              # block index beyond 16 bits
    assert call(wsb=1) == L.WC_EWORKSPACE
    assert call(cache=ctypes.byref(_cache(L, scheme=1, exact_pool=16, pool_capacity=4))) == L.WC_EINVAL
    assert L.lib.wc_dither_fill(1, 0, 0, -1, 4, p, None) == L.WC_EINVAL
    assert L.lib.wc_dither_fill(1, 0, 0, 0, 4, None, None) == L.WC_EINVAL


def test_outlier_bypass_rejects_bad_arguments():
    L = _lib()
    p = ctypes.c_void_p(16)
    sel = L.lib.wc_outlier_select
    assert sel(None, 1, 1, 64, 4, 0, 8, p, None) == L.WC_EINVAL
    assert sel(p, 1, 1, 64, 4, 0, 0, p, None) == L.WC_EINVAL          # m = 0
    assert sel(p, 1, 1, 64, 4, 0, 129, p, None) == L.WC_EINVAL        # m > d
    assert sel(p, 1, 2, 64, 4, 10, 8, p, None) == L.WC_EINVAL         # layer stride
    assert sel(p, 3, 1, 64, 4, 0, 8, p, None) == L.WC_EUNSUPPORTED    # dtype
    w = L.lib.wc_write_kv
    byp = dict(num_outliers=8, outlier_ch=16, k_outlier=16)
    assert w(ctypes.byref(_cache(L, **byp)), 0, 1, p, p, 0, 4, 0, p, p, p, None) == L.WC_EUNSUPPORTED  # fp32 in
    assert w(ctypes.byref(_cache(L, num_outliers=12, outlier_ch=16, k_outlier=16)), 0, 1, p, p, 1, 4, 0, p, p, p,
             None) == L.WC_EUNSUPPORTED
    assert w(ctypes.byref(_cache(L, scheme=1, **byp)), 0, 1, p, p, 1, 4, 0, p, p, p, None) == L.WC_EUNSUPPORTED
    assert w(ctypes.byref(_cache(L, num_outliers=8)), 0, 1, p, p, 1, 4, 0, p, p, p, None) == L.WC_EINVAL
    d = L.lib.wc_decode_attn_meter
    ws = L.wc_decode_workspace_bytes(2, 28, 4)

    def call(cache):
        return d(ctypes.byref(cache), 0, p, 1, 2, 28, p, 8, p, p, 0.088, 3, 1e-2, 28, 28, 256, 4, p, ws, None, None)

    assert call(_cache(L, num_outliers=4, outlier_ch=16, k_outlier=16)) == L.WC_EUNSUPPORTED
    assert call(_cache(L, num_outliers=16)) == L.WC_EINVAL                        # no side store


def test_tanh_gate_and_cmax_reject_bad_arguments():
    L = _lib()
    p = ctypes.c_void_p(16)
    g = L.lib.wc_gate_pagein_tanh
    c = ctypes.byref(_cache(L, scheme=1, **POOL))
    wsb = L.wc_gate_workspace_bytes(2, 4, 8)

    def call(cache=c, tau=0.2, mp=8, wsb=wsb, cm=p):
        return g(cache, 0, cm, 2, 28, p, mp, p, tau, -1, p, p, p, None, p, wsb, None)

    assert call(cm=None) == L.WC_EINVAL
    assert call(tau=-0.5) == L.WC_EINVAL
    assert call(mp=65537) == L.WC_EINVAL
    assert call(wsb=1) == L.WC_EWORKSPACE
    assert call(cache=ctypes.byref(_cache(L, scheme=1, exact_pool=16, pool_capacity=4))) == L.WC_EINVAL
    d = L.lib.wc_decode_attn_meter
    ws = L.wc_decode_workspace_bytes(2, 28, 4)
    cc = ctypes.byref(_cache(L))
    assert d(cc, 0, p, 1, 2, 28, p, 8, p, p, 0.088, 3 | L.WC_BLOCK_CMAX, 1e-2, 28, 28, 256, 4, p, ws, None,
             None) == L.WC_EINVAL                      # block maxima need the block output


def test_blackbox_schemes_reject_bad_arguments():
    L = _lib()
    p = ctypes.c_void_p(16)
    w = L.lib.wc_witness
    ok = ctypes.byref(_cache(L, scheme=L.WC_BF16_STORE))
    assert w(None, 0, 1, p, p, 1, 4, 0, p, 0, None) == L.WC_EINVAL
    assert w(ok, 0, 1, p, None, 1, 4, 0, p, 0, None) == L.WC_EINVAL
    assert w(ok, 1, 2, p, p, 1, 4, 0, p, 0, None) == L.WC_EINVAL              # layer range
    assert w(ok, 0, 1, p, p, 9, 4, 0, p, 0, None) == L.WC_EUNSUPPORTED        # dtype
    assert w(ctypes.byref(_cache(L, witness=None)), 0, 1, p, p, 1, 4, 0, p, 0, None) == L.WC_EINVAL
    assert w(ok, 0, 1, p, p, 1, 4, 0, p, 1, None) == L.WC_EINVAL              # no value witness array
    assert w(ok, 0, 1, p, p, 1, 4, 0, p, 2, None) == L.WC_EINVAL
    assert w(ok, 0, 1, p, p, 1, 0, 0, p, 0, None) == L.WC_OK                  # nothing to do
    wr = L.lib.wc_write_kv
    assert wr(ok, 0, 1, p, p, 0, 4, 0, p, p, p, None) == L.WC_EUNSUPPORTED  # the store takes bf16
    assert wr(ctypes.byref(_cache(L, scheme=L.WC_RTN_INT8, k_scale=None)), 0, 1, p, p, 1, 4, 0, p, p, p,
              None) == L.WC_EINVAL
    d = L.lib.wc_decode_attn_meter
    ws = L.wc_decode_workspace_bytes(2, 28, 4)

    def call(cache, mask=1):
        return d(ctypes.byref(cache), 0, p, 1, 2, 28, p, 8, p, p, 0.088, mask, 1e-2, 28, 28, 256, 4, p, ws, None, None)

    assert call(_cache(L, scheme=L.WC_RTN_INT8), mask=3) == L.WC_EINVAL      # Tier B needs the dither
    assert call(_cache(L, scheme=L.WC_BF16_STORE), mask=3) == L.WC_EINVAL
    assert call(_cache(L, scheme=L.WC_RTN_INT8, v_scale=None)) == L.WC_EINVAL
    assert call(_cache(L, scheme=L.WC_RTN_INT8, num_outliers=8, outlier_ch=16, k_outlier=16)) == L.WC_EUNSUPPORTED
    assert call(_cache(L), mask=1 | L.WC_METER_V) == L.WC_EINVAL              # no value witness array


def test_write_pages_rejects_bad_arguments():
    L = _lib()
    p = ctypes.c_void_p(16)
    f = L.lib.wc_write_kv_pages
    ok = ctypes.byref(_cache(L))
    assert f(None, 0, 1, p, p, 1, 4, 0, p, p, p, None) == L.WC_EINVAL
    assert f(ok, 0, 1, p, p, 1, 4, 0, None, p, p, None) == L.WC_EINVAL
    assert f(ok, 1, 2, p, p, 1, 4, 0, p, p, p, None) == L.WC_EINVAL              # layer range
    assert f(ok, 0, 1, p, p, 5, 4, 0, p, p, p, None) == L.WC_EUNSUPPORTED        # dtype
    assert f(ok, 0, 2, p, p, 1, 4, 10, p, p, p, None) == L.WC_EINVAL             # layer stride
    assert f(ctypes.byref(_cache(L, scheme=L.WC_KIVI2, page_size=32)), 0, 1, p, p, 1, 4, 0, p, p, p,
             None) == L.WC_EUNSUPPORTED
    assert f(ctypes.byref(_cache(L, scheme=L.WC_BF16_STORE)), 0, 1, p, p, 1, 4, 0, p, p, p, None) == L.WC_EUNSUPPORTED
    assert f(ctypes.byref(_cache(L, k_scale=None)), 0, 1, p, p, 1, 4, 0, p, p, p, None) == L.WC_EINVAL
    assert f(ok, 0, 1, p, p, 1, 0, 0, p, p, p, None) == L.WC_OK                  # nothing to do


def test_gate_refuses_a_host_store_the_device_cannot_map():
    """A pageable host buffer (here a numpy array) is refused with WC_EINVAL
    before any launch: every other argument is valid, so the refusal comes from
    the device-pointer lookup of host_exact_k (which fails for memory that was
    not allocated pinned, and on a machine without a GPU)."""
    import numpy as np
    L = _lib()
    p = ctypes.c_void_p(16)
    pageable = np.zeros((2, 10, 4, 16, 128), dtype=np.uint16)
    host = ctypes.c_void_p(pageable.ctypes.data)
    c = ctypes.byref(_cache(L, scheme=1, **POOL))
    wsb = L.wc_gate_workspace_bytes(2, 4, 8)
    rc = L.lib.wc_gate_pagein(c, 0, p, p, None, 2, 28, p, 8, p, 0.2, -1, host, p, p, None, None, p, wsb, None)
    assert rc == L.WC_EINVAL
    assert b"not pinned" in L.lib.wc_last_error()
    rc = L.lib.wc_gate_pagein_tanh(c, 0, p, 2, 28, p, 8, p, 0.2, -1, host, p, p, None, p, wsb, None)
    assert rc == L.WC_EINVAL
    assert b"not pinned" in L.lib.wc_last_error()


def test_gate_workspace_covers_the_sort_buffers():
    L = _lib()
    B, hkv, mp = 3, 4, 8192
    head = B * hkv * mp * 4 + B * hkv * 4
    assert L.wc_gate_workspace_bytes(B, hkv, mp) == ((head + 7) // 8) * 8 + 8 + 2 * B * hkv * mp * 8


def test_caches_with_an_exact_pool_take_bf16_keys():
    """The exact store is bf16: with exact_slot set, float32 keys are refused
    by every call that writes keys (they could not be stored exactly)."""
    L = _lib()
    p = ctypes.c_void_p(16)
    pooled = ctypes.byref(_cache(L, **POOL))
    assert L.lib.wc_write_kv(pooled, 0, 1, p, p, L.WC_F32, 4, 0, p, p, p, None) == L.WC_EUNSUPPORTED
    assert b"bf16" in L.lib.wc_last_error()
    assert L.lib.wc_write_kv(pooled, 0, 1, p, p, L.WC_BF16, 0, 0, p, p, p, None) == L.WC_OK
    assert L.lib.wc_write_kv_pages(pooled, 0, 1, p, p, L.WC_F32, 4, 0, p, p, p, None) == L.WC_EUNSUPPORTED
    store = ctypes.byref(_cache(L, scheme=L.WC_BF16_STORE, **POOL))
    assert L.lib.wc_witness(store, 0, 1, p, p, L.WC_F32, 4, 0, p, 0, None) == L.WC_EUNSUPPORTED
    # values carry no exact keys
    assert L.lib.wc_witness(ctypes.byref(_cache(L, scheme=L.WC_BF16_STORE, v_witness=16, **POOL)), 0, 1, p, p,
                            L.WC_F32, 0, 0, p, 1, None) == L.WC_OK
    no_pool = ctypes.byref(_cache(L, exact_slot=16))
    assert L.lib.wc_write_kv(no_pool, 0, 1, p, p, L.WC_BF16, 4, 0, p, p, p, None) == L.WC_EINVAL


def test_noalloc_gate_limit_and_refusal():
    """The header's WC_GATE_NOALLOC_MAX_BYTES is the binding's constant, and a
    request beyond it is refused on the host (WC_EWORKSPACE) before any
    device call."""
    L = _lib()
    txt = open(os.path.join(ROOT, "include", "witcert.h")).read()
    m = re.search(r"#define WC_GATE_NOALLOC_MAX_BYTES \(\(size_t\)(\d+) << (\d+)\)", txt)
    assert m and int(m.group(1)) << int(m.group(2)) == L.GATE_NOALLOC_MAX_BYTES
    p = ctypes.c_void_p(16)
    c = ctypes.byref(_cache(L, scheme=1, **POOL))
    assert L.wc_gate_workspace_bytes(64, 4, 65536) > L.GATE_NOALLOC_MAX_BYTES
    rc = L.lib.wc_gate_pagein_noalloc(c, 0, p, p, None, 64, 28, p, 65536, p, 0.2, -1, p, p, p, None, None, None)
    assert rc == L.WC_EWORKSPACE and b"scratch" in L.lib.wc_last_error()
    assert L.lib.wc_gate_pagein_noalloc(None, 0, p, p, None, 2, 28, p, 8, p, 0.2, -1, p, p, p, None, None,
                                        None) == L.WC_EINVAL


def test_load_floor_rejects_bad_arguments():
    L = _lib()
    f = L.lib.wc_decode_load_floor
    p = ctypes.c_void_p(16)
    ok = ctypes.byref(_cache(L))
    assert f(None, 0, 1, 8, p, 4, p, 1, 3, 1, p, None) == L.WC_EINVAL
    assert f(ok, 0, 1, 8, None, 4, p, 1, 3, 1, p, None) == L.WC_EINVAL                # page table
    assert f(ok, 0, 1, 8, p, 4, p, 1, 3, 1, None, None) == L.WC_EINVAL                # sink
    assert f(ctypes.byref(_cache(L, head_dim=64)), 0, 1, 8, p, 4, p, 1, 3, 1, p, None) == L.WC_EUNSUPPORTED
    assert f(ctypes.byref(_cache(L, scheme=2)), 0, 1, 8, p, 4, p, 1, 3, 1, p, None) == L.WC_EUNSUPPORTED
    assert f(ctypes.byref(_cache(L, num_pages=0)), 0, 1, 8, p, 4, p, 1, 3, 1, p, None) == L.WC_EUNSUPPORTED
    assert f(ok, 2, 1, 8, p, 4, p, 1, 3, 1, p, None) == L.WC_EINVAL                   # layer range
    assert f(ok, 0, 1, 7, p, 4, p, 1, 3, 1, p, None) == L.WC_EINVAL                   # Hq % Hkv
    assert f(ok, 0, 1, 8, p, 4, p, 0, 3, 1, p, None) == L.WC_EINVAL                   # n_split
    assert f(ok, 0, 1, 8, p, 4, p, 1, 1 << 9, 1, p, None) == L.WC_EINVAL              # mask bits
    assert f(ctypes.byref(_cache(L, witness=None)), 0, 1, 8, p, 4, p, 1, 1, 1, p, None) == L.WC_EINVAL
    assert f(ctypes.byref(_cache(L, k_scale=None)), 0, 1, 8, p, 4, p, 1, 0, 1, p, None) == L.WC_EINVAL
    big = ctypes.byref(_cache(L, num_pages=1 << 20, num_kv_heads=4))                  # 8 GB per layer
    assert f(big, 0, 1, 8, p, 4, p, 1, 3, 1, p, None) == L.WC_EUNSUPPORTED
    assert b"4 GB" in L.lib.wc_last_error()
    assert f(ok, 0, 0, 8, p, 4, p, 1, 3, 1, p, None) == L.WC_OK                       # nothing to do

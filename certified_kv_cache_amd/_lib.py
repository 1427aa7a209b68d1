"""ctypes binding of libwitcert.so: argument marshalling only.

Every step of the hot path runs in the HIP library; this module turns torch
tensors into pointers and streams and raises on error codes.  It never falls
back to anything: if the library is missing, importing fails loudly.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwitcert.so")

WC_OK, WC_EINVAL, WC_EUNSUPPORTED, WC_EWORKSPACE, WC_EHIP = 0, -1, -2, -3, -4
WC_DITHER_INT8, WC_FP8_E4M3, WC_KIVI2, WC_RTN_INT8, WC_BF16_STORE = 0, 1, 2, 3, 4
WC_F32, WC_BF16 = 0, 1
WC_METER_A, WC_METER_B, WC_BLOCK_CMAX, WC_METER_V = 1, 2, 4, 8
PARTIAL = 136

_c_void_p = ctypes.c_void_p
_i32, _i64, _u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64


class WcCache(ctypes.Structure):
    _fields_ = [("scheme", _i32), ("head_dim", _i32), ("num_kv_heads", _i32), ("num_bands", _i32),
                ("page_size", _i32), ("num_layers", _i32), ("num_pages", _i64),
                ("k_codes", _c_void_p), ("v_codes", _c_void_p), ("k_scale", _c_void_p),
                ("v_scale", _c_void_p), ("k_aux", _c_void_p), ("v_aux", _c_void_p),
                ("witness", _c_void_p), ("exact_slot", _c_void_p), ("exact_pool", _c_void_p),
                ("pool_capacity", _i64), ("num_outliers", _i32),
                ("reserved", _i32), ("outlier_ch", _c_void_p), ("k_outlier", _c_void_p), ("v_witness", _c_void_p)]


class WitcertError(RuntimeError):
    def __init__(self, fn, code, text):
        super().__init__(f"{fn} returned {code}: {text}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m certified_kv_cache_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = _c_void_p
    sig = {
        "wc_write_kv": [P, ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int, _i64, _i64, P, P, P, P],
        "wc_decode_attn_meter": [P, ctypes.c_int, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, ctypes.c_int,
                                 P, P, ctypes.c_float, ctypes.c_uint, ctypes.c_double, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_int, ctypes.c_int, P, ctypes.c_size_t, P, P],
        "wc_lse_merge": [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P, P, P, P, P, P],
        "wc_decode_load_floor": [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, ctypes.c_int, P, ctypes.c_int,
                                 ctypes.c_uint, ctypes.c_int, P, P],
        "wc_gate_pagein": [P, ctypes.c_int, P, P, P, ctypes.c_int, ctypes.c_int, P, ctypes.c_int, P,
                           ctypes.c_double, _i64, P, P, P, P, P, P, ctypes.c_size_t, P],
        "wc_dither_fill": [_u64, ctypes.c_int, ctypes.c_int, _i64, _i64, P, P],
        "wc_outlier_select": [P, ctypes.c_int, ctypes.c_int, _i64, ctypes.c_int, _i64, ctypes.c_int, P, P],
        "wc_witness": [P, ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int, _i64, _i64, P, ctypes.c_int, P],
        "wc_write_kv_pages": [P, ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int, _i64, _i64, P, P, P, P],
        "wc_gate_pagein_tanh": [P, ctypes.c_int, P, ctypes.c_int, ctypes.c_int, P, ctypes.c_int, P, ctypes.c_double,
                                _i64, P, P, P, P, P, ctypes.c_size_t, P],
        "wc_gate_pagein_noalloc": [P, ctypes.c_int, P, P, P, ctypes.c_int, ctypes.c_int, P, ctypes.c_int, P,
                                   ctypes.c_double, _i64, P, P, P, P, P, P],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.wc_decode_workspace_bytes.argtypes = [ctypes.c_int] * 3
    lib.wc_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.wc_gate_workspace_bytes.argtypes = [ctypes.c_int] * 3
    lib.wc_gate_workspace_bytes.restype = ctypes.c_size_t
    lib.wc_last_error.restype = ctypes.c_char_p
    lib.wc_version.restype = ctypes.c_char_p
    return lib


lib = _load()

EXPORTS = ["wc_write_kv", "wc_decode_attn_meter", "wc_decode_workspace_bytes", "wc_lse_merge", "wc_decode_load_floor",
           "wc_gate_pagein", "wc_gate_pagein_tanh", "wc_gate_pagein_noalloc", "wc_gate_workspace_bytes",
           "wc_dither_fill", "wc_outlier_select", "wc_witness", "wc_write_kv_pages", "wc_last_error", "wc_version"]

# scratch of wc_gate_pagein_noalloc (the header's WC_GATE_NOALLOC_MAX_BYTES)
GATE_NOALLOC_MAX_BYTES = 16 << 20


def _check(fn, code):
    if code != WC_OK:
        raise WitcertError(fn, code, lib.wc_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return WC_F32
    if t.dtype == torch.bfloat16:
        return WC_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


# ---------------------------------------------------------------- cache allocation
class KVCache:
    """Device tensors of one paged cache (all layers) plus its C descriptor."""

    def __init__(self, scheme, num_layers, num_pages, num_kv_heads, device="cuda", pool_capacity=0,
                 page_size=None, num_outliers=0, v_witness=False):
        self.scheme = scheme
        self.L, self.P, self.H = num_layers, num_pages, num_kv_heads
        ps = page_size or (32 if scheme == WC_KIVI2 else 16)
        self.page_size = ps
        u8 = dict(dtype=torch.uint8, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        shp = (num_layers, num_pages, num_kv_heads)
        if scheme == WC_KIVI2:
            self.k_codes = torch.zeros(shp + (128, 8), **u8)
            self.v_codes = torch.zeros(shp + (32, 32), **u8)
            self.k_aux = torch.zeros(shp + (128, 2), **f32)
            self.v_aux = torch.zeros(shp + (32, 4, 2), **f32)
            self.k_scale = self.v_scale = None
        elif scheme == WC_BF16_STORE:
            # bf16 [8-channel group in 32][32-channel group][token][8] and
            # [channel pair in 8][token group][8-channel group][channel parity][token]
            self.k_codes = torch.zeros(shp + (4, 4, 16, 8), dtype=torch.int16, device=device)
            self.v_codes = torch.zeros(shp + (4, 4, 16, 2, 4), dtype=torch.int16, device=device)
            self.k_aux = self.v_aux = None
            self.k_scale = self.v_scale = None
        else:
            # [half][32-channel group][token][16 channels] and
            # [half][token group][8-channel group][channel][token]
            self.k_codes = torch.zeros(shp + (2, 4, 16, 16), **u8)
            self.v_codes = torch.zeros(shp + (2, 4, 16, 4, 4), **u8)
            self.k_aux = self.v_aux = None
            if scheme in (WC_DITHER_INT8, WC_RTN_INT8):
                self.k_scale = torch.zeros(shp + (16,), **f32)
                self.v_scale = torch.zeros(shp + (16,), **f32)
            else:
                self.k_scale = self.v_scale = None
        self.witness = torch.zeros(shp + (ps, 8), **f32)
        # value witness ||v^ - v|| per token (the value certificate), optional
        self.v_witness = torch.zeros(shp + (ps,), **f32) if v_witness else None
        self.pool_capacity = pool_capacity
        if pool_capacity > 0:
            # repaired blocks' exact keys: bf16 [slot][token][128]
            self.exact_slot = torch.full(shp, -1, dtype=torch.int32, device=device)
            self.exact_pool = torch.zeros((pool_capacity, 16, 128), dtype=torch.bfloat16, device=device)
        else:
            self.exact_slot = self.exact_pool = None
        # outlier bypass: channels [L][Hkv][m] (filled by wc_outlier_select or
        # the caller) and the exact bf16 keys on them [L][P][Hkv][16][m]
        self.num_outliers = num_outliers
        if num_outliers > 0:
            self.outlier_ch = torch.zeros((num_layers, num_kv_heads, num_outliers), dtype=torch.int32,
                                          device=device)
            self.k_outlier = torch.zeros(shp + (16, num_outliers), dtype=torch.int16, device=device)
        else:
            self.outlier_ch = self.k_outlier = None
        self.desc = WcCache(scheme, 128, num_kv_heads, 8, ps, num_layers, num_pages,
                            *[t.data_ptr() if t is not None else None for t in
                              (self.k_codes, self.v_codes, self.k_scale, self.v_scale, self.k_aux,
                               self.v_aux, self.witness, self.exact_slot, self.exact_pool)],
                            pool_capacity, num_outliers, 0,
                            *[t.data_ptr() if t is not None else None for t in
                              (self.outlier_ch, self.k_outlier, self.v_witness)])

    def ref(self):
        return ctypes.byref(self.desc)


# ---------------------------------------------------------------- entry points
def wc_write_kv(cache, k, v, slot, pos, seed, layer0=0, stream=None):
    """k, v: [n_layers, n_tok, Hkv, 128] or [n_tok, Hkv, 128] (bf16 or fp32, contiguous)."""
    if k.dim() == 3:
        k, v = k[None], v[None]
    assert k.is_contiguous() and v.is_contiguous() and k.shape == v.shape and k.dtype == v.dtype
    n_layers, n_tok = k.shape[0], k.shape[1]
    _check("wc_write_kv", lib.wc_write_kv(cache.ref(), layer0, n_layers, _ptr(k), _ptr(v), _dtype_code(k), n_tok,
                                          n_tok * k.shape[2] * k.shape[3], _ptr(slot), _ptr(pos), _ptr(seed),
                                          _stream(stream)))


def wc_write_kv_pages(cache, k, v, pages, pos0, seed, layer0=0, stream=None):
    """k, v: [n_layers, 16 * n_pages, Hkv, 128] or [16 * n_pages, Hkv, 128]; pages, pos0 int32 [n_pages],
    seed int64 [n_pages]."""
    if k.dim() == 3:
        k, v = k[None], v[None]
    assert k.is_contiguous() and v.is_contiguous() and k.shape == v.shape and k.dtype == v.dtype
    n_layers, n_tok = k.shape[0], k.shape[1]
    assert n_tok % 16 == 0 and pages.numel() == n_tok // 16
    _check("wc_write_kv_pages", lib.wc_write_kv_pages(cache.ref(), layer0, n_layers, _ptr(k), _ptr(v), _dtype_code(k),
                                                      n_tok // 16, n_tok * k.shape[2] * k.shape[3], _ptr(pages),
                                                      _ptr(pos0), _ptr(seed), _stream(stream)))


def wc_witness(cache, x, xhat, slot, layer0=0, values=False, stream=None):
    """x, xhat: [n_layers, n_tok, Hkv, 128] or [n_tok, Hkv, 128] (same dtype, contiguous);
    values=True stores the value witness instead of the banded key witness."""
    if x.dim() == 3:
        x, xhat = x[None], xhat[None]
    assert x.is_contiguous() and xhat.is_contiguous() and x.shape == xhat.shape and x.dtype == xhat.dtype
    n_layers, n_tok = x.shape[0], x.shape[1]
    _check("wc_witness", lib.wc_witness(cache.ref(), layer0, n_layers, _ptr(x), _ptr(xhat), _dtype_code(x), n_tok,
                                        n_tok * x.shape[2] * x.shape[3], _ptr(slot), int(bool(values)),
                                        _stream(stream)))


def wc_decode_workspace_bytes(B, Hq, n_split):
    return lib.wc_decode_workspace_bytes(B, Hq, n_split)


def wc_decode_attn_meter(cache, layer, q, page_table, ctx_len, seed, partials, sm_scale, meter_mask,
                         delta_req, L, H, T, n_split, block_logrisk=None, stream=None):
    assert q.is_contiguous() and page_table.is_contiguous()
    B, Hq = q.shape[0], q.shape[1]
    _check("wc_decode_attn_meter", lib.wc_decode_attn_meter(
        cache.ref(), layer, _ptr(q), _dtype_code(q), B, Hq, _ptr(page_table), page_table.shape[1],
        _ptr(ctx_len), _ptr(seed), float(sm_scale), int(meter_mask), float(delta_req), L, H, T, n_split,
        _ptr(partials), partials.numel() * partials.element_size(), _ptr(block_logrisk), _stream(stream)))


def wc_decode_load_floor(cache, layer, Hq, page_table, ctx_len, n_split, meter_mask, sink, match_residency=True,
                         stream=None):
    assert page_table.is_contiguous()
    _check("wc_decode_load_floor", lib.wc_decode_load_floor(
        cache.ref(), layer, page_table.shape[0], Hq, _ptr(page_table), page_table.shape[1], _ptr(ctx_len), n_split,
        int(meter_mask), int(bool(match_residency)), _ptr(sink), _stream(stream)))


def wc_lse_merge(partials, B, Hq, n_split, o, lse, meter_a=None, meter_b=None, tanh_a=None, tanh_b=None,
                 meter_v=None, stream=None):
    _check("wc_lse_merge", lib.wc_lse_merge(_ptr(partials), B, Hq, n_split, _ptr(o), _ptr(lse), _ptr(meter_a),
                                            _ptr(meter_b), _ptr(tanh_a), _ptr(tanh_b), _ptr(meter_v),
                                            _stream(stream)))


def wc_gate_workspace_bytes(B, Hkv, max_pages):
    return lib.wc_gate_workspace_bytes(B, Hkv, max_pages)


def wc_gate_pagein(cache, layer, block_logrisk, lse, page_table, ctx_len, tau, host_exact_k, pool_used,
                   bytes_paged, workspace, budget_blocks=-1, selected=None, rho_fx=None, meter=None, stream=None):
    B, Hq, max_pages = block_logrisk.shape
    _check("wc_gate_pagein", lib.wc_gate_pagein(
        cache.ref(), layer, _ptr(block_logrisk), _ptr(lse), _ptr(meter), B, Hq, _ptr(page_table), max_pages,
        _ptr(ctx_len),
        float(tau), int(budget_blocks), _ptr(host_exact_k), _ptr(pool_used), _ptr(bytes_paged), _ptr(selected),
        _ptr(rho_fx), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def wc_gate_pagein_noalloc(cache, layer, block_logrisk, lse, page_table, ctx_len, tau, host_exact_k, pool_used,
                           bytes_paged, budget_blocks=-1, selected=None, rho_fx=None, meter=None, stream=None):
    B, Hq, max_pages = block_logrisk.shape
    _check("wc_gate_pagein_noalloc", lib.wc_gate_pagein_noalloc(
        cache.ref(), layer, _ptr(block_logrisk), _ptr(lse), _ptr(meter), B, Hq, _ptr(page_table), max_pages,
        _ptr(ctx_len), float(tau), int(budget_blocks), _ptr(host_exact_k), _ptr(pool_used), _ptr(bytes_paged),
        _ptr(selected), _ptr(rho_fx), _stream(stream)))


def wc_outlier_select(x, m, channels, stream=None):
    """x: [n_layers, n_tok, Hkv, 128] or [n_tok, Hkv, 128] (bf16 or fp32, contiguous);
    channels: int32 [n_layers, Hkv, m]."""
    if x.dim() == 3:
        x = x[None]
    assert x.is_contiguous() and channels.dtype == torch.int32 and channels.is_contiguous()
    n_layers, n_tok, hkv = x.shape[0], x.shape[1], x.shape[2]
    assert channels.numel() == n_layers * hkv * m
    _check("wc_outlier_select", lib.wc_outlier_select(_ptr(x), _dtype_code(x), n_layers, n_tok, hkv,
                                                      n_tok * hkv * x.shape[3], m, _ptr(channels),
                                                      _stream(stream)))


def wc_gate_pagein_tanh(cache, layer, block_cmax, page_table, ctx_len, tau, host_exact_k, pool_used, bytes_paged,
                        workspace, budget_blocks=-1, selected=None, stream=None):
    B, Hq, max_pages = block_cmax.shape
    _check("wc_gate_pagein_tanh", lib.wc_gate_pagein_tanh(
        cache.ref(), layer, _ptr(block_cmax), B, Hq, _ptr(page_table), max_pages, _ptr(ctx_len), float(tau),
        int(budget_blocks), _ptr(host_exact_k), _ptr(pool_used), _ptr(bytes_paged), _ptr(selected),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def wc_dither_fill(seed, layer, kv_head, pos0, n_pos, out, stream=None):
    _check("wc_dither_fill", lib.wc_dither_fill(int(seed), layer, kv_head, pos0, n_pos, _ptr(out), _stream(stream)))


"""Write path: quantizers and the band-norm witness.  Test infrastructure only.

Sources (WitCert pages):

* Subtractively-dithered INT8, x^ = s(round(x/s + xi) - xi) with xi
  regenerated at read time: m.montaan.com summary, Tier B paragraph.
* Witness w_{t,b} = ||r_{t,b}||, the Euclidean norm of the residual
  r_t = x^_t - x_t over band b, stored once per token at write time
  (32 B per token per head for 8 fp32 bands): summary, witness-theorem and
  implementation paragraphs.
* fp8 raw cast and kivi-2bit as black-box schemes: summary, RULER results
  paragraph ("fp8 raw", "kivi-2bit raw"); round-to-nearest INT8 ("rtn-int8")
  is the third scheme measured there.
* Any scheme given as one tensor function x^ = f(x) is metered through the
  same witness of its residual (summary implementation paragraph; the
  abstract's scheme registration).

Readings where the pages are silent:

* Scale per (token, KV head) row: s = absmax/127 and the reciprocal
  inv_s = 127/absmax, both correctly rounded float32 divisions; x/s is
  evaluated as fp32(x * inv_s).  The sum with the dither is a float32 add
  and round() is round-half-even, the result clamped to [-128, 127].
  An all-zero row stores s = 0 and code 0 (its reconstruction is 0).
* fp8 is OCP e4m3fn, round-to-nearest-even, saturating at +-448.
* 2-bit: per group, mn/mx are the group min and max, scale =
  fp32(fp32(mx - mn) / 3), code = clamp(rint(fp32(fp32(x - mn) * fp32(1/scale))),
  0, 3) (code 0 if scale is 0) and x^ = fp32(mn + fp32(code * scale)).
  Keys are grouped over 32 consecutive tokens of one channel, values over 32
  consecutive channels of one token.
* The witness is stored for keys only (32 B/token/head).
* RTN INT8 uses the same row scale as the dithered quantizer, with no
  dither: code = clamp(rint(fp32(x * inv_s)), -128, 127), x^ = s code.
"""
import numpy as np

from .rope import band_dims

F32 = np.float32


def dither_int8(x, xi):
    """Dithered INT8 of rows x (float32 [n, d]) with dither xi (float32 [n, d]).

    Returns (codes int8 [n, d], s float32 [n], inv_s float32 [n]).  The float32
    steps are the exact op sequence the GPU runs, each correctly rounded.
    """
    x = np.asarray(x, dtype=F32)
    xi = np.asarray(xi, dtype=F32)
    absmax = np.max(np.abs(x), axis=-1)
    zero = absmax == 0
    safe = np.where(zero, F32(1), absmax).astype(F32)
    s = np.where(zero, F32(0), safe / F32(127)).astype(F32)
    inv = np.where(zero, F32(0), F32(127) / safe).astype(F32)
    y = (x * inv[:, None]).astype(F32)
    y = (y + xi).astype(F32)
    code = np.clip(np.rint(y), -128, 127)
    code = np.where(zero[:, None], 0, code).astype(np.int8)
    return code, s, inv


def dequant_dither_int8(code, s, xi):
    """x^ = s (code - xi), exact in float64."""
    return s.astype(np.float64)[:, None] * (code.astype(np.float64) - xi.astype(np.float64))


def rtn_int8(x):
    """Round-to-nearest INT8 of rows x (float32 [n, d]): (codes int8, s, inv_s).

    Same float32 row scale as dither_int8; the code is the nearest level of
    x * inv_s (rint: half to even), clamped to [-128, 127]; all-zero rows code 0.
    """
    x = np.asarray(x, dtype=F32)
    absmax = np.max(np.abs(x), axis=-1)
    zero = absmax == 0
    safe = np.where(zero, F32(1), absmax).astype(F32)
    s = np.where(zero, F32(0), safe / F32(127)).astype(F32)
    inv = np.where(zero, F32(0), F32(127) / safe).astype(F32)
    y = (x * inv[:, None]).astype(F32)
    code = np.clip(np.rint(y), -128, 127)
    code = np.where(zero[:, None], 0, code).astype(np.int8)
    return code, s, inv


def dequant_rtn_int8(code, s):
    """x^ = s code, exact in float64."""
    return s.astype(np.float64)[:, None] * code.astype(np.float64)


def fp8_e4m3(x):
    """OCP e4m3fn cast by the format definition: RNE, saturating at +-448.

    Returns (code uint8, value float64).  Layout: sign bit 7, exponent bits
    6..3 (bias 7), mantissa bits 2..0; exponent field 0 is subnormal
    (m * 2**-9); the all-ones pattern S.1111.111 is NaN and never produced.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = (np.signbit(x)).astype(np.uint8)
    a = np.abs(x)
    code = np.zeros(a.shape, dtype=np.int64)
    val = np.zeros(a.shape, dtype=np.float64)
    sat = a > 448.0
    sub = (a < 2.0 ** -6) & ~sat
    nrm = ~sat & ~sub
    # subnormal range: grid step 2**-9
    qs = np.rint(a[sub] * 2.0 ** 9)
    code[sub] = qs.astype(np.int64)          # qs == 8 is the smallest normal
    val[sub] = qs * 2.0 ** -9
    # normal range: 3 mantissa bits
    an = a[nrm]
    _, e2 = np.frexp(an)                      # an = m * 2**e2, m in [0.5, 1)
    e = e2.astype(np.int64) - 1               # an in [2**e, 2**(e+1))
    q = np.rint(np.ldexp(an, -e + 3))         # in [8, 16]
    carry = q == 16
    q = np.where(carry, 8, q)
    e = np.where(carry, e + 1, e)
    code[nrm] = ((e + 7) << 3) | (q.astype(np.int64) - 8)
    val[nrm] = np.ldexp(q, e - 3)
    code[sat] = 0x7E
    val[sat] = 448.0
    code = code | (sign.astype(np.int64) << 7)
    val = np.where(sign == 1, -val, val)
    return code.astype(np.uint8), val


def fp8_e4m3_decode(code):
    """Value of e4m3fn codes (float64), by the format definition."""
    code = np.asarray(code, dtype=np.int64)
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 7
    v = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.ldexp(1.0, e - 7 - 3))
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return np.where(s == 1, -v, v)


def quant2_groups(x):
    """2-bit asymmetric quantization of groups along the last axis.

    x: float32 [..., g].  Returns (code uint8 [..., g] in 0..3, scale float32
    [...], mn float32 [...], xhat float32 [..., g]).
    """
    x = np.asarray(x, dtype=F32)
    mn = np.min(x, axis=-1).astype(F32)
    mx = np.max(x, axis=-1).astype(F32)
    rng = (mx - mn).astype(F32)
    scale = (rng / F32(3)).astype(F32)
    zero = scale == 0
    inv = np.where(zero, F32(0), F32(1) / np.where(zero, F32(1), scale)).astype(F32)
    y = ((x - mn[..., None]).astype(F32) * inv[..., None]).astype(F32)
    code = np.clip(np.rint(y), 0, 3)
    code = np.where(zero[..., None], 0, code).astype(np.uint8)
    xhat = (mn[..., None] + (code.astype(F32) * scale[..., None]).astype(F32)).astype(F32)
    return code, scale, mn, xhat


def kivi2_keys(k):
    """Keys: groups of 32 consecutive tokens per channel.  k float32 [n, d], n % 32 == 0."""
    n, d = k.shape
    assert n % 32 == 0
    g = k.reshape(n // 32, 32, d).transpose(0, 2, 1)      # [n/32, d, 32]
    code, scale, mn, xhat = quant2_groups(g)
    return (code.transpose(0, 2, 1).reshape(n, d), scale, mn,
            xhat.transpose(0, 2, 1).reshape(n, d))


def kivi2_values(v):
    """Values: groups of 32 consecutive channels per token.  v float32 [n, d]."""
    n, d = v.shape
    assert d % 32 == 0
    g = v.reshape(n, d // 32, 32)
    code, scale, mn, xhat = quant2_groups(g)
    return code.reshape(n, d), scale, mn, xhat.reshape(n, d)


def witness_v(v, vhat):
    """Value witness w^V_t = ||v^_t - v_t|| over all channels, float64 [n].

    Reading (the pages define witnesses for keys only): the value side of the
    certificate needs the size of each value's residual; values are not
    rotated by RoPE, so one norm per token suffices.
    """
    r = np.asarray(vhat, dtype=np.float64) - np.asarray(v, dtype=np.float64)
    return np.sqrt(np.sum(r * r, axis=-1))


def witness(x, xhat, num_bands=8):
    """w_{t,b} = ||xhat_t - x_t|| over band b, float64 [n, num_bands]."""
    r = np.asarray(xhat, dtype=np.float64) - np.asarray(x, dtype=np.float64)
    dims = band_dims(r.shape[-1], num_bands)
    return np.sqrt(np.sum(r[..., dims] ** 2, axis=-1))

"""Counter-hash dither, regenerated at read time.  Test infrastructure only.

WitCert (m.montaan.com summary, Tier B paragraph) quantizes with subtractive
dither x^ = s(round(x/s + xi) - xi), xi ~ U[-1/2, 1/2), and regenerates xi
deterministically when the cache is read instead of storing it; the draw is
a counter hash of (seed, layer, head, token, channel).  The pages do not fix
the generator.  Reading used here:

* The generator is the ``pcg`` hash published by Jarzynski and Olano,
  "Hash Functions for GPU Rendering", JCGT 9(3), 2020 (an RXS-M-XS output
  permutation applied to one LCG step of the input).
* A 32-bit key is chained from the sequence seed (64 bit), the layer and the
  KV head::

      key = pcg(pcg(pcg(seed_hi) ^ seed_lo) ^ layer) ^ kv_head)

* Each 32-bit hash word yields two 16-bit draws (low half = even channel),
  one word per (token, channel pair)::

      word = pcg((key + 64*t + c//2) mod 2**32),  k = (word >> 16*(c % 2)) & 0xffff

* xi = k * 2**-16 - 1/2, which lies in [-1/2, 1/2) and is exact in float32.
* The counter names (token, channel) only, as the pages' definition does:
  the key and the value at the same (token, channel) are quantized with the
  same draw.  Each tensor's residual keeps the subtractive-dither properties
  (uniform, independent of that tensor's input); Tier B concerns keys only.

t is the token's 0-based logical position in its sequence, c the channel
(0..127).  Positions up to 2**26 keep the counter inside 32 bits.

Pins (tests/test_oracle_dither.py): the hash is a bijection on 32-bit words
(checked on a sampled range), the draws are uniform (KS and chi-square),
adjacent draws are uncorrelated, and the residual of the dithered quantizer
has the variance 1/12 that Tier B assumes.
"""
import numpy as np

_M32 = np.uint64(0xFFFFFFFF)


def pcg(v):
    """pcg hash of Jarzynski and Olano (JCGT 2020), on uint32 values.

    state = v*747796405 + 2891336453; word = ((state >> ((state >> 28) + 4))
    ^ state) * 277803737; result = (word >> 22) ^ word, all modulo 2**32.
    Works on python ints or numpy integer arrays (computed in uint64 and
    masked, so no intermediate wraps early).
    """
    scalar = np.isscalar(v)
    x = np.asarray(v, dtype=np.uint64) & _M32
    state = (x * np.uint64(747796405) + np.uint64(2891336453)) & _M32
    shift = (state >> np.uint64(28)) + np.uint64(4)
    word = (((state >> shift) ^ state) * np.uint64(277803737)) & _M32
    out = ((word >> np.uint64(22)) ^ word) & _M32
    return int(out) if scalar else out.astype(np.uint32)


def stream_key(seed, layer, kv_head):
    """32-bit key of the dither of one (sequence, layer, KV head)."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    k = pcg(seed >> 32)
    k = pcg(k ^ (seed & 0xFFFFFFFF))
    k = pcg(k ^ (int(layer) & 0xFFFFFFFF))
    return pcg(k ^ (int(kv_head) & 0xFFFFFFFF))


def dither_k16(seed, layer, kv_head, t, c):
    """16-bit draw k for positions t and channels c (broadcast arrays)."""
    key = stream_key(seed, layer, kv_head)
    t = np.asarray(t, dtype=np.int64)
    c = np.asarray(c, dtype=np.int64)
    j = (np.int64(key) + 64 * t + (c >> 1)) & 0xFFFFFFFF
    word = pcg(j.astype(np.uint64)).astype(np.uint64)
    half = (c & 1).astype(np.uint64)
    return ((word >> (np.uint64(16) * half)) & np.uint64(0xFFFF)).astype(np.uint16)


def dither_xi(seed, layer, kv_head, t, c):
    """Dither xi = k * 2**-16 - 1/2 as float32 (exact) for positions t, channels c."""
    k = dither_k16(seed, layer, kv_head, t, c).astype(np.float64)
    return (k * 2.0 ** -16 - 0.5).astype(np.float32)


def dither_rows(seed, layer, kv_head, positions, d=128):
    """xi for every channel of the given token positions: float32 [n, d]."""
    t = np.asarray(positions, dtype=np.int64)[:, None]
    c = np.arange(d, dtype=np.int64)[None, :]
    return dither_xi(seed, layer, kv_head, t, c)

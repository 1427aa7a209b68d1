"""RoPE frequency bands (Lemma 1).  Test infrastructure only.

WitCert (m.montaan.com summary, witness-theorem paragraph): the witness is
position-invariant because RoPE acts unitarily within a frequency band
(Lemma 1).  Reading used here: NeoX "rotate-half" pairing, dimension i is
rotated together with i + d/2 at angle pos * base**(-2i/d); the d/2
frequency indices are cut into B contiguous bands, so band b holds the
dimensions [b*d/(2B), (b+1)*d/(2B)) and the same range shifted by d/2.
For d = 128, B = 8 that is 16 dimensions, 8 frequency pairs, per band.
"""
import numpy as np


def band_dims(d=128, num_bands=8):
    """Dimension indices of every band: int array [num_bands, d // num_bands]."""
    half = d // 2
    per = half // num_bands
    assert per * num_bands == half, "bands must split the d/2 frequencies evenly"
    out = []
    for b in range(num_bands):
        lo = np.arange(b * per, (b + 1) * per)
        out.append(np.concatenate([lo, lo + half]))
    return np.stack(out)


def rope_rotate(x, pos, base=10000.0):
    """Apply NeoX rotate-half RoPE at integer positions ``pos`` (float64).

    x: [..., n, d] with pos broadcastable to [..., n].
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
    cos, sin = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x1 * sin + x2 * cos], axis=-1)

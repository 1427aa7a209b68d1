"""Outlier bypass of the dithered INT8 keys.  Test infrastructure only.

Sources (WitCert pages):

* m.montaan.com summary, capacity paragraph: the certified INT8 cache is
  also served "with outlier bypass" (at a lower capacity gain, so the
  bypassed channels cost extra bytes); negative-results paragraph: results
  are reported per "outlier budget" m, with m = 0 meaning no bypass.
* Summary, Tier B paragraph: the variance proxy sums q_c^2 s_{c,t}^2 over
  channels, so a channel whose stored key is exact (s_{c,t} = 0) drops out.

Readings where the pages are silent:

* The bypass set O of one (layer, KV head) is the m channels of largest
  energy E_c = sum_t k_{t,c}^2 over a calibration batch of its keys (the
  prefill), ties to the lower channel.  E_c is accumulated in float32 in
  token order, E <- fp32(E + fp32(k*k)); for bf16 keys k*k is exact.
  O is kept in ascending channel order; m is 0, 8 or 16.
* Keys only (the certificate bounds the key perturbation); values keep the
  plain dithered INT8 path.
* A bypassed channel is stored exactly (bf16 side store: entry i of a token
  holds channel O[i]); its INT8 code is 0 and its reconstruction is the
  exact key, so its residual and its share of the witness are 0.  The row
  scale is the absmax of the other channels.
* Tier B: s_{c,t} = s_t off O and 0 on O, so
  varsigma_t^2 = sm^2 s_t^2 sum_{c not in O} q_c^2 / 12.  Tier A keeps the
  pages' formula (the witness already carries zeros on O).

Parity: pinned by tests/test_oracle_outlier.py (planted outliers recovered,
integer-exact energies, ties, reduction to the plain quantizer at m = 0,
exact reconstruction on O, and the Tier B variance by Monte Carlo).
"""
import numpy as np

from .quant import dither_int8

F32 = np.float32


def channel_energy(x):
    """E_c = sum_t x_{t,c}^2 in float32, accumulated in token order.  x: [n, d]."""
    x = np.asarray(x, dtype=F32)
    acc = np.zeros(x.shape[-1], dtype=F32)
    for t in range(x.shape[0]):
        acc = (acc + (x[t] * x[t]).astype(F32)).astype(F32)
    return acc


def top_energy_channels(x, m):
    """The m channels of largest channel_energy(x), ties to the lower index,
    returned in ascending channel order (int32 [m])."""
    e = channel_energy(x)
    order = sorted(range(e.shape[0]), key=lambda c: (-float(e[c]), c))
    return np.array(sorted(order[:m]), dtype=np.int32)


def bypass_mask(d, channels):
    mask = np.zeros(d, dtype=bool)
    mask[np.asarray(channels, dtype=np.int64)] = True
    return mask


def dither_int8_bypass(x, xi, channels):
    """Dithered INT8 of key rows x [n, d] with the channels O stored exactly.

    Returns (codes int8 [n, d] with 0 on O, s [n], inv_s [n], side float32
    [n, m] = x[:, O]).  Off O the codes and scale are those of the plain
    quantizer applied to the row with its O entries replaced by 0 (a zero
    neither raises the absmax nor, with |xi| <= 1/2, rounds to a nonzero code).
    """
    x = np.asarray(x, dtype=F32)
    O = np.asarray(channels, dtype=np.int64)
    mask = bypass_mask(x.shape[-1], O)
    xin = np.where(mask[None, :], F32(0), x).astype(F32)
    code, s, inv = dither_int8(xin, xi)
    code = np.where(mask[None, :], 0, code).astype(np.int8)
    return code, s, inv, x[:, O].copy()


def dequant_bypass(code, s, xi, side, channels):
    """k^ = s (code - xi) off O and the exact side store on O (float64)."""
    khat = np.asarray(s, dtype=np.float64)[:, None] * (np.asarray(code, dtype=np.float64) -
                                                       np.asarray(xi, dtype=np.float64))
    khat[:, np.asarray(channels, dtype=np.int64)] = np.asarray(side, dtype=np.float64)
    return khat

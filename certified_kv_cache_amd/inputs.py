"""Seeded synthetic inputs shared by the tests, the oracle checks and bench.py.

This module holds input synthesis only: random draws, the RoPE rotation the
workloads apply before caching, bf16 rounding, paging.  It holds none of the
quantization, meter or gate arithmetic, and imports neither the oracle nor
the HIP library.

Workloads (shapes of Qwen2.5-7B attention: 28 query heads, 4 KV heads,
d = 128, RoPE base 10000; the pages' RULER/Qwen runs are replaced by these
synthetic stand-ins):

* ``tiny``   -- one query head, one KV head, S = 256, fp32 N(0,1), RoPE on K.
* ``layer``  -- one layer, batch 1, 28q/4kv, S = 4096, bf16 N(0,1) plus two
  outlier channels per KV head scaled by 20 (before RoPE, K and V).
* ``decode`` -- batch B, 28q/4kv, S tokens per sequence, bf16 N(0,1), paged
  at 16 tokens with a random permutation of the physical pages.
* ``prefill``-- 28 layers x 4 KV heads x n tokens, bf16 N(0, sigma_c^2) with
  sigma_c^2 log-uniform in [0.1, 10] per (layer, head, channel).

Small workloads use numpy's PCG64 so CPU and GPU runs see identical bytes;
the large ones draw with torch on the target device from a seeded generator.
"""
import numpy as np

ROPE_BASE = 10000.0


# ---------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(x):
    """Round float32 to bf16 (nearest even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- RoPE (synthesis)
def apply_rope_np(x, pos, base=ROPE_BASE):
    """NeoX rotate-half RoPE on float64 [..., n, d] at positions pos [n]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    inv = base ** (-np.arange(half) * 2.0 / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
    shape = (1,) * (x.ndim - 2) + ang.shape
    c, s = np.cos(ang).reshape(shape), np.sin(ang).reshape(shape)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


# ---------------------------------------------------------------- small workloads
def tiny(seed=1, S=256, d=128):
    """Single head, S cached tokens, fp32.  Returns dict of float32 arrays.

    k, v: [S, 1, d] (k rotated at positions 0..S-1); q: [1, 1, d].
    """
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((S, 1, d))
    v = rng.standard_normal((S, 1, d))
    q = rng.standard_normal((1, 1, d))
    k = apply_rope_np(k.transpose(1, 0, 2), np.arange(S)).transpose(1, 0, 2)
    return dict(k=k.astype(np.float32), v=v.astype(np.float32), q=q.astype(np.float32),
                dtype="f32")


def layer(seed=2, S=4096, Hq=28, Hkv=4, d=128, outliers=2, outlier_scale=20.0, batch=1):
    """One layer, bf16.  k, v: uint16 bf16 bits [batch*S, Hkv, d]; q: [batch, Hq, d].

    Draw float32 N(0,1); scale ``outliers`` seeded channels per KV head by
    ``outlier_scale`` (K and V); rotate K in float64; round to bf16.
    """
    rng = np.random.default_rng(seed)
    n = batch * S
    k = rng.standard_normal((n, Hkv, d)).astype(np.float32).astype(np.float64)
    v = rng.standard_normal((n, Hkv, d)).astype(np.float32).astype(np.float64)
    for g in range(Hkv):
        ch = rng.choice(d, size=outliers, replace=False)
        k[:, g, ch] *= outlier_scale
        v[:, g, ch] *= outlier_scale
    pos = np.tile(np.arange(S), batch)
    k = apply_rope_np(k.transpose(1, 0, 2), pos).transpose(1, 0, 2)
    q = rng.standard_normal((batch, Hq, d)).astype(np.float32)
    return dict(k=f32_to_bf16_bits(k.astype(np.float32)), v=f32_to_bf16_bits(v.astype(np.float32)),
                q=f32_to_bf16_bits(q), dtype="bf16")


def page_table(seed, ctx_lens, page_size=16, num_pages=None, extra_pages=0):
    """Random physical page assignment for sequences of the given lengths.

    Returns (table int32 [B, max_pages] with -1 padding, num_pages).
    Physical pages are a random permutation of range(num_pages).
    """
    rng = np.random.default_rng(seed)
    pages = [-(-int(s) // page_size) for s in ctx_lens]
    total = sum(pages)
    if num_pages is None:
        num_pages = total + extra_pages
    perm = rng.permutation(num_pages)[:total].astype(np.int32)
    maxp = max(pages) if pages else 0
    tab = np.full((len(pages), max(maxp, 1)), -1, dtype=np.int32)
    off = 0
    for b, p in enumerate(pages):
        tab[b, :p] = perm[off:off + p]
        off += p
    return tab, num_pages


def seeds(batch, base=1234):
    """One 64-bit dither seed per sequence: base + b."""
    return (np.arange(batch, dtype=np.uint64) + np.uint64(base)).astype(np.uint64)


# ---------------------------------------------------------------- large workloads (torch)
def _torch_rope(x, pos, base=ROPE_BASE):
    import torch
    d = x.shape[-1]
    half = d // 2
    inv = base ** (-torch.arange(half, dtype=torch.float64, device=x.device) * 2.0 / d)
    ang = pos.to(torch.float64)[:, None] * inv[None, :]
    c = torch.cos(ang)[:, None, :]
    s = torch.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return torch.cat([x1 * c - x2 * s, x1 * s + x2 * c], dim=-1)


def decode_kv_torch(seed, batch, S, Hkv=4, d=128, device="cuda", chunk=8192):
    """bf16 K (RoPE'd at positions 0..S-1 of each sequence) and V, [batch*S, Hkv, d].

    Drawn with a seeded torch generator on ``device``, chunk by chunk.
    """
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    n = batch * S
    k = torch.empty((n, Hkv, d), dtype=torch.bfloat16, device=device)
    v = torch.empty((n, Hkv, d), dtype=torch.bfloat16, device=device)
    for t0 in range(0, n, chunk):
        t1 = min(n, t0 + chunk)
        kk = torch.randn((t1 - t0, Hkv, d), generator=gen, device=device, dtype=torch.float32)
        vv = torch.randn((t1 - t0, Hkv, d), generator=gen, device=device, dtype=torch.float32)
        pos = torch.arange(t0, t1, device=device) % S
        kk = _torch_rope(kk.to(torch.float64), pos)
        k[t0:t1] = kk.to(torch.float32).to(torch.bfloat16)
        v[t0:t1] = vv.to(torch.bfloat16)
    return k, v


def ragged_kv_torch(seed, ctx_lens, Hkv=4, d=128, device="cuda", chunk=8192):
    """bf16 K, V [sum(ctx_lens), Hkv, d] for a ragged batch, sequences back to
    back, K RoPE'd at each sequence's own positions 0..S_b-1."""
    import torch
    lens = torch.as_tensor(np.asarray(ctx_lens, dtype=np.int64), device=device)
    n = int(lens.sum().item())
    starts = torch.cumsum(lens, 0) - lens
    pos_all = torch.arange(n, device=device) - torch.repeat_interleave(starts, lens)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    k = torch.empty((n, Hkv, d), dtype=torch.bfloat16, device=device)
    v = torch.empty((n, Hkv, d), dtype=torch.bfloat16, device=device)
    for t0 in range(0, n, chunk):
        t1 = min(n, t0 + chunk)
        kk = torch.randn((t1 - t0, Hkv, d), generator=gen, device=device, dtype=torch.float32)
        vv = torch.randn((t1 - t0, Hkv, d), generator=gen, device=device, dtype=torch.float32)
        k[t0:t1] = _torch_rope(kk.to(torch.float64), pos_all[t0:t1]).to(torch.float32).to(torch.bfloat16)
        v[t0:t1] = vv.to(torch.bfloat16)
    return k, v


def query_torch(seed, batch, Hq=28, d=128, device="cuda"):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) + 7919)
    return torch.randn((batch, Hq, d), generator=gen, device=device).to(torch.bfloat16)


def prefill_kv_torch(seed, layers=28, n_tok=4096, Hkv=4, d=128, device="cuda"):
    """bf16 K, V [layers, n_tok, Hkv, d], N(0, sigma^2) with per-(layer, head,
    channel) variance log-uniform in [0.1, 10]."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    logv = torch.empty((2, layers, 1, Hkv, d), device=device).uniform_(
        float(np.log(0.1)), float(np.log(10.0)), generator=gen)
    sd = torch.exp(0.5 * logv)
    k = (torch.randn((layers, n_tok, Hkv, d), generator=gen, device=device) * sd[0]).to(torch.bfloat16)
    v = (torch.randn((layers, n_tok, Hkv, d), generator=gen, device=device) * sd[1]).to(torch.bfloat16)
    return k, v


def plant_needles_torch(k, q, batch, S, Hkv=4, sm=1.0 / np.sqrt(128), sink=8.0, needle=6.0, n_needles=4, seed=0):
    """Structured variant of a decode workload: per (sequence, KV head) the key
    at position 0 becomes a sink and `n_needles` seeded positions become
    needles, by adding a multiple of u, the unit vector of the mean of the
    group's queries, sized so that the mean query's logit rises by `sink`
    (`needle`).  k: bf16 [batch*S, Hkv, d] (returned modified copy); q: [batch, Hq, d]."""
    import torch
    G = q.shape[1] // Hkv
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed) + 31337)
    out = k.clone()
    for b in range(batch):
        pos = torch.randperm(S - 1, generator=gen)[:n_needles] + 1
        for g in range(Hkv):
            qm = q[b, g * G:(g + 1) * G].float().mean(0)
            nrm = float(qm.norm())
            if nrm == 0.0:
                continue
            u = qm / nrm
            for t, gain in [(0, sink)] + [(int(p), needle) for p in pos]:
                row = b * S + t
                out[row, g] = (out[row, g].float() + (gain / (sm * nrm)) * u).to(out.dtype)
    return out

"""Decode attention over the compressed cache and the WitCert meter.

Test infrastructure only.  Everything here is float64.

Sources (WitCert pages):

* Tier A, the black-box logit bound (m.montaan.com summary, Theorem 2
  paragraph): for any query q and cached token t with residual r_t,
  eps_t <= (1/sqrt d) sum_b ||q_b|| w_{t,b}.
* Tier B, the dithered-INT8 certificate (summary, Tier B paragraph):
  varsigma_t^2 = (1/d) sum_c q_c^2 s_{c,t}^2 / 12 and, with probability at least
  1 - delta_loc jointly over the S cached tokens,
  eps_t <= u_t = sqrt(2 varsigma_t^2 log(2S/delta_loc)), with
  delta_loc = delta_req / (L H T).
* Aggregation into a TV bound (summary, improvements list):
  TV <= min(1, (A^2 - 1)/2) with A = sum_t p~_t exp(c_t).
* KV splits merged by log-sum-exp, output and certificate together
  (summary implementation paragraph; paperswithlean Figure 2 caption).
* Gate risk per block (summary implementation paragraph; Figure 5
  caption): the block's share of the meter.
* The deterministic tanh bound that the certificate is compared against
  (summary, page-in paragraph; paperswithlean results and the coverage
  table, where it is the delta = 0 reference).  The pages give no formula.
  Derivation used here: if every logit moves by eps_t with |eps_t| <= c_t,
  the log-ratio log(p~_t / p_t) spans at most 2 max_t c_t, and a log-ratio
  range D gives TV <= tanh(D / 4) (attained by two groups of tokens at the
  two ends of the range), so TV <= tanh(max_t c_t / 2).  It is evaluated per
  tier: with Tier A's c it is deterministic (delta = 0).

Readings taken where the pages leave a step open:

* Logits are l_t = sm_scale * q . k_t; the pages' 1/sqrt(d) is sm_scale, and
  both tiers scale with sm_scale (they reduce to the pages at sm_scale =
  1/sqrt d).
* p~ is the compressed attention softmax(l~) and c_t the tier's per-token
  logit bound.  A = 1 + E with E = sum_t p~_t expm1(c_t), so
  (A^2 - 1)/2 = E (1 + E/2) =: R.  R is reported unclamped; the TV bound is
  min(1, R).
* Tier B uses s_{c,t} = s_t (one scale per token and KV head), S = the
  sequence's full context length, H = query heads; with the outlier bypass
  (oracle/outlier.py) s_{c,t} = 0 on the bypassed channels.
* Repaired (exact) tokens have c_t = 0 in both tiers and k^ = k.
* The value-side certificate (the pages report joint K+V coverage but
  define no value bound): with the value witness w^V_t = ||v^_t - v_t||,
  ||sum_t p~_t v^_t - sum_t p~_t v_t|| <= E_V = sum_t p~_t w^V_t by the
  triangle inequality (deterministic, any value quantizer).  With the key
  side's TV it bounds the whole output error:
  ||o~ - o|| <= E_V + 2 TV max_t ||v_t||, since sum_t (p~_t - p_t) v_t has norm
  at most 2 TV max ||v_t||.
* The block risk used by the gate is rho_{h,j} = sum_{t in block j}
  p~_t expm1(c_t) for the gate's tier, so that sum_j rho_{h,j} = E_h.
"""
import numpy as np

from .rope import band_dims


def delta_loc(delta_req, L, H, T):
    """Per-cell failure budget delta_req / (L H T)."""
    return float(delta_req) / (float(L) * float(H) * float(T))


def cells(requests, L, H, T):
    """Number of monitored (request, layer, head, step) cells."""
    return int(requests) * int(L) * int(H) * int(T)


def tier_a(q, w, sm_scale, num_bands=8):
    """a[h, t] = sm_scale * sum_b ||q_{h,b}|| w[t, b].

    q: [Hq, d] (all heads sharing one KV head), w: [S, num_bands].
    """
    q = np.asarray(q, dtype=np.float64)
    dims = band_dims(q.shape[-1], num_bands)
    qn = np.sqrt(np.sum(q[:, dims] ** 2, axis=-1))          # [Hq, B]
    return sm_scale * qn @ np.asarray(w, dtype=np.float64).T  # [Hq, S]


def tier_b_sigma2(q, s, sm_scale, bypass=None):
    """Variance proxy varsigma^2[h, t] = sm^2 sum_c q_c^2 s_{c,t}^2 / 12.

    s_{c,t} = s_t, except on the outlier-bypass channels ``bypass`` (stored
    exactly, s_{c,t} = 0), which drop out of the sum.
    """
    q = np.array(q, dtype=np.float64)
    if bypass is not None and len(bypass):
        q[:, np.asarray(bypass, dtype=np.int64)] = 0.0
    s = np.asarray(s, dtype=np.float64)
    return sm_scale ** 2 * np.sum(q ** 2, axis=-1)[:, None] * (s[None, :] ** 2) / 12.0


def tier_b(q, s, sm_scale, log_term, bypass=None):
    """u[h, t] = sqrt(2 varsigma^2 log_term); log_term = log(2 S / delta_loc)."""
    return np.sqrt(2.0 * tier_b_sigma2(q, s, sm_scale, bypass) * log_term)


def softmax(l):
    m = np.max(l, axis=-1, keepdims=True)
    e = np.exp(l - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def meter_from(p_tilde, c):
    """E = sum_t p~_t expm1(c_t), R = E (1 + E/2) = (A^2 - 1)/2, TV bound min(1, R)."""
    E = np.sum(p_tilde * np.expm1(c), axis=-1)
    R = E * (1.0 + 0.5 * E)
    return E, R, np.minimum(1.0, R)


def tv(p, p_tilde):
    """True total variation 1/2 sum |p - p~|."""
    return 0.5 * np.sum(np.abs(p - p_tilde), axis=-1)


def v_certificate(p_tilde, wv):
    """E_V = sum_t p~_t w^V_t (value witness wv [S])."""
    return np.asarray(p_tilde, dtype=np.float64) @ np.asarray(wv, dtype=np.float64)


def tanh_bound(c):
    """TV <= tanh(max_t c_t / 2) for per-token logit bounds c [..., S] (0 if S = 0)."""
    c = np.asarray(c, dtype=np.float64)
    cm = np.max(c, axis=-1, initial=0.0)
    return np.tanh(0.5 * cm)


def decode_group(q, k, khat, v, vhat, w, sm_scale, k_scale=None, log_term=None,
                 repaired=None, page_size=16, gate_tier="auto", num_bands=8, bypass=None, wv=None):
    """Decode of the query heads sharing one KV head, over S cached tokens.

    q [G, d]; k, khat, v, vhat [S, d]; w [S, B]; k_scale [S] (dithered INT8,
    enables Tier B); repaired bool [S] (exact tokens: k^ = k and c = 0);
    bypass: the outlier-bypass channels of the keys (Tier B drops them).
    Returns a dict of float64 arrays, per head unless noted:
      o_tilde [G, d]  compressed output sum_t p~_t v^_t (what the GPU returns)
      lse [G]         log sum_t exp(l~_t)
      E_A, R_A [G]    Tier A meter;  E_B, R_B [G] Tier B (NaN if no k_scale)
      T_A, T_B [G]    tanh bounds tanh(max_t c_t / 2) of each tier (T_B NaN if no k_scale)
      block_cmax [G, P]  per page max of the gate tier's c (the tanh gate's input)
      E_V [G]         value certificate sum_t p~_t w^V_t (wv given; else from vhat - v)
      dv_true [G]     ||sum_t p~_t (v^_t - v_t)||, what E_V bounds
      tv_true [G]     TV between exact and compressed attention
      o_exact [G, d]  exact attention output
      a, u [G, S]     per-token bounds; eps [G, S] = |l~ - l|
      block_risk [G, P]  per page share of E for the gate tier
    """
    q = np.asarray(q, dtype=np.float64)
    S = khat.shape[0]
    khat = np.array(khat, dtype=np.float64)
    rep = np.zeros(S, dtype=bool) if repaired is None else np.asarray(repaired, dtype=bool)
    khat[rep] = np.asarray(k, dtype=np.float64)[rep]
    l_exact = sm_scale * q @ np.asarray(k, dtype=np.float64).T
    l_tilde = sm_scale * q @ khat.T
    p = softmax(l_exact)
    pt = softmax(l_tilde)
    m = np.max(l_tilde, axis=-1)
    lse = m + np.log(np.sum(np.exp(l_tilde - m[:, None]), axis=-1))
    a = tier_a(q, w, sm_scale, num_bands)
    a[:, rep] = 0.0
    E_A, R_A, _ = meter_from(pt, a)
    if k_scale is not None and log_term is not None:
        u = tier_b(q, k_scale, sm_scale, log_term, bypass)
        u[:, rep] = 0.0
        E_B, R_B, _ = meter_from(pt, u)
    else:
        u = np.full_like(a, np.nan)
        E_B = R_B = np.full(q.shape[0], np.nan)
    use_b = (gate_tier == "B") or (gate_tier == "auto" and k_scale is not None and log_term is not None)
    cg = u if use_b else a
    P = -(-S // page_size)
    contrib = pt * np.expm1(cg)
    pad = P * page_size - S
    contrib = np.concatenate([contrib, np.zeros((q.shape[0], pad))], axis=1)
    block_risk = contrib.reshape(q.shape[0], P, page_size).sum(-1)
    cpad = np.concatenate([cg, np.zeros((q.shape[0], pad))], axis=1)
    block_cmax = cpad.reshape(q.shape[0], P, page_size).max(-1)
    rv = np.asarray(vhat, dtype=np.float64) - np.asarray(v, dtype=np.float64)
    wv_ = np.sqrt(np.sum(rv * rv, axis=-1)) if wv is None else np.asarray(wv, dtype=np.float64)
    return dict(o_tilde=pt @ np.asarray(vhat, dtype=np.float64), lse=lse,
                E_V=pt @ wv_, dv_true=np.linalg.norm(pt @ rv, axis=-1),
                E_A=E_A, R_A=R_A, E_B=E_B, R_B=R_B, tv_true=tv(p, pt),
                T_A=tanh_bound(a), T_B=tanh_bound(u) if use_b else np.full(q.shape[0], np.nan),
                block_cmax=block_cmax,
                o_exact=p @ np.asarray(v, dtype=np.float64), a=a, u=u,
                eps=np.abs(l_tilde - l_exact), block_risk=block_risk,
                p_tilde=pt, p=p)


def split_ranges(num_pages, n_split):
    """Page ranges of the KV splits: split i covers [i*P//n, (i+1)*P//n)."""
    return [(i * num_pages // n_split, (i + 1) * num_pages // n_split) for i in range(n_split)]


def split_partials(q, khat, vhat, c_a, c_b, sm_scale, n_split, page_size=16, wv=None):
    """Per-split partials (m, l, o, N_A, N_B, C_A, C_B) of one KV head's query group.

    m = max l~ in the split, l = sum exp(l~ - m), o = sum exp(l~ - m) v^,
    N_X = sum exp(l~ - m) expm1(c_X), C_X = max c_X over the split's tokens,
    N_V = sum exp(l~ - m) w^V (value witness wv, zeros if not given).
    Empty splits have m = -inf, l = 0, C_X = 0, N_V = 0.
    c_a, c_b: [G, S] per-token bounds (already zero on repaired tokens).
    """
    q = np.asarray(q, dtype=np.float64)
    S = khat.shape[0]
    wv = np.zeros(S) if wv is None else np.asarray(wv, dtype=np.float64)
    l_tilde = sm_scale * q @ np.asarray(khat, dtype=np.float64).T
    P = -(-S // page_size)
    parts = []
    for lo, hi in split_ranges(P, n_split):
        t0, t1 = lo * page_size, min(hi * page_size, S)
        G = q.shape[0]
        if t1 <= t0:
            parts.append(dict(m=np.full(G, -np.inf), l=np.zeros(G), o=np.zeros((G, vhat.shape[1])),
                              N_A=np.zeros(G), N_B=np.zeros(G), C_A=np.zeros(G), C_B=np.zeros(G),
                              N_V=np.zeros(G)))
            continue
        ls = l_tilde[:, t0:t1]
        m = np.max(ls, axis=-1)
        e = np.exp(ls - m[:, None])
        parts.append(dict(m=m, l=e.sum(-1), o=e @ np.asarray(vhat[t0:t1], dtype=np.float64),
                          N_A=np.sum(e * np.expm1(c_a[:, t0:t1]), -1),
                          N_B=np.sum(e * np.expm1(c_b[:, t0:t1]), -1),
                          C_A=np.max(c_a[:, t0:t1], -1), C_B=np.max(c_b[:, t0:t1], -1),
                          N_V=e @ wv[t0:t1]))
    return parts


def lse_merge(parts):
    """Merge split partials by log-sum-exp: output, LSE and both meters.

    M = max_s m_s, w_s = exp(m_s - M), L = sum w_s l_s, o = sum w_s o_s / L,
    E_X = sum w_s N_X,s / L, LSE = M + log L, R_X = E_X (1 + E_X / 2),
    T_X = tanh(max_s C_X,s / 2), E_V = sum w_s N_V,s / L.
    """
    m = np.stack([p["m"] for p in parts])
    M = np.max(m, axis=0)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    wts = np.where(np.isfinite(m), np.exp(m - Ms), 0.0)
    L = np.sum(wts * np.stack([p["l"] for p in parts]), axis=0)
    o = np.sum(wts[..., None] * np.stack([p["o"] for p in parts]), axis=0)
    NA = np.sum(wts * np.stack([p["N_A"] for p in parts]), axis=0)
    NB = np.sum(wts * np.stack([p["N_B"] for p in parts]), axis=0)
    NV = np.sum(wts * np.stack([p["N_V"] for p in parts]), axis=0)
    Ls = np.where(L > 0, L, 1.0)
    E_A = np.where(L > 0, NA / Ls, 0.0)
    E_B = np.where(L > 0, NB / Ls, 0.0)
    CA = np.max(np.stack([p["C_A"] for p in parts]), axis=0)
    CB = np.max(np.stack([p["C_B"] for p in parts]), axis=0)
    return dict(o=np.where((L > 0)[:, None], o / Ls[:, None], 0.0),
                lse=np.where(L > 0, M + np.log(Ls), -np.inf),
                E_A=E_A, R_A=E_A * (1 + 0.5 * E_A), E_B=E_B, R_B=E_B * (1 + 0.5 * E_B),
                T_A=np.tanh(0.5 * CA), T_B=np.tanh(0.5 * CB), E_V=np.where(L > 0, NV / Ls, 0.0))

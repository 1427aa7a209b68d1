"""Meter-driven gate: which blocks to page in.  Test infrastructure only.

WitCert (m.montaan.com summary implementation paragraph; paperswithlean
Problem/Approach and the Figure 2 and Figure 5 captions): a gate pages in
exact blocks from a CPU backing store when the meter exceeds a threshold,
repairs at block granularity, zeroes the repaired witnesses, and the repair
persists; it is risk-ranked where the witness is saturated (tau >= 1) and
certified where it is informative (tau < 1).

Reading: R = E (1 + E/2) <= tau  <=>  E <= E_tau = sqrt(1 + 2 tau) - 1,
so the gate works on E.  Per (sequence, KV head) with its G query heads:

1. rho_fx[h, j] = ceil(rho[h, j] * 2**40), capped at 2**47, where rho[h, j]
   is block j's share of E_h (its risk);
2. X_h = sum_j rho_fx[h, j]; T = floor(E_tau * 2**40);
3. trigger if max_h X_h > T;
4. rank the unrepaired blocks with nonzero risk by max_h rho_fx[h, j],
   descending, ties to the lower block index;
5. repair the shortest prefix of that ranking after which every head has
   X_h - sum_{j in prefix} rho_fx[h, j] <= T; a budget caps the prefix.

All of it is integer arithmetic, so the decision is exact given rho_fx.

The tanh gate (the comparison the summary's page-in paragraph makes against
the certificate): the tanh bound tanh(max_t c_t / 2) (oracle/meter.py) is
<= tau for every head exactly when no unrepaired token has
c_t > c* = 2 artanh(tau), so it repairs every unrepaired block whose largest
per-token bound over the group's heads exceeds c*, ranked by that value
(descending, ties to the lower block), capped by the budget.  c* and the
comparisons are float32, the precision of the per-block maxima the kernel
hands over (its decision is taken on those values).
"""
import math

import numpy as np

FX_BITS = 40
FX_CAP = 1 << 47


def e_tau(tau):
    """E threshold equivalent to R <= tau."""
    return math.sqrt(1.0 + 2.0 * float(tau)) - 1.0


def threshold_fx(tau):
    """T = floor(E_tau * 2**40) as a python int."""
    return int(math.floor(e_tau(tau) * float(1 << FX_BITS)))


def rho_to_fx(rho):
    """ceil(rho * 2**40) capped at 2**47, for float arrays (rho >= 0 or NaN/inf)."""
    rho = np.asarray(rho, dtype=np.float64)
    out = np.zeros(rho.shape, dtype=np.uint64)
    big = ~(rho < FX_CAP / float(1 << FX_BITS))   # also catches inf and NaN
    pos = (rho > 0) & ~big
    out[pos] = np.ceil(rho[pos] * float(1 << FX_BITS)).astype(np.uint64)
    out[big] = np.uint64(FX_CAP)
    return out


def select(rho_fx, repaired, T, budget=-1):
    """Blocks to repair, in rank order, for one (sequence, KV head).

    rho_fx: integer array [G, P]; repaired: bool [P] (already exact);
    T: threshold; budget: max blocks (-1 = none).  Returns a list of ints.
    """
    rho = [[int(x) for x in row] for row in np.asarray(rho_fx)]
    G = len(rho)
    P = len(rho[0]) if G else 0
    X = [sum(row) for row in rho]
    if not X or max(X) <= T:
        return []
    cand = [j for j in range(P) if not repaired[j] and max(rho[h][j] for h in range(G)) > 0]
    cand.sort(key=lambda j: (-max(rho[h][j] for h in range(G)), j))
    rem = list(X)
    chosen = []
    for j in cand:
        if all(r <= T for r in rem):
            break
        if budget >= 0 and len(chosen) >= budget:
            break
        chosen.append(j)
        for h in range(G):
            rem[h] -= rho[h][j]
    return chosen


def tanh_threshold_f32(tau):
    """c* = 2 artanh(tau) rounded to float32; +inf for tau >= 1 (the bound never exceeds 1)."""
    if tau >= 1.0:
        return np.float32(np.inf)
    return np.float32(2.0 * math.atanh(float(tau)))


def select_tanh(cmax, repaired, tau, budget=-1):
    """Blocks the tanh gate repairs, in rank order, for one (sequence, KV head).

    cmax: float32 [G, P] per-block largest bound of each head; repaired: bool [P].
    """
    cm = np.max(np.asarray(cmax, dtype=np.float32), axis=0) if len(cmax) else np.zeros(0, np.float32)
    cs = tanh_threshold_f32(tau)
    cand = [j for j in range(cm.shape[0]) if not repaired[j] and cm[j] > cs]
    cand.sort(key=lambda j: (-float(cm[j]), j))
    if budget >= 0:
        cand = cand[:budget]
    return cand

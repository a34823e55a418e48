"""Decision margins that make bit-exact parity of reuse decisions and top-k sets well posed.

The GPU accumulates in fp32 and the oracle in fp64, so a score within rounding
error of the k-th/(k+1)-th boundary, or a cosine within rounding error of tau,
could flip a decision.  Before a parity comparison, the inputs are adjusted with
the oracle (never with the GPU path):
  * cosine: |c - tau| >= 1e-4, else the unit's q_prev gets a fresh draw;
  * scores: for each query that will score a unit (q_prev at step 0, q_t at
    step 1) let t be the midpoint of the r-th and (r+1)-th largest scores for
    each boundary rank r (k by default); every key with |s_j - t| < delta_u gets
    a fresh draw of the same norm class, until none is left.  delta_u =
    max(1e-2, 4 * gamma_d * max_j sum_i |q_i k_ji|), gamma_d = d u / (1 - d u),
    u = 2^-24 (the standard bound for recursive fp32 summation).
"""
from __future__ import annotations

import numpy as np

import oracle

COS_MARGIN = 1e-4


def gamma(d: int) -> float:
    u = 2.0 ** -24
    return d * u / (1 - d * u)


def near_boundary_rows(qg: np.ndarray, K: np.ndarray, ranks) -> set:
    s = oracle.token_scores(qg, K)
    n = s.shape[0]
    absdot = np.abs(K) @ np.abs(qg).T  # [N, g]
    delta = max(1e-2, 4 * gamma(qg.shape[1]) * float(absdot.max()))
    order = np.argsort(-s, kind="stable")
    bad = set()
    for r in ranks:
        if r < 1 or r >= n:
            continue
        t = 0.5 * (s[order[r - 1]] + s[order[r]])
        bad |= set(np.nonzero(np.abs(s - t) < delta)[0].tolist())
    return bad


def enforce_margins(problem, layer: int, units=None, extra_ranks=(), max_rounds: int = 40, tau=None):
    """Resample q_prev / key rows of the listed (b, kvh) units until every decision has a margin."""
    p = problem
    tau = p.tau if tau is None else tau
    g = p.g
    if units is None:
        units = [(b, h) for b in range(p.batch) for h in range(p.hkv)]
    units = list(units)
    # cosine margins
    for _ in range(max_rounds):
        q = oracle.as_f64(p.q(layer), p.dtype)
        qp = oracle.as_f64(p.q_prev(layer), p.dtype)
        redo = [(b, h) for b, h in units
                if abs(oracle.group_cosine(q[b, h * g:(h + 1) * g], qp[b, h * g:(h + 1) * g]) - tau) < COS_MARGIN]
        if not redo:
            break
        for b, h in redo:
            p.resample_q_prev(layer, b, h)
    else:
        raise RuntimeError("cosine margins not reached")
    ranks = [p.topk, *extra_ranks]
    for b, h in units:
        for _ in range(max_rounds):
            K = oracle.as_f64(p.kv("k", layer, b, h), p.dtype)
            bad = set()
            for qq in (qp, q):
                bad |= near_boundary_rows(qq[b, h * g:(h + 1) * g], K, ranks)
            if not bad:
                break
            p.resample_k_rows(layer, b, h, sorted(bad))
        else:
            raise RuntimeError(f"score margins not reached for unit {(b, h)}")
    return p

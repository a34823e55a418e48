"""Decision margins that make bit-exact parity of reuse decisions and top-k sets well posed.

Test infrastructure, as the rest of this package: only the tests, the smoke
check and the benchmark's CPU baseline use it; it adjusts seeded inputs with
the oracle's own arithmetic and never with the GPU path.

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

from . import clo_oracle as oracle

COS_MARGIN = 1e-4


def gamma(d: int) -> float:
    u = 2.0 ** -24
    return d * u / (1 - d * u)


def score_delta(qgs, K: np.ndarray) -> float:
    """delta_u for the queries that score a unit."""
    m = 0.0
    for qg in qgs:
        m = max(m, float((np.abs(K) @ np.abs(qg).T).max()))
    return max(1e-2, 4 * gamma(qgs[0].shape[1]) * m)


def boundaries(qgs, K: np.ndarray, ranks):
    """For each query: its scores and the midpoints between the r-th and (r+1)-th largest score."""
    out = []
    for qg in qgs:
        s = oracle.token_scores(qg, K)
        order = np.argsort(-s, kind="stable")
        ts = [0.5 * (s[order[r - 1]] + s[order[r]]) for r in ranks if 1 <= r < s.shape[0]]
        out.append((s, ts))
    return out


def near_boundary_rows(qg: np.ndarray, K: np.ndarray, ranks) -> set:
    """Rows whose score lies within delta_u of a rank boundary (for one query)."""
    delta = score_delta([qg], K)
    (s, ts), = boundaries([qg], K, ranks)
    bad = set()
    for t in ts:
        bad |= set(np.nonzero(np.abs(s - t) < delta)[0].tolist())
    return bad


def _redraw_keeping_sides(p, layer, b, h, K, qgs, row, bounds, delta, max_tries=4000):
    """Draw new rounds of one key row until, for every query and boundary, its score
    is on the same side as before and at least delta away."""
    sides = [[s[row] > t for t in ts] for s, ts in bounds]
    rnd = p.k_row_round(layer, b, h, row)
    for _ in range(max_tries):
        rnd += 1
        cand = oracle.as_f64(p.k_row_draw(layer, b, h, row, rnd), p.dtype)
        ok = True
        for qg, (s, ts), sd in zip(qgs, bounds, sides):
            sc = float(np.max(qg @ cand))
            for t, above in zip(ts, sd):
                if (sc > t + delta) if above else (sc < t - delta):
                    continue
                ok = False
                break
            if not ok:
                break
        if ok:
            p.set_k_row_round(layer, b, h, row, rnd)
            K[row] = cand
            return
    raise RuntimeError(f"no redraw of key row {row} keeps its side")


def enforce_margins(problem, layer: int, units=None, extra_ranks=(), max_rounds: int = 40, tau=None):
    """Redraw q_prev / key rows of the listed (b, kvh) units until every decision has a margin.

    A key within delta_u of a rank boundary is redrawn until it lands on the same
    side of every boundary, at least delta_u away: the number of keys above each
    boundary is unchanged, so the boundaries stay where they are and the band
    around them empties."""
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
        qgs = [qp[b, h * g:(h + 1) * g], q[b, h * g:(h + 1) * g]]
        K = oracle.as_f64(p.kv("k", layer, b, h), p.dtype)
        for _ in range(max_rounds):
            delta = score_delta(qgs, K)
            bounds = boundaries(qgs, K, ranks)
            bad = set()
            for s, ts in bounds:
                for t in ts:
                    bad |= set(np.nonzero(np.abs(s - t) < delta)[0].tolist())
                # a key between two boundaries of one query (the k-th key when ranks k-1
                # and k are both guarded) stays; its neighbours are moved away instead
                if len(ts) > 1:
                    lo_t, hi_t = min(ts), max(ts)
                    bad -= set(np.nonzero((s > lo_t) & (s < hi_t))[0].tolist())
            if not bad:
                break
            for row in sorted(bad):
                _redraw_keeping_sides(p, layer, b, h, K, qgs, row, bounds, delta)
        else:
            raise RuntimeError(f"score margins not reached for unit {(b, h)}")
    return p


def _redraw_keeping_sides_pairs(p, layer, b, h, K, pairs, row, bounds, delta, max_tries=2000):
    """_redraw_keeping_sides for queries that each score only a prefix of the rows
    (pairs of query group and row count); a row past a prefix is free there.

    With many queries a key that sits above some boundaries and below others (a
    heavy hitter) rarely finds a draw on the same side of all of them; then the
    first draw at least delta away from every boundary is taken, on either side.
    The boundaries may then move by one rank, and the caller checks again."""
    sides = [[s[row] > t for t in ts] if row < n else None for (s, ts), (_, n) in zip(bounds, pairs)]
    rnd = p.k_row_round(layer, b, h, row)
    for keep_sides in (True, False):
        for _ in range(max_tries):
            rnd += 1
            cand = oracle.as_f64(p.k_row_draw(layer, b, h, row, rnd), p.dtype)
            ok = True
            for (qg, n), (s, ts), sd in zip(pairs, bounds, sides):
                if sd is None:
                    continue
                sc = float(np.max(qg @ cand))
                for t, above in zip(ts, sd):
                    if keep_sides:
                        good = (sc > t + delta) if above else (sc < t - delta)
                    else:
                        good = abs(sc - t) >= delta
                    if not good:
                        ok = False
                        break
                if not ok:
                    break
            if ok:
                p.set_k_row_round(layer, b, h, row, rnd)
                K[row] = cand
                return
    raise RuntimeError(f"no redraw of key row {row} clears the boundaries")


def enforce_walk_margins(problem, layer: int, steps: int, tau=None, max_rounds: int = 40):
    """Margins for a multi-step run over a growing context (steps 0..steps; step t
    sees the first context - steps + t key rows and queries with p.q_walk(layer, t)).

    Cosines: step by step, a unit's step-t query is redrawn while its cosine with
    the previous step's query or with the query of its last miss under the
    refresh policy lies within 1e-4 of tau (so both reference policies decide
    with a margin).  Scores: as enforce_margins, for every step's query over the
    rows present at that step."""
    p = problem
    tau = p.tau if tau is None else tau
    g = p.g
    n0 = p.context - steps
    units = [(b, h) for b in range(p.batch) for h in range(p.hkv)]
    last_miss = {u: 0 for u in units}
    qf = lambda t: oracle.as_f64(p.q_walk(layer, t), p.dtype)  # noqa: E731
    for t in range(1, steps + 1):
        for _ in range(max_rounds):
            qt, qp = qf(t), qf(t - 1)
            redo = []
            for b, h in units:
                sl = slice(h * g, (h + 1) * g)
                qr = qf(last_miss[(b, h)])[b, sl]
                c1 = oracle.group_cosine(qt[b, sl], qp[b, sl])
                c2 = oracle.group_cosine(qt[b, sl], qr)
                if abs(c1 - tau) < COS_MARGIN or abs(c2 - tau) < COS_MARGIN:
                    redo.append((b, h))
            if not redo:
                break
            for b, h in redo:
                p.resample_walk(layer, b, h, t)
        else:
            raise RuntimeError(f"cosine margins not reached at step {t}")
        qt = qf(t)
        for b, h in units:
            sl = slice(h * g, (h + 1) * g)
            if oracle.group_cosine(qt[b, sl], qf(last_miss[(b, h)])[b, sl]) < tau:
                last_miss[(b, h)] = t
    qs = [qf(t) for t in range(steps + 1)]
    for b, h in units:
        sl = slice(h * g, (h + 1) * g)
        pairs = [(qs[t][b, sl], n0 + t) for t in range(steps + 1)]
        K = oracle.as_f64(p.kv("k", layer, b, h), p.dtype)
        for _ in range(max_rounds):
            delta = score_delta([q for q, _ in pairs], K)
            bounds = [boundaries([q], K[:n], [p.topk])[0] for q, n in pairs]
            bad = set()
            for s, ts in bounds:
                for t in ts:
                    bad |= set(np.nonzero(np.abs(s - t) < delta)[0].tolist())
            if not bad:
                break
            for row in sorted(bad):
                _redraw_keeping_sides_pairs(p, layer, b, h, K, pairs, row, bounds, delta)
        else:
            raise RuntimeError(f"score margins not reached for unit {(b, h)}")
    return p


def enforce_block_margins(problem, layer: int, block_size: int, units=None, max_rounds: int = 40):
    """Margins for block selection: for each query that scores a unit (q_prev at
    step 0, q_t at step 1), t = the midpoint between the (k/B)-th and (k/B+1)-th
    largest block maxima (full blocks of B tokens); every token of the full blocks
    within delta_u of t is redrawn on its side of t.  A block's max is above t
    exactly when one of its tokens is, so the chosen blocks stay and the band
    around t empties."""
    p = problem
    g = p.g
    if units is None:
        units = [(b, h) for b in range(p.batch) for h in range(p.hkv)]
    q = oracle.as_f64(p.q(layer), p.dtype)
    qp = oracle.as_f64(p.q_prev(layer), p.dtype)
    kb = p.topk // block_size
    for b, h in units:
        qgs = [qp[b, h * g:(h + 1) * g], q[b, h * g:(h + 1) * g]]
        K = oracle.as_f64(p.kv("k", layer, b, h), p.dtype)
        nb = K.shape[0] // block_size
        if nb <= kb:
            continue
        for _ in range(max_rounds):
            delta = score_delta(qgs, K)
            bounds, bad = [], set()
            for qg in qgs:
                s = oracle.token_scores(qg, K)
                bm = np.sort(s[:nb * block_size].reshape(nb, block_size).max(axis=1))[::-1]
                t = 0.5 * (bm[kb - 1] + bm[kb])
                bounds.append((s, [t]))
                bad |= set(np.nonzero(np.abs(s[:nb * block_size] - t) < delta)[0].tolist())
            if not bad:
                break
            for row in sorted(bad):
                _redraw_keeping_sides(p, layer, b, h, K, qgs, row, bounds, delta)
        else:
            raise RuntimeError(f"block margins not reached for unit {(b, h)}")
    return p

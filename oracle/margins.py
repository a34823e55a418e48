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


def abs_sums(qgs, K: np.ndarray) -> np.ndarray:
    """Per key row, the largest sum_i |q_i k_ji| over the queries' heads."""
    Ka = np.abs(K)
    return np.max(np.stack([(Ka @ np.abs(qg).T).max(axis=1) for qg in qgs]), axis=0)


def delta_of(m: float, d: int) -> float:
    return max(1e-2, 4 * gamma(d) * m)


def score_delta(qgs, K: np.ndarray) -> float:
    """delta_u for the queries that score a unit."""
    return delta_of(float(abs_sums(qgs, K).max()), qgs[0].shape[1])


def midpoints(s: np.ndarray, ranks):
    """Midpoints between the r-th and (r+1)-th largest of the scores s, per rank r."""
    rs = [r for r in ranks if 1 <= r < s.shape[0]]
    if not rs:
        return []
    part = np.partition(-s, sorted({r - 1 for r in rs} | set(rs)))
    return [-0.5 * (part[r - 1] + part[r]) for r in rs]


def boundaries(qgs, K: np.ndarray, ranks):
    """For each query: its scores and the midpoints between the r-th and (r+1)-th largest score."""
    out = []
    for qg in qgs:
        s = oracle.token_scores(qg, K)
        out.append((s, midpoints(s, ranks)))
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


def for_units(fn, units, workers: int = 1):
    """fn(b, h) for every unit, on `workers` threads (each with a one-thread BLAS);
    the first exception is raised.  Units touch disjoint resample records."""
    units = list(units)
    if workers <= 1 or len(units) <= 1:
        return [fn(b, h) for b, h in units]
    import concurrent.futures as cf

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    try:
        if ctx:
            ctx.__enter__()
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            return list(ex.map(lambda u: fn(*u), units))
    finally:
        if ctx:
            ctx.__exit__(None, None, None)


def enforce_margins(problem, layer: int, units=None, extra_ranks=(), max_rounds: int = 40, tau=None,
                    workers: int = 1):
    """Redraw q_prev / key rows of the listed (b, kvh) units until every decision has a margin.

    A key within delta_u of a rank boundary is redrawn until it lands on the same
    side of every boundary, at least delta_u away: the number of keys above each
    boundary is unchanged, so the boundaries stay where they are and the band
    around them empties.  workers > 1 treats the units' keys on that many
    threads."""
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

    def one(b, h):
        qgs = [qp[b, h * g:(h + 1) * g], q[b, h * g:(h + 1) * g]]
        K = oracle.as_f64(p.kv("k", layer, b, h, threads=1 if workers > 1 else None), p.dtype)
        # scores and row bounds are kept up to date for the redrawn rows only
        A = abs_sums(qgs, K)
        S = [oracle.token_scores(qg, K) for qg in qgs]
        for _ in range(max_rounds):
            delta = delta_of(float(A.max()), K.shape[1])
            bounds = [(s, midpoints(s, ranks)) for s in S]
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
            rows = np.asarray(sorted(bad), dtype=np.int64)
            _redraw_rows_keeping_sides(p, layer, b, h, K, qgs, rows, bounds, delta)
            A[rows] = abs_sums(qgs, K[rows])
            for s, qg in zip(S, qgs):
                s[rows] = (K[rows] @ qg.T).max(axis=1)
        else:
            raise RuntimeError(f"score margins not reached for unit {(b, h)}")

    for_units(one, units, workers)
    return p


def _redraw_rows_keeping_sides(p, layer, b, h, K, qgs, rows, bounds, delta, batch: int = 32,
                               max_rounds: int = 4096, keep_rounds=None):
    """_redraw_keeping_sides for many rows at once: candidate rounds are drawn
    `batch` at a time for every row still open, and each row takes the first
    round (above every listed row's current one) that keeps its side of every
    boundary at least delta away.  With keep_rounds, a row still open after that
    many rounds takes the first draw at least delta away from every boundary on
    either side (a side that is rare for every query at once, such as above
    the block-maximum boundary near the top percent of the scores, is then left):
    the boundaries may move by a rank, and the caller checks again."""
    rows = np.asarray(sorted(rows), dtype=np.int64)
    sides = [np.stack([s[rows] > t for t in ts], axis=1) if ts else np.zeros((rows.size, 0), bool)
             for s, ts in bounds]
    base = max(p.k_row_round(layer, b, h, int(r)) for r in rows)
    open_ = np.ones(rows.size, dtype=bool)
    for start in range(base + 1, base + 1 + max_rounds, batch):
        idx = np.nonzero(open_)[0]
        if idx.size == 0:
            return
        either = keep_rounds is not None and start - base > keep_rounds
        rr = np.repeat(rows[idx], batch)
        rnds = np.tile(np.arange(start, start + batch), idx.size)
        cand = oracle.as_f64(p.k_rows_draw(layer, b, h, rr, rnds), p.dtype).reshape(idx.size, batch, -1)
        ok = np.ones((idx.size, batch), dtype=bool)
        for qg, (s, ts), sd in zip(qgs, bounds, sides):
            sc = (cand @ qg.T).max(axis=2)  # [rows, batch]
            for j, t in enumerate(ts):
                if either:
                    ok &= np.abs(sc - t) >= delta
                else:
                    above = sd[idx, j][:, None]
                    ok &= np.where(above, sc > t + delta, sc < t - delta)
        for n, i in enumerate(idx):
            hit = np.nonzero(ok[n])[0]
            if hit.size:
                j = int(hit[0])
                p.set_k_row_round(layer, b, h, int(rows[i]), start + j)
                K[rows[i]] = cand[n, j]
                open_[i] = False
    raise RuntimeError(f"no redraw keeps the side of key rows {rows[open_][:5].tolist()}")


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


def enforce_block_margins(problem, layer: int, block_size: int, units=None, max_rounds: int = 40,
                          workers: int = 1):
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

    def one(b, h):
        qgs = [qp[b, h * g:(h + 1) * g], q[b, h * g:(h + 1) * g]]
        K = oracle.as_f64(p.kv("k", layer, b, h, threads=1 if workers > 1 else None), p.dtype)
        nb = K.shape[0] // block_size
        if nb <= kb:
            return
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
            _redraw_rows_keeping_sides(p, layer, b, h, K, qgs, sorted(bad), bounds, delta, keep_rounds=1024)
        else:
            raise RuntimeError(f"block margins not reached for unit {(b, h)}")

    for_units(one, units, workers)
    return p

"""Pins for the CPU oracle: checks against facts fixed outside the oracle itself.

Each pin takes an object `O` exposing the oracle's functions (group_cosine,
reuse_decision, token_scores, select_topk, attend, decode_unit, decode_layer,
as_f64), so the same pins run against the real oracle (all must pass) and
against deliberately broken copies of it (each must fail at least one pin).

Sources of truth used here, none of which is the oracle's own code:
  * hand-derived closed forms for tiny inputs (values written as exact
    expressions of e, sqrt and the sigmoid);
  * library routines for special cases the method reduces to: torch's
    scaled_dot_product_attention (float64, CPU) for k = N, torch.topk for
    distinct scores, scipy's cosine distance;
  * brute force over all k-subsets for tiny selections;
  * invariants (softmax sums to 1, convex hull, scale and permutation
    behaviour, k = 1 returns the row);
  * the worked examples stored as text under tests/golden/ (each file names
    the passage of the pages it follows and how its values were derived).
"""
from __future__ import annotations

import ast
import itertools
import json
import math
import operator
import os

import numpy as np


def sigmoid(x: float) -> float:
    return 1.0 / (1.0 + math.exp(-x))


def close(a, b, tol=1e-9):
    return np.allclose(np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64), rtol=0, atol=tol)


# ---------------------------------------------------------------- cosine / reuse
def pin_cosine_closed_forms(O):
    # q = (1,0) against (3,1): 3/sqrt(10); against (1,1): 1/sqrt(2); against (-1,0): -1
    q = np.array([[1.0, 0.0]])
    assert close(O.group_cosine(q, np.array([[3.0, 1.0]])), 3 / math.sqrt(10))
    assert close(O.group_cosine(q, np.array([[1.0, 1.0]])), 1 / math.sqrt(2))
    assert close(O.group_cosine(q, np.array([[-1.0, 0.0]])), -1.0)
    assert O.reuse_decision(3 / math.sqrt(10), 0.8) is True
    assert O.reuse_decision(1 / math.sqrt(2), 0.8) is False


def pin_cosine_group_concatenated(O):
    # q = ((2,0),(0,1)), q_prev = ((1,0),(1,0)): concatenated (2,0,0,1).(1,0,1,0)
    # = 2, norms sqrt(5) and sqrt(2) -> 2/sqrt(10).  The per-head mean would be
    # 0.5 and the per-head min 0, so at tau = 0.6 only the concatenated reading hits.
    q = np.array([[2.0, 0.0], [0.0, 1.0]])
    qp = np.array([[1.0, 0.0], [1.0, 0.0]])
    c = O.group_cosine(q, qp)
    assert close(c, 2 / math.sqrt(10))
    assert O.reuse_decision(c, 0.6) is True


def pin_cosine_invariants(O):
    rng = np.random.default_rng(1)
    for _ in range(20):
        g, d = rng.integers(1, 6), rng.integers(1, 130)
        a = rng.standard_normal((g, d))
        b = rng.standard_normal((g, d))
        c = O.group_cosine(a, b)
        # scipy's cosine distance on the flattened vectors
        from scipy.spatial.distance import cosine

        assert close(c, 1.0 - cosine(a.reshape(-1), b.reshape(-1)), 1e-12)
        # scale invariance and the two extreme cases
        assert close(O.group_cosine(3.5 * a, 0.25 * b), c, 1e-12)
        assert close(O.group_cosine(a, 7.0 * a), 1.0, 1e-12)
        assert close(O.group_cosine(a, -a), -1.0, 1e-12)
        assert -1.0 - 1e-12 <= c <= 1.0 + 1e-12
    z = np.zeros((2, 4))
    assert O.group_cosine(z, np.ones((2, 4))) == 0.0


def pin_reuse_threshold(O):
    # inclusive at equality, never on NaN, +inf forces a miss, -inf a hit
    assert O.reuse_decision(0.8, 0.8) is True
    assert O.reuse_decision(0.8 - 1e-12, 0.8) is False
    assert O.reuse_decision(float("nan"), 0.8) is False
    assert O.reuse_decision(1.0, float("inf")) is False
    assert O.reuse_decision(-1.0, float("-inf")) is True


# ---------------------------------------------------------------- scoring / top-k
def pin_t1_selection(O):
    # g=1, d=2: q=(sqrt2,0), K rows (1,0),(0,1),(-1,0),(2,0): scores sqrt2,0,-sqrt2,2sqrt2
    q = np.array([[math.sqrt(2), 0.0]])
    K = np.array([[1.0, 0.0], [0.0, 1.0], [-1.0, 0.0], [2.0, 0.0]])
    s = O.token_scores(q, K)
    assert close(s, [math.sqrt(2), 0.0, -math.sqrt(2), 2 * math.sqrt(2)])
    assert list(O.select_topk(s, 2)) == [0, 3]


def pin_t2_group_max(O):
    # g=2: q_a=(1,0), q_b=(0,1); K=(3,0),(0,2.5),(1.5,1.5),(-1,-1).
    # max over heads: 3, 2.5, 1.5, -1 -> {0,1}; a sum over heads would give {0,2}.
    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    K = np.array([[3.0, 0.0], [0.0, 2.5], [1.5, 1.5], [-1.0, -1.0]])
    s = O.token_scores(q, K)
    assert close(s, [3.0, 2.5, 1.5, -1.0])
    assert list(O.select_topk(s, 2)) == [0, 1]


def pin_topk_vs_torch(O):
    import torch

    rng = np.random.default_rng(2)
    for n in (1, 7, 64, 1000, 4099):
        s = rng.standard_normal(n) * 10
        for k in sorted({1, max(1, n // 10), n // 2 or 1, n}):
            ref = torch.topk(torch.from_numpy(s), k).indices.numpy()
            assert list(O.select_topk(s, k)) == sorted(ref.tolist())


def pin_topk_bruteforce_with_ties(O):
    # Enumerate every k-subset; exactly one has each member ahead of each
    # non-member under (score descending, index ascending).
    rng = np.random.default_rng(3)
    for _ in range(60):
        n = int(rng.integers(1, 8))
        s = rng.integers(-2, 3, size=n).astype(np.float64)  # many ties
        k = int(rng.integers(1, n + 1))
        ahead = lambda i, j: (s[i] > s[j]) or (s[i] == s[j] and i < j)  # noqa: E731
        good = [S for S in itertools.combinations(range(n), k)
                if all(ahead(i, j) for i in S for j in range(n) if j not in S)]
        assert len(good) == 1
        assert list(O.select_topk(s, k)) == list(good[0])


def pin_topk_invariants(O):
    rng = np.random.default_rng(4)
    n, k = 500, 50
    s = rng.standard_normal(n)
    idx = O.select_topk(s, k)
    assert len(idx) == k and np.all(np.diff(idx) > 0)
    mask = np.zeros(n, bool)
    mask[idx] = True
    assert s[mask].min() > s[~mask].max()
    perm = rng.permutation(n)
    idx_p = O.select_topk(s[perm], k)  # s[perm][i] = s[perm[i]]
    assert sorted(perm[idx_p].tolist()) == idx.tolist()
    # scaling the query by a positive factor keeps the selection
    q = rng.standard_normal((3, 16))
    K = rng.standard_normal((n, 16))
    assert list(O.select_topk(O.token_scores(2.5 * q, K), k)) == list(O.select_topk(O.token_scores(q, K), k))


# ---------------------------------------------------------------- attention
def pin_t1_attention(O):
    # idx {0,3}: logits (1, 2) at d=2 -> p = (1/(1+e), e/(1+e)); V rows (1,0),(0,2)
    e = math.e
    q = np.array([[math.sqrt(2), 0.0]])
    Kc = np.array([[1.0, 0.0], [2.0, 0.0]])
    Vc = np.array([[1.0, 0.0], [0.0, 2.0]])
    out, p = O.attend(q, Kc, Vc, return_p=True)
    assert close(p[0], [1 / (1 + e), e / (1 + e)], 1e-12)
    assert close(out[0], [1 / (1 + e), 2 * e / (1 + e)], 1e-12)
    # zero-padded to d=128: logits sqrt2/sqrt128 = 1/8 and 2sqrt2/sqrt128 = 1/4
    pad = lambda a: np.pad(a, ((0, 0), (0, 126)))  # noqa: E731
    out, p = O.attend(pad(q), pad(Kc), pad(Vc), return_p=True)
    p1 = sigmoid(0.125)
    assert close(p[0], [1 - p1, p1], 1e-12)
    assert close(out[0, :2], [1 - p1, 2 * p1], 1e-12)
    assert close(out[0, 2:], 0.0)


def pin_t2_attention(O):
    # Kc = (3,0),(0,2.5); Vc = (1,2),(3,4)
    # head a logits (3/sqrt d, 0); head b logits (0, 2.5/sqrt d); o = (1,2) + 2 p_1 (1,1)
    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    Kc = np.array([[3.0, 0.0], [0.0, 2.5]])
    Vc = np.array([[1.0, 2.0], [3.0, 4.0]])
    for d in (2, 128):
        pad = lambda a: np.pad(a, ((0, 0), (0, d - 2)))  # noqa: E731
        out = O.attend(pad(q), pad(Kc), pad(Vc))
        pa1 = sigmoid(-3 / math.sqrt(d))
        pb1 = sigmoid(2.5 / math.sqrt(d))
        assert close(out[0, :2], [1 + 2 * pa1, 2 + 2 * pa1], 1e-12)
        assert close(out[1, :2], [1 + 2 * pb1, 2 + 2 * pb1], 1e-12)


def pin_attention_invariants(O):
    rng = np.random.default_rng(5)
    for _ in range(10):
        g, k, d = int(rng.integers(1, 6)), int(rng.integers(1, 300)), int(rng.integers(2, 130))
        q = rng.standard_normal((g, d)) * 3
        Kc = rng.standard_normal((k, d))
        Vc = rng.standard_normal((k, d))
        out, p = O.attend(q, Kc, Vc, return_p=True)
        assert p.shape == (g, k)
        assert np.all(np.abs(p.sum(axis=1) - 1.0) < 1e-12)
        assert np.all(p >= 0)
        assert np.all(out <= Vc.max(axis=0) + 1e-12) and np.all(out >= Vc.min(axis=0) - 1e-12)
        same = np.tile(Vc[:1], (k, 1))
        assert close(O.attend(q, Kc, same), np.tile(Vc[:1], (g, 1)), 1e-12)
        assert np.array_equal(O.attend(q, Kc[:1], Vc[:1]), np.tile(Vc[:1], (g, 1)))


def _sdpa_dense(q, K, V):
    """Dense GQA decode attention from torch (float64, CPU): q [B,Hq,d], K,V [B,Hkv,N,d]."""
    import torch
    import torch.nn.functional as F

    qt = torch.from_numpy(q)[:, :, None, :]  # [B,Hq,1,d]
    g = q.shape[1] // K.shape[1]
    Kt = torch.from_numpy(K).repeat_interleave(g, dim=1).contiguous()
    Vt = torch.from_numpy(V).repeat_interleave(g, dim=1).contiguous()
    return F.scaled_dot_product_attention(qt, Kt, Vt)[:, :, 0, :].numpy()


def pin_dense_limit_gqa(O):
    # k = N with every unit missing is plain dense attention (GQA: head h reads KV head h // g)
    rng = np.random.default_rng(6)
    for (B, Hq, Hkv, N, d) in [(2, 8, 2, 37, 16), (1, 10, 2, 64, 8), (2, 4, 4, 19, 32)]:
        q = rng.standard_normal((B, Hq, d)).astype(np.float32)
        qp = rng.standard_normal((B, Hq, d)).astype(np.float32)
        K = rng.standard_normal((B, Hkv, N, d)).astype(np.float32) * 2
        V = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
        res = O.decode_layer(q, qp, lambda b, h: (K[b, h], V[b, h]), Hkv, N, float("inf"), "f32")
        ref = _sdpa_dense(q.astype(np.float64), K.astype(np.float64), V.astype(np.float64))
        g = Hq // Hkv
        for (b, h), r in res.items():
            assert r["reuse"] is False
            assert list(r["idx"]) == list(range(N))
            assert close(r["out"], ref[b, h * g:(h + 1) * g], 1e-10)


def pin_sparse_equals_dense_on_selection(O):
    # top-k attention equals dense attention restricted to the selected tokens
    rng = np.random.default_rng(7)
    B, Hq, Hkv, N, d, k = 1, 4, 2, 50, 8, 7
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    K = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    V = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    res = O.decode_layer(q, q, lambda b, h: (K[b, h], V[b, h]), Hkv, k, float("inf"), "f32")
    g = Hq // Hkv
    for (b, h), r in res.items():
        sel = np.asarray(r["idx"])
        ref = _sdpa_dense(q[:, h * g:(h + 1) * g].astype(np.float64),
                          K[:, h:h + 1][:, :, sel].astype(np.float64), V[:, h:h + 1][:, :, sel].astype(np.float64))
        assert close(r["out"], ref[b], 1e-10)
        # brute force: the selection is the top-k of the per-token max over the group
        s = np.max(K[b, h].astype(np.float64) @ q[b, h * g:(h + 1) * g].astype(np.float64).T, axis=1)
        assert sorted(np.argsort(-s)[:k].tolist()) == sel.tolist()


def pin_two_step_reuse(O):
    # step 0: every unit misses (tau = +inf) with q_prev as the query; step 1:
    # a hit reuses step 0's selection, a miss selects afresh.
    rng = np.random.default_rng(8)
    B, Hq, Hkv, N, d, k = 2, 4, 2, 40, 8, 5
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    qp = rng.standard_normal((B, Hq, d)).astype(np.float32)
    K = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    V = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    kv = lambda b, h: (K[b, h], V[b, h])  # noqa: E731
    s0 = O.decode_layer(qp, qp, kv, Hkv, k, float("inf"), "f32")
    idx0 = np.stack([np.stack([s0[(b, h)]["idx"] for h in range(Hkv)]) for b in range(B)])
    hit = O.decode_layer(q, qp, kv, Hkv, k, -1.5, "f32", idx_prev=idx0)
    miss = O.decode_layer(q, qp, kv, Hkv, k, 1.5, "f32", idx_prev=idx0)
    g = Hq // Hkv
    for b in range(B):
        for h in range(Hkv):
            qg = q[b, h * g:(h + 1) * g].astype(np.float64)
            assert hit[(b, h)]["reuse"] is True and list(hit[(b, h)]["idx"]) == list(idx0[b, h])
            ref = _sdpa_dense(qg[None], K[b:b + 1, h:h + 1][:, :, idx0[b, h]].astype(np.float64),
                              V[b:b + 1, h:h + 1][:, :, idx0[b, h]].astype(np.float64))
            assert close(hit[(b, h)]["out"], ref[0], 1e-10)
            assert miss[(b, h)]["reuse"] is False
            s = np.max(K[b, h].astype(np.float64) @ qg.T, axis=1)
            assert list(miss[(b, h)]["idx"]) == sorted(np.argsort(-s)[:k].tolist())


# ---------------------------------------------------------------- many steps, growing context
# A 2-D unit (g = 1, d = 2) whose query turns by 30 degrees per step, with three
# initial key rows and one appended before each step, tau = 0.8.  cos(q_t, q_{t-1})
# = cos 30 = 0.866 always hits; against the query of the last miss, step 2 sees
# cos 60 = 0.5 and misses, step 3 sees cos 30 again and hits.
_S3 = math.sqrt(3.0)
_WALK_Q = [np.array([[1.0, 0.0]]), np.array([[_S3 / 2, 0.5]]), np.array([[0.5, _S3 / 2]]), np.array([[0.0, 1.0]])]
_WALK_K = np.array([[1.0, 0.0], [0.0, 1.0], [-1.0, 0.0], [0.5, 0.5], [0.0, 2.0], [-1.0, -1.0]])
_WALK_V = np.array([[1.0, 0.0], [0.0, 1.0], [5.0, 5.0], [7.0, 7.0], [2.0, 3.0], [9.0, 9.0]])


def pin_multistep_reference_policies_k1(O):
    # k = 1: the output is the selected V row.  Step 0 (rows 0-2, q = (1,0)) selects
    # row 0.  "previous" hits every step and keeps row 0.  "refresh" misses at step 2,
    # where the scores of rows 0-4 are 1/2, sqrt3/2, -1/2, (1+sqrt3)/4, sqrt3: the
    # row appended before step 2 wins; step 3 hits and keeps it.
    prev = O.decode_steps_unit(_WALK_Q, _WALK_K, _WALK_V, 3, 1, 0.8, "previous")
    ref = O.decode_steps_unit(_WALK_Q, _WALK_K, _WALK_V, 3, 1, 0.8, "refresh")
    assert [r["reuse"] for r in prev] == [False, True, True, True]
    assert [r["reuse"] for r in ref] == [False, True, False, True]
    assert [list(r["idx"]) for r in prev] == [[0], [0], [0], [0]]
    assert [list(r["idx"]) for r in ref] == [[0], [0], [4], [4]]
    for r in prev:
        assert close(r["out"], [[1.0, 0.0]])
    for r, want in zip(ref, ([1.0, 0.0], [1.0, 0.0], [2.0, 3.0], [2.0, 3.0])):
        assert close(r["out"], [want])
    assert close([r["cos"] for r in ref[1:]], [_S3 / 2, 0.5, _S3 / 2])


def pin_multistep_reference_policies_k2(O):
    # k = 2 (scale 1/sqrt2): with two rows a, b the weights are sigma((l_a - l_b)/sqrt2).
    r2 = math.sqrt(2.0)
    prev = O.decode_steps_unit(_WALK_Q, _WALK_K, _WALK_V, 3, 2, 0.8, "previous")
    ref = O.decode_steps_unit(_WALK_Q, _WALK_K, _WALK_V, 3, 2, 0.8, "refresh")
    assert [list(r["idx"]) for r in prev] == [[0, 1]] * 4
    assert [list(r["idx"]) for r in ref] == [[0, 1], [0, 1], [1, 4], [1, 4]]
    # rows 0 and 1 (V = (1,0), (0,1)): o = (p0, 1 - p0), p0 = sigma((q.r0 - q.r1)/sqrt2)
    for t, diff in enumerate((1.0, _S3 / 2 - 0.5, 0.5 - _S3 / 2, -1.0)):
        p0 = sigmoid(diff / r2)
        assert close(prev[t]["out"], [[p0, 1 - p0]])
    # refresh, steps 2 and 3: rows 1 and 4 (V = (0,1), (2,3)): o = (2 p4, p1 + 3 p4)
    for t, (l1, l4) in ((2, (_S3 / 2, _S3)), (3, (1.0, 2.0))):
        p1 = sigmoid((l1 - l4) / r2)
        p4 = 1 - p1
        assert close(ref[t]["out"], [[2 * p4, p1 + 3 * p4]])


def pin_multistep_limits(O):
    # tau = +inf: every step selects afresh over the keys present at that step
    # (brute force) and attends them (torch SDPA); tau = -1.5: every later step
    # keeps step 0's selection and attends it with its own query.
    rng = np.random.default_rng(11)
    g, d, n0, T, k = 3, 16, 40, 5, 6
    K = rng.standard_normal((n0 + T, d))
    V = rng.standard_normal((n0 + T, d))
    qs = [rng.standard_normal((g, d)) for _ in range(T + 1)]
    for policy in ("previous", "refresh"):
        fresh = O.decode_steps_unit(qs, K, V, n0, k, float("inf"), policy)
        keep = O.decode_steps_unit(qs, K, V, n0, k, -1.5, policy)
        s0 = np.max(K[:n0] @ qs[0].T, axis=1)
        sel0 = sorted(np.argsort(-s0)[:k].tolist())
        for t in range(T + 1):
            s = np.max(K[:n0 + t] @ qs[t].T, axis=1)
            sel = sorted(np.argsort(-s)[:k].tolist())
            assert fresh[t]["reuse"] is False and list(fresh[t]["idx"]) == sel
            ref = _sdpa_dense(qs[t][None], K[None, None, sel], V[None, None, sel])
            assert close(fresh[t]["out"], ref[0], 1e-10)
            assert list(keep[t]["idx"]) == sel0
            assert keep[t]["reuse"] is (t > 0)
            ref = _sdpa_dense(qs[t][None], K[None, None, sel0], V[None, None, sel0])
            assert close(keep[t]["out"], ref[0], 1e-10)


# ---------------------------------------------------------------- per-head thresholds, persistent choice
def pin_per_head_thresholds(O):
    # two KV heads whose groups have the same cosine 3/sqrt(10) = 0.9487 with the
    # previous query: thresholds (0.9, 0.95) make the first a hit and the second a
    # miss; equal thresholds behave like the single threshold.
    B, Hkv, g, d, N, k = 1, 2, 1, 2, 4, 2
    q = np.array([[[1.0, 0.0], [1.0, 0.0]]], dtype=np.float32)
    qp = np.array([[[3.0, 1.0], [3.0, 1.0]]], dtype=np.float32)
    K = np.array([[1.0, 0.0], [0.0, 1.0], [-1.0, 0.0], [2.0, 0.0]], dtype=np.float32)
    V = np.array([[1.0, 0.0], [0.0, 1.0], [5.0, 5.0], [0.0, 2.0]], dtype=np.float32)
    kv = lambda b, h: (K, V)  # noqa: E731
    idx_prev = np.array([[[1, 2], [1, 2]]])
    r = O.decode_layer(q, qp, kv, Hkv, k, [0.9, 0.95], "f32", idx_prev=idx_prev)
    assert r[(0, 0)]["reuse"] is True and list(r[(0, 0)]["idx"]) == [1, 2]
    assert r[(0, 1)]["reuse"] is False and list(r[(0, 1)]["idx"]) == [0, 3]
    for t in (0.9, 0.95):
        a = O.decode_layer(q, qp, kv, Hkv, k, [t, t], "f32", idx_prev=idx_prev)
        b = O.decode_layer(q, qp, kv, Hkv, k, t, "f32", idx_prev=idx_prev)
        for u in a:
            assert a[u]["reuse"] == b[u]["reuse"] and list(a[u]["idx"]) == list(b[u]["idx"])


def pin_plan_persistent(O):
    # closed form: 2 layers x 3 heads; the three lowest similarities are slots
    # (1,0)=0.1, (0,2)=0.2 and the tie 0.5 between (0,1) and (1,2) goes to (0,1)
    s = np.array([[0.9, 0.5, 0.2], [0.1, 0.7, 0.5]])
    assert O.plan_persistent(s, 0) == [0, 0]
    assert O.plan_persistent(s, 3) == [0b110, 0b001]
    assert O.plan_persistent(s, 6) == [0b111, 0b111]
    # brute force: among all subsets of the same size, the chosen one has the
    # smallest total similarity, and with ties the lexicographically first slots
    rng = np.random.default_rng(12)
    for _ in range(30):
        L, H = rng.integers(1, 4), rng.integers(1, 4)
        s = rng.integers(0, 4, size=(L, H)).astype(np.float64) / 4  # many ties
        n = int(rng.integers(0, L * H + 1))
        masks = O.plan_persistent(s, n)
        chosen = sorted(l * H + h for l in range(L) for h in range(H) if masks[l] >> h & 1)
        assert len(chosen) == n
        flat = s.reshape(-1)
        best = min(itertools.combinations(range(L * H), n), key=lambda c: (sum(flat[list(c)]), c))
        assert chosen == list(best)


# ---------------------------------------------------------------- quantized host formats
def raises(exc, fn, *args) -> bool:
    try:
        fn(*args)
    except exc:
        return True
    return False


def pin_quantize_closed_forms(O):
    # m = 1: 127 * 2^-7 = 0.99 < 1 <= 127 * 2^-6 = 1.98, so e = -6 and q = x * 64
    q, e = O.quantize_row([1.0, -0.5, 0.25, 0.0])
    assert e == -6 and list(q) == [64, -32, 16, 0]
    # m exactly 127 * 2^-6 stays at e = -6 (q = 127); the next float up needs e = -5
    q, e = O.quantize_row([127 * 2.0 ** -6, 1.0])
    assert e == -6 and list(q) == [127, 64]
    q, e = O.quantize_row([np.nextafter(127 * 2.0 ** -6, 2.0), 1.0])
    assert e == -5 and list(q) == [64, 32]
    # halves round to even: with e = -1 (m = 63.5) x = 0.75 -> 1.5 -> 2, x = 1.25 -> 2.5 -> 2, -0.25 -> -0.5 -> 0
    q, e = O.quantize_row([63.5, 0.75, 1.25, -0.25])
    assert e == -1 and list(q) == [127, 2, 2, 0]
    # zero rows and the smallest exponent
    q, e = O.quantize_row([0.0, 0.0])
    assert e == 0 and list(q) == [0, 0]
    q, e = O.quantize_row([2.0 ** -130, -(2.0 ** -125)])
    assert e == -120 and list(q) == [0, 0]
    assert list(O.dequantize_row([64, -32, 16], -6)) == [1.0, -0.5, 0.25]


def pin_quantize_invariants(O):
    rng = np.random.default_rng(13)
    for _ in range(200):
        x = rng.standard_normal(128) * 2.0 ** rng.integers(-20, 20)
        q, e = O.quantize_row(x)
        m = np.max(np.abs(x))
        assert np.max(np.abs(q)) <= 127 and m <= 127 * 2.0 ** e and not m <= 127 * 2.0 ** (e - 1)
        xd = O.dequantize_row(q, e)
        assert np.max(np.abs(xd - x)) <= 2.0 ** (e - 1)  # round to nearest
        # every dequantized value fits bfloat16 exactly (at most 8 significant bits)
        mant = np.abs(xd[xd != 0]) / 2.0 ** np.floor(np.log2(np.abs(xd[xd != 0])))
        assert np.all(mant * 128 == np.round(mant * 128))
        # scaling by a power of two shifts e and keeps q
        q2, e2 = O.quantize_row(x * 8.0)
        assert e2 == e + 3 and list(q2) == list(q)


def pin_quantized_rows_closed_form(O):
    # quantized_rows works row by row: row 0 (max 1) gets e = -6, so 0.3 becomes
    # rint(19.2) / 64 = 19/64; row 1 (max 100) gets e = 0, so 0.3 becomes 0.  A
    # column-wise or transposed rule would give column 1 (max 0.3, e = -8) the
    # value rint(76.8) / 256 = 77/256 in both rows.
    X = np.array([[1.0, 0.3, 0.0, -0.5], [100.0, 0.3, -7.0, 0.0]])
    got = O.quantized_rows(X)
    assert got.shape == X.shape
    want = np.array([[1.0, 19 / 64, 0.0, -0.5], [100.0, 0.0, -7.0, 0.0]])
    assert np.array_equal(got, want)
    # rows that each fit their own scale come back unchanged (row 0: e = 0, row 1:
    # e = -16, values 64 * 2^-16 and -16 * 2^-16); one scale per column would
    # flush 2^-10 to 0 next to 64
    Y = np.array([[64.0, -32.0, 16.0], [2.0 ** -10, 0.0, -(2.0 ** -12)]])
    assert np.array_equal(O.quantized_rows(Y), Y)


def pin_quantize4_closed_forms(O):
    # 4-bit values, M = 7: m = 1 has 7 * 2^-3 = 0.875 < 1 <= 7 * 2^-2 = 1.75, so
    # e = -2 and q = x * 4
    assert O.quant_max(4) == 7 and O.quant_max(8) == 127
    q, e = O.quantize_row([1.0, -0.5, 0.25, 0.0], 4)
    assert e == -2 and list(q) == [4, -2, 1, 0]
    # m exactly 7 * 2^-2 keeps e = -2 (q = 7); the next float up needs e = -1,
    # where 1.75+ / 0.5 = 3.5+ rounds up to 4
    q, e = O.quantize_row([1.75, 1.0], 4)
    assert e == -2 and list(q) == [7, 4]
    q, e = O.quantize_row([np.nextafter(1.75, 2.0), 1.0], 4)
    assert e == -1 and list(q) == [4, 2]
    # ties to even at e = -1 (m = 3.5): 0.75 -> 1.5 -> 2, 1.25 -> 2.5 -> 2, -0.25 -> -0.5 -> 0
    q, e = O.quantize_row([3.5, 0.75, 1.25, -0.25], 4)
    assert e == -1 and list(q) == [7, 2, 2, 0]
    # m = 300: 7 * 32 = 224 < 300 <= 448 = 7 * 64, so e = 6; 300 / 64 = 4.6875 -> 5
    q, e = O.quantize_row([300.0, -1.0, 0.5], 4)
    assert e == 6 and list(q) == [5, 0, 0]
    # zero rows and the smallest exponent
    q, e = O.quantize_row([0.0, 0.0], 4)
    assert e == 0 and list(q) == [0, 0]
    q, e = O.quantize_row([2.0 ** -130, -(2.0 ** -125)], 4)
    assert e == -120 and list(q) == [0, 0]
    for bad in (0, 2, 16):
        assert raises(ValueError, O.quantize_row, [1.0], bad)


def pin_quantize4_invariants(O):
    rng = np.random.default_rng(14)
    for _ in range(200):
        x = rng.standard_normal(128) * 2.0 ** rng.integers(-20, 20)
        q, e = O.quantize_row(x, 4)
        m = np.max(np.abs(x))
        assert np.max(np.abs(q)) <= 7 and m <= 7 * 2.0 ** e and not m <= 7 * 2.0 ** (e - 1)
        assert np.max(np.abs(O.dequantize_row(q, e) - x)) <= 2.0 ** (e - 1)
        # the 8-bit exponent of the same row is 4 lower (127 / 7 lies between 2^4 and 2^5)
        # or 5 lower, and the 4-bit grid is a subset of the 8-bit one
        q8, e8 = O.quantize_row(x, 8)
        assert e - e8 in (4, 5)
        q2, e2 = O.quantize_row(x * 0.25, 4)
        assert e2 == e - 2 and list(q2) == list(q)
    # quantized_rows takes the width along: 0.3 next to 1 becomes 1/4 with 4 bits
    assert np.array_equal(O.quantized_rows(np.array([[1.0, 0.3]]), 4), np.array([[1.0, 0.25]]))


def pin_pack_int4(O):
    # value 2j in the low half of byte j, value 2j+1 in the high half, two's complement
    assert O.pack_int4([1, -1, 7, -7]) == bytes([0xF1, 0x97])
    assert O.pack_int4([4, -2, 1, 0]) == bytes([0xE4, 0x01])
    assert O.pack_int4([-8, 0, 0, -8]) == bytes([0x08, 0x80])
    # every pair of codes round-trips through the nibbles
    for a in range(-8, 8):
        for b in range(-8, 8):
            byte = O.pack_int4([a, b])[0]
            lo, hi = byte & 0xF, byte >> 4
            assert (lo - 16 if lo >= 8 else lo, hi - 16 if hi >= 8 else hi) == (a, b)
    for bad in ([1], [8, 0], [0, -9]):
        assert raises(ValueError, O.pack_int4, bad)


# ---------------------------------------------------------------- block selection
def pin_select_blocks_closed_form(O):
    # blocks of 2 over 9 tokens: (0.1, 0.9) -> 0.9, (0.2, 0.3) -> 0.3, (0.8, 0.85) -> 0.85,
    # (0.0, 0.05) -> 0.05; token 8 (0.7) is a partial tail block and never taken.  The two
    # best blocks are 0 and 2; token-level top-4 would be tokens 1, 4, 5, 8.
    s = np.array([0.1, 0.9, 0.2, 0.3, 0.8, 0.85, 0.0, 0.05, 0.7])
    assert list(O.select_blocks(s, 4, 2)) == [0, 1, 4, 5]
    assert list(O.select_topk(s, 4)) == [1, 4, 5, 8]
    # equal block scores go to the lower block
    assert list(O.select_blocks(np.array([0.5, 0.0, 0.0, 0.5, 0.5, 0.0]), 2, 2)) == [0, 1]
    # blocks of 3 over 7 tokens: (1, 5, 2) -> 5, (9, 0, 0) -> 9; the tail token 6 never counts
    assert list(O.select_blocks(np.array([1.0, 5.0, 2.0, 9.0, 0.0, 0.0, 99.0]), 3, 3)) == [3, 4, 5]


def pin_select_blocks_invariants(O):
    rng = np.random.default_rng(14)
    for _ in range(50):
        bs = int(rng.integers(1, 9))
        n = int(rng.integers(bs, 200))
        nb = n // bs
        kb = int(rng.integers(1, nb + 1))
        s = rng.integers(0, 6, size=n).astype(np.float64)  # many ties
        sel = O.select_blocks(s, kb * bs, bs)
        assert len(sel) == kb * bs and np.all(np.diff(sel) > 0) and sel.max() < nb * bs
        blocks = sorted(set((sel // bs).tolist()))
        assert len(blocks) == kb and all(set(range(b * bs, b * bs + bs)) <= set(sel.tolist()) for b in blocks)
        bmax = s[:nb * bs].reshape(nb, bs).max(axis=1)
        chosen = set(blocks)
        for b in range(nb):
            for c in chosen:
                if b not in chosen:
                    assert bmax[c] > bmax[b] or (bmax[c] == bmax[b] and c < b)
        if bs == 1:
            assert list(sel) == list(O.select_topk(s, kb))


# ---------------------------------------------------------------- attention rows apart from scored keys, blocks in a layer
# T1's unit: q = (sqrt2, 0); exact keys (1,0), (0,1), (-1,0), (2,0) score sqrt2, 0,
# -sqrt2, 2 sqrt2, so k = 2 selects rows {0, 3}.  Attention reads other rows:
# K_attn has the selected rows halved, (0.5,0) and (1,0) (logits 1/2 and 1 at
# d = 2, weights sigma(-1/2) and sigma(1/2)), and a large row 1, (5,0), that the
# exact keys never select (scoring K_attn would take {1, 3}); V_attn rows 0 and 3
# are (10,0) and (0,20).
_T1_Q = np.array([[math.sqrt(2.0), 0.0]])
_T1_K = np.array([[1.0, 0.0], [0.0, 1.0], [-1.0, 0.0], [2.0, 0.0]])
_T1_V = np.array([[1.0, 0.0], [0.0, 1.0], [5.0, 5.0], [0.0, 2.0]])
_T1_KA = np.array([[0.5, 0.0], [5.0, 0.0], [-0.5, 0.0], [1.0, 0.0]])
_T1_VA = np.array([[10.0, 0.0], [3.0, 3.0], [7.0, 7.0], [0.0, 20.0]])
_T1_OUT_A = [10 * sigmoid(-0.5), 20 * sigmoid(0.5)]


def pin_decode_unit_attn_rows(O):
    r = O.decode_unit(_T1_Q, _T1_Q, _T1_K, _T1_V, 2, math.inf, K_attn=_T1_KA, V_attn=_T1_VA)
    assert r["reuse"] is False and list(r["idx"]) == [0, 3]
    assert close(r["out"], [_T1_OUT_A], 1e-12)
    # without separate rows: T1's own attention, weights sigma(-1) and sigma(1) on V rows (1,0), (0,2)
    r = O.decode_unit(_T1_Q, _T1_Q, _T1_K, _T1_V, 2, math.inf)
    assert close(r["out"], [[sigmoid(-1.0), 2 * sigmoid(1.0)]], 1e-12)
    # a reused unit attends its previous selection in the separate rows too
    r = O.decode_unit(_T1_Q, _T1_Q, _T1_K, _T1_V, 2, -1.5, idx_prev=np.array([0, 3]), K_attn=_T1_KA,
                      V_attn=_T1_VA)
    assert r["reuse"] is True and close(r["out"], [_T1_OUT_A], 1e-12)


def pin_decode_layer_attn_rows(O):
    # a layer of two units (B = 1, Hkv = 2, g = 1, fp32, q = (1, 0) exact) on T1's
    # keys: scores 1, 0, -1, 2 select {0, 3} in both.  attn_kv_of gives unit (0, 1)
    # the separate rows and leaves unit (0, 0) alone.  Unit (0, 0): logits 1/sqrt2,
    # 2/sqrt2 on V rows (1,0), (0,2); unit (0, 1): logits (1/2)/sqrt2, 1/sqrt2 on
    # V_attn rows (10,0), (0,20).
    q = np.array([[[1.0, 0.0], [1.0, 0.0]]], dtype=np.float32)
    K32, V32 = _T1_K.astype(np.float32), _T1_V.astype(np.float32)
    res = O.decode_layer(q, q, lambda b, h: (K32, V32), 2, 2, math.inf, "f32",
                         attn_kv_of=lambda b, h: (_T1_KA, _T1_VA) if h == 1 else None)
    assert list(res[(0, 0)]["idx"]) == [0, 3] and list(res[(0, 1)]["idx"]) == [0, 3]
    p = sigmoid(1 / math.sqrt(2.0))
    assert close(res[(0, 0)]["out"], [[1 - p, 2 * p]], 1e-12)
    p = sigmoid(0.5 / math.sqrt(2.0))
    assert close(res[(0, 1)]["out"], [[10 * (1 - p), 20 * p]], 1e-12)


def pin_decode_layer_blocks(O):
    # B = 1, Hkv = 2, g = 1, d = 2, N = 5, k = 2, blocks of 2 (token 4 is a tail
    # block, never selectable); values exact in fp32.
    # unit 0: q = (1, 0); scores 1/8, 7/8, 3/4, 13/16, 3 -> blocks 7/8, 13/16 ->
    #   block 0 = tokens {0, 1} (token top-2 would be {1, 4}); logits (1/8, 7/8)/sqrt2
    #   on V rows (1,0), (0,1): o = (1 - p, p), p = sigma((3/4)/sqrt2).
    # unit 1: q = (0, 1); scores 1/4, 1/8, 1/2, 3/8, 9 -> blocks 1/4, 1/2 -> block 1 =
    #   tokens {2, 3} (token top-2: {2, 4}); logits (1/2, 3/8)/sqrt2 on V rows (2,0),
    #   (0,2): o = (2 p2, 2 (1 - p2)), p2 = sigma((1/8)/sqrt2).
    q = np.array([[[1.0, 0.0], [0.0, 1.0]]], dtype=np.float32)
    K = {0: np.array([[0.125, 0], [0.875, 0], [0.75, 0], [0.8125, 0], [3.0, 0]], dtype=np.float32),
         1: np.array([[0, 0.25], [0, 0.125], [0, 0.5], [0, 0.375], [0, 9.0]], dtype=np.float32)}
    V = {0: np.array([[1, 0], [0, 1], [4, 4], [6, 6], [8, 8]], dtype=np.float32),
         1: np.array([[1, 0], [0, 1], [2, 0], [0, 2], [5, 5]], dtype=np.float32)}
    kv = lambda b, h: (K[h], V[h])  # noqa: E731
    res = O.decode_layer(q, q, kv, 2, 2, math.inf, "f32", block_size=2)
    assert list(res[(0, 0)]["idx"]) == [0, 1] and list(res[(0, 1)]["idx"]) == [2, 3]
    p = sigmoid(0.75 / math.sqrt(2.0))
    assert close(res[(0, 0)]["out"], [[1 - p, p]], 1e-12)
    p2 = sigmoid(0.125 / math.sqrt(2.0))
    assert close(res[(0, 1)]["out"], [[2 * p2, 2 * (1 - p2)]], 1e-12)
    tok = O.decode_layer(q, q, kv, 2, 2, math.inf, "f32")
    assert list(tok[(0, 0)]["idx"]) == [1, 4] and list(tok[(0, 1)]["idx"]) == [2, 4]


def pin_bf16_decoding(O):
    # IEEE facts about bfloat16 bit patterns
    bits = np.array([0x3F80, 0xC000, 0x3FC0, 0x0000, 0x8000, 0x7F7F, 0x0001, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 1.5, 0.0, -0.0, (2 - 2 ** -7) * 2.0 ** 127, 2.0 ** -133, 3.140625]
    got = O.as_f64(bits, "bf16")
    assert list(got) == want
    assert np.signbit(got[4])
    f = np.array([0.1, -3.25], dtype=np.float32)
    assert list(O.as_f64(f, "f32")) == [float(np.float32(0.1)), -3.25]


# ---------------------------------------------------------------- worked examples (tests/golden)
GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
_BINOPS = {ast.Add: operator.add, ast.Sub: operator.sub, ast.Mult: operator.mul, ast.Div: operator.truediv,
           ast.Pow: operator.pow}
_FUNCS = {"sqrt": math.sqrt, "exp": math.exp, "sigmoid": sigmoid}


def golden_value(x):
    """A fixture number: a JSON number, or a closed form written as text over
    + - * / **, sqrt, exp, sigmoid and inf (evaluated here, nothing else is
    allowed)."""
    if isinstance(x, (int, float)) and not isinstance(x, bool):
        return float(x)
    if isinstance(x, list):
        return [golden_value(v) for v in x]

    def ev(n):
        if isinstance(n, ast.Expression):
            return ev(n.body)
        if isinstance(n, ast.Constant) and isinstance(n.value, (int, float)):
            return float(n.value)
        if isinstance(n, ast.Name) and n.id == "inf":
            return math.inf
        if isinstance(n, ast.BinOp) and type(n.op) in _BINOPS:
            return _BINOPS[type(n.op)](ev(n.left), ev(n.right))
        if isinstance(n, ast.UnaryOp) and isinstance(n.op, (ast.USub, ast.UAdd)):
            v = ev(n.operand)
            return -v if isinstance(n.op, ast.USub) else v
        if (isinstance(n, ast.Call) and isinstance(n.func, ast.Name) and n.func.id in _FUNCS
                and len(n.args) == 1 and not n.keywords):
            return _FUNCS[n.func.id](ev(n.args[0]))
        raise ValueError(f"not a closed form: {x!r}")

    return ev(ast.parse(str(x), mode="eval"))


def golden(name):
    with open(os.path.join(GOLDEN_DIR, name)) as f:
        return json.load(f)


def golden_array(x):
    return np.array(golden_value(x), dtype=np.float64)


def pin_golden_reuse(O):
    for c in golden("reuse_test.json")["cases"]:
        cos = O.group_cosine(golden_array(c["q"]), golden_array(c["q_prev"]))
        assert close(cos, golden_value(c["cos"]), 1e-12), c
        assert O.reuse_decision(cos, golden_value(c["tau"])) is c["reuse"], c


def pin_golden_selection(O):
    fx = golden("selection.json")
    for c in fx["cases"]:
        s = O.token_scores(golden_array(c["q"]), golden_array(c["K"]))
        assert close(s, golden_array(c["scores"]), 1e-12), c["name"]
        assert list(O.select_topk(s, c["k"])) == c["idx"], c["name"]
    for c in fx["block_cases"]:
        assert list(O.select_blocks(golden_array(c["scores"]), c["k"], c["block_size"])) == c["idx"], c


def pin_golden_attention(O):
    for c in golden("attention.json")["cases"]:
        d = c["d"]
        pad = lambda a: np.pad(golden_array(a), ((0, 0), (0, d - len(a[0]))))  # noqa: E731
        out, p = O.attend(pad(c["q"]), pad(c["Kc"]), pad(c["Vc"]), return_p=True)
        assert close(p, golden_array(c["p"]), 1e-12), c["name"]
        w = len(c["out"][0])
        assert close(out[:, :w], golden_array(c["out"]), 1e-12), c["name"]
        assert close(out[:, w:], 0.0), c["name"]


def pin_golden_decode_step(O):
    fx = golden("decode_step.json")
    K, V = golden_array(fx["K"]), golden_array(fx["V"])
    for c in fx["cases"]:
        r = O.decode_unit(golden_array(c["q"]), golden_array(c["q_prev"]), K, V, fx["k"], golden_value(c["tau"]),
                          idx_prev=np.array(c["idx_prev"]))
        assert close(r["cos"], golden_value(c["cos"]), 1e-12), c["name"]
        assert r["reuse"] is c["reuse"] and list(r["idx"]) == c["idx"], c["name"]
        assert close(r["out"], golden_array(c["out"]), 1e-12), c["name"]


def pin_golden_growing_context(O):
    fx = golden("growing_context.json")
    qs = [golden_array(q) for q in fx["queries"]]
    K, V = golden_array(fx["K"]), golden_array(fx["V"])
    for policy, want in fx["policies"].items():
        res = O.decode_steps_unit(qs, K, V, fx["n0"], fx["k"], golden_value(fx["tau"]), policy)
        assert [r["reuse"] for r in res] == want["reuse"], policy
        assert [list(r["idx"]) for r in res] == want["idx"], policy
        assert close([r["cos"] for r in res], golden_array(want["cos"]), 1e-12), policy
        for r, o in zip(res, want["out"]):
            assert close(r["out"], golden_array(o), 1e-12), policy


def pin_golden_int8_rows(O):
    for c in golden("int8_rows.json")["cases"]:
        x = golden_array(c["x"])
        q, e = O.quantize_row(x)
        assert e == c["e"] and list(q) == c["q"], c
        assert list(O.dequantize_row(q, e)) == [v * 2.0 ** c["e"] for v in c["q"]], c


def pin_golden_int4_rows(O):
    for c in golden("int4_rows.json")["cases"]:
        x = golden_array(c["x"])
        q, e = O.quantize_row(x, 4)
        assert e == c["e"] and list(q) == c["q"], c
        assert O.pack_int4(q).hex() == c["bytes"], c


ALL_PINS = [
    pin_cosine_closed_forms,
    pin_cosine_group_concatenated,
    pin_cosine_invariants,
    pin_reuse_threshold,
    pin_t1_selection,
    pin_t2_group_max,
    pin_topk_vs_torch,
    pin_topk_bruteforce_with_ties,
    pin_topk_invariants,
    pin_t1_attention,
    pin_t2_attention,
    pin_attention_invariants,
    pin_dense_limit_gqa,
    pin_sparse_equals_dense_on_selection,
    pin_two_step_reuse,
    pin_multistep_reference_policies_k1,
    pin_multistep_reference_policies_k2,
    pin_multistep_limits,
    pin_per_head_thresholds,
    pin_plan_persistent,
    pin_quantize_closed_forms,
    pin_quantize_invariants,
    pin_quantized_rows_closed_form,
    pin_quantize4_closed_forms,
    pin_quantize4_invariants,
    pin_pack_int4,
    pin_select_blocks_closed_form,
    pin_select_blocks_invariants,
    pin_decode_unit_attn_rows,
    pin_decode_layer_attn_rows,
    pin_decode_layer_blocks,
    pin_bf16_decoding,
    pin_golden_reuse,
    pin_golden_selection,
    pin_golden_attention,
    pin_golden_decode_step,
    pin_golden_growing_context,
    pin_golden_int8_rows,
    pin_golden_int4_rows,
]

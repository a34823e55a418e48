"""Plant plausible mistakes in copies of the oracle; each must fail at least one pin.

This shows the pins are strong enough to catch a dropped term, a wrong sign or
index, or a transposed operand anywhere in the oracle's arithmetic.
"""
import math
import types

import numpy as np
import pytest

import oracle
from oracle import clo_oracle as base
from tests.oracle_pins import ALL_PINS


def _ns(**over):
    ns = types.SimpleNamespace(**{n: getattr(base, n) for n in (
        "as_f64", "group_cosine", "reuse_decision", "token_scores", "select_topk",
        "attend", "decode_unit", "decode_layer")})
    for k, v in over.items():
        setattr(ns, k, v)
    # decode_unit/decode_layer must route through the (possibly mutated) namespace
    def decode_unit(q_group, q_prev_group, K, V, k, tau, idx_prev=None):
        c = ns.group_cosine(q_group, q_prev_group)
        reuse = ns.reuse_decision(c, tau)
        sel = np.asarray(idx_prev) if reuse else ns.select_topk(ns.token_scores(q_group, K), k)
        return {"cos": c, "reuse": reuse, "idx": sel,
                "out": ns.attend(q_group, np.asarray(K, float)[sel], np.asarray(V, float)[sel])}

    def decode_layer(q, q_prev, kv_of, hkv, k, tau, dtype, idx_prev=None, units=None, head_of=None,
                     tau_of=None):
        qf, qpf = ns.as_f64(q, dtype), ns.as_f64(q_prev, dtype)
        B, Hq, _ = qf.shape
        g = Hq // hkv
        res = {}
        for b in range(B):
            for h in range(hkv):
                heads = head_of(h, g, hkv, Hq) if head_of else list(range(h * g, (h + 1) * g))
                K, V = kv_of(b, h)
                t = (tau_of or (lambda tau, h: float(tau[h]) if np.ndim(tau) else float(tau)))(tau, h)
                res[(b, h)] = ns.decode_unit(qf[b, heads], qpf[b, heads], ns.as_f64(K, dtype), ns.as_f64(V, dtype),
                                             k, t, None if idx_prev is None else idx_prev[b, h])
        return res

    def decode_steps_unit(queries, K, V, n0, k, tau, policy="previous", grow=1, lag=0, rules=None):
        # rules maps a policy to when the reference is replaced: "previous" every
        # step, "refresh" on a miss, "never" only at the cold step
        rule = (rules or {}).get(policy, policy)
        results, ref, sel = [], None, None
        for t, qg in enumerate(queries):
            n = n0 + grow * t - (lag if t else 0)
            if t == 0:
                r = ns.decode_unit(qg, qg, K[:n], V[:n], k, math.inf)
            else:
                r = ns.decode_unit(qg, ref, K[:n], V[:n], k, tau, sel)
            sel = r["idx"]
            if t == 0 or rule == "previous" or (rule == "refresh" and not r["reuse"]):
                ref = qg
            results.append(r)
        return results

    if "decode_unit" not in over:
        ns.decode_unit = decode_unit
    if "decode_layer" not in over:
        ns.decode_layer = decode_layer
    steps_kw = over.get("steps_kw")
    if steps_kw is not None:
        ns.decode_steps_unit = lambda *a, **kw: decode_steps_unit(*a, **{**kw, **steps_kw})
    elif "decode_steps_unit" not in over:
        ns.decode_steps_unit = decode_steps_unit
    if "head_of" in over:
        ns.decode_layer = lambda *a, **kw: decode_layer(*a, head_of=over["head_of"], **kw)
    if "tau_of" in over:
        ns.decode_layer = lambda *a, **kw: decode_layer(*a, tau_of=over["tau_of"], **kw)
    for name in ("plan_persistent", "quantize_row", "dequantize_row", "select_blocks"):
        if name not in over:
            setattr(ns, name, getattr(base, name))
    return ns


def m_sum_over_heads(q_group, K):
    return (np.asarray(K, float) @ np.asarray(q_group, float).T).sum(axis=1)


def m_mean_head_cosine(a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    cs = [base.group_cosine(a[i:i + 1], b[i:i + 1]) for i in range(a.shape[0])]
    return float(np.mean(cs))


def m_strict_reuse(c, tau):
    return bool(c > tau)


def m_no_scale(q_group, Kc, Vc, return_p=False):
    q = np.asarray(q_group, float)
    return base.attend(q * math.sqrt(q.shape[1]), Kc, Vc, return_p)


def m_softmax_wrong_axis(q_group, Kc, Vc, return_p=False):
    q, Kc, Vc = (np.asarray(x, float) for x in (q_group, Kc, Vc))
    lg = (Kc @ q.T) / math.sqrt(q.shape[1])
    e = np.exp(lg - lg.max(axis=1, keepdims=True))
    p = e / e.sum(axis=1, keepdims=True)
    out = p.T @ Vc
    return (out, p.T) if return_p else out


def m_values_from_keys(q_group, Kc, Vc, return_p=False):
    return base.attend(q_group, Kc, Kc, return_p)


def m_ties_to_larger_index(s, k):
    s = np.asarray(s, float)
    n = s.shape[0]
    order = np.lexsort((-np.arange(n), -s))
    return np.sort(order[:k])


def m_unsorted_topk(s, k):
    return np.argsort(-np.asarray(s, float), kind="stable")[:k]


def m_smallest_k(s, k):
    return base.select_topk(-np.asarray(s, float), k)


def m_head_modulo(h, g, hkv, hq):
    return [x for x in range(hq) if x % hkv == h]


def m_bf16_low_half(a, dtype):
    if dtype == "bf16":
        return np.asarray(a, np.uint16).astype(np.float64)
    return base.as_f64(a, dtype)


def m_cos_no_prev_norm(a, b):
    a, b = np.asarray(a, float).reshape(-1), np.asarray(b, float).reshape(-1)
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(a)))


def m_plan_highest_first(s_hat, n):
    return base.plan_persistent(-np.asarray(s_hat, float), n)


def m_plan_ties_to_higher_index(s_hat, n):
    s = np.asarray(s_hat, float)
    L, H = s.shape
    order = sorted(range(L * H), key=lambda i: (s.reshape(-1)[i], -i))
    masks = [0] * L
    for i in order[:n]:
        masks[i // H] |= 1 << (i % H)
    return masks


def m_quant_floor(x):
    q, e = base.quantize_row(x)
    return np.floor(np.asarray(x, float) * 2.0 ** -e).astype(np.int64), e


def m_quant_exponent_low(x):
    q, e = base.quantize_row(x)
    e -= 1
    return np.clip(np.rint(np.asarray(x, float) * 2.0 ** -e), -127, 127).astype(np.int64), e


def m_quant_half_away(x):
    q, e = base.quantize_row(x)
    y = np.asarray(x, float) * 2.0 ** -e
    return (np.sign(y) * np.floor(np.abs(y) + 0.5)).astype(np.int64), e


def m_blocks_sum(s, k, bs):
    s = np.asarray(s, float)
    nb = s.shape[0] // bs
    bsum = s[:nb * bs].reshape(nb, bs).sum(axis=1)
    blocks = np.sort(base.select_topk(bsum, k // bs))
    return (blocks[:, None] * bs + np.arange(bs)[None, :]).reshape(-1)


def m_blocks_tail_selectable(s, k, bs):
    s = np.asarray(s, float)
    nb = -(-s.shape[0] // bs)
    pad = np.concatenate([s, np.full(nb * bs - s.shape[0], -np.inf)])
    bmax = pad.reshape(nb, bs).max(axis=1)
    blocks = np.sort(base.select_topk(bmax, k // bs))
    out = (blocks[:, None] * bs + np.arange(bs)[None, :]).reshape(-1)
    return out


def m_blocks_ties_high(s, k, bs):
    s = np.asarray(s, float)
    nb = s.shape[0] // bs
    bmax = s[:nb * bs].reshape(nb, bs).max(axis=1)
    order = np.lexsort((-np.arange(nb), -bmax))[:k // bs]
    blocks = np.sort(order)
    return (blocks[:, None] * bs + np.arange(bs)[None, :]).reshape(-1)


MUTANTS = {
    "score_sum_over_heads": dict(token_scores=m_sum_over_heads),
    "cosine_mean_of_heads": dict(group_cosine=m_mean_head_cosine),
    "cosine_wrong_norm": dict(group_cosine=m_cos_no_prev_norm),
    "reuse_strict": dict(reuse_decision=m_strict_reuse),
    "attention_no_scale": dict(attend=m_no_scale),
    "softmax_over_heads": dict(attend=m_softmax_wrong_axis),
    "values_from_keys": dict(attend=m_values_from_keys),
    "ties_to_larger_index": dict(select_topk=m_ties_to_larger_index),
    "topk_unsorted": dict(select_topk=m_unsorted_topk),
    "topk_smallest": dict(select_topk=m_smallest_k),
    "gqa_head_modulo": dict(head_of=m_head_modulo),
    "bf16_decoded_as_int": dict(as_f64=m_bf16_low_half),
    # many steps: the context does not grow, grows one step late, or the
    # reference is kept / replaced at the wrong steps
    "tau_heads_ignored": dict(tau_of=lambda tau, h: float(np.max(tau)) if np.ndim(tau) else float(tau)),
    "tau_heads_reversed": dict(tau_of=lambda tau, h: float(tau[::-1][h]) if np.ndim(tau) else float(tau)),
    "plan_highest_similarity": dict(plan_persistent=m_plan_highest_first),
    "plan_ties_to_higher_index": dict(plan_persistent=m_plan_ties_to_higher_index),
    "quant_floor": dict(quantize_row=m_quant_floor),
    "quant_exponent_low": dict(quantize_row=m_quant_exponent_low),
    "quant_ties_away": dict(quantize_row=m_quant_half_away),
    "dequant_wrong_sign_exponent": dict(dequantize_row=lambda q, e: np.asarray(q, float) * 2.0 ** -e),
    "blocks_scored_by_sum": dict(select_blocks=m_blocks_sum),
    "blocks_tail_selectable": dict(select_blocks=m_blocks_tail_selectable),
    "blocks_ties_to_higher": dict(select_blocks=m_blocks_ties_high),
    "steps_context_fixed": dict(steps_kw=dict(grow=0)),
    "steps_context_one_late": dict(steps_kw=dict(lag=1)),
    "steps_refresh_never_updates": dict(steps_kw=dict(rules={"refresh": "never"})),
    "steps_refresh_as_previous": dict(steps_kw=dict(rules={"refresh": "previous"})),
    "steps_previous_as_refresh": dict(steps_kw=dict(rules={"previous": "refresh"})),
}


def test_unmutated_namespace_passes():
    ns = _ns()
    for pin in ALL_PINS:
        pin(ns)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    ns = _ns(**MUTANTS[name])
    failed = []
    for pin in ALL_PINS:
        try:
            pin(ns)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"

"""Plant plausible mistakes in the oracle's own source; each must fail at least one pin.

Every mutant is a fresh copy of oracle/clo_oracle.py, executed as a module of
its own after one or more text edits (each edit site must occur exactly once),
or with one function replaced.  The oracle's functions look each other up in
their module, so a mutant goes through the real decode_unit, decode_layer and
decode_steps_unit: a dropped term, a wrong sign or index, or a transposed
operand anywhere in the arithmetic, or in the way those compositions route
their arguments, must be caught by the pins.
"""
import os
import types

import numpy as np
import pytest

from oracle import clo_oracle as base
from tests.oracle_pins import ALL_PINS

SRC_PATH = base.__file__
with open(SRC_PATH, encoding="utf-8") as _f:
    SRC = _f.read()


def mutant_module(edits=(), funcs=None, name="clo_oracle_mutant"):
    """A copy of the oracle with text edits [(old, new), ...] and function replacements."""
    src = SRC
    for old, new in edits:
        n = src.count(old)
        assert n == 1, f"mutation site {old!r} occurs {n} times in {os.path.basename(SRC_PATH)}"
        src = src.replace(old, new)
    mod = types.ModuleType(name)
    mod.__file__ = SRC_PATH
    exec(compile(src, f"<{name}>", "exec"), mod.__dict__)
    for fname, f in (funcs or {}).items():
        assert hasattr(mod, fname), fname
        setattr(mod, fname, f)
    return mod


def m_mean_head_cosine(a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    return float(np.mean([base.group_cosine(a[i:i + 1], b[i:i + 1]) for i in range(a.shape[0])]))


E = lambda old, new: dict(edits=[(old, new)])  # noqa: E731

MUTANTS = {
    # reuse test
    "cosine_mean_of_heads": dict(funcs=dict(group_cosine=m_mean_head_cosine)),
    "cosine_wrong_norm": E("nb = math.sqrt(float(np.sum(b * b)))", "nb = math.sqrt(float(np.sum(a * a)))"),
    "reuse_strict": E("return bool(c >= tau)", "return bool(c > tau)"),
    # scoring and top-k
    "score_sum_over_heads": E("return per_head.max(axis=1)", "return per_head.sum(axis=1)"),
    "ties_to_larger_index": E('order = np.argsort(-s, kind="stable")',
                              'order = s.shape[0] - 1 - np.argsort(-s[::-1], kind="stable")'),
    "topk_unsorted": E("return np.sort(order[:k]).astype(np.int64)", "return order[:k].astype(np.int64)"),
    "topk_smallest": E('order = np.argsort(-s, kind="stable")', 'order = np.argsort(s, kind="stable")'),
    # attention
    "attention_no_scale": E("logits = (Kc @ q.T) / math.sqrt(d)", "logits = Kc @ q.T"),
    "softmax_over_heads": dict(edits=[("m = logits.max(axis=0, keepdims=True)", "m = logits.max(axis=1, keepdims=True)"),
                                      ("p = e / e.sum(axis=0, keepdims=True)", "p = e / e.sum(axis=1, keepdims=True)")]),
    "values_from_keys": E("out = p.T @ Vc", "out = p.T @ Kc"),
    # bf16 decoding
    "bf16_decoded_as_int": E("return (bits * np.uint32(65536)).view(np.float32).astype(np.float64)",
                             "return bits.astype(np.float64)"),
    # one unit: rows attention reads apart from the scored keys, block selection
    "attend_scored_keys": E("Kc = np.asarray(K if K_attn is None else K_attn, dtype=np.float64)[sel]",
                            "Kc = np.asarray(K, dtype=np.float64)[sel]"),
    "attend_exact_values": E("Vc = np.asarray(V if V_attn is None else V_attn, dtype=np.float64)[sel]",
                             "Vc = np.asarray(V, dtype=np.float64)[sel]"),
    "score_attention_rows": E("s = token_scores(q_group, K)", "s = token_scores(q_group, K if K_attn is None else K_attn)"),
    "unit_ignores_block_size": E("sel = select_topk(s, k) if block_size <= 1 else select_blocks(s, k, block_size)",
                                 "sel = select_topk(s, k)"),
    # one layer: GQA grouping, thresholds, previous selections, routing of the unit's arguments
    "gqa_head_modulo": E("decode_unit(qf[b, kvh * g:(kvh + 1) * g], qpf[b, kvh * g:(kvh + 1) * g],",
                         "decode_unit(qf[b, kvh::hkv], qpf[b, kvh::hkv],"),
    "tau_heads_ignored": E("tau_u = float(tau[kvh]) if np.ndim(tau) else float(tau)", "tau_u = float(np.max(tau))"),
    "tau_heads_reversed": E("tau_u = float(tau[kvh]) if np.ndim(tau) else float(tau)",
                            "tau_u = float(tau[::-1][kvh]) if np.ndim(tau) else float(tau)"),
    "previous_selection_of_head_0": E("prev = None if idx_prev is None else idx_prev[b, kvh]",
                                      "prev = None if idx_prev is None else idx_prev[b, 0]"),
    "layer_ignores_attention_rows": E("ka = attn_kv_of(b, kvh) if attn_kv_of else None", "ka = None"),
    "layer_ignores_block_size": E("*(ka if ka is not None else (None, None)), block_size=block_size)",
                                  "*(ka if ka is not None else (None, None)))"),
    # persistent-head planning
    "plan_highest_similarity": E("key=lambda i: (s.reshape(-1)[i], i)", "key=lambda i: (-s.reshape(-1)[i], i)"),
    "plan_ties_to_higher_index": E("key=lambda i: (s.reshape(-1)[i], i)", "key=lambda i: (s.reshape(-1)[i], -i)"),
    # int8 rows
    "quant_floor": E("q = np.rint(x * 2.0 ** -e).astype(np.int64)", "q = np.floor(x * 2.0 ** -e).astype(np.int64)"),
    "quant_exponent_low": E("e = max(e, QUANT_MIN_EXP)", "e = max(e, QUANT_MIN_EXP) - 1"),
    "quant_ties_away": E("q = np.rint(x * 2.0 ** -e).astype(np.int64)",
                         "q = (np.sign(x) * np.floor(np.abs(x * 2.0 ** -e) + 0.5)).astype(np.int64)"),
    "dequant_wrong_sign_exponent": E("return np.asarray(q, dtype=np.float64) * 2.0 ** e",
                                     "return np.asarray(q, dtype=np.float64) * 2.0 ** -e"),
    "quantized_rows_by_column": E("    for i in range(X.shape[0]):\n        out[i] = dequantize_row(*quantize_row(X[i], bits))",
                                  "    for i in range(X.shape[1]):\n        out[:, i] = dequantize_row(*quantize_row(X[:, i], bits))"),
    # 4-bit rows: the range's exponent off by one, 8 levels, the width dropped
    # on the way through quantized_rows, the nibbles swapped or unsigned
    "quant_range_exponent_high": E("f = math.frexp(M)[1] - 1", "f = math.frexp(M)[1]"),
    "quant4_eight_levels": E("return 2 ** (bits - 1) - 1", "return 2 ** (bits - 1) - (1 if bits == 8 else 0)"),
    "quantized_rows_drops_width": E("out[i] = dequantize_row(*quantize_row(X[i], bits))",
                                    "out[i] = dequantize_row(*quantize_row(X[i]))"),
    "pack_nibbles_swapped": E("(q[2 * j] & 0xF) | ((q[2 * j + 1] & 0xF) << 4)",
                              "((q[2 * j] & 0xF) << 4) | (q[2 * j + 1] & 0xF)"),
    "pack_offset_binary": E("(q[2 * j] & 0xF) | ((q[2 * j + 1] & 0xF) << 4)",
                            "((q[2 * j] + 8) & 0xF) | (((q[2 * j + 1] + 8) & 0xF) << 4)"),
    # block selection
    "blocks_scored_by_sum": E("bscore = s[:nb * block_size].reshape(nb, block_size).max(axis=1)",
                              "bscore = s[:nb * block_size].reshape(nb, block_size).sum(axis=1)"),
    "blocks_tail_selectable": dict(edits=[
        ("nb = s.shape[0] // block_size", "nb = -(-s.shape[0] // block_size)"),
        ("bscore = s[:nb * block_size].reshape(nb, block_size).max(axis=1)",
         "bscore = np.concatenate([s, np.full(nb * block_size - s.shape[0], -np.inf)]).reshape(nb, block_size).max(axis=1)")]),
    "blocks_ties_to_higher": E("blocks = np.sort(select_topk(bscore, k // block_size))",
                               "blocks = np.sort(nb - 1 - select_topk(bscore[::-1], k // block_size))"),
    # many steps: the context does not grow, grows one step late, or the
    # reference is kept / replaced at the wrong steps
    "steps_context_fixed": E("n = n0 + t", "n = n0"),
    "steps_context_one_late": E("n = n0 + t", "n = n0 + max(t - 1, 0)"),
    "steps_refresh_never_updates": E('if policy == "previous" or not r["reuse"]:', 'if policy == "previous" or t == 0:'),
    "steps_refresh_as_previous": E('if policy == "previous" or not r["reuse"]:', "if True:"),
    "steps_previous_as_refresh": E('if policy == "previous" or not r["reuse"]:', 'if not r["reuse"]:'),
}


def test_unmutated_copy_passes():
    mod = mutant_module()
    for pin in ALL_PINS:
        pin(mod)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = mutant_module(name=f"mutant_{name}", **MUTANTS[name])
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"

"""Parity at the five workload shapes, in the launch configuration bench.py times.

Every unit of configs 1, 2 and 3 is compared with the oracle at both steps of
the two-step protocol (reuse decision and selection bit-exact, cache rows bit
for bit, outputs within tolerance).  Configs 4 and 5 run all 48 layers through
the three-stream layer loop with the bench's distinct data layers (8 for
config 4, 16 for config 5); 8 layers with 8 different data layers are
compared (config 5: all their units; config 4: every miss unit and some reuse
units of each), and every unit of those
layers is checked for its reuse decision and a valid selection.  Config 3's
shape is also run with int8 and int4 host KV and with 16-token blocks on sampled
units, and config 5's loop with int4 host KV on 3 of those layers.
Each case logs its largest normwise output error against the tolerance.

The oracle and the margin work run per unit on a pool of threads (each with a
one-thread BLAS): the oracle itself is unchanged, only units run side by side.
"""
import gc
import math
import os

import numpy as np
import pytest

import gen
import oracle
from oracle.margins import COS_MARGIN, enforce_block_margins, enforce_margins, for_units
from tests.gpu_common import compare, log, log_worst, merge_worst, snapshot

pytestmark = pytest.mark.gpu

try:
    WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))
except (AttributeError, OSError):
    WORKERS = 8


class _Prev:
    """idx_prev for decode_layer restricted to one unit."""

    def __init__(self, idx):
        self.idx = idx

    def __getitem__(self, key):
        return self.idx


def check_unit(p, layer, bufs, got0, got1, b, h, q, qp, block_size=1, quant_bits=0, tag=""):
    """Both steps of one unit against the oracle; returns the two compare() results."""
    K = p.kv("k", layer, b, h, threads=1)
    V = p.kv("v", layer, b, h, threads=1)
    kv = lambda bb, hh: (K, V)  # noqa: E731
    attn = cache_of = None
    if quant_bits and not bufs.is_persistent(h):
        Kq = oracle.quantized_rows(oracle.as_f64(K, p.dtype), quant_bits)
        Vq = oracle.quantized_rows(oracle.as_f64(V, p.dtype), quant_bits)
        attn = lambda bb, hh: (Kq, Vq)  # noqa: E731
        cache_of = attn
    u = [(b, h)]
    r0 = oracle.decode_layer(qp, qp, kv, p.hkv, p.topk, math.inf, p.dtype, units=u, attn_kv_of=attn,
                             block_size=block_size)
    r1 = oracle.decode_layer(q, qp, kv, p.hkv, p.topk, p.tau, p.dtype, idx_prev=_Prev(r0[(b, h)]["idx"]), units=u,
                             attn_kv_of=attn, block_size=block_size)
    e0 = compare(p, bufs, got0, r0, kv, f"{tag} step0", cache_of=cache_of)
    e1 = compare(p, bufs, got1, r1, kv, f"{tag} step1", cache_of=cache_of)
    if r1[(b, h)]["reuse"]:
        assert np.array_equal(got1["idx"][b, h], got0["idx"][b, h]), f"{tag} ({b}, {h}): hit changed idx"
    return e0, e1


def check_units(p, layer, bufs, got0, got1, units, tag, **kw):
    q, qp = p.q(layer), p.q_prev(layer)
    res = for_units(lambda b, h: check_unit(p, layer, bufs, got0, got1, b, h, q, qp, tag=tag, **kw), units,
                    WORKERS)
    log_worst(tag, "step0", merge_worst(r[0] for r in res), p.dtype)
    log_worst(tag, "step1", merge_worst(r[1] for r in res), p.dtype)


def check_all_units(p, layer, got, step, block_size=1):
    """Properties of every unit: reuse decisions equal the oracle's; selections valid."""
    g = p.g
    tau = p.tau if step == 1 else math.inf
    q = oracle.as_f64(p.q(layer) if step == 1 else p.q_prev(layer), p.dtype)
    qp = oracle.as_f64(p.q_prev(layer), p.dtype)
    for b in range(p.batch):
        for h in range(p.hkv):
            c = oracle.group_cosine(q[b, h * g:(h + 1) * g], qp[b, h * g:(h + 1) * g])
            assert bool(got["reuse"][b, h]) == oracle.reuse_decision(c, tau), (layer, b, h)
            idx = got["idx"][b, h]
            assert idx.shape[0] == p.topk and idx[0] >= 0 and idx[-1] < p.context
            assert np.all(np.diff(idx) > 0), (layer, b, h)
            if block_size > 1:
                blk = idx.reshape(-1, block_size)
                assert np.all(blk == blk[:, :1] + np.arange(block_size)), (layer, b, h)


def unit_classes(p, layer):
    g = p.g
    q = oracle.as_f64(p.q(layer), p.dtype)
    qp = oracle.as_f64(p.q_prev(layer), p.dtype)
    miss, hit = [], []
    for b in range(p.batch):
        for h in range(p.hkv):
            c = oracle.group_cosine(q[b, h * g:(h + 1) * g], qp[b, h * g:(h + 1) * g])
            (hit if oracle.reuse_decision(c, p.tau) else miss).append((b, h))
    return miss, hit


def sample_units(p, layer, n_miss, n_hit, seed=0):
    miss, hit = unit_classes(p, layer)
    rng = np.random.default_rng(seed)
    pick = lambda xs, n: [xs[i] for i in sorted(rng.choice(len(xs), size=min(n, len(xs)), replace=False))]  # noqa
    return pick(miss, n_miss) + pick(hit, n_hit)


def enforce_cos_all(p, layer):
    """Cosine margins on every unit of a layer (only q_prev redraws; cheap)."""
    all_units = [(b, h) for b in range(p.batch) for h in range(p.hkv)]
    g = p.g
    for _ in range(20):
        q = oracle.as_f64(p.q(layer), p.dtype)
        qp = oracle.as_f64(p.q_prev(layer), p.dtype)
        redo = [(b, h) for b, h in all_units
                if abs(oracle.group_cosine(q[b, h * g:(h + 1) * g], qp[b, h * g:(h + 1) * g]) - p.tau) < COS_MARGIN]
        if not redo:
            return
        for b, h in redo:
            p.resample_q_prev(layer, b, h)
    raise RuntimeError("cosine margins")


def _release():
    import torch

    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _run_single_layer(p, host_format=0, block_size=1):
    from top_sparse_attention_02_amd import workload

    bufs = workload.load_layer(p, 0, host_format=host_format)
    if block_size > 1:
        bufs.set_block_size(block_size)
    bufs.step0()
    got0 = snapshot(bufs)
    bufs.step1()
    got1 = snapshot(bufs)
    return bufs, got0, got1


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_single_layer_configs_every_unit(need_gpu, cfg):
    p = gen.config(cfg)
    tag = f"full config {cfg}"
    enforce_cos_all(p, 0)
    units = [(b, h) for b in range(p.batch) for h in range(p.hkv)]
    log(f"[{tag}] margins for all {len(units)} units on {WORKERS} threads")
    enforce_margins(p, 0, units=units, workers=WORKERS)
    log(f"[{tag}] generating, loading, two steps on the GPU")
    bufs, got0, got1 = _run_single_layer(p)
    log(f"[{tag}] oracle")
    check_units(p, 0, bufs, got0, got1, units, tag)
    check_all_units(p, 0, got0, 0)
    check_all_units(p, 0, got1, 1)
    del bufs, got0, got1
    _release()


QUANT = {"int8_host_kv": 8, "int4_host_kv": 4}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("variant", ["int8_host_kv", "int4_host_kv", "blocks_16"])
def test_config3_shape_variants(need_gpu, variant):
    from top_sparse_attention_02_amd import clo

    bs = 16 if variant == "blocks_16" else 1
    bits = QUANT.get(variant, 0)
    host_format = {8: clo.CLO_HOST_INT8, 4: clo.CLO_HOST_INT4}.get(bits, clo.CLO_HOST_NATIVE)
    p = gen.config(3) if bs == 1 else gen.config(3, topk=gen.config(3).topk // bs * bs)
    tag = f"config 3 {variant}"
    enforce_cos_all(p, 0)
    units = sample_units(p, 0, n_miss=12, n_hit=12, seed=3)
    log(f"[{tag}] margins for {len(units)} sampled units (k={p.topk})")
    if bs > 1:
        enforce_block_margins(p, 0, bs, units=units, workers=WORKERS)
    else:
        enforce_margins(p, 0, units=units, workers=WORKERS)
    bufs, got0, got1 = _run_single_layer(p, host_format=host_format, block_size=bs)
    log(f"[{tag}] oracle")
    check_units(p, 0, bufs, got0, got1, units, tag, block_size=bs, quant_bits=bits)
    check_all_units(p, 0, got0, 0, block_size=bs)
    check_all_units(p, 0, got1, 1, block_size=bs)
    del bufs, got0, got1
    _release()


# the bench's distinct data layers (layer l holds data layer l % D), and 8 layers
# over 8 different data layers
DATA_LAYERS = {4: 8, 5: 16}
LAYERS_CHECKED = {4: [0, 9, 18, 27, 36, 45, 6, 15], 5: [0, 17, 34, 3, 20, 37, 6, 47]}
# with int4 host KV, three of them, those with the most offloaded heads (the
# oracle dequantizes every row of an offloaded unit, one row at a time)
LAYERS_CHECKED_QUANT = {5: [34, 3, 47]}


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("cfg,bits", [(4, 0), (5, 0), (5, 4)], ids=["config4", "config5", "config5_int4_host_kv"])
def test_layer_loop_configs_full_size(need_gpu, cfg, bits):
    import torch

    from top_sparse_attention_02_amd import clo, workload

    host_format = {8: clo.CLO_HOST_INT8, 4: clo.CLO_HOST_INT4}.get(bits, clo.CLO_HOST_NATIVE)
    p = gen.config(cfg, data_layers=DATA_LAYERS[cfg])
    checked = LAYERS_CHECKED_QUANT[cfg] if bits else LAYERS_CHECKED[cfg]
    assert len({p.data_layer(l) for l in checked}) == len(checked)
    tag = f"full config {cfg}" + (f" int{bits} host KV" if bits else "")
    samples = {}
    for l in checked:
        enforce_cos_all(p, l)
        if cfg == 5:
            samples[l] = [(b, h) for b in range(p.batch) for h in range(p.hkv)]
        else:
            miss, hit = unit_classes(p, l)
            samples[l] = miss + sample_units(p, l, n_miss=0, n_hit=4, seed=l)
        enforce_margins(p, l, units=samples[l], workers=WORKERS)
    mixes = [(bool(p.persistent[l].any()), bool((~p.persistent[l]).any())) for l in checked]
    assert any(a for a, _ in mixes) and any(b for _, b in mixes), "persistent and offloaded heads both covered"
    log(f"[{tag}] generating and loading 48 layers ({p.data_layers} data layers)")
    layers = workload.load_layers(p, host_format=host_format)
    loop = workload.LayerLoop(layers)
    loop.step(cold=True)
    torch.cuda.synchronize()
    loop.check()
    got0 = {l: snapshot(layers[l]) for l in checked}
    loop.step()
    torch.cuda.synchronize()
    loop.check()
    got1 = {l: snapshot(layers[l]) for l in checked}
    for l in checked:
        n_p = sum(1 for b, h in samples[l] if layers[l].is_persistent(h))
        log(f"[{tag}] oracle, layer {l}: {len(samples[l])} units ({n_p} of persistent heads)")
        check_units(p, l, layers[l], got0[l], got1[l], samples[l], f"{tag} layer {l}", quant_bits=bits)
        check_all_units(p, l, got0[l], 0)
        check_all_units(p, l, got1[l], 1)
    del layers, loop, got0, got1
    _release()

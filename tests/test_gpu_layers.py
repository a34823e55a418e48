"""Multi-layer decode step (layer-ahead selection and gather on their own streams,
ordered by device flags) and the device-side wait/signal protocol."""
import math

import numpy as np
import pytest

import gen
from tests.gpu_common import compare, log, oracle_steps, snapshot
from oracle.margins import enforce_margins

pytestmark = pytest.mark.gpu


def multi_layer_problem():
    return gen.Problem(name="layers", layers=6, data_layers=3, batch=2, hq=10, hkv=2, d=128, context=3000,
                       topk=300, dtype="bf16", tau=0.8, seed=0x5EED0200, qprev_model="target_cos", low_frac=0.5,
                       heavy_frac=0.005,
                       persistent=np.array([[1, 0], [0, 0], [0, 1], [1, 0], [0, 0], [0, 1]], dtype=bool))


def enforce_all_layers(p):
    # aliased layers score the same keys with different queries: repeat until no layer resamples
    for _ in range(10):
        snap = {k: dict(v) for k, v in p.k_resample.items()}
        for l in range(p.layers):
            enforce_margins(p, l)
        if {k: dict(v) for k, v in p.k_resample.items()} == snap:
            return p
    raise RuntimeError("margins did not settle")


@pytest.mark.parametrize("select_streams,gather,select,attend", [
    (1, "resident", "per-layer", "per-layer"), (2, "resident", "per-layer", "per-layer"),
    (3, "resident", "per-layer", "batched"), (1, "per-layer", "per-layer", "per-layer"),
    (1, "resident", "batched", "per-layer"), (1, "per-layer", "batched", "per-layer"),
    (1, "resident", "batched", "batched")])
def test_layer_loop_matches_sequential_and_oracle(need_gpu, select_streams, gather, select, attend):
    import torch

    from top_sparse_attention_02_amd import workload

    p = enforce_all_layers(multi_layer_problem())
    layers = workload.load_layers(p)
    # three batches of selections over the 6 layers (the default sizing takes them in one),
    # attention in batches of 3, 2 and 1 layers
    loop = workload.LayerLoop(layers, select_streams=select_streams, gather=gather, select=select,
                              select_batches=(1, 2, 3) if select == "batched" else None, attend=attend,
                              attend_batches=(3, 2, 1))
    assert loop.attend == (attend if gather == "resident" else "per-layer")
    log(f"[case layer loop, {select_streams} select streams, {gather} gather, {select} selection, "
        f"{attend} attention] cold step")
    loop.step(cold=True)
    torch.cuda.synchronize()
    loop.check()
    a0 = [snapshot(b) for b in layers]
    log("[case layer loop] steady step")
    loop.step()
    torch.cuda.synchronize()
    loop.check()
    a1 = [snapshot(b) for b in layers]
    # the same steps, layer by layer on one stream with the fused entry point
    for b in layers:
        b.step0()
    b0 = [snapshot(b) for b in layers]
    for b in layers:
        b.step1()
    b1 = [snapshot(b) for b in layers]
    for l in range(p.layers):
        for key in a0[l]:
            assert np.array_equal(a0[l][key], b0[l][key]), (l, key)
            assert np.array_equal(a1[l][key], b1[l][key]), (l, key)
    # and the oracle, layer by layer
    for l in range(p.layers):
        r0, r1, kv = oracle_steps(p, l)
        compare(p, layers[l], a0[l], r0, kv, f"layer {l} step0")
        compare(p, layers[l], a1[l], r1, kv, f"layer {l} step1")


def wide_layer_problem():
    # 64 units per layer (16 sequences x 4 KV heads): the most a batched selection
    # takes, and the resident gather's grid for layers of 64 units or more
    return gen.Problem(name="layers_wide", layers=3, batch=16, hq=16, hkv=4, d=128, context=1500, topk=150,
                       dtype="bf16", tau=0.8, seed=0x5EED0202, qprev_model="target_cos", low_frac=0.5,
                       heavy_frac=0.005,
                       persistent=np.array([[0, 1, 0, 0], [0, 0, 0, 0], [1, 0, 0, 1]], dtype=bool))


@pytest.mark.parametrize("host_kv,units,blocks", [("int8", 4, 32), ("int4", 4, 32), ("int8", 64, 40),
                                                  ("int4", 64, 40)])
def test_layer_loop_quantized_host_kv_matches_sequential(need_gpu, host_kv, units, blocks):
    """The three-stream loop over layers whose offloaded KV is quantized in host memory
    (the dequantizing gather inside the resident launch, its in-LDS unit list and the
    fused reuse-select launch) equals the fused step run layer after layer on one
    stream, bit for bit, for layers of 4 units and of 64 (the resident gather's grid
    of 32 and of 40 blocks)."""
    import torch

    from top_sparse_attention_02_amd import clo, workload

    p = enforce_all_layers(multi_layer_problem() if units == 4 else wide_layer_problem())
    assert p.batch * p.hkv == units
    fmt = clo.CLO_HOST_INT8 if host_kv == "int8" else clo.CLO_HOST_INT4
    layers = workload.load_layers(p, host_format=fmt)
    loop = workload.LayerLoop(layers)
    assert loop.plan_blocks == blocks and loop.select == "batched"
    log(f"[case layer loop, {host_kv} host KV, {units} units per layer] cold + steady step")
    loop.step(cold=True)
    loop.step()
    torch.cuda.synchronize()
    loop.check()
    a1 = [snapshot(b) for b in layers]
    for b in layers:
        b.step0()
    for b in layers:
        b.step1()
    b1 = [snapshot(b) for b in layers]
    for l in range(p.layers):
        for key in a1[l]:
            assert np.array_equal(a1[l][key], b1[l][key]), (l, key)


def test_resident_gather_with_a_layer_without_offloaded_heads(need_gpu):
    """The resident gather walks a layer whose heads are all persistent (nothing to
    gather: its counters live in the plan) between layers that gather; three steps
    in a row equal the per-layer gathers bit for bit."""
    import torch

    from top_sparse_attention_02_amd import workload

    p = gen.Problem(name="layers_pers", layers=4, batch=2, hq=8, hkv=2, d=128, context=2500, topk=250,
                    dtype="bf16", tau=0.8, seed=0x5EED0201, qprev_model="target_cos", low_frac=0.5,
                    persistent=np.array([[0, 1], [1, 1], [0, 0], [1, 1]], dtype=bool))
    p = enforce_all_layers(p)
    got = {}
    for mode in ("resident", "per-layer"):
        layers = workload.load_layers(p)
        loop = workload.LayerLoop(layers, gather=mode)
        log(f"[case layers without offloaded heads, {mode}]")
        loop.step(cold=True)
        loop.step()
        loop.step()
        torch.cuda.synchronize()
        loop.check()
        got[mode] = [snapshot(b) for b in layers]
    for l in range(p.layers):
        for key in got["resident"][l]:
            assert np.array_equal(got["resident"][l][key], got["per-layer"][l][key]), (l, key)


def test_resident_gather_wait_times_out_without_hanging(need_gpu):
    """A plan whose selection flags are never set: every block gives up after its
    bounded wait, CLO_E_TIMEOUT lands in the error word, each layer is still
    signalled, and the launch ends."""
    import torch

    from top_sparse_attention_02_amd import clo, workload
    from tests.gpu_common import small_problem

    p = small_problem("resident_timeout", batch=1, hq=4, hkv=2, context=700, topk=70, dtype="f32",
                      persistent=[0, 1])
    bufs = [workload.load_layer(p, 0) for _ in range(2)]
    flags = torch.zeros(2, 2, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    plan = torch.zeros(clo.clo_gather_plan_size(2), dtype=torch.uint8, device="cuda")
    blocks = clo.clo_gather_plan([(b.shape, b.layer(), b.reuse, b.ws, flags[0, l], flags[1, l])
                                  for l, b in enumerate(bufs)], plan)
    clo.clo_gather_layers(plan, 2, blocks, 1, 5, error_word=err, spin_limit=2000)
    torch.cuda.synchronize()
    assert int(err.item()) == clo.CLO_E_TIMEOUT
    assert flags[1].tolist() == [5, 5]


def test_consumer_sees_rows_written_before_the_flag(need_gpu):
    """Delay the producer (gather) on its stream; the consumer (attention) must still
    read the freshly gathered rows because it waits for the producer's flag."""
    import torch

    from top_sparse_attention_02_amd import clo, workload
    from tests.gpu_common import small_problem

    p = small_problem("delay", batch=2, hq=8, hkv=2, context=4000, topk=400, dtype="bf16", persistent=[0, 0],
                      qprev_model="independent")
    enforce_margins(p, 0)
    bufs = workload.load_layer(p, 0)
    bufs.step0()
    torch.cuda.synchronize()
    ref = snapshot(bufs)
    # wipe the cache and output, then redo gather + attention on two streams
    bufs.k_cache.zero_()
    bufs.v_cache.zero_()
    bufs.out.zero_()
    flag = torch.zeros(2, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    sp, sc = torch.cuda.Stream(), torch.cuda.Stream()
    shape, layer = bufs.shape_with(math.inf), bufs.layer()
    torch.cuda.synchronize()
    with torch.cuda.stream(sp):
        torch.cuda._sleep(50_000_000)  # tens of milliseconds before the producer starts
    clo.clo_gather_kv(shape, layer, None, bufs.ws, sync=clo.Sync(signal_flag=flag[0], signal_value=7), stream=sp)
    clo.clo_sparse_attn(shape, layer, bufs.q_prev, bufs.out, bufs.ws,
                        sync=clo.Sync(wait_flag=flag[0], wait_value=7, error_word=err), stream=sc)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got = snapshot(bufs)
    assert np.array_equal(got["k_cache"], ref["k_cache"])
    assert np.array_equal(got["out"], ref["out"])


def test_never_signalled_flag_times_out_without_hanging(need_gpu):
    import torch

    from top_sparse_attention_02_amd import clo, workload
    from tests.gpu_common import small_problem

    p = small_problem("timeout", batch=1, hq=4, hkv=1, context=500, topk=50, dtype="f32", persistent=[0])
    bufs = workload.load_layer(p, 0)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    clo.clo_gather_kv(bufs.shape_with(math.inf), bufs.layer(), None, bufs.ws,
                      sync=clo.Sync(wait_flag=flag[0], wait_value=1, error_word=err, spin_limit=2000))
    torch.cuda.synchronize()
    assert int(err.item()) == clo.CLO_E_TIMEOUT


def test_reuse_select_wait_times_out_without_hanging(need_gpu):
    """The wait folded into clo_reuse_select's single-block launch is bounded too: a flag
    that is never set (tiny spin limit) ends in CLO_E_TIMEOUT, and the selection still
    runs, equal to the oracle's."""
    import torch

    import oracle
    from top_sparse_attention_02_amd import clo, workload
    from tests.gpu_common import small_problem

    p = small_problem("rsel_timeout", batch=1, hq=4, hkv=2, context=600, topk=60, dtype="f32", persistent=[1, 0])
    enforce_margins(p, 0)
    bufs = workload.load_layer(p, 0)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    sig = torch.zeros(1, dtype=torch.int32, device="cuda")
    clo.clo_reuse_select(bufs.shape_with(math.inf), bufs.layer(), bufs.q_prev, bufs.q_prev, bufs.reuse, bufs.cos,
                         bufs.ws, sync=clo.Sync(wait_flag=flag[0], wait_value=1, error_word=err, spin_limit=2000,
                                                signal_flag=sig[0], signal_value=4))
    torch.cuda.synchronize()
    assert int(err.item()) == clo.CLO_E_TIMEOUT
    assert int(sig.item()) == 4
    qp = p.q_prev(0)
    for h in range(p.hkv):
        ref = oracle.decode_unit(qp[0, h * 2:(h + 1) * 2], qp[0, h * 2:(h + 1) * 2],
                                 oracle.as_f64(p.kv("k", 0, 0, h), "f32"), oracle.as_f64(p.kv("v", 0, 0, h), "f32"),
                                 p.topk, math.inf)
        assert np.array_equal(bufs.idx[0, h].cpu().numpy(), ref["idx"])


def test_already_signalled_flag_does_not_wait(need_gpu):
    import time

    import torch

    from top_sparse_attention_02_amd import clo

    flag = torch.full((1,), 5, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    shape = clo.Shape(0, 4, 1, 10, 1, 0.8, clo.CLO_F32)  # empty batch: only the wait and the signal run
    t = time.perf_counter()
    clo.clo_gather_kv(shape, clo.Layer(), None, None,
                      sync=clo.Sync(wait_flag=flag[0], wait_value=5, signal_flag=flag[0], signal_value=9,
                                    error_word=err))
    torch.cuda.synchronize()
    assert time.perf_counter() - t < 0.5
    assert int(err.item()) == 0 and int(flag.item()) == 9

"""GPU parity: the HIP path through the C ABI against the CPU oracle on seeded inputs.

Reuse decisions, top-k index sets and gathered cache rows must match bit for
bit; attention outputs within 1e-4 (fp32) / 2e-2 (bf16), normwise per output
row.  Sizes span several work items of every kernel plus ragged tails.
"""
import math

import numpy as np
import pytest

import oracle
from tests.gpu_common import log, log_worst, run_and_check, small_problem, snapshot, compare, oracle_steps
from oracle.margins import enforce_margins

pytestmark = pytest.mark.gpu

CASES = {
    # fp32, group 4, both KV heads persistent (config-1 style), ragged N
    "f32_g4_persistent": dict(batch=2, hq=8, hkv=2, context=5000, topk=500, dtype="f32", persistent=[1, 1]),
    # bf16, group 2, mixed persistent mask, heavy-hitter keys
    "bf16_g2_mixed": dict(batch=2, hq=8, hkv=4, context=3000, topk=301, dtype="bf16", persistent=[1, 0, 1, 0],
                          heavy_frac=0.01),
    # bf16, group 5 (Qwen2.5-14B grouping), host-resident heads only
    "bf16_g5_host": dict(batch=3, hq=10, hkv=2, context=4100, topk=410, dtype="bf16", persistent=[0, 0],
                         heavy_frac=0.005),
    # fp32, group 8, previous query mixed from the current one
    "f32_g8": dict(batch=1, hq=16, hkv=2, context=777, topk=78, dtype="f32", persistent=[0, 1], qprev_model="mix"),
    # bf16, group 1 (MHA), independent previous query: every unit misses at step 1
    "bf16_g1": dict(batch=2, hq=4, hkv=4, context=2049, topk=205, dtype="bf16", persistent=[0, 0, 1, 1],
                    qprev_model="independent"),
    # more than one score chunk per unit and a top-k spanning several 4096-key tiles
    "bf16_g4_long": dict(batch=1, hq=8, hkv=2, context=20000, topk=2000, dtype="bf16", persistent=[0, 1]),
    # long context: the multi-block top-k (17 chunks of 16384 keys, ragged last chunk)
    "bf16_g5_multiblock": dict(batch=1, hq=10, hkv=2, context=270000, topk=27000, dtype="bf16",
                               persistent=[0, 1], heavy_frac=0.005),
    "f32_g4_multiblock": dict(batch=2, hq=8, hkv=2, context=262145, topk=26215, dtype="f32", persistent=[1, 0]),
    # 24 attention chunks, merged by two chunk groups
    "bf16_g4_two_groups": dict(batch=2, hq=8, hkv=2, context=60001, topk=6001, dtype="bf16", persistent=[1, 0]),
    # either side of the switch between the single-block and the multi-block top-k
    # (7 chunks of 16384 keys; 7 chunks and one key)
    "bf16_g4_single_at_switch": dict(batch=1, hq=8, hkv=2, context=114688, topk=11469, dtype="bf16",
                                     persistent=[0, 1]),
    "bf16_g4_multi_at_switch": dict(batch=1, hq=8, hkv=2, context=114689, topk=11469, dtype="bf16",
                                    persistent=[1, 0]),
    # either side of the one-launch top-k's limit (128 chunks of 16384 keys; 128 chunks and
    # one key: the top-k then runs its three radix passes and the write launch by launch)
    "bf16_g4_fused_at_limit": dict(batch=2, hq=4, hkv=1, context=128 * 16384, topk=209716, dtype="bf16",
                                   persistent=[0]),
    "bf16_g4_passes_past_limit": dict(batch=2, hq=4, hkv=1, context=128 * 16384 + 1, topk=209716,
                                      dtype="bf16", persistent=[1]),
    # 20 and 18 units with offloaded heads: the step overlapped over 8 unit ranges
    # of 2-3 units on the helper streams (smaller layers run in order)
    "bf16_g4_overlapped": dict(batch=5, hq=16, hkv=4, context=3001, topk=301, dtype="bf16",
                               persistent=[0, 1, 0, 0], heavy_frac=0.01),
    "f32_g2_overlapped": dict(batch=9, hq=4, hkv=2, context=2000, topk=200, dtype="f32", persistent=[0, 0]),
    # 256 units: one resident gather launch for the 8 ranges, selected in groups of 1, 1, 2 and 4 ranges
    "bf16_g4_resident": dict(batch=64, hq=16, hkv=4, context=2000, topk=200, dtype="bf16",
                             persistent=[0, 1, 0, 0], heavy_frac=0.01),
    "f32_g2_resident": dict(batch=130, hq=4, hkv=2, context=1500, topk=150, dtype="f32", persistent=[0, 0]),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_decode_step_matches_oracle(need_gpu, name):
    p = small_problem(name, **CASES[name])
    enforce_margins(p, 0)
    run_and_check(p)


EDGE = {
    "k_equals_n": dict(batch=1, hq=8, hkv=2, context=300, topk=300, dtype="bf16", persistent=[0, 1]),
    "k_one": dict(batch=2, hq=8, hkv=2, context=1000, topk=1, dtype="f32", persistent=[1, 0]),
    "n_one": dict(batch=1, hq=4, hkv=1, context=1, topk=1, dtype="f32", persistent=[0]),
    "n_small_ragged": dict(batch=3, hq=6, hkv=3, context=67, topk=13, dtype="bf16", persistent=[0, 1, 0]),
}


@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_shapes(need_gpu, name):
    p = small_problem(name, **EDGE[name])
    enforce_margins(p, 0)
    run_and_check(p)


def test_dense_limit_equals_full_attention(need_gpu):
    """k = N with tau = +inf is dense GQA attention: compare with torch SDPA in float64 on the CPU."""
    import torch
    import torch.nn.functional as F

    p = small_problem("dense", batch=2, hq=8, hkv=2, context=700, topk=700, dtype="f32", persistent=[0, 1])
    bufs, got0, _ = run_and_check(p)
    qp = oracle.as_f64(p.q_prev(0), "f32")
    K = np.stack([np.stack([oracle.as_f64(p.kv("k", 0, b, h), "f32") for h in range(2)]) for b in range(2)])
    V = np.stack([np.stack([oracle.as_f64(p.kv("v", 0, b, h), "f32") for h in range(2)]) for b in range(2)])
    ref = F.scaled_dot_product_attention(torch.from_numpy(qp)[:, :, None],
                                         torch.from_numpy(K).repeat_interleave(4, 1).contiguous(),
                                         torch.from_numpy(V).repeat_interleave(4, 1).contiguous())[:, :, 0].numpy()
    err = np.abs(got0["out"] - ref).max() / np.abs(ref).max()
    assert err < 1e-4


@pytest.mark.parametrize("context", [3000, 300000])
def test_ties_go_to_the_smaller_index(need_gpu, context):
    """Duplicate the k-th key into two low-scoring rows (one before it): exact ties on both sides
    (single-block top-k at N = 3000, multi-block across chunks at N = 300000)."""
    from top_sparse_attention_02_amd import workload

    p = small_problem(f"ties{context}", batch=1, hq=4, hkv=2, context=context, topk=context // 10, dtype="bf16",
                      persistent=[0, 1], qprev_model="independent")
    enforce_margins(p, 0, extra_ranks=(p.topk - 1,))
    bufs = workload.load_layer(p, 0)
    qp = oracle.as_f64(p.q_prev(0), "bf16")
    planted = {}
    for h in range(2):
        K = p.kv("k", 0, 0, h)
        s = oracle.token_scores(qp[0, h * 2:(h + 1) * 2], oracle.as_f64(K, "bf16"))
        order = np.argsort(-s, kind="stable")
        r = int(order[p.topk - 1])  # the k-th key
        low = [int(j) for j in order[::-1][:50]]
        x = min(j for j in low if j < r) if any(j < r for j in low) else None
        y = max(j for j in low if j > r)
        targets = [t for t in (x, y) if t is not None]
        for t in targets:
            K[t] = K[r]
        planted[h] = (r, targets, K)
        if bufs.is_persistent(h):
            bufs.k_hbm[0, bufs.slot(h)].copy_(workload.stored_tensor(K, "bf16"))
        else:
            bufs.host_view("k", 0, h)[:] = K
            bufs.k_score[0, bufs.slot(h)].copy_(workload.stored_tensor(K, "bf16"))
    bufs.step0()
    got = snapshot(bufs)
    for h, (r, targets, K) in planted.items():
        V = p.kv("v", 0, 0, h)
        ref = oracle.decode_unit(qp[0, h * 2:(h + 1) * 2], qp[0, h * 2:(h + 1) * 2], oracle.as_f64(K, "bf16"),
                                 oracle.as_f64(V, "bf16"), p.topk, math.inf)
        winner = min([r, *targets])
        assert winner in ref["idx"] and all(t not in ref["idx"] for t in [r, *targets] if t != winner)
        assert np.array_equal(got["idx"][0, h], ref["idx"])


@pytest.mark.parametrize("batch", [2, 5, 64])
def test_standalone_entry_points_equal_fused_step(need_gpu, batch):
    """clo_reuse_test + clo_topk_select + clo_gather_kv + clo_sparse_attn == clo_decode_step, bit for bit,
    for a layer of 8 units (the step in order on one stream), of 20 units (overlapped over unit
    ranges, a gather launch per range) and of 256 units (one resident gather launch)."""
    from top_sparse_attention_02_amd import clo, workload

    p = small_problem(f"split{batch}", batch=batch, hq=8, hkv=4, context=3000, topk=300, dtype="bf16",
                      persistent=[0, 1, 0, 1])
    enforce_margins(p, 0)
    bufs = workload.load_layer(p, 0)
    bufs.step0()
    bufs.step1()
    fused = snapshot(bufs)
    # redo step 1 through the separate calls, starting from step 0's state
    bufs.step0()
    shape = bufs.shape_with(p.tau)
    layer = bufs.layer()
    clo.clo_reuse_test(shape, bufs.q, bufs.q_prev, bufs.reuse, bufs.cos)
    clo.clo_topk_select(shape, layer, bufs.q, bufs.reuse, bufs.ws)
    clo.clo_gather_kv(shape, layer, bufs.reuse, bufs.ws)
    clo.clo_sparse_attn(shape, layer, bufs.q, bufs.out, bufs.ws)
    split = snapshot(bufs)
    for key in fused:
        assert np.array_equal(fused[key], split[key]), key


@pytest.mark.parametrize("batch", [5, 64])
def test_every_unit_reusing_gathers_nothing(need_gpu, batch):
    """A steady step whose every unit reuses (q = q_prev): the overlapped step (20 units: a
    gather launch per range; 256 units: the resident gather, every range with nothing to
    gather but its flags still raised) keeps the cold step's selections and cache rows and
    attends them, equal to the oracle's reuse step."""
    import torch

    from top_sparse_attention_02_amd import clo, workload

    p = small_problem(f"allhit{batch}", batch=batch, hq=16, hkv=4, context=1500, topk=150, dtype="bf16",
                      persistent=[0, 1, 0, 0])
    enforce_margins(p, 0)
    bufs = workload.load_layer(p, 0)
    bufs.step0()
    cold = snapshot(bufs)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    bufs.decode_step(bufs.q_prev, bufs.q_prev, bufs.tau, sync=clo.Sync(error_word=err))
    got = snapshot(bufs)
    assert int(err.item()) == 0
    assert got["reuse"].all()
    for key in ("idx", "k_cache", "v_cache", "out"):
        assert np.array_equal(got[key], cold[key]), key
    qp = p.q_prev(0)
    kv = lambda b, h: (p.kv("k", 0, b, h), p.kv("v", 0, b, h))  # noqa: E731
    ref = oracle.decode_layer(qp, qp, kv, p.hkv, p.topk, p.tau, p.dtype, idx_prev=cold["idx"])
    assert all(r["reuse"] for r in ref.values())
    log_worst(p.name, "all reuse", compare(p, bufs, got, ref, kv, "all reuse", check_cos=False), p.dtype)


@pytest.mark.parametrize("batch", [5, 64])
def test_last_step_gather_time_is_reported(need_gpu, batch):
    """clo_last_step_gather_ms after an overlapped step (20 units: range gathers on two
    streams; 256 units: the resident gather) is a positive GPU time no longer than the step
    itself, as timed with events on the caller's stream around it."""
    import torch

    from top_sparse_attention_02_amd import clo, workload

    p = small_problem(f"gtime{batch}", batch=batch, hq=16, hkv=4, context=3000, topk=300, dtype="bf16",
                      persistent=[0, 1, 0, 0])
    bufs = workload.load_layer(p, 0)
    bufs.step0()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    bufs.step1()
    e1.record()
    torch.cuda.synchronize()
    g = clo.clo_last_step_gather_ms()
    log(f"[case gather time, {batch * 4} units] gather {g:.4f} ms of a {e0.elapsed_time(e1):.4f} ms step")
    assert 0.0 < g <= e0.elapsed_time(e1) + 1e-3


def test_concurrent_steps_on_two_streams_equal_sequential_steps(need_gpu):
    """Two host threads, each on its own stream, run overlapped steps of their own layer at
    the same time (256 units: the resident gather; 20 units: a gather launch per range): the
    calls share the device's helper streams under its lock and keep their flags in their own
    workspaces, so every step's outputs equal the same steps run one after another."""
    import threading

    import torch

    from top_sparse_attention_02_amd import workload

    probs = [small_problem("conc64", batch=64, hq=16, hkv=4, context=1500, topk=150, dtype="bf16",
                           persistent=[0, 1, 0, 0]),
             small_problem("conc5", batch=5, hq=16, hkv=4, context=2000, topk=200, dtype="bf16",
                           persistent=[0, 0, 1, 0])]
    bufs = [workload.load_layer(p, 0) for p in probs]
    for b in bufs:
        b.step0()
        b.step1()
    ref = [snapshot(b) for b in bufs]
    streams = [torch.cuda.Stream() for _ in bufs]
    errors = []

    def run(i):
        try:
            with torch.cuda.stream(streams[i]):
                for _ in range(6):
                    bufs[i].step0(stream=streams[i])
                    bufs[i].step1(stream=streams[i])
            streams[i].synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads) and not errors, errors
    for i, b in enumerate(bufs):
        got = snapshot(b)
        for key in ref[i]:
            assert np.array_equal(ref[i][key], got[key]), (probs[i].name, key)


@pytest.mark.parametrize("batch", [5, 64])
def test_caller_spin_limit_bounds_only_the_callers_wait(need_gpu, batch):
    """A tiny sync.spin_limit on a flag that is already up bounds the caller's own wait
    only: the overlapped step's internal waits (the resident gather's and the attention
    stream's, 256 units) keep the library's bound, so the step reports no time-out and
    equals the step without sync bit for bit."""
    import torch

    from top_sparse_attention_02_amd import clo, workload

    p = small_problem(f"spin{batch}", batch=batch, hq=16, hkv=4, context=1500, topk=150, dtype="bf16",
                      persistent=[0, 1, 0, 0])
    bufs = workload.load_layer(p, 0)
    bufs.step0()
    bufs.step1()
    ref = snapshot(bufs)
    flag = torch.ones(1, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    bufs.step0()
    bufs.decode_step(bufs.q, bufs.q_prev, bufs.tau,
                     sync=clo.Sync(wait_flag=flag[0], wait_value=1, error_word=err, spin_limit=1))
    got = snapshot(bufs)
    assert int(err.item()) == 0
    for key in ref:
        assert np.array_equal(ref[key], got[key]), key


@pytest.mark.parametrize("name,kw", [
    # config-1 shape: 8 units, 2 attention chunks
    ("inorder_f32", dict(batch=1, hq=32, hkv=8, context=4096, topk=410, dtype="f32", persistent=[1] * 8)),
    # 12 chunks per unit, bf16, group 5
    ("inorder_bf16", dict(batch=2, hq=10, hkv=2, context=30000, topk=3000, dtype="bf16", persistent=[1, 1])),
    # 70 units: the reuse test and unit lists in launches of their own
    ("inorder_wide", dict(batch=35, hq=4, hkv=2, context=700, topk=70, dtype="bf16", persistent=[1, 1])),
])
def test_in_order_step_equals_separate_calls(need_gpu, name, kw):
    """Layers without offloaded heads run the whole step in order on one stream (the reuse
    test and unit lists in one launch up to 64 units).  Its outputs equal a separate
    clo_sparse_attn call's bit for bit, and both steps the oracle's."""
    from top_sparse_attention_02_amd import clo, workload

    p = small_problem(name, **kw)
    enforce_margins(p, 0)
    bufs = workload.load_layer(p, 0)
    log(f"[case {name}] U={p.batch * p.hkv} k={p.topk}")
    bufs.step0()
    got0 = snapshot(bufs)
    bufs.step1()
    fused = snapshot(bufs)
    shape, layer = bufs.shape_with(p.tau), bufs.layer()
    bufs.out.zero_()
    clo.clo_sparse_attn(shape, layer, bufs.q, bufs.out, bufs.ws)
    split = snapshot(bufs)
    assert np.array_equal(fused["out"], split["out"])
    r0, r1, kv = oracle_steps(p, 0)
    compare(p, bufs, got0, r0, kv, "step0")
    compare(p, bufs, fused, r1, kv, "step1")


@pytest.mark.parametrize("batch,hkv,persistent", [(2, 4, [1, 0, 0, 1]), (8, 8, [0, 0, 1, 0, 0, 0, 0, 1]),
                                                  (9, 8, [0, 1, 0, 0, 0, 0, 1, 0])])
def test_reuse_select_equals_fused_step(need_gpu, batch, hkv, persistent):
    """clo_reuse_select (reuse test + top-k in one call; one fused launch for the reuse
    test and unit lists up to 64 units, separate launches above) + gather + attention
    == clo_decode_step, bit for bit, at 8, 64 and 72 units (either side of the 64-unit
    bound); its wait on an already-set flag passes through."""
    import torch

    from top_sparse_attention_02_amd import clo, workload

    p = small_problem(f"rsel{batch}", batch=batch, hq=2 * hkv, hkv=hkv, context=2100, topk=210, dtype="bf16",
                      persistent=persistent)
    enforce_margins(p, 0)
    bufs = workload.load_layer(p, 0)
    bufs.step0()
    bufs.step1()
    fused = snapshot(bufs)
    bufs.step0()
    shape = bufs.shape_with(p.tau)
    layer = bufs.layer()
    flag = torch.full((1,), 3, dtype=torch.int32, device="cuda")
    sig = torch.zeros(1, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    bufs.cos.fill_(-7.0)
    clo.clo_reuse_select(shape, layer, bufs.q, bufs.q_prev, bufs.reuse, bufs.cos, bufs.ws,
                         sync=clo.Sync(wait_flag=flag, wait_value=3, error_word=err, signal_flag=sig,
                                       signal_value=5))
    clo.clo_gather_kv(shape, layer, bufs.reuse, bufs.ws)
    clo.clo_sparse_attn(shape, layer, bufs.q, bufs.out, bufs.ws)
    split = snapshot(bufs)
    assert int(err.item()) == 0 and int(sig.item()) == 5
    for key in fused:
        assert np.array_equal(fused[key], split[key]), key


def test_zero_copy_gather_equals_hbm_gather(need_gpu):
    """The gather reads the same bytes from pinned host memory as from an HBM copy."""
    import torch

    from top_sparse_attention_02_amd import clo, workload

    p = small_problem("zc", batch=2, hq=8, hkv=2, context=4000, topk=400, dtype="bf16", persistent=[0, 0])
    bufs = workload.load_layer(p, 0)
    bufs.step0()
    host = snapshot(bufs)
    k_dev = bufs.k_score
    v_dev = torch.empty_like(k_dev)
    from top_sparse_attention_02_amd.hip_host import copy_h2d

    copy_h2d(v_dev.data_ptr(), bufs.v_host.ptr, v_dev.numel() * 2)
    bufs.k_cache.zero_()
    bufs.v_cache.zero_()
    layer = bufs.layer()
    layer.k_host, layer.v_host = k_dev, v_dev
    clo.clo_gather_kv(bufs.shape_with(math.inf), layer, None, bufs.ws)
    dev = snapshot(bufs)
    assert np.array_equal(host["k_cache"], dev["k_cache"])
    assert np.array_equal(host["v_cache"], dev["v_cache"])


def test_per_head_thresholds(need_gpu):
    """Each KV head decides with its own threshold (host array in the shape)."""
    from top_sparse_attention_02_amd import workload

    p = small_problem("tau_heads", batch=3, hq=16, hkv=4, context=3000, topk=300, dtype="bf16",
                      persistent=[1, 0, 0, 1], qprev_model="target_cos", low_frac=0.3)
    taus = [0.3, 0.8, 0.95, 0.5]
    # margins against each head's own threshold
    for h, t in enumerate(taus):
        enforce_margins(p, 0, units=[(b, h) for b in range(p.batch)], tau=t)
    log(f"[case tau_heads] thresholds {taus}")
    bufs = workload.load_layer(p, 0)
    bufs.shape.tau_heads = taus
    bufs.step0()
    got0 = snapshot(bufs)
    bufs.step1()
    got1 = snapshot(bufs)
    r0, _, kv = oracle_steps(p, 0)
    idx0 = np.zeros((p.batch, p.hkv, p.topk), dtype=np.int64)
    for (b, h), r in r0.items():
        idx0[b, h] = r["idx"]
    r1 = oracle.decode_layer(p.q(0), p.q_prev(0), kv, p.hkv, p.topk, taus, p.dtype, idx_prev=idx0)
    compare(p, bufs, got0, r0, kv, "step0")
    compare(p, bufs, got1, r1, kv, "step1")
    # the thresholds change decisions: a unit's outcome follows its own head's tau
    c = got1["cos"]
    for b in range(p.batch):
        for h in range(p.hkv):
            assert bool(got1["reuse"][b, h]) == (c[b, h] >= taus[h])
    assert len({bool(x) for x in got1["reuse"].reshape(-1)}) == 2


@pytest.mark.parametrize("bs,dtype", [(16, "bf16"), (64, "f32"), (3, "bf16")])
def test_block_selection(need_gpu, bs, dtype):
    """Token blocks as the selection unit (full blocks only, ragged tail ignored)."""
    from oracle.margins import enforce_block_margins
    from top_sparse_attention_02_amd import workload

    p = small_problem(f"blocks_{bs}_{dtype}", batch=2, hq=8, hkv=2, context=5007, topk=40 * bs, dtype=dtype,
                      persistent=[0, 1])
    enforce_margins(p, 0)
    enforce_block_margins(p, 0, bs)
    log(f"[case blocks {bs} {dtype}] N={p.context} k={p.topk}")
    bufs = workload.load_layer(p, 0)
    bufs.set_block_size(bs)
    bufs.step0()
    got0 = snapshot(bufs)
    bufs.step1()
    got1 = snapshot(bufs)
    memo = {}

    def kv(b, h):
        if (b, h) not in memo:
            memo[(b, h)] = (p.kv("k", 0, b, h), p.kv("v", 0, b, h))
        return memo[(b, h)]

    qp, q = p.q_prev(0), p.q(0)
    r0 = oracle.decode_layer(qp, qp, kv, p.hkv, p.topk, math.inf, p.dtype, block_size=bs)
    idx0 = np.zeros((p.batch, p.hkv, p.topk), dtype=np.int64)
    for (b, h), r in r0.items():
        idx0[b, h] = r["idx"]
    r1 = oracle.decode_layer(q, qp, kv, p.hkv, p.topk, p.tau, p.dtype, idx_prev=idx0, block_size=bs)
    compare(p, bufs, got0, r0, kv, "step0")
    compare(p, bufs, got1, r1, kv, "step1")
    # every selection is whole blocks
    for b in range(p.batch):
        for h in range(p.hkv):
            sel = got1["idx"][b, h]
            assert np.all(sel.reshape(-1, bs) == (sel.reshape(-1, bs)[:, :1] + np.arange(bs)))
    # step 1 again through clo_reuse_select (its single-block reuse test and unit
    # lists clear the block-key histograms), the gather and attention: bit for bit
    from top_sparse_attention_02_amd import clo

    bufs.step0()
    shape, layer = bufs.shape_with(p.tau), bufs.layer()
    clo.clo_reuse_select(shape, layer, bufs.q, bufs.q_prev, bufs.reuse, bufs.cos, bufs.ws)
    clo.clo_gather_kv(shape, layer, bufs.reuse, bufs.ws)
    clo.clo_sparse_attn(shape, layer, bufs.q, bufs.out, bufs.ws)
    split = snapshot(bufs)
    for key in got1:
        assert np.array_equal(got1[key], split[key]), key

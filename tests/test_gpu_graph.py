"""GPU: a decode step captured into a HIP graph replays bit for bit like the eager step.

Each replay follows eager work of the program's own (a cold step that rewrites
every selection and cache row) and a synchronization, and every replay is
checked against the eager steady step: a graph that kept stale state, or a
library call that recorded a memset, would show up on the replays after the first.
"""
import numpy as np
import pytest

from tests.gpu_common import log, small_problem, snapshot
from oracle.margins import enforce_margins

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,kw", [
    # fp32, every head persistent: one stream, the single-block reuse test + lists
    ("graph_f32_persistent", dict(batch=1, hq=32, hkv=8, context=4096, topk=410, dtype="f32", persistent=[1] * 8)),
    # bf16 with offloaded heads, 8 units: the step in order on one stream, gather included
    ("graph_bf16_mixed", dict(batch=2, hq=8, hkv=4, context=3000, topk=300, dtype="bf16", persistent=[1, 0, 0, 1])),
    # 20 units, which run overlapped on helper streams when launched eagerly: under
    # capture the step runs in order (the eager reference is the overlapped step)
    ("graph_bf16_overlapped", dict(batch=5, hq=8, hkv=4, context=3000, topk=300, dtype="bf16",
                                   persistent=[1, 0, 0, 1])),
])
def test_graph_replays_equal_eager_step(need_gpu, name, kw):
    import torch

    from top_sparse_attention_02_amd import workload

    p = small_problem(name, **kw)
    enforce_margins(p, 0)
    bufs = workload.load_layer(p, 0)
    bufs.step0()
    bufs.step1()
    eager = snapshot(bufs)
    bufs.step0()
    log(f"[case {name}] capture")
    g = workload.capture_step(bufs.step1)
    for rep in range(4):
        bufs.step0()  # eager work between replays: every unit misses and rewrites its rows
        torch.cuda.synchronize()
        g.replay()
        got = snapshot(bufs)
        for key in eager:
            assert np.array_equal(eager[key], got[key]), (rep, key)
    log(f"[case {name}] 4 replays equal the eager step")

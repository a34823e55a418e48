"""Decode steps of every overlapped schedule, run with error words, for
tests/test_gpu_shared_queue.py.  The test runs them in its own process and, as
`python -m tests.shared_queue_steps OUT.npz`, in child processes: one whose
streams all share one hardware queue (GPU_MAX_HW_QUEUES=1 in its environment),
where kernels start in the order they were enqueued, so a kernel that polls a
flag finishes only if it was enqueued after the kernels that raise it; and one
with CLO_STEP_IN_ORDER=1, where clo_decode_step runs every kernel in order on
the caller's stream."""
from __future__ import annotations

import math
import os
import sys
import time

import numpy as np

import gen
from tests.gpu_common import small_problem, snapshot


def layer_problem(name: str, batch: int) -> gen.Problem:
    # 4 KV heads, one persistent: batch 64 gives 256 units (one resident gather
    # launch), batch 5 gives 20 (a gather launch per unit range)
    return small_problem(name, batch=batch, hq=16, hkv=4, context=1500, topk=150, dtype="bf16",
                         persistent=[0, 1, 0, 0])


def loop_problem() -> gen.Problem:
    return gen.Problem(name="shared_queue_loop", layers=4, data_layers=4, batch=2, hq=10, hkv=2, d=128,
                       context=3000, topk=300, dtype="bf16", tau=0.8, seed=0x5EED0500, qprev_model="target_cos",
                       low_frac=0.5, heavy_frac=0.005,
                       persistent=np.array([[1, 0], [0, 0], [0, 1], [0, 0]], dtype=bool))


LAYER_CASES = (("resident", 64), ("ranges", 5))


def run_steps(log=print) -> dict:
    """A cold and a steady step of each single-layer case and of a 4-layer loop
    (batched selection, resident gather, batched attention).  Returns
    {case: {output: array, "err": error word, "seconds": wall time, "mode": the
    schedule clo_decode_step_schedule reports (single-layer cases)}}."""
    import torch

    from top_sparse_attention_02_amd import clo, workload

    res = {}
    for name, batch in LAYER_CASES:
        b = workload.load_layer(layer_problem(f"shared_queue_{name}", batch), 0)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for cold in (True, False):
            b.decode_step(b.q_prev if cold else b.q, b.q_prev, math.inf if cold else b.tau,
                          sync=clo.Sync(error_word=err))
        torch.cuda.synchronize()
        res[name] = dict(snapshot(b), err=int(err.item()), seconds=time.perf_counter() - t0,
                         mode=clo.clo_decode_step_schedule(b.shape, b.mask)["mode"])
        log(f"  {name}: {res[name]['mode']}, error word {res[name]['err']}, {res[name]['seconds']:.3f} s")
    layers = workload.load_layers(loop_problem())
    loop = workload.LayerLoop(layers, gather="resident", select="batched", select_batches=(1, 3),
                              attend="batched", attend_batches=(2, 2))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    loop.step(cold=True)
    loop.step()
    torch.cuda.synchronize()
    case = {"err": int(loop.error.item()), "seconds": time.perf_counter() - t0}
    for l, b in enumerate(layers):
        case.update({f"{l}_{k}": v for k, v in snapshot(b).items()})
    res["loop"] = case
    log(f"  loop: error word {case['err']}, {case['seconds']:.3f} s")
    return res


def main(path: str):
    env = {k: os.environ[k] for k in ("GPU_MAX_HW_QUEUES", "CLO_STEP_IN_ORDER") if k in os.environ}
    print(f"steps with {env}", flush=True)
    res = run_steps(log=lambda m: print(m, flush=True))
    np.savez(path, **{f"{c}__{k}": np.asarray(v) for c, d in res.items() for k, v in d.items()})


if __name__ == "__main__":
    main(sys.argv[1])

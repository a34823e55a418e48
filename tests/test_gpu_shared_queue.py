"""GPU: the decode schedules complete when their streams share one hardware
queue, and CLO_STEP_IN_ORDER=1 runs the step in order with the same results.

HIP maps the streams of a process beyond GPU_MAX_HW_QUEUES onto shared hardware
queues, which start kernels in the order they were enqueued.  The overlapped
step and the layer loop hand work between streams with flags that consumer
kernels poll, so each consumer must be enqueued after its producers; one
enqueued ahead of them on a shared queue would wait out its bound (CLO_E_TIMEOUT)
and then read stale selections.  A child process with GPU_MAX_HW_QUEUES=1 runs
the resident-gather step, the range-gather step and a 4-layer loop: no wait may
time out, and every output must equal the same steps run in this process.  A
child with CLO_STEP_IN_ORDER=1 (the switch for tools that run one kernel at a
time) must report and run the single-layer steps in order, with the same
outputs.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

from tests.gpu_common import log
from tests.shared_queue_steps import LAYER_CASES, layer_problem, run_steps

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OVERLAPPED = {"resident": "one resident gather launch", "ranges": "a gather launch per unit range"}


@pytest.fixture(scope="module")
def same_steps_here(need_gpu):
    """The steps run in this process, on separate hardware queues."""
    log("[case shared queue] the steps in this process")
    return run_steps(log=log)


@pytest.mark.parametrize("env,modes", [
    ({"GPU_MAX_HW_QUEUES": "1"}, OVERLAPPED),
    ({"CLO_STEP_IN_ORDER": "1"}, {name: "in order" for name, _ in LAYER_CASES}),
], ids=["one_hardware_queue", "step_in_order"])
def test_steps_in_a_child_process_equal_the_steps_here(need_gpu, tmp_path, same_steps_here, env, modes):
    from top_sparse_attention_02_amd import clo

    for name, batch in LAYER_CASES:
        p = layer_problem(f"shared_queue_{name}", batch)
        shape = clo.Shape(batch=p.batch, n_q_heads=p.hq, n_kv_heads=p.hkv, context=p.context, topk=p.topk,
                          tau=p.tau, dtype=clo.CLO_BF16)
        assert clo.clo_decode_step_schedule(shape, persistent_mask=p.persistent_mask_bits(0))["mode"] == OVERLAPPED[name]
    out = tmp_path / "steps.npz"
    log(f"[case {env}] child process: resident-gather step (256 units), range-gather step (20 units), "
        "4-layer loop")
    r = subprocess.run([sys.executable, "-u", "-m", "tests.shared_queue_steps", str(out)], cwd=ROOT,
                       env=dict(os.environ, **env), capture_output=True, text=True, timeout=100)
    log(r.stdout.strip())
    assert r.returncode == 0, r.stderr[-3000:]
    got = dict(np.load(out))
    for case, outputs in same_steps_here.items():
        assert int(got[f"{case}__err"]) == 0, (case, clo.clo_status_string(int(got[f"{case}__err"])))
        assert outputs["err"] == 0, case
        if case in modes:
            assert str(got[f"{case}__mode"]) == modes[case], case
        for key, value in outputs.items():
            if key in ("err", "seconds", "mode"):
                continue
            assert np.array_equal(got[f"{case}__{key}"], np.asarray(value)), (case, key)

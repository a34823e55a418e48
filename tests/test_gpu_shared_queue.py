"""GPU: the overlapped decode schedules complete when their streams share one
hardware queue.

HIP maps the streams of a process beyond GPU_MAX_HW_QUEUES onto shared hardware
queues, which start kernels in the order they were enqueued.  The overlapped
step and the layer loop hand work between streams with flags that consumer
kernels poll, so each consumer must be enqueued after its producers; one
enqueued ahead of them on a shared queue would wait out its bound (CLO_E_TIMEOUT)
and then read stale selections.  A child process with GPU_MAX_HW_QUEUES=1 runs
the resident-gather step, the range-gather step and a 4-layer loop: no wait may
time out, and every output must equal the same steps run in this process.
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


def test_overlapped_steps_complete_on_one_hardware_queue(need_gpu, tmp_path):
    from top_sparse_attention_02_amd import clo

    modes = {}
    for name, batch in LAYER_CASES:
        p = layer_problem(f"shared_queue_{name}", batch)
        shape = clo.Shape(batch=p.batch, n_q_heads=p.hq, n_kv_heads=p.hkv, context=p.context, topk=p.topk,
                          tau=p.tau, dtype=clo.CLO_BF16)
        modes[name] = clo.clo_decode_step_schedule(shape, persistent_mask=p.persistent_mask_bits(0))["mode"]
    assert modes == {"resident": "one resident gather launch", "ranges": "a gather launch per unit range"}
    out = tmp_path / "steps.npz"
    log("[case one hardware queue] child process: resident-gather step (256 units), range-gather step "
        "(20 units), 4-layer loop")
    r = subprocess.run([sys.executable, "-u", "-m", "tests.shared_queue_steps", str(out)], cwd=ROOT,
                       env=dict(os.environ, GPU_MAX_HW_QUEUES="1"), capture_output=True, text=True, timeout=100)
    log(r.stdout.strip())
    assert r.returncode == 0, r.stderr[-3000:]
    got = dict(np.load(out))
    log("[case one hardware queue] the same steps in this process")
    ref = run_steps(log=log)
    for case, outputs in ref.items():
        assert int(got[f"{case}__err"]) == 0, (case, clo.clo_status_string(int(got[f"{case}__err"])))
        assert outputs["err"] == 0, case
        for key, value in outputs.items():
            if key in ("err", "seconds"):
                continue
            assert np.array_equal(got[f"{case}__{key}"], np.asarray(value)), (case, key)

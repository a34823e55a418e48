"""GPU: the multi-layer selection (clo_select_plan + clo_select_layers).

Batches of layers take the reuse test, scoring and top-k in three launches;
their reuse flags, cosines and selections must equal clo_reuse_select run on
each layer alone, bit for bit, for both top-k kernels (contexts of fewer than 8
chunks of 16384 keys and of more), for cold and steady steps, and for layers of
persistent, offloaded and mixed heads.  A wait that is never satisfied must end
at its bound with CLO_E_TIMEOUT and every layer still signalled; a launch shaped
for another context, or reaching past the plan's layers, must report CLO_E_ARG
and end.
"""
import math

import numpy as np
import pytest

import gen
from tests.gpu_common import log

pytestmark = pytest.mark.gpu

PERSISTENT = np.array([[1, 0], [0, 0], [1, 1], [0, 1], [0, 0]], dtype=bool)


def _problem(context):
    topk = math.ceil(context / 10)
    return gen.Problem(name=f"sel_layers_{context}", layers=5, batch=2, hq=8, hkv=2, d=128, context=context,
                       topk=topk, dtype="bf16", tau=0.8, seed=0x5EED0300 + context % 997, qprev_model="target_cos",
                       low_frac=0.5, heavy_frac=0.005, persistent=PERSISTENT)


def _state(layers):
    import torch

    torch.cuda.synchronize()
    return [(b.reuse.cpu().numpy().copy(), b.cos.cpu().numpy().copy(), b.idx.cpu().numpy().copy()) for b in layers]


def _per_layer(clo, layers, cold):
    for b in layers:
        shape = b.shape_with(math.inf if cold else b.tau)
        clo.clo_reuse_select(shape, b.layer(), b.q_prev if cold else b.q, b.q_prev, b.reuse, b.cos, b.ws)


def _plan(clo, layers, cold, flags, room=0):
    import torch

    plan = torch.zeros(clo.clo_select_plan_size(len(layers) + room), dtype=torch.uint8, device="cuda")
    items = [(b.shape_with(math.inf if cold else b.tau), b.layer(), b.q_prev if cold else b.q, b.q_prev, b.reuse,
              b.cos, b.ws, flags[0, l], flags[1, l]) for l, b in enumerate(layers)]
    clo.clo_select_plan(items, plan)
    return plan


def _reset(layers):
    for b in layers:
        b.reuse.fill_(7)
        b.cos.fill_(-2.0)
        b.idx.fill_(-1)


@pytest.mark.parametrize("context", [3000, 131073])
def test_select_layers_equal_per_layer_calls(need_gpu, context):
    import torch

    from top_sparse_attention_02_amd import clo, workload

    p = _problem(context)
    log(f"[case select layers N={context}] 5 layers, batches (2, 3) and (5)")
    layers = workload.load_layers(p)
    # per layer: cold step, then steady step
    _per_layer(clo, layers, True)
    cold_ref = _state(layers)
    _per_layer(clo, layers, False)
    steady_ref = _state(layers)
    for batches in ((2, 3), (5,)):
        flags = torch.zeros(2, len(layers), dtype=torch.int32, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        _reset(layers)
        for cold, ref, value in ((True, cold_ref, 1), (False, steady_ref, 2)):
            plan = _plan(clo, layers, cold, flags)
            first = 0
            for n in batches:
                clo.clo_select_layers(layers[0].shape, plan, first, n, 0, value, error_word=err)
                first += n
            got = _state(layers)
            assert int(err.item()) == 0
            assert flags[1].tolist() == [value] * len(layers)
            for l, (a, b) in enumerate(zip(got, ref)):
                for name, x, y in zip(("reuse", "cos", "idx"), a, b):
                    assert np.array_equal(x, y), (batches, "cold" if cold else "steady", l, name)
        hits = sum(int(r.sum()) for r, _, _ in steady_ref)
        log(f"[case select layers N={context}] batches {batches}: equal ({hits} of 20 units reuse at the steady step)")


def test_select_layers_wait_times_out_and_signals(need_gpu):
    import torch

    from top_sparse_attention_02_amd import clo, workload

    p = _problem(3000)
    layers = workload.load_layers(p)
    flags = torch.zeros(2, len(layers), dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    plan = _plan(clo, layers, True, flags)
    # wait flags stay 0: every layer's wait for 1 ends at its bound
    clo.clo_select_layers(layers[0].shape, plan, 0, len(layers), 1, 3, error_word=err, spin_limit=2000)
    torch.cuda.synchronize()
    assert int(err.item()) == clo.CLO_E_TIMEOUT
    assert flags[1].tolist() == [3] * len(layers)
    assert all(int(b.reuse.sum()) == 0 for b in layers)  # cold plan: every unit selected


def test_select_layers_report_a_launch_shaped_for_another_context(need_gpu):
    import torch

    from top_sparse_attention_02_amd import clo, workload

    p = _problem(131073)
    layers = workload.load_layers(p)
    flags = torch.zeros(2, len(layers), dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    plan = _plan(clo, layers, True, flags)
    other = clo.Shape(**layers[0].shape.__dict__)
    other.context = 2 * 131073  # 17 chunks of keys per unit instead of 9
    other.topk = math.ceil(other.context / 10)
    clo.clo_select_layers(other, plan, 0, len(layers), 0, 1, error_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) == clo.CLO_E_ARG
    assert flags[1].tolist() == [1] * len(layers)


def test_select_layers_refuse_layers_past_the_plan(need_gpu):
    import torch

    from top_sparse_attention_02_amd import clo, workload

    p = _problem(3000)
    layers = workload.load_layers(p)
    flags = torch.zeros(2, len(layers), dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    plan = _plan(clo, layers, True, flags, room=3)  # room for 8 layers, 5 written
    clo.clo_select_layers(layers[0].shape, plan, 3, 4, 0, 1, error_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) == clo.CLO_E_ARG
    assert flags[1].tolist() == [0] * len(layers)
    # the plan still works for the layers it holds
    err.zero_()
    clo.clo_select_layers(layers[0].shape, plan, 0, 5, 0, 2, error_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0 and flags[1].tolist() == [2] * len(layers)

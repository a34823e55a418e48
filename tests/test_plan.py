"""clo_plan_persistent (host-only, no GPU) against the oracle's plan_persistent."""
import math

import numpy as np
import pytest

import oracle
from top_sparse_attention_02_amd import clo


@pytest.mark.parametrize("seed", range(20))
def test_plan_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    L, H = int(rng.integers(1, 50)), int(rng.integers(1, 9))
    # coarse values: many ties, exactly representable in float32
    s = (rng.integers(0, 16, size=(L, H)) / 16).astype(np.float32)
    n = int(rng.integers(0, L * H + 1))
    assert clo.clo_plan_persistent(s, n) == oracle.plan_persistent(s, n)


def test_plan_config_sized():
    # 48 layers x 8 KV heads, 183 persistent slots (47.6%)
    rng = np.random.default_rng(3)
    s = rng.uniform(0.2, 1.0, size=(48, 8)).astype(np.float32)
    masks = clo.clo_plan_persistent(s, 183)
    assert masks == oracle.plan_persistent(s, 183)
    assert sum(bin(m).count("1") for m in masks) == 183


@pytest.mark.parametrize("n", [-1, 17])
def test_plan_rejects_bad_counts(n):
    with pytest.raises(clo.CloError) as e:
        clo.clo_plan_persistent(np.zeros((2, 8), np.float32), n)
    assert e.value.status == clo.CLO_E_ARG


def test_plan_rejects_nan():
    s = np.zeros((2, 4), np.float32)
    s[1, 2] = math.nan
    with pytest.raises(clo.CloError) as e:
        clo.clo_plan_persistent(s, 3)
    assert e.value.status == clo.CLO_E_ARG and "NaN" in str(e.value)


def test_default_selection_batches_cover_the_layers():
    from top_sparse_attention_02_amd.workload import default_select_batches

    assert default_select_batches(8, 48) == (3, 3, 6, 12, 24)   # B=1, 8 KV heads
    assert default_select_batches(64, 48)[:6] == (1, 1, 2, 4, 8, 16)
    for units in (1, 4, 8, 16, 64, 512):
        for n in (1, 6, 48, 200):
            sizes = default_select_batches(units, n)
            assert sum(sizes) >= n and all(1 <= x <= 64 for x in sizes)


def test_default_attend_batches_cover_the_layers():
    """The loop's attention batches: 8 layers each, the last layers 4, 2, 1 and 1;
    every size within 1..64 (the multi-layer attention's limit) and, once cut to
    the layer count, covering every layer exactly once."""
    from top_sparse_attention_02_amd.workload import _cover, default_attend_batches

    assert default_attend_batches(48) == (8, 8, 8, 8, 8, 4, 2, 1, 1)
    for n in (1, 2, 3, 6, 8, 9, 48, 200):
        sizes = _cover(default_attend_batches(n), n)
        assert sum(sizes) == n and all(1 <= x <= 64 for x in sizes), (n, sizes)

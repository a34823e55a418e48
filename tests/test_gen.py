"""The seeded input generator: reproducibility, published generator values, data-model statistics."""
import math

import numpy as np

import gen


def test_splitmix64_reference_values():
    # SplitMix64 seeded with 0 (Steele et al. 2014; Vigna's reference splitmix64.c):
    # the first three outputs of the stream
    assert [int(x) for x in gen.u64_stream(0, 3)] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_based_slices_and_threads():
    key = gen.derive_key(123, 4, 5)
    full = gen.normal_stream(key, 1001)
    assert np.array_equal(gen.normal_stream(key, 500, first=501), full[501:])
    p = gen.Problem(name="t", layers=1, batch=1, hq=4, hkv=2, d=128, context=3000, topk=300,
                    dtype="bf16", tau=0.8, seed=9, qprev_model="independent", heavy_frac=0.01)
    a = np.empty((3000, 128), np.uint16)
    b = np.empty((3000, 128), np.uint16)
    p.fill("k", 0, 0, 1, a.ctypes.data, threads=1)
    p.fill("k", 0, 0, 1, b.ctypes.data, threads=7)
    assert np.array_equal(a, b)


def test_normal_moments():
    z = gen.normal_stream(gen.derive_key(77), 2_000_000)
    assert abs(z.mean()) < 3e-3
    assert abs(z.var() - 1) < 5e-3
    assert abs(np.mean(z ** 4) - 3) < 3e-2


def test_bf16_rounding_is_nearest_even():
    v = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.0, 3.140625, 1 + 2 ** -9])
    assert gen.round_to(v, "bf16").tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC000, 0x4049, 0x3F80]


def test_config_data_models():
    c1, c2, c3, c4, c5 = (gen.config(i) for i in range(1, 6))
    assert [c.topk for c in (c1, c2, c3, c4, c5)] == [410, 3277, 13108, 26215, 52429]
    assert c1.persistent.all() and not c3.persistent.any()
    assert c2.persistent.sum() == 2 and (c2.persistent == c2.persistent[0]).all()
    assert c4.persistent.sum() == 183 and c5.persistent.sum() == 183
    assert len(c2.heavy_rows(0, 3)) == math.ceil(0.01 * 32768)
    assert len(c4.heavy_rows(0, 0)) == math.ceil(0.005 * 262144)
    # config 3: exactly 20% of units low, targets inside their windows
    t = np.array([c3.cos_target(0, b, h) for b in range(64) for h in range(8)])
    low = t < 0.7
    assert low.sum() == round(0.2 * 512)
    assert t[low].min() >= 0.2 and t[low].max() <= 0.6
    assert t[~low].min() >= 0.801 and t[~low].max() <= 0.98
    # config 1: previous-step query heads are unit vectors
    qp = gen.stored_to_f64(c1.q_prev(0), "f32")
    assert np.allclose(np.linalg.norm(qp, axis=-1), 1.0, atol=1e-6)


def test_resample_changes_only_listed_rows():
    p = gen.config(2, batch=1, context=2048, topk=205)
    before = p.kv("k", 0, 0, 0)
    p.resample_k_rows(0, 0, 0, [5, 700])
    after = p.kv("k", 0, 0, 0)
    diff = np.nonzero((before != after).any(axis=1))[0].tolist()
    assert diff == [5, 700]


def test_rows_draw_matches_single_row_draws():
    # the vectorized redraw used by the margins gives the same stored values as
    # drawing each row on its own, heavy-hitter scale included
    p = gen.config(2, batch=1, context=4096, topk=410)
    rows = np.array([0, 5, 4095, 77, 5], dtype=np.int64)
    rnds = np.array([1, 1, 3, 7, 2], dtype=np.int64)
    got = p.k_rows_draw(0, 0, 3, rows, rnds)
    want = np.stack([p.k_row_draw(0, 0, 3, int(r), int(n)) for r, n in zip(rows, rnds)])
    assert np.array_equal(got, want)
    # and a row set to a round through the resample record comes out of fill so
    p.set_k_row_round(0, 0, 3, 77, 7)
    assert np.array_equal(p.kv("k", 0, 0, 3)[77], want[3])

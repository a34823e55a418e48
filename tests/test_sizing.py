"""Sizing checks against the figures the pages print, and the benchmark's byte accounting.

* KV-cache offloading article ("KV Cache Offloading 完全拆解"), section on how large
  the KV cache is: bytes per token per layer = 2 * n_kv * d_head * b; a 70B-class GQA
  model (n_kv = 8, d_head = 128, fp16, 80 layers) holds about 320 KB per token, and one
  128K-token request about 39 GB (binary units).
* CLO synthesis page, section 3.4 (attack point 7): Qwen2.5-14B at 512K holds 93.75 GB
  of KV cache -- exact for 512,000 tokens counted in GiB with the decode-layer shape the
  Qwen2.5-14B workloads here use (48 layers, 8 KV heads, d = 128, bf16).
* CLO synthesis section 2.2 (only the top-10% rows move): the host bytes of a step are
  k / N of the KV of the miss units of offloaded heads; bench.py's accounting must give
  exactly that, and the algorithmic bytes DESIGN quotes for the B=64, N=131072 step.
"""
import math
from types import SimpleNamespace

import numpy as np
import pytest

import gen

GIB = 1 << 30


def kv_bytes_per_token_layer(n_kv: int, d_head: int, b: int) -> int:
    return 2 * n_kv * d_head * b


def test_seventy_b_example():
    per_token = kv_bytes_per_token_layer(8, 128, 2) * 80
    assert per_token == 327_680                       # "≈ 320 KB/token"
    assert per_token / 1024 == 320.0
    request = 128_000 * per_token
    assert round(request / GIB) == 39                 # "128000 × 320 KB ≈ 39 GB"


def test_qwen_512k_footprint_matches_the_motivating_example():
    p = gen.config(5)
    assert (p.layers, p.hkv, p.d, p.dtype) == (48, 8, 128, "bf16")
    per_token = kv_bytes_per_token_layer(p.hkv, p.d, 2) * p.layers
    assert 512_000 * per_token / GIB == 93.75         # exact
    # the workload's own context (2^19 tokens) is 96 GiB = 103.1 GB
    assert p.context * per_token == 96 * GIB


class _Layer(SimpleNamespace):
    def is_persistent(self, h):
        return bool((self.mask >> h) & 1)


def _layer(B, Hq, Hkv, N, k, dtype, mask, reuse, host_format=0):
    import torch

    return _Layer(B=B, Hq=Hq, Hkv=Hkv, N=N, k=k, dtype=dtype, mask=mask, host_format=host_format,
                  reuse=torch.from_numpy(reuse.astype(np.uint8)))


def test_host_bytes_are_top_k_fraction_of_miss_units_kv():
    import bench

    rng = np.random.default_rng(7)
    for B, Hq, Hkv, N, dtype, mask in [(4, 32, 8, 40960, "bf16", 0b00000110), (2, 10, 2, 5000, "f32", 0b01)]:
        k = math.ceil(N / 10)
        reuse = rng.random((B, Hkv)) < 0.6
        lay = _layer(B, Hq, Hkv, N, k, dtype, mask, reuse)
        tot = bench.algorithmic_bytes([lay])
        b = 4 if dtype == "f32" else 2
        offl = np.array([not ((mask >> h) & 1) for h in range(Hkv)])
        miss_offl = int((~reuse & offl[None, :]).sum())
        unit_kv = N * kv_bytes_per_token_layer(1, 128, b)  # one (sequence, KV head)
        assert tot["misses_host"] == miss_offl
        assert tot["host_bytes"] * N == miss_offl * unit_kv * k   # host bytes = k/N of their KV
        # int8 host rows: half the bytes of bf16
        tot8 = bench.algorithmic_bytes([_layer(B, Hq, Hkv, N, k, dtype, mask, reuse, host_format=1)])
        assert tot8["host_bytes"] * b == tot["host_bytes"]


def test_algorithmic_bytes_of_the_b64_n131072_step():
    import bench

    B, Hkv, N, k = 64, 8, 131072, 13108
    reuse = np.ones((B, Hkv), dtype=bool)
    reuse.flat[np.random.default_rng(3).choice(B * Hkv, size=102, replace=False)] = False
    tot = bench.algorithmic_bytes([_layer(B, 32, Hkv, N, k, "bf16", 0, reuse)])
    assert tot["host_bytes"] == 684_552_192          # 102 x 13108 rows x 512 B
    assert tot["score_bytes"] == 3_422_552_064       # 102 x 131072 keys x 256 B
    assert tot["misses"] == 102 and tot["hits"] == 410

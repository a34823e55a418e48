"""Quantized host KV (CLO_HOST_INT8, CLO_HOST_INT4) on the GPU against the oracle.

Rows quantize to 8- or 4-bit values with one power-of-two scale per row; the
gather dequantizes them exactly into the HBM cache.  Quantized values (4-bit:
the packed bytes) and exponents, selections and cache rows must equal the
oracle's bit for bit; outputs (the oracle attending the dequantized rows of
offloaded heads) within the usual tolerances."""
import math

import numpy as np
import pytest

import oracle
from tests.gpu_common import compare, log, small_problem, snapshot, to_numpy
from oracle.margins import enforce_margins, enforce_walk_margins

pytestmark = pytest.mark.gpu


FORMATS = {8: 1, 4: 2}  # bits -> clo host format (CLO_HOST_INT8, CLO_HOST_INT4)


def _rows(rng, n, dtype, bits):
    M = oracle.quant_max(bits)
    x = rng.standard_normal((n, 128)) * 2.0 ** rng.integers(-30, 30, size=(n, 1)).astype(np.float64)
    x[0] = 0.0                                     # zero row
    x[1] = rng.standard_normal(128) * 2.0 ** -125  # below the smallest exponent
    x[2, :] = 0.0
    x[2, 5] = M * 2.0 ** -6                        # exactly at an exponent boundary
    x[3, :] = 0.0
    x[3, 7] = -M * 2.0 ** -6                       # a negative one
    x[3, 8] = 2.0 ** -7                            # a tie: 1/2 -> 0
    if dtype == "f32":
        return x.astype(np.float32)
    b = x.astype(np.float32).view(np.uint32)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)  # bf16 patterns, RNE


def _want_bytes(q, bits):
    """The oracle's values as the format's bytes."""
    if bits == 8:
        return np.asarray(q, dtype=np.int64).astype(np.int8).view(np.uint8)
    return np.frombuffer(oracle.pack_int4(q), dtype=np.uint8)


@pytest.mark.parametrize("where", ["host", "device", "host_records"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("bits", [8, 4])
def test_quantize_rows_match_oracle(need_gpu, bits, dtype, where):
    import torch

    from top_sparse_attention_02_amd import clo, workload
    from top_sparse_attention_02_amd.hip_host import HostBuffer

    fmt, rb = FORMATS[bits], 128 * bits // 8  # row bytes
    rng = np.random.default_rng(21 + bits)
    n = 1000
    x = _rows(rng, n, dtype, bits)
    src = workload.host_rows_tensor(x, dtype)
    exp = torch.zeros(n, dtype=torch.int8, device="cuda")
    if where == "host":
        host = HostBuffer(n * rb)
        clo.clo_quantize_rows(src, n, workload.clo_dtype(dtype), host.ptr, exp, dst_stride=rb, host_format=fmt)
        torch.cuda.synchronize()
        q = host.numpy(np.uint8, (n, rb)).copy()
    elif where == "host_records":
        # the V half of records: rows 2 * rb bytes apart, K halves untouched
        host = HostBuffer(n * 2 * rb)
        host.numpy(np.uint8, (n * 2 * rb,))[:] = 99
        clo.clo_quantize_rows(src, n, workload.clo_dtype(dtype), host.ptr + rb, exp, dst_stride=2 * rb,
                              host_format=fmt)
        torch.cuda.synchronize()
        rec = host.numpy(np.uint8, (n, 2, rb))
        assert np.all(rec[:, 0] == 99)
        q = rec[:, 1].copy()
    else:
        dst = torch.zeros(n, rb, dtype=torch.uint8, device="cuda")
        clo.clo_quantize_rows(src, n, workload.clo_dtype(dtype), dst, exp, dst_stride=rb, host_format=fmt)
        q = dst.cpu().numpy()
    e = exp.cpu().numpy()
    xf = oracle.as_f64(x, dtype)
    for i in range(n):
        rq, re = oracle.quantize_row(xf[i], bits)
        assert e[i] == re and np.array_equal(q[i], _want_bytes(rq, bits)), f"row {i}"


def _quant_problem(name, **kw):
    return small_problem(name, **kw)


CASES = {
    "bf16_g4_mixed": dict(batch=2, hq=8, hkv=2, context=3000, topk=300, dtype="bf16", persistent=[1, 0],
                          heavy_frac=0.005),
    "f32_g5_host": dict(batch=2, hq=10, hkv=2, context=2500, topk=250, dtype="f32", persistent=[0, 0]),
    # 24 units: overlapped, a gather launch per range; 256 units: one resident gather launch
    "bf16_g4_overlapped": dict(batch=6, hq=16, hkv=4, context=2000, topk=200, dtype="bf16", persistent=[0, 1, 0, 0]),
    "bf16_g4_resident": dict(batch=64, hq=16, hkv=4, context=1200, topk=120, dtype="bf16", persistent=[0, 0, 1, 0]),
}


def _cache_of(p, kvs, bits):
    memo = {}

    def f(b, h):
        if (b, h) not in memo:
            K, V = kvs(b, h)
            memo[(b, h)] = (oracle.quantized_rows(oracle.as_f64(K, p.dtype), bits),
                            oracle.quantized_rows(oracle.as_f64(V, p.dtype), bits))
        return memo[(b, h)]
    return f


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("bits", [8, 4])
def test_quantized_host_decode_matches_oracle(need_gpu, bits, name):
    from top_sparse_attention_02_amd import workload

    p = _quant_problem(f"int{bits}_" + name, **CASES[name])
    enforce_margins(p, 0)
    log(f"[case int{bits} {name}] B={p.batch} Hq={p.hq} Hkv={p.hkv} N={p.context} k={p.topk} {p.dtype}")
    bufs = workload.load_layer(p, 0, host_format=FORMATS[bits])
    bufs.step0()
    got0 = snapshot(bufs)
    bufs.step1()
    got1 = snapshot(bufs)
    memo = {}

    def kv(b, h):
        if (b, h) not in memo:
            memo[(b, h)] = (p.kv("k", 0, b, h), p.kv("v", 0, b, h))
        return memo[(b, h)]

    cache_of = _cache_of(p, kv, bits)
    attn = lambda b, h: None if bufs.is_persistent(h) else cache_of(b, h)  # noqa: E731
    qp, q = p.q_prev(0), p.q(0)
    r0 = oracle.decode_layer(qp, qp, kv, p.hkv, p.topk, math.inf, p.dtype, attn_kv_of=attn)
    idx0 = np.zeros((p.batch, p.hkv, p.topk), dtype=np.int64)
    for (b, h), r in r0.items():
        idx0[b, h] = r["idx"]
    r1 = oracle.decode_layer(q, qp, kv, p.hkv, p.topk, p.tau, p.dtype, idx_prev=idx0, attn_kv_of=attn)
    compare(p, bufs, got0, r0, kv, "step0", cache_of=cache_of)
    compare(p, bufs, got1, r1, kv, "step1", cache_of=cache_of)


@pytest.mark.parametrize("bits", [8, 4])
def test_quantized_growing_context(need_gpu, bits):
    from top_sparse_attention_02_amd import workload

    steps = 5
    p = _quant_problem(f"int{bits}_growing", batch=2, hq=8, hkv=2, context=3000 + steps, topk=300, dtype="bf16",
                       persistent=[0, 1], low_frac=0.2)
    enforce_walk_margins(p, 0, steps)
    log(f"[case int{bits} growing] N={p.context - steps}+{steps}")
    run = workload.GrowingRun(p, 0, steps, "refresh", host_format=FORMATS[bits])
    g, n0 = p.g, p.context - steps
    kvs = {(b, h): (p.kv("k", 0, b, h), p.kv("v", 0, b, h)) for b in range(p.batch) for h in range(p.hkv)}
    kv = lambda b, h: kvs[(b, h)]  # noqa: E731
    cache_of = _cache_of(p, kv, bits)
    qs = [oracle.as_f64(p.q_walk(0, t), p.dtype) for t in range(steps + 1)]
    ref = {}
    for (b, h), (K, V) in kvs.items():
        Ka, Va = cache_of(b, h) if not run.bufs.is_persistent(h) else (oracle.as_f64(K, p.dtype),
                                                                      oracle.as_f64(V, p.dtype))
        sl = slice(h * g, (h + 1) * g)
        # scoring reads the exact keys, attention the (dequantized) rows of the host copy
        res, r_ref, sel = [], None, None
        for t in range(steps + 1):
            n = n0 + t
            Kf, Vf = oracle.as_f64(K, p.dtype)[:n], oracle.as_f64(V, p.dtype)[:n]
            if t == 0:
                r = oracle.decode_unit(qs[0][b, sl], qs[0][b, sl], Kf, Vf, p.topk, math.inf, None, Ka[:n], Va[:n])
            else:
                r = oracle.decode_unit(qs[t][b, sl], r_ref, Kf, Vf, p.topk, p.tau, sel, Ka[:n], Va[:n])
            sel = r["idx"]
            if not r["reuse"]:
                r_ref = qs[t][b, sl]
            res.append(r)
        ref[(b, h)] = res
    for t in range(steps + 1):
        run.step(t)
        got = snapshot(run.bufs)
        compare(p, run.bufs, got, {u: r[t] for u, r in ref.items()}, kv, f"step{t}", check_cos=t > 0,
                cache_of=cache_of)
    # the appended rows were quantized on the GPU into pinned memory, exponents into HBM
    b = run.bufs
    for (bb, h), (K, V) in kvs.items():
        if b.is_persistent(h):
            continue
        s = b.slot(h)
        for which, X, exps in (("k", K, b.k_exp), ("v", V, b.v_exp)):
            hv = b.host_view(which, bb, h)
            ex = exps[bb, s].cpu().numpy()
            for row in range(n0, p.context):
                rq, re = oracle.quantize_row(oracle.as_f64(X[row], p.dtype), bits)
                got = hv[row].view(np.uint8)
                assert ex[row] == re and np.array_equal(got, _want_bytes(rq, bits)), (which, bb, h, row)

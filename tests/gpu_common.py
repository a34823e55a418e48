"""Shared helpers of the GPU parity tests: run the two-step protocol on the GPU
through the C ABI and compare every observable output with the CPU oracle."""
from __future__ import annotations

import math
import zlib
import sys

import numpy as np

import gen
import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2}


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def small_problem(name, **kw) -> gen.Problem:
    base = dict(name=name, layers=1, d=128, tau=0.8, seed=zlib.crc32(name.encode()), qprev_model="target_cos",
                low_frac=0.5)
    base.update(kw)
    if "persistent" in base:
        base["persistent"] = np.asarray(base["persistent"], dtype=bool).reshape(1, -1)
    return gen.Problem(**base)


def to_numpy(t, dtype):
    """Device tensor of stored values -> numpy array of the stored representation."""
    import torch

    t = t.detach().cpu()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def snapshot(bufs):
    """Read every observable output of the last step back to the host."""
    import torch

    torch.cuda.synchronize()
    s = {
        "reuse": bufs.reuse.cpu().numpy().astype(bool),
        "cos": bufs.cos.cpu().numpy().astype(np.float64),
        "idx": bufs.idx.cpu().numpy().astype(np.int64),
        "out": oracle.as_f64(to_numpy(bufs.out, bufs.dtype), bufs.dtype),
    }
    if bufs.H:
        s["k_cache"] = to_numpy(bufs.k_cache, bufs.dtype)
        s["v_cache"] = to_numpy(bufs.v_cache, bufs.dtype)
    return s


def oracle_steps(p: gen.Problem, layer: int, units=None):
    """Oracle results of step 0 (tau = inf, q_prev as query) and step 1 for the listed units."""
    q, qp = p.q(layer), p.q_prev(layer)
    cache = {}

    def kv(b, h):
        if (b, h) not in cache:
            cache[(b, h)] = (p.kv("k", layer, b, h), p.kv("v", layer, b, h))
        return cache[(b, h)]

    r0 = oracle.decode_layer(qp, qp, kv, p.hkv, p.topk, math.inf, p.dtype, units=units)
    idx0 = np.zeros((p.batch, p.hkv, p.topk), dtype=np.int64)
    for (b, h), r in r0.items():
        idx0[b, h] = r["idx"]
    r1 = oracle.decode_layer(q, qp, kv, p.hkv, p.topk, p.tau, p.dtype, idx_prev=idx0, units=units)
    return r0, r1, kv


def compare(p: gen.Problem, bufs, got, ref, kv, step: str, units=None, check_cos=None, cache_of=None):
    """Assert GPU outputs of one step equal the oracle's (decisions and indices bit-exact).

    cache_of(b, kvh): the float64 rows a miss unit's cache must hold (default: the
    stored K and V, bit for bit).  Returns the largest normwise output error and
    cosine difference met (the headroom under the tolerances)."""
    g = p.g
    check_cos = (step == "step1") if check_cos is None else check_cos
    tol = TOL[p.dtype]
    worst = {"out_err": 0.0, "cos_err": 0.0, "units": 0}
    for (b, h), r in ref.items():
        where = f"{step} unit (b={b}, kvh={h})"
        assert bool(got["reuse"][b, h]) == r["reuse"], f"{where}: reuse {got['reuse'][b, h]} vs {r['reuse']}"
        if check_cos:
            assert abs(got["cos"][b, h] - r["cos"]) <= 1e-5, f"{where}: cos {got['cos'][b, h]} vs {r['cos']}"
            worst["cos_err"] = max(worst["cos_err"], abs(got["cos"][b, h] - r["cos"]))
        gi = got["idx"][b, h]
        if not np.array_equal(gi, r["idx"]):
            missing = sorted(set(r["idx"].tolist()) - set(gi.tolist()))[:5]
            extra = sorted(set(gi.tolist()) - set(r["idx"].tolist()))[:5]
            raise AssertionError(f"{where}: idx differs (missing {missing}, extra {extra})")
        if not bufs.is_persistent(h) and not r["reuse"]:
            s = bufs.slot(h)
            if cache_of is not None:
                Kq, Vq = cache_of(b, h)
                assert np.array_equal(oracle.as_f64(got["k_cache"][b, s], p.dtype), Kq[r["idx"]]), \
                    f"{where}: K cache rows differ from the dequantized rows"
                assert np.array_equal(oracle.as_f64(got["v_cache"][b, s], p.dtype), Vq[r["idx"]]), \
                    f"{where}: V cache rows differ from the dequantized rows"
            else:
                K, V = kv(b, h)
                assert np.array_equal(got["k_cache"][b, s], K[r["idx"]]), f"{where}: K cache rows differ"
                assert np.array_equal(got["v_cache"][b, s], V[r["idx"]]), f"{where}: V cache rows differ"
        o = got["out"][b, h * g:(h + 1) * g]
        ro = r["out"]
        err = np.abs(o - ro).max(axis=1) / np.maximum(np.abs(ro).max(axis=1), 1e-30)
        assert err.max() <= tol, f"{where}: output error {err.max():.3e} > {tol}"
        worst["out_err"] = max(worst["out_err"], float(err.max()))
        worst["units"] += 1
    return worst


def merge_worst(results):
    """Largest errors over many compare() results."""
    out = {"out_err": 0.0, "cos_err": 0.0, "units": 0}
    for r in results:
        out["out_err"] = max(out["out_err"], r["out_err"])
        out["cos_err"] = max(out["cos_err"], r["cos_err"])
        out["units"] += r["units"]
    return out


def log_worst(case: str, step: str, worst, dtype: str):
    tol = TOL[dtype]
    log(f"[{case}] {step}: {worst['units']} units, max normwise output error {worst['out_err']:.3e} "
        f"(tolerance {tol:g}, headroom {tol / max(worst['out_err'], 1e-30):.1f}x), max cosine difference "
        f"{worst['cos_err']:.2e} (tolerance 1e-5)")


def run_and_check(p: gen.Problem, layer: int = 0, units=None, bufs=None):
    """Two-step protocol on the GPU vs the oracle; returns the GPU snapshots."""
    from top_sparse_attention_02_amd import workload

    log(f"[case {p.name}] B={p.batch} Hq={p.hq} Hkv={p.hkv} N={p.context} k={p.topk} {p.dtype} "
        f"mask={p.persistent_mask_bits(layer):#x}")
    bufs = workload.load_layer(p, layer, bufs)
    bufs.step0()
    got0 = snapshot(bufs)
    bufs.step1()
    got1 = snapshot(bufs)
    r0, r1, kv = oracle_steps(p, layer, units)
    log_worst(p.name, "step0", compare(p, bufs, got0, r0, kv, "step0"), p.dtype)
    log_worst(p.name, "step1", compare(p, bufs, got1, r1, kv, "step1"), p.dtype)
    # hit units keep step 0's selection and cache rows
    for (b, h), r in r1.items():
        if r["reuse"]:
            assert np.array_equal(got1["idx"][b, h], got0["idx"][b, h])
    return bufs, got0, got1

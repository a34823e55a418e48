"""Seeded synthetic inputs for the CLO decode step (test and benchmark infrastructure).

This module builds the inputs only: queries, previous-step queries, keys and
values, heavy-hitter rows and persistent-head masks, at the decode-layer shapes
of Llama3-8B (32 query / 8 KV heads) and Qwen2.5-14B (40 query / 8 KV heads),
d = 128, that the CLO evaluation uses (CLO per-paper synthesis page, section
3.1 "attack point 1").  It holds none of the decode step's arithmetic: no
cosine test, no scoring, no selection, no attention.  Both the HIP path and the
CPU oracle consume what it produces.

Random numbers come from the counter-based SplitMix64 / Box-Muller generator
in ``synth.c``; every element is a pure function of (seed, tensor tag, layer,
sequence, head, resample round, flat index), so results do not depend on the
thread count or on which slice is generated first.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libclogen.so")
_lib = None

MASK64 = (1 << 64) - 1

# tensor tags for key derivation
TAG_Q, TAG_QPREV, TAG_K, TAG_V, TAG_HEAVY, TAG_PERSIST, TAG_LOW, TAG_COS, TAG_WALK, TAG_VOLATILE = range(1, 11)

F32, BF16 = "f32", "bf16"


def build(verbose: bool = False) -> str:
    """Compile synth.c into libclogen.so with gcc (always rebuilds)."""
    import subprocess

    src = os.path.join(_HERE, "synth.c")
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        u64, i64, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        L.gen_u64.restype = u64
        L.gen_u64.argtypes = [u64, u64]
        L.gen_mix.restype = u64
        L.gen_mix.argtypes = [u64]
        L.gen_u64_fill.argtypes = [vp, i64, u64, i64]
        L.gen_uniform_f64.argtypes = [vp, i64, u64, i64]
        L.gen_normal_f64.argtypes = [vp, i64, u64, i64]
        L.gen_normal_rows.argtypes = [vp, vp, vp, i64, i64]
        L.gen_fill_rows.argtypes = [vp, i64, i64, u64, vp, ctypes.c_int, ctypes.c_int]
        L.gen_round.argtypes = [vp, vp, i64, ctypes.c_int]
        L.gen_copy.argtypes = [vp, vp, i64, ctypes.c_int]
        _lib = L
    return _lib


def default_threads() -> int:
    n = os.environ.get("OMP_NUM_THREADS")
    try:
        n = int(n) if n else (os.cpu_count() or 1)
    except ValueError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def mix(z: int) -> int:
    return int(lib().gen_mix(z & MASK64))


def derive_key(seed: int, *fields: int) -> int:
    """Chain a 64-bit stream key from the seed and integer fields."""
    z = seed & MASK64
    for f in fields:
        z = mix(z ^ mix((int(f) * 0x9E3779B97F4A7C15 + 0x632BE59BD9B4E019) & MASK64))
    return z


def u64_stream(key: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    if n:
        lib().gen_u64_fill(out.ctypes.data, n, key, first)
    return out


def uniform_stream(key: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    if n:
        lib().gen_uniform_f64(out.ctypes.data, n, key, first)
    return out


def normal_stream(key: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    if n:
        lib().gen_normal_f64(out.ctypes.data, n, key, first)
    return out


def storage_dtype(dtype: str):
    return np.float32 if dtype == F32 else np.uint16


def elem_bytes(dtype: str) -> int:
    return 4 if dtype == F32 else 2


def round_to(values: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values to the stored dtype (fp32, or bf16 bit patterns)."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, dtype=storage_dtype(dtype))
    if v.size:
        lib().gen_round(out.ctypes.data, v.ctypes.data, v.size, 0 if dtype == F32 else 1)
    return out


def smallest_by_key(key: int, n: int, m: int) -> np.ndarray:
    """m distinct positions of range(n), chosen by a seeded random key order."""
    if m <= 0:
        return np.zeros(0, dtype=np.int64)
    order = np.argsort(u64_stream(key, n), kind="stable")
    return order[:m].astype(np.int64)


@dataclass
class Problem:
    """One decode-step workload: shapes, data model and seeded contents.

    Layout of stored tensors (row-major): q and q_prev [B, Hq, d]; K and V of
    one (layer, sequence, KV head) unit [N, d].  Query head h belongs to KV head
    h // g with g = Hq / Hkv.
    """

    name: str
    layers: int
    batch: int
    hq: int
    hkv: int
    d: int
    context: int
    topk: int
    dtype: str
    tau: float
    seed: int
    qprev_model: str  # "mix" | "independent" | "target_cos"
    heavy_frac: float = 0.0
    heavy_scale: float = 4.0
    persistent: Optional[np.ndarray] = None  # bool [layers, hkv]
    low_frac: float = 0.2
    low_range: Tuple[float, float] = (0.2, 0.6)
    high_range: Tuple[float, float] = (0.801, 0.98)
    data_layers: Optional[int] = None  # K/V of layer l are those of layer l % data_layers
    # head-dependent similarity: a fraction of the (data layer, KV head) slots are
    # "volatile" -- their units draw the low cosine class with probability
    # volatile_low, the other slots less often, so that low_frac holds overall
    volatile_frac: float = 0.0
    volatile_low: float = 0.6
    slot_seed: Optional[int] = None  # seed of the volatile-slot draw (default: seed)
    k_resample: Dict[Tuple[int, int, int], Dict[int, int]] = field(default_factory=dict)
    qprev_round: Dict[Tuple[int, int, int], int] = field(default_factory=dict)
    walk_round: Dict[Tuple[int, int, int, int], int] = field(default_factory=dict)

    def __post_init__(self):
        assert self.hq % self.hkv == 0
        if self.persistent is None:
            self.persistent = np.zeros((self.layers, self.hkv), dtype=bool)
        self.persistent = np.asarray(self.persistent, dtype=bool).reshape(self.layers, self.hkv)
        self._cos_targets = None

    # ---- shape helpers -------------------------------------------------
    @property
    def g(self) -> int:
        return self.hq // self.hkv

    @property
    def units_per_layer(self) -> int:
        return self.batch * self.hkv

    def persistent_heads(self, layer: int):
        return [h for h in range(self.hkv) if self.persistent[layer, h]]

    def host_heads(self, layer: int):
        return [h for h in range(self.hkv) if not self.persistent[layer, h]]

    def persistent_mask_bits(self, layer: int) -> int:
        bits = 0
        for h in self.persistent_heads(layer):
            bits |= 1 << h
        return bits

    def data_layer(self, layer: int) -> int:
        return layer % self.data_layers if self.data_layers else layer

    # ---- queries ---------------------------------------------------------
    def q_f64(self, layer: int) -> np.ndarray:
        out = np.empty((self.batch, self.hq, self.d))
        for b in range(self.batch):
            for h in range(self.hq):
                out[b, h] = normal_stream(derive_key(self.seed, TAG_Q, layer, b, h), self.d)
        return out

    def q(self, layer: int) -> np.ndarray:
        """Current-step query, stored dtype, [B, Hq, d]."""
        return round_to(self.q_f64(layer), self.dtype)

    def volatile_slots(self) -> np.ndarray:
        """bool [layers, hkv]: the volatile (layer, KV head) slots, periodic over the
        data layers like the persistent mask."""
        if "_volatile" not in self.__dict__:
            period = self.data_layers or self.layers
            n = int(round(self.volatile_frac * period * self.hkv))
            seed = self.slot_seed if self.slot_seed is not None else self.seed
            base = np.zeros(period * self.hkv, dtype=bool)
            base[smallest_by_key(derive_key(seed, TAG_VOLATILE), period * self.hkv, n)] = True
            base = base.reshape(period, self.hkv)
            self.__dict__["_volatile"] = np.stack([base[l % period] for l in range(self.layers)])
        return self.__dict__["_volatile"]

    def low_probability(self, layer: int, kvh: int) -> float:
        """P(low cosine class) of a unit of this slot under the volatile-slot model."""
        if self.volatile_slots()[layer, kvh]:
            return self.volatile_low
        v = self.volatile_frac
        return max(0.0, (self.low_frac - v * self.volatile_low) / (1.0 - v))

    def cos_target(self, layer: int, b: int, kvh: int) -> float:
        """Target group cosine of a unit under the 80/20 correlation model (exactly
        round(low_frac * units) low units; with volatile slots, each unit low with
        its slot's probability)."""
        if self._cos_targets is None and self.volatile_frac > 0:
            U = self.layers * self.batch * self.hkv
            u = uniform_stream(derive_key(self.seed, TAG_COS), U)
            w = uniform_stream(derive_key(self.seed, TAG_LOW), U)
            t = np.empty(U)
            for i in range(U):
                l, h = i // (self.batch * self.hkv), i % self.hkv
                lo, hi = self.low_range if w[i] < self.low_probability(l, h) else self.high_range
                t[i] = lo + (hi - lo) * u[i]
            self._cos_targets = t
        if self._cos_targets is None:
            U = self.layers * self.batch * self.hkv
            n_low = int(round(self.low_frac * U))
            low = set(smallest_by_key(derive_key(self.seed, TAG_LOW), U, n_low).tolist())
            u = uniform_stream(derive_key(self.seed, TAG_COS), U)
            t = np.empty(U)
            for i in range(U):
                lo, hi = self.low_range if i in low else self.high_range
                t[i] = lo + (hi - lo) * u[i]
            self._cos_targets = t
        return float(self._cos_targets[(layer * self.batch + b) * self.hkv + kvh])

    def q_prev(self, layer: int) -> np.ndarray:
        """Previous-step query, stored dtype, [B, Hq, d]."""
        q_stored = self.q(layer)
        qf = stored_to_f64(q_stored, self.dtype)
        out = np.empty_like(qf)
        g, d = self.g, self.d
        for b in range(self.batch):
            for kvh in range(self.hkv):
                r = self.qprev_round.get((layer, b, kvh), 0)
                heads = range(kvh * g, (kvh + 1) * g)
                if self.qprev_model == "mix":
                    for h in heads:
                        n = normal_stream(derive_key(self.seed, TAG_QPREV, layer, b, h, r), d)
                        v = 0.9 * qf[b, h] + 0.44 * n
                        out[b, h] = v / np.sqrt(np.dot(v, v))
                elif self.qprev_model == "independent":
                    for h in heads:
                        out[b, h] = normal_stream(derive_key(self.seed, TAG_QPREV, layer, b, h, r), d)
                elif self.qprev_model == "target_cos":
                    c = self.cos_target(layer, b, kvh)
                    qg = qf[b, kvh * g:(kvh + 1) * g].reshape(-1)
                    qn = np.sqrt(np.dot(qg, qg))
                    qhat = qg / qn
                    n = normal_stream(derive_key(self.seed, TAG_QPREV, layer, b, kvh, r), g * d)
                    w = n - np.dot(n, qhat) * qhat
                    w /= np.sqrt(np.dot(w, w))
                    out[b, kvh * g:(kvh + 1) * g] = (qn * (c * qhat + math.sqrt(1 - c * c) * w)).reshape(g, d)
                else:
                    raise ValueError(self.qprev_model)
        return round_to(out, self.dtype)

    # ---- many decode steps ----------------------------------------------
    def walk_cos(self, layer: int, b: int, kvh: int, t: int) -> float:
        """Target cosine between a unit's query groups at steps t-1 and t: the
        80/20 model drawn afresh per (unit, step) -- "low" with probability
        low_frac, uniform in the class's range."""
        u = uniform_stream(derive_key(self.seed, TAG_WALK, layer, b, kvh, t), 2)
        lo, hi = self.low_range if u[0] < self.low_frac else self.high_range
        return float(lo + (hi - lo) * u[1])

    def q_walk(self, layer: int, t: int) -> np.ndarray:
        """Query at decode step t of a multi-step run, stored dtype, [B, Hq, d].

        Step 0 is q(layer); step t turns each unit's concatenated query group of
        step t-1 (its stored values) by the target cosine walk_cos towards a fresh
        direction orthogonal to it, keeping its norm."""
        cache = self.__dict__.setdefault("_walk_cache", {})
        if (layer, t) in cache:
            return cache[(layer, t)]
        if t == 0:
            out = self.q(layer)
        else:
            prev = stored_to_f64(self.q_walk(layer, t - 1), self.dtype)
            res = np.empty_like(prev)
            g, d = self.g, self.d
            for b in range(self.batch):
                for kvh in range(self.hkv):
                    c = self.walk_cos(layer, b, kvh, t)
                    r = self.walk_round.get((layer, b, kvh, t), 0)
                    qg = prev[b, kvh * g:(kvh + 1) * g].reshape(-1)
                    qn = np.sqrt(np.dot(qg, qg))
                    qhat = qg / qn
                    n = normal_stream(derive_key(self.seed, TAG_WALK, layer, b, kvh, t, r + 1), g * d)
                    w = n - np.dot(n, qhat) * qhat
                    w /= np.sqrt(np.dot(w, w))
                    res[b, kvh * g:(kvh + 1) * g] = (qn * (c * qhat + math.sqrt(1 - c * c) * w)).reshape(g, d)
            out = round_to(res, self.dtype)
        cache[(layer, t)] = out
        return out

    def resample_walk(self, layer: int, b: int, kvh: int, t: int) -> None:
        """Fresh direction for a unit's step-t query (later steps follow from it)."""
        key = (layer, b, kvh, t)
        self.walk_round[key] = self.walk_round.get(key, 0) + 1
        cache = self.__dict__.get("_walk_cache", {})
        for k in [k for k in cache if k[0] == layer and k[1] >= t]:
            del cache[k]

    # ---- keys and values -----------------------------------------------
    def heavy_rows(self, layer: int, b: int) -> np.ndarray:
        if self.heavy_frac <= 0:
            return np.zeros(0, dtype=np.int64)
        m = int(math.ceil(self.heavy_frac * self.context))
        dl = self.data_layer(layer)
        return np.sort(smallest_by_key(derive_key(self.seed, TAG_HEAVY, dl, b), self.context, m))

    def _row_scale(self, layer: int, b: int) -> Optional[np.ndarray]:
        key = (self.data_layer(layer), b)
        cache = self.__dict__.setdefault("_scale_cache", {})
        if key not in cache:
            rows = self.heavy_rows(layer, b)
            if rows.size == 0:
                cache[key] = None
            else:
                s = np.ones(self.context, dtype=np.float32)
                s[rows] = self.heavy_scale
                cache[key] = s
        return cache[key]

    def fill(self, which: str, layer: int, b: int, kvh: int, out_ptr: int, threads: Optional[int] = None):
        """Write the [N, d] K or V block of one unit to raw memory at out_ptr."""
        tag = TAG_K if which == "k" else TAG_V
        dl = self.data_layer(layer)
        scale = self._row_scale(layer, b) if which == "k" else None
        L = lib()
        dt = 0 if self.dtype == F32 else 1
        nt = threads or default_threads()
        L.gen_fill_rows(out_ptr, self.context, self.d, derive_key(self.seed, tag, dl, b, kvh, 0),
                        scale.ctypes.data if scale is not None else None, dt, nt)
        if which == "k":
            over = self.k_resample.get((dl, b, kvh))
            if over:
                eb = elem_bytes(self.dtype)
                one = np.empty(self.d, dtype=storage_dtype(self.dtype))
                for row, r in over.items():
                    # row `row` of the round-r stream, same norm class
                    key = derive_key(self.seed, tag, dl, b, kvh, r)
                    vals = normal_stream(key, self.d, first=row * self.d)
                    if scale is not None:
                        vals = vals * float(scale[row])
                    one[:] = round_to(vals, self.dtype)
                    ctypes.memmove(out_ptr + row * self.d * eb, one.ctypes.data, self.d * eb)

    def kv(self, which: str, layer: int, b: int, kvh: int, threads: Optional[int] = None) -> np.ndarray:
        out = np.empty((self.context, self.d), dtype=storage_dtype(self.dtype))
        self.fill(which, layer, b, kvh, out.ctypes.data, threads)
        return out

    def k_row_draw(self, layer: int, b: int, kvh: int, row: int, rnd: int) -> np.ndarray:
        """Stored values of key row `row` of a unit as drawn in resample round `rnd`."""
        dl = self.data_layer(layer)
        vals = normal_stream(derive_key(self.seed, TAG_K, dl, b, kvh, rnd), self.d, first=row * self.d)
        scale = self._row_scale(layer, b)
        if scale is not None:
            vals = vals * float(scale[row])
        return round_to(vals, self.dtype)

    def k_rows_draw(self, layer: int, b: int, kvh: int, rows, rnds) -> np.ndarray:
        """Stored values [n, d] of key rows rows[i] of a unit as drawn in resample
        rounds rnds[i] (k_row_draw for many rows and rounds in one call)."""
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        rnds = np.asarray(rnds, dtype=np.int64)
        dl = self.data_layer(layer)
        keymap = {int(r): derive_key(self.seed, TAG_K, dl, b, kvh, int(r)) for r in np.unique(rnds)}
        keys = np.array([keymap[int(r)] for r in rnds], dtype=np.uint64)
        vals = np.empty((rows.shape[0], self.d))
        if rows.shape[0]:
            lib().gen_normal_rows(vals.ctypes.data, keys.ctypes.data, rows.ctypes.data, rows.shape[0], self.d)
        scale = self._row_scale(layer, b)
        if scale is not None:
            vals *= scale[rows].astype(np.float64)[:, None]
        return round_to(vals, self.dtype)

    def k_row_round(self, layer: int, b: int, kvh: int, row: int) -> int:
        return self.k_resample.get((self.data_layer(layer), b, kvh), {}).get(int(row), 0)

    def set_k_row_round(self, layer: int, b: int, kvh: int, row: int, rnd: int) -> None:
        self.k_resample.setdefault((self.data_layer(layer), b, kvh), {})[int(row)] = int(rnd)

    def resample_k_rows(self, layer: int, b: int, kvh: int, rows) -> None:
        """Give the listed key rows of a unit a fresh draw (next resample round)."""
        dl = self.data_layer(layer)
        over = self.k_resample.setdefault((dl, b, kvh), {})
        for r in rows:
            r = int(r)
            over[r] = over.get(r, 0) + 1

    def resample_q_prev(self, layer: int, b: int, kvh: int) -> None:
        key = (layer, b, kvh)
        self.qprev_round[key] = self.qprev_round.get(key, 0) + 1


def stored_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact value of stored elements (fp32, or bf16 bit patterns) as fp64."""
    if dtype == F32:
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def topk_count(context: int, frac: float = 0.1) -> int:
    """k for a 'top 10%' selection: the ceiling of frac * N."""
    return int(math.ceil(frac * context - 1e-9))


def _persistent_slots(seed: int, layers: int, hkv: int, count: int) -> np.ndarray:
    m = np.zeros(layers * hkv, dtype=bool)
    m[smallest_by_key(derive_key(seed, TAG_PERSIST), layers * hkv, count)] = True
    return m.reshape(layers, hkv)


def config(cfg: int, **overrides) -> Problem:
    """The five benchmark workloads (plus keyword overrides for smaller variants).

    1: one layer, B=1, 32Q/8KV, d=128, N=4096, fp32, k=410, q_prev mixed from
       q_t per head, tau 0.8, every KV head persistent.
    2: Llama3-8B layer, B=16, N=32768, bf16, 1% heavy-hitter keys at 4x norm,
       2 of 8 heads persistent, independent q_prev.
    3: Llama3-8B layer, B=64, N=131072, bf16, 80% of units with cos in
       [0.801, 0.98] and 20% in [0.2, 0.6], no persistent heads.
    4: Qwen2.5-14B, 48 layers, B=8, 40Q/8KV, N=262144, bf16, 0.5% heavy
       hitters, 183 of 384 (layer, KV head) slots persistent (~47.6%).
    5: Qwen2.5-14B, 48 layers, B=1, N=524288, bf16, same data model as 4.
    """
    seed = 0x5EED0000 + cfg
    if cfg == 1:
        p = dict(name="cfg1", layers=1, batch=1, hq=32, hkv=8, d=128, context=4096, dtype=F32,
                 tau=0.8, seed=seed, qprev_model="mix")
    elif cfg == 2:
        p = dict(name="cfg2", layers=1, batch=16, hq=32, hkv=8, d=128, context=32768, dtype=BF16,
                 tau=0.8, seed=seed, qprev_model="independent", heavy_frac=0.01)
    elif cfg == 3:
        p = dict(name="cfg3", layers=1, batch=64, hq=32, hkv=8, d=128, context=131072, dtype=BF16,
                 tau=0.8, seed=seed, qprev_model="target_cos")
    elif cfg == 4:
        p = dict(name="cfg4", layers=48, batch=8, hq=40, hkv=8, d=128, context=262144, dtype=BF16,
                 tau=0.8, seed=seed, qprev_model="target_cos", heavy_frac=0.005)
    elif cfg == 5:
        p = dict(name="cfg5", layers=48, batch=1, hq=40, hkv=8, d=128, context=524288, dtype=BF16,
                 tau=0.8, seed=seed, qprev_model="target_cos", heavy_frac=0.005)
    else:
        raise ValueError(f"unknown config {cfg}")
    p.update(overrides)
    if "topk" not in p:
        p["topk"] = topk_count(p["context"])
    if "persistent" not in p:
        L, H = p["layers"], p["hkv"]
        period = p.get("data_layers") or L  # aliased layers share data, so they share the mask
        if cfg == 1:
            p["persistent"] = np.ones((L, H), dtype=bool)
        elif cfg == 2:
            p["persistent"] = _persistent_slots(seed, 1, H, 2).repeat(L, axis=0)
        elif cfg == 3:
            p["persistent"] = np.zeros((L, H), dtype=bool)
        else:
            # ~47.6% of (layer, KV head) slots keep their full KV in HBM
            base = _persistent_slots(seed, period, H, int(round(0.476 * period * H)))
            p["persistent"] = np.stack([base[l % period] for l in range(L)])
    return Problem(**p)

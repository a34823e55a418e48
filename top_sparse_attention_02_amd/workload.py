"""Device/pinned buffers of one layer in the library's layout, and loading synthetic workloads into them.

`LayerBuffers` allocates every tensor a decode step reads or writes (device
memory from torch, K/V of non-persistent heads in pinned host memory) in the
row-major layouts include/clo.h documents.  `load_layer` fills them from a
seeded `gen.Problem`; `decode_step` drives the two-step protocol: step 0 (cold,
every unit misses, q_prev as the query) and step 1 (the steady decode step).
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch

from . import clo
from .hip_host import HostBuffer, copy_h2d, hipHostMallocMapped

HEAD_DIM = 128


def torch_dtype(dtype: str):
    return torch.float32 if dtype == "f32" else torch.bfloat16


def clo_dtype(dtype: str) -> int:
    return clo.CLO_F32 if dtype == "f32" else clo.CLO_BF16


def quant_row_bytes(host_format: int) -> int:
    """Bytes of one quantized row of HEAD_DIM values (a record holds a K and a V row)."""
    return HEAD_DIM // 2 if host_format == clo.CLO_HOST_INT4 else HEAD_DIM


def elem_bytes(dtype: str) -> int:
    return 4 if dtype == "f32" else 2


class LayerBuffers:
    """All buffers of one layer for batch B, Hq/Hkv heads, context N and top-k k."""

    def __init__(self, batch: int, hq: int, hkv: int, context: int, topk: int, dtype: str, persistent_mask: int,
                 tau: float, device: str = "cuda", host_flags: int = hipHostMallocMapped,
                 share: Optional["LayerBuffers"] = None, host_format: int = clo.CLO_HOST_NATIVE):
        self.B, self.Hq, self.Hkv, self.N, self.k = batch, hq, hkv, context, topk
        self.dtype, self.tau, self.mask = dtype, tau, persistent_mask
        self.host_format = host_format
        self.P = bin(persistent_mask).count("1")
        self.H = hkv - self.P
        tdt = torch_dtype(dtype)
        d = HEAD_DIM
        dev = torch.device(device)
        self.q = torch.zeros(batch, hq, d, dtype=tdt, device=dev)
        self.q_prev = torch.zeros_like(self.q)
        self.out = torch.zeros_like(self.q)
        self.reuse = torch.zeros(batch, hkv, dtype=torch.uint8, device=dev)
        self.cos = torch.zeros(batch, hkv, dtype=torch.float32, device=dev)
        self.idx = torch.zeros(batch, hkv, topk, dtype=torch.int32, device=dev)
        # inputs (full K/V): shared with `share` when layers alias the same data
        self.shared = share is not None
        self.k_exp = self.v_exp = None
        if share is not None:
            assert share.mask == persistent_mask and share.N == context and share.B == batch
            self.k_hbm, self.v_hbm = share.k_hbm, share.v_hbm
            self.k_host, self.v_host, self.k_score = share.k_host, share.v_host, share.k_score
            self.host_format, self.k_exp, self.v_exp = share.host_format, share.k_exp, share.v_exp
        else:
            self.k_hbm = self.v_hbm = None
            if self.P:
                self.k_hbm = torch.empty(batch, self.P, context, d, dtype=tdt, device=dev)
                self.v_hbm = torch.empty_like(self.k_hbm)
            self.k_host = self.v_host = self.k_score = None
            if self.H:
                if host_format != clo.CLO_HOST_NATIVE:
                    # one record per token (256 bytes with int8, 128 with int4): K values, then V values
                    self.k_host = HostBuffer(batch * self.H * context * 2 * quant_row_bytes(host_format), host_flags)
                else:
                    nb = batch * self.H * context * d * elem_bytes(dtype)
                    self.k_host = HostBuffer(nb, host_flags)
                    self.v_host = HostBuffer(nb, host_flags)
                self.k_score = torch.empty(batch, self.H, context, d, dtype=tdt, device=dev)
                if host_format != clo.CLO_HOST_NATIVE:
                    self.k_exp = torch.zeros(batch, self.H, context, dtype=torch.int8, device=dev)
                    self.v_exp = torch.zeros_like(self.k_exp)
        # outputs and per-layer state
        self.k_cache = self.v_cache = None
        if self.H:
            self.k_cache = torch.zeros(batch, self.H, topk, d, dtype=tdt, device=dev)
            self.v_cache = torch.zeros_like(self.k_cache)
        self.shape = clo.Shape(batch, hq, hkv, context, topk, tau, clo_dtype(dtype))
        ws = clo.clo_workspace_size(self.shape)
        self.ws = torch.zeros(max(ws, 256), dtype=torch.uint8, device=dev)

    def set_block_size(self, block_size: int):
        """Select token blocks of this size (0/1 = tokens); grows the workspace when needed."""
        self.shape.block_size = block_size
        need = clo.clo_workspace_size(self.shape)
        if need > self.ws.numel():
            self.ws = torch.zeros(need, dtype=torch.uint8, device=self.ws.device)

    # ----------------------------------------------------------------- views
    def layer(self) -> clo.Layer:
        return clo.Layer(self.mask, self.k_hbm, self.v_hbm, self.k_host, self.v_host, self.k_score, self.k_cache,
                         self.v_cache, self.idx, self.host_format, self.k_exp, self.v_exp)

    def shape_with(self, tau: float) -> clo.Shape:
        """The layer's shape with threshold tau (+inf: every unit misses, whatever
        the per-head thresholds)."""
        s = clo.Shape(**self.shape.__dict__)
        s.tau = tau
        if math.isinf(tau):
            s.tau_heads = None
        return s

    def slot(self, kvh: int) -> int:
        """Rank of KV head kvh among the persistent or the non-persistent heads."""
        pers = (self.mask >> kvh) & 1
        return sum(1 for h in range(kvh) if ((self.mask >> h) & 1) == pers)

    def is_persistent(self, kvh: int) -> bool:
        return bool((self.mask >> kvh) & 1)

    def host_view(self, which: str, b: int, kvh: int) -> np.ndarray:
        """numpy view of a non-persistent unit's pinned K or V: [N, d] rows, or the
        quantized values ([N, d] int8; [N, d/2] uint8 bytes of two 4-bit values)."""
        if self.host_format != clo.CLO_HOST_NATIVE:
            rb = quant_row_bytes(self.host_format)
            unit = self.N * 2 * rb
            off = (b * self.H + self.slot(kvh)) * unit
            npdt = np.int8 if self.host_format == clo.CLO_HOST_INT8 else np.uint8
            rec = self.k_host.numpy(npdt, (self.N, 2, rb), offset=off)
            return rec[:, 0 if which == "k" else 1, :]
        buf = self.k_host if which == "k" else self.v_host
        npdt, eb = (np.float32 if self.dtype == "f32" else np.uint16), elem_bytes(self.dtype)
        unit = self.N * HEAD_DIM * eb
        off = (b * self.H + self.slot(kvh)) * unit
        return buf.numpy(npdt, (self.N, HEAD_DIM), offset=off)

    # ----------------------------------------------------------------- steps
    def decode_step(self, q, q_prev, tau: float, stream=None, sync=None):
        clo.clo_decode_step(self.shape_with(tau), self.layer(), q, q_prev, self.out, self.reuse, self.cos, self.ws,
                            sync=sync, stream=stream)

    def step0(self, stream=None):
        """Cold step: every unit misses and selects with q_prev as its query."""
        self.decode_step(self.q_prev, self.q_prev, math.inf, stream)

    def step1(self, stream=None):
        """Steady decode step: q_t against q_prev with the real threshold."""
        self.decode_step(self.q, self.q_prev, self.tau, stream)


def capture_step(step) -> "torch.cuda.CUDAGraph":
    """Capture one call of `step` (a function that enqueues a whole decode step on
    the current stream, e.g. LayerBuffers.step1) into a HIP graph; replay() then
    launches all of its kernels at once.  The library records no memset or copy,
    synchronizes nothing and, under capture, runs the step in order on the
    capturing stream, so the step captures whole; validation runs on the host at
    capture time only, and the buffers must stay where they were when captured."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # one eager call first: the library creates its helper streams outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # relaxed: the host-side pointer checks of the library's entry points
    # (hipPointerGetAttributes) run during the capture, and they enqueue nothing
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        step()
    torch.cuda.synchronize()
    return g


def stored_tensor(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to(device)


def load_layer(problem, layer: int, bufs: Optional[LayerBuffers] = None, threads: Optional[int] = None,
               log=None, share: Optional[LayerBuffers] = None, host_flags: int = hipHostMallocMapped,
               host_format: int = clo.CLO_HOST_NATIVE) -> LayerBuffers:
    """Allocate (unless given) and fill the buffers of one layer of `problem`.

    With `share`, the layer reuses that layer's K/V buffers (aliased data) and
    only its queries are loaded.  With a quantized host format the offloaded
    rows are quantized by clo_quantize_rows on the GPU straight into pinned
    memory."""
    p = problem
    mask = p.persistent_mask_bits(layer)
    if bufs is None:
        bufs = LayerBuffers(p.batch, p.hq, p.hkv, p.context, p.topk, p.dtype, mask, p.tau, share=share,
                            host_flags=host_flags, host_format=host_format)
    assert bufs.mask == mask
    bufs.q.copy_(stored_tensor(p.q(layer), p.dtype))
    bufs.q_prev.copy_(stored_tensor(p.q_prev(layer), p.dtype))
    if bufs.shared:
        return bufs
    eb = elem_bytes(p.dtype)
    unit_bytes = p.context * HEAD_DIM * eb
    staging = None
    q8 = bufs.host_format != clo.CLO_HOST_NATIVE  # a quantized host format
    rb = quant_row_bytes(bufs.host_format) if q8 else 0
    dev_stage = torch.empty(p.context, HEAD_DIM, dtype=torch_dtype(p.dtype), device=bufs.q.device) if q8 else None
    for b in range(p.batch):
        for kvh in range(p.hkv):
            if q8 and not bufs.is_persistent(kvh):
                if staging is None:
                    staging = HostBuffer(unit_bytes)
                s = bufs.slot(kvh)
                rec = bufs.k_host.ptr + (b * bufs.H + s) * p.context * 2 * rb  # the unit's records
                for which, exp, half in (("k", bufs.k_exp, 0), ("v", bufs.v_exp, rb)):
                    p.fill(which, layer, b, kvh, staging.ptr, threads)
                    copy_h2d(dev_stage.data_ptr(), staging.ptr, unit_bytes)
                    if which == "k":
                        bufs.k_score[b, s].copy_(dev_stage)
                    clo.clo_quantize_rows(dev_stage, p.context, clo_dtype(p.dtype), rec + half, exp[b, s],
                                          dst_stride=2 * rb, host_format=bufs.host_format)
                torch.cuda.synchronize()
                continue
            if bufs.is_persistent(kvh):
                if staging is None:
                    staging = HostBuffer(unit_bytes)
                s = bufs.slot(kvh)
                for which, dst in (("k", bufs.k_hbm), ("v", bufs.v_hbm)):
                    p.fill(which, layer, b, kvh, staging.ptr, threads)
                    copy_h2d(dst[b, s].data_ptr(), staging.ptr, unit_bytes)
            else:
                off = (b * bufs.H + bufs.slot(kvh)) * unit_bytes
                p.fill("k", layer, b, kvh, bufs.k_host.ptr + off, threads)
                p.fill("v", layer, b, kvh, bufs.v_host.ptr + off, threads)
        if log:
            log(f"  generated sequence {b + 1}/{p.batch}")
    if bufs.H and not q8:
        copy_h2d(bufs.k_score.data_ptr(), bufs.k_host.ptr, bufs.B * bufs.H * unit_bytes)
    if staging is not None:
        staging.close()
    torch.cuda.synchronize()
    return bufs


def load_layers(problem, log=None, threads: Optional[int] = None, host_flags: int = hipHostMallocMapped,
                host_format: int = clo.CLO_HOST_NATIVE):
    """Buffers of every layer; layers with the same data layer share their K/V."""
    first = {}
    layers = []
    for l in range(problem.layers):
        dl = problem.data_layer(l)
        bufs = load_layer(problem, l, threads=threads, share=first.get(dl), host_flags=host_flags,
                          host_format=host_format)
        first.setdefault(dl, bufs)
        layers.append(bufs)
        if log:
            log(f"  layer {l + 1}/{problem.layers} ready (data layer {dl})")
    torch.cuda.synchronize()
    return layers


def default_select_batches(units: int, n_layers: int):
    """Selection batch sizes of the 48-layer loop: a first batch of about 24
    units (at least one layer), the same again, then doubling, at most 64 layers
    per call.  Measured on MI355X (ms per 48-layer step): B=1, N=524288 (8 units
    per layer) 17.89 with 3, 3, 6, 12, 24 against 18.09 with 1, 1, 2, 4, 8, 16, 16
    (int4 rows: 8.10 against 8.15); B=8, N=262144 (64 units) 76.2 with 1, 1, 2, 4,
    8, 16, 16 against 76.6 with 3, 3, 6, 12, 24.  With the attention batched too, at
    B=1: 17.84 (int4 rows 7.02) with 3, 3, 6, 12, 24 against 17.90-17.91 (7.40-7.44)
    with 2, 2, 4, 8, 16, 16 or 4, 4, 8, 16, 16, 18.04 (7.09) with 6, 6, 12, 24 and
    17.95 (7.62) with 3, 6, 12, 27; re-measured side by side, 17.83-17.84 with 3, 3,
    6, 12, 24 against 17.88-17.89 with 1, 2, 3, 6, 12, 24, 17.92-17.94 with 1, 2,
    4, 8, 16, 17 and 18.02 with 2, 3, 6, 12, 25."""
    f = max(1, -(-24 // max(1, units)))
    sizes, n = [f, f], f
    while sum(sizes) < n_layers:
        n = min(2 * n, 64)
        sizes.append(n)
    return tuple(sizes)


def default_attend_batches(n_layers: int):
    """Attention batch sizes of the 48-layer loop (clo_attend_layers): batches of
    8 layers, the last layers in batches of 4, 2, 1 and 1 so that little
    attention is left once the gather has read the last layer."""
    sizes, left = [], n_layers
    tail = [n for n in (4, 2, 1, 1) if n <= n_layers]
    body = n_layers - sum(tail)
    while body > 0:
        sizes.append(min(8, body))
        body -= sizes[-1]
    return tuple(sizes + tail)


def batched_attend_ok(layers) -> bool:
    """Whether clo_attend_layers takes these layers: one batch, head and top-k shape."""
    b = layers[0]
    return all((x.B, x.Hq, x.Hkv, x.k, x.dtype) == (b.B, b.Hq, b.Hkv, b.k, b.dtype) for x in layers)


def batched_select_ok(layers) -> bool:
    """Whether clo_select_layers takes these layers: bf16, at most 64 units per
    layer, token top-k, at most 128 chunks of 16384 keys, one shape for all."""
    b = layers[0]
    same = all((x.B, x.Hq, x.Hkv, x.N, x.k) == (b.B, b.Hq, b.Hkv, b.N, b.k) for x in layers)
    return (same and b.dtype == "bf16" and b.B * b.Hkv <= 64 and (b.shape.block_size or 1) <= 1
            and -(-b.N // 16384) <= 128)


def _cover(sizes, n_layers: int):
    """Consecutive batches covering n_layers: the given sizes, the last cut to
    fit or repeated until every layer is covered."""
    out, left = [], n_layers
    for n in sizes:
        if left <= 0:
            break
        out.append(min(int(n), left))
        left -= out[-1]
    while left > 0:
        out.append(min(int(sizes[-1]), left))
        left -= out[-1]
    return out


class LayerLoop:
    """A multi-layer decode step on streams ordered only by device flags.

    select: reuse test, scoring and top-k of layer l (one clo_reuse_select), then
            flag sel[l] = epoch;
            with select_streams > 1 the layers alternate between that many
            streams (slower on MI355X: at B=1, N=524288 two streams gave 38.9
            against 46.6 steps/s and at B=8, N=262144 10.3 against 12.2, the
            concurrent scorings and top-k passes slowing each other and the
            gather more than the overlap gains);
    gather: waits for sel[l], reads layer l's selected rows from host memory,
            then flag gat[l] = epoch -- by default one resident launch per step
            over all layers (clo_gather_layers), whose blocks run from one
            layer's tail straight into the next layer; gather="per-layer" uses
            one clo_gather_kv launch per layer instead;
    attend: waits for gat[l], attention of layer l, then flag att[l] = epoch;
            with attend="batched" (the default) consecutive layers are attended
            by one clo_attend_layers call each (sizes `attend_batches`, by
            default default_attend_batches), which waits for every gat[l] of
            its layers and sets their att[l], four launches per call instead
            of four per layer.
    With select="batched" the selections run as clo_select_layers calls over
    consecutive layers (sizes `select_batches`, by default
    default_select_batches: small first so that the gather starts early, larger
    after), four launches per call instead of four per layer; each layer still
    waits for its own att[l] and sets its own sel[l].
    The selection of layer l in the next step waits for att[l] of this step
    before overwriting layer l's selections.  Selection and gathering of layer
    l+1 therefore run while layer l is attended (one-layer-ahead prefetch and
    beyond); the host never waits inside a step.  Every layer has its own
    workspace, selections and cache, so selections on different streams share
    only read-only inputs.
    """

    def __init__(self, layers, spin_limit: int = 0, select_streams: int = 1, gather: str = "resident",
                 select: str = "batched", select_batches=None, attend: str = "batched", attend_batches=None,
                 gather_blocks: int = 0):
        if gather not in ("resident", "per-layer"):
            raise ValueError(gather)
        if select not in ("per-layer", "batched"):
            raise ValueError(select)
        if attend not in ("per-layer", "batched"):
            raise ValueError(attend)
        if select == "batched" and not batched_select_ok(layers):
            select = "per-layer"  # shapes the multi-layer selection does not take
        if attend == "batched" and (gather != "resident" or not batched_attend_ok(layers)):
            attend = "per-layer"  # the per-layer gathers each hand their layer to its attention
        self.layers = layers
        L = len(layers)
        dev = layers[0].q.device
        self.flags = torch.zeros(3, L, dtype=torch.int32, device=dev)
        self.error = torch.zeros(1, dtype=torch.int32, device=dev)
        self.s_selects = [torch.cuda.Stream(device=dev) for _ in range(max(1, select_streams))]
        self.s_gather = torch.cuda.Stream(device=dev)
        self.s_attend = torch.cuda.Stream(device=dev)
        self.epoch = 0
        self.spin_limit = spin_limit
        self.gather = gather
        self.plan = None
        if gather == "resident":
            self.plan = torch.zeros(clo.clo_gather_plan_size(L), dtype=torch.uint8, device=dev)
            items = [(b.shape, b.layer(), b.reuse, b.ws, self._flag(0, l), self._flag(1, l))
                     for l, b in enumerate(layers)]
            self.plan_blocks = clo.clo_gather_plan(items, self.plan)
            if gather_blocks:  # the resident gather's grid instead of the plan's suggestion
                self.plan_blocks = int(gather_blocks)
        self.select = select
        self.sel_plans = {}
        if select == "batched":
            if select_batches is None:
                select_batches = default_select_batches(layers[0].B * layers[0].Hkv, L)
            self.batches = _cover(select_batches, L)
            # one plan for steady steps (each layer's query and threshold) and one for
            # cold steps (every unit misses: tau = +inf, q_prev as the query)
            for cold in (False, True):
                plan = torch.zeros(clo.clo_select_plan_size(L), dtype=torch.uint8, device=dev)
                items = []
                for l, b in enumerate(layers):
                    shape = b.shape_with(math.inf if cold else b.tau)
                    items.append((shape, b.layer(), b.q_prev if cold else b.q, b.q_prev, b.reuse, b.cos, b.ws,
                                  self._flag(2, l), self._flag(0, l)))
                clo.clo_select_plan(items, plan)
                self.sel_plans[cold] = plan
        self.attend = attend
        self.att_plans = {}
        if attend == "batched":
            self.att_batches = _cover(attend_batches or default_attend_batches(L), L)
            # steady steps attend with each layer's query, cold steps with q_prev
            for cold in (False, True):
                plan = torch.zeros(clo.clo_attend_plan_size(L), dtype=torch.uint8, device=dev)
                items = [(b.shape, b.layer(), b.q_prev if cold else b.q, b.out, b.ws, self._flag(1, l),
                          self._flag(2, l)) for l, b in enumerate(layers)]
                clo.clo_attend_plan(items, plan)
                self.att_plans[cold] = plan

    def _flag(self, kind: int, l: int):
        return self.flags[kind, l]

    def step(self, cold: bool = False):
        """Enqueue one decode step over all layers (cold: every unit misses)."""
        # the loop's streams start after work already queued on the current stream
        cur = torch.cuda.current_stream()
        for st in (*self.s_selects, self.s_gather, self.s_attend):
            st.wait_stream(cur)
        self.epoch += 1
        e = self.epoch
        sp = self.spin_limit
        resident = self.gather == "resident"
        calls = []
        if self.select == "batched":
            # each layer waits for its att[l] of the previous step (flags start at 0)
            plan, first = self.sel_plans[cold], 0
            for n in self.batches:
                clo.clo_select_layers(self.layers[0].shape, plan, first, n, e - 1, e, error_word=self.error,
                                      spin_limit=sp, stream=self.s_selects[0])
                first += n
        for l, b in enumerate(self.layers):
            tau = math.inf if cold else b.tau
            q = b.q_prev if cold else b.q
            shape, layer = b.shape_with(tau), b.layer()
            # waits for the previous step's attention of this layer, signals sel[l]
            sel_sync = clo.Sync(signal_flag=self._flag(0, l), signal_value=e)
            if e > 1:
                sel_sync = clo.Sync(wait_flag=self._flag(2, l), wait_value=e - 1, error_word=self.error,
                                    spin_limit=sp, signal_flag=self._flag(0, l), signal_value=e)
            s_sel = self.s_selects[l % len(self.s_selects)]
            if self.select != "batched":
                clo.clo_reuse_select(shape, layer, q, b.q_prev, b.reuse, b.cos, b.ws, sync=sel_sync, stream=s_sel)
            if not resident:
                clo.clo_gather_kv(shape, layer, b.reuse, b.ws,
                                  sync=clo.Sync(wait_flag=self._flag(0, l), wait_value=e,
                                                signal_flag=self._flag(1, l), signal_value=e,
                                                error_word=self.error, spin_limit=sp),
                                  stream=self.s_gather)
                self._attend(b, shape, layer, q, l, e)
            else:
                calls.append((b, shape, layer, q, l))
        if resident:
            # every selection is enqueued before the gather that waits for it
            clo.clo_gather_layers(self.plan, len(self.layers), self.plan_blocks, e, e, error_word=self.error,
                                  spin_limit=sp, stream=self.s_gather)
            if self.attend == "batched":
                plan, first = self.att_plans[cold], 0
                for n in self.att_batches:
                    clo.clo_attend_layers(self.layers[0].shape, plan, first, n, e, e, error_word=self.error,
                                          spin_limit=sp, stream=self.s_attend)
                    first += n
            else:
                for b, shape, layer, q, l in calls:
                    self._attend(b, shape, layer, q, l, e)
        # the caller's stream continues after the last attention
        cur.wait_stream(self.s_attend)

    def _attend(self, b, shape, layer, q, l, e):
        clo.clo_sparse_attn(shape, layer, q, b.out, b.ws,
                            sync=clo.Sync(wait_flag=self._flag(1, l), wait_value=e, signal_flag=self._flag(2, l),
                                          signal_value=e, error_word=self.error, spin_limit=self.spin_limit),
                            stream=self.s_attend)

    def check(self):
        """Raise if any device-side wait timed out (call after a synchronize)."""
        v = int(self.error.item())
        if v:
            raise RuntimeError(f"device-side wait failed with status {v} ({clo.clo_status_string(v)})")


def host_rows_tensor(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Stored rows (fp32, or bf16 bit patterns) from pinned or pageable memory -> device tensor."""
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.int16) if dtype == "bf16" else a)
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to(device)


class GrowingRun:
    """Multi-step decoding of one layer over a growing context.

    The layer's buffers hold capacity C = problem.context rows per (sequence,
    head).  The run starts with the first n0 = C - steps rows (the rows after
    them are cleared) and before step t >= 1 appends row n0 + t - 1 of every
    unit with clo_append_kv, so step t decodes over n0 + t rows.  Step 0 is a
    cold step (every unit misses, q_0 as its own reference); step t >= 1
    compares q_t = problem.q_walk(layer, t) with the reference: the previous
    step's query ("previous") or the query of the unit's last miss ("refresh",
    kept on the GPU by clo_update_reference).
    """

    def __init__(self, problem, layer: int, steps: int, policy: str = "previous",
                 host_flags: int = hipHostMallocMapped, host_format: int = clo.CLO_HOST_NATIVE):
        if policy not in ("previous", "refresh"):
            raise ValueError(policy)
        p = problem
        self.p, self.layer, self.steps, self.policy = p, layer, steps, policy
        self.C = p.context
        self.n0 = p.context - steps
        assert self.n0 >= p.topk
        b = self.bufs = load_layer(p, layer, host_flags=host_flags, host_format=host_format)
        dev = b.q.device
        tdt = torch_dtype(p.dtype)
        n0 = self.n0
        # the rows appended during the run, [steps, B, Hkv, d], taken from the loaded
        # buffers; the buffers then hold only the first n0 rows
        self.k_new = torch.zeros(steps, b.B, b.Hkv, HEAD_DIM, dtype=tdt, device=dev)
        self.v_new = torch.zeros_like(self.k_new)
        for h in range(b.Hkv):
            s = b.slot(h)
            if b.is_persistent(h):
                self.k_new[:, :, h] = b.k_hbm[:, s, n0:].transpose(0, 1)
                self.v_new[:, :, h] = b.v_hbm[:, s, n0:].transpose(0, 1)
            else:
                self.k_new[:, :, h] = b.k_score[:, s, n0:].transpose(0, 1)
                for bb in range(b.B):
                    self.v_new[:, bb, h] = host_rows_tensor(p.kv("v", layer, bb, h)[n0:], p.dtype, dev)
        self.qs = torch.stack([stored_tensor(p.q_walk(layer, t), p.dtype, dev) for t in range(steps + 1)])
        self.q_ref = torch.zeros_like(b.q)
        self.reset()

    def reset(self, policy: Optional[str] = None):
        """Clear the rows the run appends, so that it can start again (optionally
        with another reference policy)."""
        if policy is not None:
            if policy not in ("previous", "refresh"):
                raise ValueError(policy)
            self.policy = policy
        b, n0 = self.bufs, self.n0
        torch.cuda.synchronize()
        for h in range(b.Hkv):
            s = b.slot(h)
            if b.is_persistent(h):
                b.k_hbm[:, s, n0:] = 0
                b.v_hbm[:, s, n0:] = 0
            else:
                b.k_score[:, s, n0:] = 0
                for bb in range(b.B):
                    b.host_view("k", bb, h)[n0:] = 0
                    b.host_view("v", bb, h)[n0:] = 0
        torch.cuda.synchronize()

    def shape(self, t: int, tau: float) -> clo.Shape:
        s = clo.Shape(**self.bufs.shape.__dict__)
        s.context, s.capacity, s.tau = self.n0 + t, self.C, tau
        return s

    def step(self, t: int, stream=None):
        """Enqueue step t (steps run in order 0, 1, ..., steps)."""
        b = self.bufs
        q = self.qs[t]
        if t == 0:
            s = self.shape(0, math.inf)
            clo.clo_decode_step(s, b.layer(), q, q, b.out, b.reuse, b.cos, b.ws, stream=stream)
            clo.clo_update_reference(s, q, None, self.q_ref, stream=stream)
            return
        s = self.shape(t, b.tau)
        clo.clo_append_kv(s, b.layer(), self.k_new[t - 1], self.v_new[t - 1], self.n0 + t - 1, stream=stream)
        ref = self.qs[t - 1] if self.policy == "previous" else self.q_ref
        clo.clo_decode_step(s, b.layer(), q, ref, b.out, b.reuse, b.cos, b.ws, stream=stream)
        if self.policy == "refresh":
            clo.clo_update_reference(s, q, b.reuse, self.q_ref, stream=stream)

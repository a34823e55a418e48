"""Python binding of libclo.so: the same entry points as include/clo.h, argument marshalling only.

Every step of the decode path runs in the HIP kernels behind the C ABI; this
module only turns torch tensors / pinned host buffers into pointers and checks
the returned status.  Importing it without a built libclo.so raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libclo.so")

CLO_F32, CLO_BF16 = 0, 1
CLO_HOST_NATIVE, CLO_HOST_INT8, CLO_HOST_INT4 = 0, 1, 2
CLO_OK, CLO_E_ARG, CLO_E_UNSUPPORTED, CLO_E_WORKSPACE, CLO_E_HIP, CLO_E_TIMEOUT, CLO_E_INDEX = range(7)

# every function include/clo.h declares
EXPORTS = ("clo_workspace_size", "clo_reuse_test", "clo_topk_select", "clo_reuse_select", "clo_gather_kv",
           "clo_sparse_attn", "clo_decode_step", "clo_decode_step_static", "clo_append_kv", "clo_update_reference", "clo_plan_persistent", "clo_quantize_rows",
           "clo_stream_read", "clo_status_string", "clo_last_error", "clo_gather_plan_size", "clo_gather_plan",
           "clo_gather_layers", "clo_select_plan_size", "clo_select_plan", "clo_select_layers",
           "clo_attend_plan_size", "clo_attend_plan", "clo_attend_layers", "clo_decode_step_schedule",
           "clo_last_step_gather_ms")

CLO_STEP_IN_ORDER, CLO_STEP_RANGE_GATHERS, CLO_STEP_RESIDENT_GATHER = range(3)
STEP_MODES = {CLO_STEP_IN_ORDER: "in order", CLO_STEP_RANGE_GATHERS: "a gather launch per unit range",
              CLO_STEP_RESIDENT_GATHER: "one resident gather launch"}


class CloError(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        super().__init__(f"{func}: status {status} ({msg})")
        self.status = status


class clo_shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("context", ctypes.c_int64), ("topk", ctypes.c_int64),
                ("tau", ctypes.c_float), ("dtype", ctypes.c_int32), ("capacity", ctypes.c_int64),
                ("tau_heads", ctypes.POINTER(ctypes.c_float)), ("block_size", ctypes.c_int32)]


class clo_layer(ctypes.Structure):
    _fields_ = [("persistent_mask", ctypes.c_uint64), ("k_hbm", ctypes.c_void_p), ("v_hbm", ctypes.c_void_p),
                ("k_host", ctypes.c_void_p), ("v_host", ctypes.c_void_p), ("k_score", ctypes.c_void_p),
                ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p), ("idx", ctypes.c_void_p),
                ("host_format", ctypes.c_int32), ("k_host_exp", ctypes.c_void_p), ("v_host_exp", ctypes.c_void_p)]


class clo_sync(ctypes.Structure):
    _fields_ = [("wait_flag", ctypes.c_void_p), ("wait_value", ctypes.c_uint32),
                ("signal_flag", ctypes.c_void_p), ("signal_value", ctypes.c_uint32),
                ("error_word", ctypes.c_void_p), ("spin_limit", ctypes.c_uint32)]


class clo_gather_layer(ctypes.Structure):
    _fields_ = [("shape", ctypes.POINTER(clo_shape)), ("layer", ctypes.POINTER(clo_layer)), ("reuse", ctypes.c_void_p),
                ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t), ("wait_flag", ctypes.c_void_p),
                ("signal_flag", ctypes.c_void_p)]


class clo_select_layer(ctypes.Structure):
    _fields_ = [("shape", ctypes.POINTER(clo_shape)), ("layer", ctypes.POINTER(clo_layer)), ("q", ctypes.c_void_p),
                ("q_prev", ctypes.c_void_p), ("reuse", ctypes.c_void_p), ("cos", ctypes.c_void_p),
                ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t), ("wait_flag", ctypes.c_void_p),
                ("signal_flag", ctypes.c_void_p)]


class clo_step_schedule(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("ranges", ctypes.c_int32), ("gather_blocks", ctypes.c_int32),
                ("gather_blocks_in_flight", ctypes.c_int32), ("host_bytes_per_gather_block", ctypes.c_int64),
                ("host_bytes_in_flight", ctypes.c_int64)]


class clo_attend_layer(ctypes.Structure):
    _fields_ = [("shape", ctypes.POINTER(clo_shape)), ("layer", ctypes.POINTER(clo_layer)), ("q", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t),
                ("wait_flag", ctypes.c_void_p), ("signal_flag", ctypes.c_void_p)]


_lib = None


def load():
    """Load libclo.so; raise ImportError when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libclo.so is not built ({LIB_PATH}); run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, st = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        P = ctypes.POINTER
        L.clo_workspace_size.restype = sz
        L.clo_workspace_size.argtypes = [P(clo_shape)]
        L.clo_reuse_test.restype = st
        L.clo_reuse_test.argtypes = [P(clo_shape), vp, vp, vp, vp, P(clo_sync), vp]
        L.clo_topk_select.restype = st
        L.clo_topk_select.argtypes = [P(clo_shape), P(clo_layer), vp, vp, vp, sz, P(clo_sync), vp]
        L.clo_reuse_select.restype = st
        L.clo_reuse_select.argtypes = [P(clo_shape), P(clo_layer), vp, vp, vp, vp, vp, sz, P(clo_sync), vp]
        L.clo_gather_kv.restype = st
        L.clo_gather_kv.argtypes = [P(clo_shape), P(clo_layer), vp, vp, sz, P(clo_sync), vp]
        L.clo_sparse_attn.restype = st
        L.clo_sparse_attn.argtypes = [P(clo_shape), P(clo_layer), vp, vp, vp, sz, P(clo_sync), vp]
        L.clo_decode_step.restype = st
        L.clo_decode_step.argtypes = [P(clo_shape), P(clo_layer), vp, vp, vp, vp, vp, vp, sz, P(clo_sync), vp]
        L.clo_decode_step_schedule.restype = st
        L.clo_decode_step_schedule.argtypes = [P(clo_shape), ctypes.c_uint64, ctypes.c_int32, P(clo_step_schedule)]
        L.clo_last_step_gather_ms.restype = st
        L.clo_last_step_gather_ms.argtypes = [P(ctypes.c_float)]
        L.clo_decode_step_static.restype = st
        L.clo_decode_step_static.argtypes = [P(clo_shape), P(clo_layer), vp, vp, vp, vp, vp, P(clo_sync), vp]
        L.clo_append_kv.restype = st
        L.clo_append_kv.argtypes = [P(clo_shape), P(clo_layer), vp, vp, ctypes.c_int64, P(clo_sync), vp]
        L.clo_update_reference.restype = st
        L.clo_update_reference.argtypes = [P(clo_shape), vp, vp, vp, P(clo_sync), vp]
        L.clo_quantize_rows.restype = st
        L.clo_quantize_rows.argtypes = [vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, vp, ctypes.c_int64, vp,
                                        P(clo_sync), vp]
        L.clo_stream_read.restype = st
        L.clo_stream_read.argtypes = [vp, ctypes.c_size_t, ctypes.c_int32, vp, vp]
        L.clo_plan_persistent.restype = st
        L.clo_plan_persistent.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp]
        L.clo_gather_plan_size.restype = sz
        L.clo_gather_plan_size.argtypes = [ctypes.c_int32]
        L.clo_gather_plan.restype = st
        L.clo_gather_plan.argtypes = [P(clo_gather_layer), ctypes.c_int32, vp, sz, P(ctypes.c_int32)]
        L.clo_select_plan_size.restype = sz
        L.clo_select_plan_size.argtypes = [ctypes.c_int32]
        L.clo_select_plan.restype = st
        L.clo_select_plan.argtypes = [P(clo_select_layer), ctypes.c_int32, vp, sz]
        L.clo_select_layers.restype = st
        L.clo_select_layers.argtypes = [P(clo_shape), vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32,
                                        ctypes.c_uint32, vp, ctypes.c_uint32, vp]
        L.clo_attend_plan_size.restype = sz
        L.clo_attend_plan_size.argtypes = [ctypes.c_int32]
        L.clo_attend_plan.restype = st
        L.clo_attend_plan.argtypes = [P(clo_attend_layer), ctypes.c_int32, vp, sz]
        L.clo_attend_layers.restype = st
        L.clo_attend_layers.argtypes = [P(clo_shape), vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32,
                                        ctypes.c_uint32, vp, ctypes.c_uint32, vp]
        L.clo_gather_layers.restype = st
        L.clo_gather_layers.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint32, vp,
                                        ctypes.c_uint32, vp]
        L.clo_status_string.restype = ctypes.c_char_p
        L.clo_status_string.argtypes = [st]
        L.clo_last_error.restype = st
        L.clo_last_error.argtypes = [ctypes.c_char_p, sz]
        _lib = L
    return _lib


def ptr(x) -> Optional[int]:
    """Address of a torch tensor, a pinned HostBuffer, an int, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if hasattr(x, "ptr"):
        return x.ptr
    raise TypeError(f"cannot take the address of {type(x)}")


def nbytes(x, given: Optional[int] = None) -> int:
    """Size of a workspace: `given` when stated, else the tensor's or buffer's size (0 for a raw address)."""
    if given is not None:
        return int(given)
    if x is None or isinstance(x, int):
        return 0
    if hasattr(x, "numel") and hasattr(x, "element_size"):
        return x.numel() * x.element_size()
    return int(getattr(x, "nbytes"))


def stream_handle(stream) -> Optional[int]:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def clo_last_error():
    """(status, message) of the calling thread's last non-OK call."""
    buf = ctypes.create_string_buffer(512)
    st = load().clo_last_error(buf, 512)
    return st, buf.value.decode()


def last_error() -> str:
    return clo_last_error()[1]


def _check(status: int, func: str):
    if status != CLO_OK:
        raise CloError(status, func, last_error() or load().clo_status_string(status).decode())


@dataclass
class Shape:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    context: int
    topk: int
    tau: float
    dtype: int
    head_dim: int = 128
    capacity: int = 0  # rows allocated per (sequence, head); 0 = context
    tau_heads: Optional[Sequence[float]] = None  # per-KV-head thresholds; None = tau for every head
    block_size: int = 0  # selection granularity in tokens (0/1 = single tokens)

    def c(self) -> clo_shape:
        th = None
        if self.tau_heads is not None:
            if len(self.tau_heads) != self.n_kv_heads:
                # the library reads exactly n_kv_heads thresholds from the array
                raise ValueError(f"tau_heads has {len(self.tau_heads)} entries, n_kv_heads is {self.n_kv_heads}")
            th = (ctypes.c_float * len(self.tau_heads))(*[float(x) for x in self.tau_heads])
        cs = clo_shape(self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim, self.context, self.topk,
                       self.tau, self.dtype, self.capacity,
                       ctypes.cast(th, ctypes.POINTER(ctypes.c_float)) if th is not None else None,
                       int(self.block_size))
        cs._tau_heads = th  # keeps the array alive while the struct is in use
        return cs


@dataclass
class Layer:
    persistent_mask: int = 0
    k_hbm: object = None
    v_hbm: object = None
    k_host: object = None
    v_host: object = None
    k_score: object = None
    k_cache: object = None
    v_cache: object = None
    idx: object = None
    host_format: int = 0  # CLO_HOST_NATIVE, CLO_HOST_INT8 or CLO_HOST_INT4
    k_host_exp: object = None
    v_host_exp: object = None

    def c(self) -> clo_layer:
        return clo_layer(self.persistent_mask, ptr(self.k_hbm), ptr(self.v_hbm), ptr(self.k_host), ptr(self.v_host),
                         ptr(self.k_score), ptr(self.k_cache), ptr(self.v_cache), ptr(self.idx), self.host_format,
                         ptr(self.k_host_exp), ptr(self.v_host_exp))


@dataclass
class Sync:
    wait_flag: object = None
    wait_value: int = 0
    signal_flag: object = None
    signal_value: int = 0
    error_word: object = None
    spin_limit: int = 0

    def c(self) -> clo_sync:
        return clo_sync(ptr(self.wait_flag), self.wait_value, ptr(self.signal_flag), self.signal_value,
                        ptr(self.error_word), self.spin_limit)


def _sync(s: Optional[Sync]):
    return ctypes.byref(s.c()) if s is not None else None


def clo_workspace_size(shape: Shape) -> int:
    return int(load().clo_workspace_size(ctypes.byref(shape.c())))


def clo_reuse_test(shape: Shape, q, q_prev, reuse, cos=None, sync: Optional[Sync] = None, stream=None):
    _check(load().clo_reuse_test(ctypes.byref(shape.c()), ptr(q), ptr(q_prev), ptr(reuse), ptr(cos), _sync(sync),
                                 stream_handle(stream)), "clo_reuse_test")


def clo_topk_select(shape: Shape, layer: Layer, q, reuse, ws, sync: Optional[Sync] = None, stream=None,
                    ws_bytes: Optional[int] = None):
    _check(load().clo_topk_select(ctypes.byref(shape.c()), ctypes.byref(layer.c()), ptr(q), ptr(reuse), ptr(ws),
                                  nbytes(ws, ws_bytes), _sync(sync), stream_handle(stream)), "clo_topk_select")


def clo_reuse_select(shape: Shape, layer: Layer, q, q_prev, reuse, cos, ws, sync: Optional[Sync] = None,
                     stream=None, ws_bytes: Optional[int] = None):
    _check(load().clo_reuse_select(ctypes.byref(shape.c()), ctypes.byref(layer.c()), ptr(q), ptr(q_prev), ptr(reuse),
                                   ptr(cos), ptr(ws), nbytes(ws, ws_bytes), _sync(sync), stream_handle(stream)),
           "clo_reuse_select")


def clo_gather_kv(shape: Shape, layer: Layer, reuse, ws, sync: Optional[Sync] = None, stream=None,
                  ws_bytes: Optional[int] = None):
    _check(load().clo_gather_kv(ctypes.byref(shape.c()), ctypes.byref(layer.c()), ptr(reuse), ptr(ws),
                                nbytes(ws, ws_bytes), _sync(sync), stream_handle(stream)), "clo_gather_kv")


def clo_sparse_attn(shape: Shape, layer: Layer, q, out, ws, sync: Optional[Sync] = None, stream=None,
                    ws_bytes: Optional[int] = None):
    _check(load().clo_sparse_attn(ctypes.byref(shape.c()), ctypes.byref(layer.c()), ptr(q), ptr(out), ptr(ws),
                                  nbytes(ws, ws_bytes), _sync(sync), stream_handle(stream)),
           "clo_sparse_attn")


def clo_decode_step_schedule(shape: Shape, persistent_mask: int = 0, host_format: int = CLO_HOST_NATIVE) -> dict:
    """How clo_decode_step runs a layer of this shape (host-only)."""
    out = clo_step_schedule()
    _check(load().clo_decode_step_schedule(ctypes.byref(shape.c()), int(persistent_mask), int(host_format),
                                           ctypes.byref(out)), "clo_decode_step_schedule")
    return {"mode": STEP_MODES[out.mode], "ranges": out.ranges, "gather_blocks": out.gather_blocks,
            "gather_blocks_in_flight": out.gather_blocks_in_flight,
            "host_bytes_per_gather_block": out.host_bytes_per_gather_block,
            "host_bytes_in_flight": out.host_bytes_in_flight}


def clo_last_step_gather_ms() -> float:
    """GPU ms of the gather inside the last overlapped clo_decode_step on this device."""
    v = ctypes.c_float()
    _check(load().clo_last_step_gather_ms(ctypes.byref(v)), "clo_last_step_gather_ms")
    return float(v.value)


def clo_decode_step(shape: Shape, layer: Layer, q, q_prev, out, reuse, cos, ws, sync: Optional[Sync] = None,
                    stream=None, ws_bytes: Optional[int] = None):
    _check(load().clo_decode_step(ctypes.byref(shape.c()), ctypes.byref(layer.c()), ptr(q), ptr(q_prev), ptr(out),
                                  ptr(reuse), ptr(cos), ptr(ws), nbytes(ws, ws_bytes), _sync(sync),
                                  stream_handle(stream)), "clo_decode_step")


def clo_decode_step_static(shape: Shape, layer: Layer, q, q_prev, out, reuse, cos, sync: Optional[Sync] = None,
                           stream=None):
    _check(load().clo_decode_step_static(ctypes.byref(shape.c()), ctypes.byref(layer.c()), ptr(q), ptr(q_prev),
                                         ptr(out), ptr(reuse), ptr(cos), _sync(sync), stream_handle(stream)),
           "clo_decode_step_static")


CLO_STATIC_SCRATCH_BYTES = 32 << 20


def clo_gather_plan_size(n_layers: int) -> int:
    return int(load().clo_gather_plan_size(int(n_layers)))


def clo_gather_plan(items, plan, plan_bytes: Optional[int] = None) -> int:
    """items: (shape, layer, reuse, ws, wait_flag, signal_flag) per layer, in gather order.
    Writes the plan (device memory) and returns the grid size for clo_gather_layers."""
    n = len(items)
    arr = (clo_gather_layer * max(n, 1))()
    keep = []
    for i, (shape, layer, reuse, ws, wait_flag, signal_flag) in enumerate(items):
        cs, cl = shape.c(), layer.c()
        keep += [cs, cl]
        arr[i] = clo_gather_layer(ctypes.pointer(cs), ctypes.pointer(cl), ptr(reuse), ptr(ws), nbytes(ws),
                                  ptr(wait_flag), ptr(signal_flag))
    blocks = ctypes.c_int32(0)
    _check(load().clo_gather_plan(arr, n, ptr(plan), nbytes(plan, plan_bytes), ctypes.byref(blocks)),
           "clo_gather_plan")
    return int(blocks.value)


def clo_gather_layers(plan, n_layers: int, blocks: int, wait_value: int, signal_value: int, error_word=None,
                      spin_limit: int = 0, stream=None):
    _check(load().clo_gather_layers(ptr(plan), int(n_layers), int(blocks), int(wait_value), int(signal_value),
                                    ptr(error_word), int(spin_limit), stream_handle(stream)), "clo_gather_layers")


def clo_select_plan_size(n_layers: int) -> int:
    return int(load().clo_select_plan_size(int(n_layers)))


def clo_select_plan(items, plan, plan_bytes: Optional[int] = None):
    """items: (shape, layer, q, q_prev, reuse, cos, ws, wait_flag, signal_flag) per layer.
    Writes the plan (device memory)."""
    n = len(items)
    arr = (clo_select_layer * max(n, 1))()
    keep = []
    for i, (shape, layer, q, q_prev, reuse, cos, ws, wait_flag, signal_flag) in enumerate(items):
        cs, cl = shape.c(), layer.c()
        keep += [cs, cl]
        arr[i] = clo_select_layer(ctypes.pointer(cs), ctypes.pointer(cl), ptr(q), ptr(q_prev), ptr(reuse), ptr(cos),
                                  ptr(ws), nbytes(ws), ptr(wait_flag), ptr(signal_flag))
    _check(load().clo_select_plan(arr, n, ptr(plan), nbytes(plan, plan_bytes)), "clo_select_plan")


def clo_select_layers(shape: Shape, plan, first: int, count: int, wait_value: int, signal_value: int,
                      error_word=None, spin_limit: int = 0, stream=None):
    _check(load().clo_select_layers(ctypes.byref(shape.c()), ptr(plan), int(first), int(count), int(wait_value),
                                    int(signal_value), ptr(error_word), int(spin_limit), stream_handle(stream)),
           "clo_select_layers")


def clo_attend_plan_size(n_layers: int) -> int:
    return int(load().clo_attend_plan_size(int(n_layers)))


def clo_attend_plan(items, plan, plan_bytes: Optional[int] = None):
    """items: (shape, layer, q, out, ws, wait_flag, signal_flag) per layer.
    Writes the plan (device memory)."""
    n = len(items)
    arr = (clo_attend_layer * max(n, 1))()
    keep = []
    for i, (shape, layer, q, out, ws, wait_flag, signal_flag) in enumerate(items):
        cs, cl = shape.c(), layer.c()
        keep += [cs, cl]
        arr[i] = clo_attend_layer(ctypes.pointer(cs), ctypes.pointer(cl), ptr(q), ptr(out), ptr(ws), nbytes(ws),
                                  ptr(wait_flag), ptr(signal_flag))
    _check(load().clo_attend_plan(arr, n, ptr(plan), nbytes(plan, plan_bytes)), "clo_attend_plan")


def clo_attend_layers(shape: Shape, plan, first: int, count: int, wait_value: int, signal_value: int,
                      error_word=None, spin_limit: int = 0, stream=None):
    _check(load().clo_attend_layers(ctypes.byref(shape.c()), ptr(plan), int(first), int(count), int(wait_value),
                                    int(signal_value), ptr(error_word), int(spin_limit), stream_handle(stream)),
           "clo_attend_layers")


def clo_append_kv(shape: Shape, layer: Layer, k_new, v_new, position: int, sync: Optional[Sync] = None,
                  stream=None):
    _check(load().clo_append_kv(ctypes.byref(shape.c()), ctypes.byref(layer.c()), ptr(k_new), ptr(v_new),
                                int(position), _sync(sync), stream_handle(stream)), "clo_append_kv")


def clo_update_reference(shape: Shape, q, reuse, q_ref, sync: Optional[Sync] = None, stream=None):
    _check(load().clo_update_reference(ctypes.byref(shape.c()), ptr(q), ptr(reuse), ptr(q_ref), _sync(sync),
                                       stream_handle(stream)), "clo_update_reference")


def clo_quantize_rows(src, n_rows: int, dtype: int, dst, dst_exp, dst_stride: int = 128,
                      host_format: int = CLO_HOST_INT8, sync: Optional[Sync] = None, stream=None):
    _check(load().clo_quantize_rows(ptr(src), int(n_rows), int(dtype), int(host_format), ptr(dst), int(dst_stride),
                                    ptr(dst_exp), _sync(sync), stream_handle(stream)), "clo_quantize_rows")


def clo_stream_read(src, nbytes_: int, blocks: int, sink, stream=None):
    """Measurement helper: stream-read nbytes_ of device memory (HBM read ceiling)."""
    _check(load().clo_stream_read(ptr(src), int(nbytes_), int(blocks), ptr(sink), stream_handle(stream)),
           "clo_stream_read")


def clo_plan_persistent(s_hat, n_persist: int):
    """Persistent-head masks from per-(layer, KV head) mean similarities s_hat [L, Hkv] (host)."""
    import numpy as np

    a = np.ascontiguousarray(np.asarray(s_hat, dtype=np.float32))
    L, H = a.shape
    masks = (ctypes.c_uint64 * max(L, 1))()
    _check(load().clo_plan_persistent(a.ctypes.data, L, H, int(n_persist), ctypes.cast(masks, ctypes.c_void_p)),
           "clo_plan_persistent")
    return [int(masks[i]) for i in range(L)]


def clo_status_string(status: int) -> str:
    return load().clo_status_string(status).decode()

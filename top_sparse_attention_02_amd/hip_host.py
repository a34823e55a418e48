"""Pinned host memory and raw HIP copies through the HIP runtime (ctypes).

Plumbing for callers of the library: the non-persistent heads' full K/V live
in pinned host memory that the GPU reads directly (zero-copy).  torch supplies
device memory and streams; this module supplies pinned host buffers with an
explicit coherence flag and bulk copies.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_hip = None

hipHostMallocDefault = 0x0
hipHostMallocPortable = 0x1
hipHostMallocMapped = 0x2
hipHostMallocNumaUser = 0x20000000
hipHostMallocCoherent = 0x40000000
hipHostMallocNonCoherent = 0x80000000

hipMallocSignalMemory = 0x2  # hipExtMallocWithFlags: memory hipStreamWaitValue32 can wait on
hipStreamWaitValueGte = 0x0
hipDeviceAttributeCanUseStreamWaitValue = 10013

hipMemcpyHostToDevice = 1
hipMemcpyDeviceToHost = 2
hipMemcpyDefault = 4


def hip():
    global _hip
    if _hip is None:
        for name in ("libamdhip64.so", "/opt/rocm/lib/libamdhip64.so"):
            try:
                _hip = ctypes.CDLL(name)
                break
            except OSError:
                continue
        if _hip is None:
            raise ImportError("libamdhip64.so (HIP runtime) not found")
        vp, sz, u = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint
        _hip.hipHostMalloc.argtypes = [ctypes.POINTER(vp), sz, u]
        _hip.hipHostFree.argtypes = [vp]
        _hip.hipMemcpy.argtypes = [vp, vp, sz, ctypes.c_int]
        _hip.hipMemcpyAsync.argtypes = [vp, vp, sz, ctypes.c_int, vp]
        _hip.hipGetErrorString.restype = ctypes.c_char_p
        _hip.hipGetErrorString.argtypes = [ctypes.c_int]
        _hip.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(vp), vp, u]
        _hip.hipExtMallocWithFlags.argtypes = [ctypes.POINTER(vp), sz, u]
        _hip.hipStreamWriteValue32.argtypes = [vp, vp, ctypes.c_uint32, u]
        _hip.hipStreamWaitValue32.argtypes = [vp, vp, ctypes.c_uint32, u, ctypes.c_uint32]
        _hip.hipDeviceGetAttribute.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int, ctypes.c_int]
    return _hip


def check(err: int, what: str):
    if err != 0:
        msg = hip().hipGetErrorString(err).decode()
        raise RuntimeError(f"{what}: HIP error {err} ({msg})")


class HostBuffer:
    """Pinned, device-mapped host memory of `nbytes` bytes (freed on close/GC)."""

    def __init__(self, nbytes: int, flags: int = hipHostMallocMapped):
        self.nbytes = int(nbytes)
        self.flags = flags
        p = ctypes.c_void_p()
        check(hip().hipHostMalloc(ctypes.byref(p), max(self.nbytes, 1), flags), f"hipHostMalloc({nbytes})")
        self.ptr = p.value

    def device_ptr(self) -> int:
        d = ctypes.c_void_p()
        check(hip().hipHostGetDevicePointer(ctypes.byref(d), self.ptr, 0), "hipHostGetDevicePointer")
        return d.value

    def numpy(self, dtype, shape=None, offset: int = 0) -> np.ndarray:
        dtype = np.dtype(dtype)
        count = (self.nbytes - offset) // dtype.itemsize if shape is None else int(np.prod(shape))
        raw = (ctypes.c_char * (count * dtype.itemsize)).from_address(self.ptr + offset)
        a = np.frombuffer(raw, dtype=dtype, count=count)
        return a if shape is None else a.reshape(shape)

    def close(self):
        if getattr(self, "ptr", None):
            check(hip().hipHostFree(self.ptr), "hipHostFree")
            self.ptr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def copy_h2d(dst_dev_ptr: int, src_host_ptr: int, nbytes: int):
    check(hip().hipMemcpy(dst_dev_ptr, src_host_ptr, nbytes, hipMemcpyHostToDevice), "hipMemcpy H2D")


def copy_d2h(dst_host_ptr: int, src_dev_ptr: int, nbytes: int):
    check(hip().hipMemcpy(dst_host_ptr, src_dev_ptr, nbytes, hipMemcpyDeviceToHost), "hipMemcpy D2H")


def copy_async(dst: int, src: int, nbytes: int, stream_handle: int):
    check(hip().hipMemcpyAsync(dst, src, nbytes, hipMemcpyDefault, stream_handle), "hipMemcpyAsync")


# ---------------------------------------------------------------- stream memory operations
# Signal-memory words are never freed: they stay allocated until the process ends.
_signal_words = []


def can_wait_value(device: int = 0) -> bool:
    """Whether the device supports hipStreamWaitValue32."""
    v = ctypes.c_int(0)
    check(hip().hipDeviceGetAttribute(ctypes.byref(v), hipDeviceAttributeCanUseStreamWaitValue, device),
          "hipDeviceGetAttribute")
    return bool(v.value)


def signal_word() -> int:
    """Address of an 8-byte word of signal memory (hipExtMallocWithFlags with
    hipMallocSignalMemory), the memory hipStreamWaitValue32 waits on; kept until
    the process ends."""
    p = ctypes.c_void_p()
    check(hip().hipExtMallocWithFlags(ctypes.byref(p), 8, hipMallocSignalMemory), "hipExtMallocWithFlags(signal)")
    _signal_words.append(p.value)
    return p.value


def stream_write_value32(stream_handle: int, ptr: int, value: int):
    """After the stream's earlier work, the command processor writes `value` to *ptr."""
    check(hip().hipStreamWriteValue32(stream_handle, ptr, value, 0), "hipStreamWriteValue32")


def stream_wait_value32(stream_handle: int, ptr: int, value: int):
    """The stream's later work waits until *ptr >= value (signal memory)."""
    check(hip().hipStreamWaitValue32(stream_handle, ptr, value, hipStreamWaitValueGte, 0xFFFFFFFF),
          "hipStreamWaitValue32")

"""Minimal HIP runtime access through ctypes: device memory, copies, streams, events
and stream capture into graphs. Plumbing for callers that do not want PyTorch in
the process (the benchmark: PyTorch ships its own HIP runtime, and the library then
runs on that copy instead of the system one it was built against).
No compute happens here.
"""

from __future__ import annotations

import ctypes
from typing import Callable

import numpy as np

_vp = ctypes.c_void_p
_H2D, _D2H, _D2D = 1, 2, 3


class HipError(RuntimeError):
    pass


_UNIT = 2 << 20  # 2 MiB
_CONTIGUOUS = 0x4  # hipDeviceMallocContiguous


class Hip:
    def __init__(self, path: str = "libamdhip64.so.7"):
        self.lib = ctypes.CDLL(path)
        L = self.lib
        sig = {
            "hipMalloc": [ctypes.POINTER(_vp), ctypes.c_size_t],
            "hipExtMallocWithFlags": [ctypes.POINTER(_vp), ctypes.c_size_t, ctypes.c_uint],
            "hipFree": [_vp],
            "hipMemcpy": [_vp, _vp, ctypes.c_size_t, ctypes.c_int],
            "hipMemset": [_vp, ctypes.c_int, ctypes.c_size_t],
            "hipMemcpyAsync": [_vp, _vp, ctypes.c_size_t, ctypes.c_int, _vp],
            "hipDeviceSynchronize": [],
            "hipStreamCreate": [ctypes.POINTER(_vp)],
            "hipStreamSynchronize": [_vp],
            "hipEventCreate": [ctypes.POINTER(_vp)],
            "hipEventCreateWithFlags": [ctypes.POINTER(_vp), ctypes.c_uint],
            "hipEventRecord": [_vp, _vp],
            "hipEventRecordWithFlags": [_vp, _vp, ctypes.c_uint],
            "hipEventSynchronize": [_vp],
            "hipEventElapsedTime": [ctypes.POINTER(ctypes.c_float), _vp, _vp],
            "hipStreamBeginCapture": [_vp, ctypes.c_int],
            "hipStreamEndCapture": [_vp, ctypes.POINTER(_vp)],
            "hipGraphInstantiate": [ctypes.POINTER(_vp), _vp, _vp, _vp, ctypes.c_size_t],
            "hipGraphLaunch": [_vp, _vp],
            "hipGetErrorString": [ctypes.c_int],
            "hipGetLastError": [],
            "hipGetDeviceCount": [ctypes.POINTER(ctypes.c_int)],
            "hipHostMalloc": [ctypes.POINTER(_vp), ctypes.c_size_t, ctypes.c_uint],
            "hipHostFree": [_vp],
            "hipStreamWaitEvent": [_vp, _vp, ctypes.c_uint],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_char_p if name == "hipGetErrorString" else ctypes.c_int
        self._graphs = []

    def check(self, rc: int, what: str) -> None:
        if rc != 0:
            self.lib.hipGetLastError()  # the failure is reported here; do not leave it for the next caller
            raise HipError(f"{what}: {self.lib.hipGetErrorString(rc).decode()}")

    def device_count(self) -> int:
        n = ctypes.c_int(0)
        rc = self.lib.hipGetDeviceCount(ctypes.byref(n))
        return n.value if rc == 0 else 0

    # memory
    def malloc(self, nbytes: int, contiguous: bool = False) -> int:
        """Device memory from hipMalloc, or with `contiguous` physically contiguous in whole 2 MiB
        units where the driver can provide them (hipDeviceMallocContiguous; hipMalloc otherwise).
        Measured on the split attention's workspace, whose partial results are written and read
        back within one call: 1 x 32K calls at ~9.2 us from contiguous units, 9.6 or 10.7 us from
        scattered pages depending on where they land. The full-cache scan's logits go the other
        way (8 x 16K..64K ragged: 73 us written to scattered pages, 84 us to contiguous units)."""
        n = max(int(nbytes), 256)
        p = _vp()
        if contiguous:
            if self.lib.hipExtMallocWithFlags(ctypes.byref(p), (n + _UNIT - 1) // _UNIT * _UNIT, _CONTIGUOUS) == 0:
                return p.value
            self.lib.hipGetLastError()  # the refused contiguous request is not an error of the next call
        self.check(self.lib.hipMalloc(ctypes.byref(p), n), "hipMalloc")
        return p.value

    def memset(self, ptr: int, value: int, nbytes: int) -> None:
        self.check(self.lib.hipMemset(ptr, value, nbytes), "hipMemset")

    def free(self, ptr: int) -> None:
        self.check(self.lib.hipFree(ptr), "hipFree")

    def to_device(self, dst: int, a: np.ndarray) -> None:
        a = np.ascontiguousarray(a)
        self.check(self.lib.hipMemcpy(dst, a.ctypes.data, a.nbytes, _H2D), "hipMemcpy H2D")

    def to_host(self, a: np.ndarray, src: int) -> np.ndarray:
        self.check(self.lib.hipMemcpy(a.ctypes.data, src, a.nbytes, _D2H), "hipMemcpy D2H")
        return a

    def copy(self, dst: int, src: int, nbytes: int) -> None:
        self.check(self.lib.hipMemcpy(dst, src, nbytes, _D2D), "hipMemcpy D2D")

    def host_malloc(self, nbytes: int) -> int:
        """Pinned host memory (hipHostMalloc, default flags: mapped into the device's address space)."""
        p = _vp()
        self.check(self.lib.hipHostMalloc(ctypes.byref(p), max(int(nbytes), 256), 0), "hipHostMalloc")
        return p.value

    def wait(self, stream: int, event: int) -> None:
        """`stream` waits for the work recorded in `event`."""
        self.check(self.lib.hipStreamWaitEvent(stream, event, 0), "hipStreamWaitEvent")

    # streams and events
    def stream(self) -> int:
        s = _vp()
        self.check(self.lib.hipStreamCreate(ctypes.byref(s)), "hipStreamCreate")
        return s.value

    def sync(self, stream: int | None = None) -> None:
        if stream is None:
            self.check(self.lib.hipDeviceSynchronize(), "hipDeviceSynchronize")
        else:
            self.check(self.lib.hipStreamSynchronize(stream), "hipStreamSynchronize")

    def event(self, light: bool = False) -> int:
        """A timing event; `light` ones skip the system-scope cache release on record
        (hipEventDisableSystemFence), so bracketing a kernel adds little to it."""
        e = _vp()
        if light:
            self.check(self.lib.hipEventCreateWithFlags(ctypes.byref(e), 0x20000000), "hipEventCreateWithFlags")
        else:
            self.check(self.lib.hipEventCreate(ctypes.byref(e)), "hipEventCreate")
        return e.value

    def record(self, event: int, stream: int, external: bool = False) -> None:
        """Record `event` on `stream`; `external` makes it an event node of a graph being captured."""
        if external:
            self.check(self.lib.hipEventRecordWithFlags(event, stream, 1), "hipEventRecordWithFlags")
        else:
            self.check(self.lib.hipEventRecord(event, stream), "hipEventRecord")

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        self.check(self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b), "hipEventElapsedTime")
        return ms.value

    # graphs
    def capture(self, stream: int, fn: Callable[[], None]) -> int:
        """Capture everything `fn` enqueues on `stream` into an instantiated graph."""
        self.check(self.lib.hipStreamBeginCapture(stream, 0), "hipStreamBeginCapture")
        try:
            fn()
        finally:
            g = _vp()
            rc = self.lib.hipStreamEndCapture(stream, ctypes.byref(g))
        self.check(rc, "hipStreamEndCapture")
        ge = _vp()
        self.check(self.lib.hipGraphInstantiate(ctypes.byref(ge), g, None, None, 0), "hipGraphInstantiate")
        self._graphs.append(g)
        return ge.value

    def launch(self, graph_exec: int, stream: int) -> None:
        self.check(self.lib.hipGraphLaunch(graph_exec, stream), "hipGraphLaunch")


class HostArray:
    """Pinned host memory with a shape and dtype, viewable as a numpy array."""

    def __init__(self, hip: Hip, shape, dtype):
        self.hip = hip
        self.shape = tuple(int(x) for x in shape)
        self.dtype = np.dtype(dtype)
        self.nbytes = int(np.prod(self.shape, dtype=np.int64)) * self.dtype.itemsize
        self.ptr = hip.host_malloc(self.nbytes)

    def data_ptr(self) -> int:
        return self.ptr

    def numpy(self) -> np.ndarray:
        buf = (ctypes.c_char * self.nbytes).from_address(self.ptr)
        return np.frombuffer(buf, dtype=self.dtype).reshape(self.shape)


class DevArray:
    """A device allocation with a shape and a host dtype (for copies back)."""

    def __init__(self, hip: Hip, shape, dtype, zero: bool = False, contiguous: bool = False):
        self.hip = hip
        self.shape = tuple(int(x) for x in shape)
        self.dtype = np.dtype(dtype)
        self.nbytes = int(np.prod(self.shape, dtype=np.int64)) * self.dtype.itemsize
        self.ptr = hip.malloc(self.nbytes, contiguous)
        if zero:
            hip.memset(self.ptr, 0, self.nbytes)

    @classmethod
    def from_host(cls, hip: Hip, a: np.ndarray) -> "DevArray":
        d = cls(hip, a.shape, a.dtype)
        hip.to_device(d.ptr, a)
        return d

    def data_ptr(self) -> int:
        return self.ptr

    def offset(self, index: int) -> int:
        """Address of sub-array `index` along the first axis."""
        return self.ptr + index * (self.nbytes // self.shape[0])

    def numpy(self) -> np.ndarray:
        return self.hip.to_host(np.empty(self.shape, self.dtype), self.ptr)

    def clone(self) -> "DevArray":
        d = DevArray(self.hip, self.shape, self.dtype)
        self.hip.copy(d.ptr, self.ptr, self.nbytes)
        return d


class DevView:
    """Bytes [offset, offset + nbytes) of a device allocation, which it keeps alive."""

    def __init__(self, parent: DevArray, offset: int, nbytes: int):
        if offset < 0 or nbytes < 0 or offset + nbytes > parent.nbytes:
            raise ValueError(f"view [{offset}, {offset + nbytes}) outside a {parent.nbytes}-byte allocation")
        self.parent, self.offset, self.nbytes = parent, int(offset), int(nbytes)
        self.ptr = parent.ptr + self.offset

    def data_ptr(self) -> int:
        return self.ptr


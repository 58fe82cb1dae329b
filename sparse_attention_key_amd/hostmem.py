"""Page-locked host memory mapped into the GPU address space, for an index
that lives in host memory and is read by the scan over the host link (the
offloaded setting the method targets).  Plumbing over the HIP runtime; the
scan kernels themselves only see a device address.
"""
from __future__ import annotations

import ctypes

class PinnedHost:
    """hipHostMalloc'd page-locked host memory mapped into the device address
    space (the host-resident index of the scan)."""

    MAPPED, COHERENT, NONCOHERENT = 0x2, 0x40000000, 0x80000000

    def __init__(self, nbytes: int, coherent: bool = False):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipHostMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t, ctypes.c_uint]
        self.hip.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_uint]
        self.hip.hipHostFree.argtypes = [ctypes.c_void_p]
        self.hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
        h = ctypes.c_void_p()
        flags = self.MAPPED | (self.COHERENT if coherent else self.NONCOHERENT)
        rc = self.hip.hipHostMalloc(ctypes.byref(h), nbytes, flags)
        if rc != 0:
            raise RuntimeError(f"hipHostMalloc({nbytes}) failed: {rc}")
        d = ctypes.c_void_p()
        rc = self.hip.hipHostGetDevicePointer(ctypes.byref(d), h, 0)
        if rc != 0:
            raise RuntimeError(f"hipHostGetDevicePointer failed: {rc}")
        self.host, self.dev, self.nbytes = h.value, d.value, nbytes

    def copy_from_device(self, offset: int, src_ptr: int, nbytes: int, stream):
        rc = self.hip.hipMemcpyAsync(self.host + offset, src_ptr, nbytes, 2, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"hipMemcpyAsync D2H failed: {rc}")

    def copy_to_device(self, dst_ptr: int, offset: int, nbytes: int, stream):
        rc = self.hip.hipMemcpyAsync(dst_ptr, self.host + offset, nbytes, 1, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"hipMemcpyAsync H2D failed: {rc}")

    def free(self):
        if self.host:
            self.hip.hipHostFree(self.host)
            self.host = None



    def __del__(self):
        try:
            self.free()
        except Exception:
            pass

"""ctypes binding of libdsa_roofline.so (include/dsa_roofline.h): the
benchmark's ceiling probes -- streaming HBM read and copy, a BF16 MFMA loop
and random 256-byte row gathers -- measured on the GPU that runs the path.
Argument marshalling only."""
import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa_roofline.so")
EXPORTS = ("dsa_roofline_read", "dsa_roofline_write", "dsa_roofline_copy", "dsa_roofline_mfma",
           "dsa_roofline_mfma_flops", "dsa_roofline_gather", "dsa_roofline_kv_gather",
           "dsa_roofline_floor")


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.dsa_roofline_read.restype = i32
    lib.dsa_roofline_read.argtypes = [vp, sz, vp, vp]
    lib.dsa_roofline_write.restype = i32
    lib.dsa_roofline_write.argtypes = [vp, sz, vp]
    lib.dsa_roofline_copy.restype = i32
    lib.dsa_roofline_copy.argtypes = [vp, vp, sz, vp]
    lib.dsa_roofline_mfma.restype = i32
    lib.dsa_roofline_mfma.argtypes = [vp, i32, i32, vp]
    lib.dsa_roofline_mfma_flops.restype = ctypes.c_double
    lib.dsa_roofline_mfma_flops.argtypes = [i32, i32]
    lib.dsa_roofline_gather.restype = i32
    lib.dsa_roofline_gather.argtypes = [vp, sz, vp, i32, vp, vp]
    lib.dsa_roofline_kv_gather.restype = i32
    lib.dsa_roofline_kv_gather.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp]
    lib.dsa_roofline_floor.restype = i32
    lib.dsa_roofline_floor.argtypes = [vp, vp, i32, i32, vp]
    return lib


LIB = _load()


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ok(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with status {rc}")


def read(src, sink):
    _ok(LIB.dsa_roofline_read(src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(),
                              _stream()), "dsa_roofline_read")


def write(dst):
    _ok(LIB.dsa_roofline_write(dst.data_ptr(), dst.numel() * dst.element_size(), _stream()),
        "dsa_roofline_write")


def copy(src, dst):
    _ok(LIB.dsa_roofline_copy(src.data_ptr(), dst.data_ptr(), src.numel() * src.element_size(),
                              _stream()), "dsa_roofline_copy")


def mfma(sink, workgroups, iters):
    _ok(LIB.dsa_roofline_mfma(sink.data_ptr(), workgroups, iters, _stream()), "dsa_roofline_mfma")
    return LIB.dsa_roofline_mfma_flops(workgroups, iters)


def gather(buf, rows, sink):
    _ok(LIB.dsa_roofline_gather(buf.data_ptr(), buf.numel() * buf.element_size(), rows.data_ptr(),
                                rows.numel(), sink.data_ptr(), _stream()), "dsa_roofline_gather")


def floor(word, sink, workgroups, threads):
    _ok(LIB.dsa_roofline_floor(word.data_ptr(), sink.data_ptr(), workgroups, threads, _stream()),
        "dsa_roofline_floor")


def kv_gather(k_cache, v_cache, indices, S, sink, wave_rows=False):
    B, L, H_kv, D = k_cache.shape
    rows, k = indices.shape[0] * indices.shape[1], indices.shape[-1]
    _ok(LIB.dsa_roofline_kv_gather(k_cache.data_ptr(), v_cache.data_ptr(), indices.data_ptr(), rows,
                                   k, S, H_kv, L, int(bool(wave_rows)), sink.data_ptr(),
                                   _stream()),
        "dsa_roofline_kv_gather")

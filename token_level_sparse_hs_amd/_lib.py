"""ctypes binding of libhysparse (argument marshalling only).

Every step of the computation runs in the HIP library; this module turns
torch tensors into device pointers, sizes and allocates the workspace with
torch (device memory is PyTorch's job here) and passes the current HIP stream.
It fails loudly when the library is missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int32, c_int64, c_size_t, c_uint32, c_void_p, POINTER

import torch

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libhysparse.so")

HS_OK, HS_ERR_INVALID_ARG, HS_ERR_UNSUPPORTED, HS_ERR_WORKSPACE, HS_ERR_HIP, HS_ERR_INTERNAL = range(6)
HS_OP_FULL_ATTN_SELECT, HS_OP_SPARSE_ATTN_REUSE, HS_OP_DECODE_STEP = range(3)
HS_FLAG_EXACT_RESCAN = 1
HS_FLAG_PROB_SCORE = 2
HS_FLAG_FP8_KV = 4
HS_FLAG_BLOCK_SELECT = 8
HS_FLAG_HEAD_UNION = 16

EXPORTED = ("hs_workspace_size", "hs_full_attn_select", "hs_sparse_attn_reuse", "hs_decode_step",
            "hs_kv_fp8_size", "hs_kv_fp8_convert", "hs_select_diagnostics", "hs_gather_probe", "hs_kv_bridge", "hs_decode_step_noalloc",
            "hs_timing_enable", "hs_timing_read", "hs_status_string", "hs_last_error", "hs_version")


class HsShape(ctypes.Structure):
    _fields_ = [
        ("batch", c_int32), ("n_q", c_int32), ("n_kv", c_int32), ("kv_capacity", c_int32),
        ("q_heads", c_int32), ("kv_heads", c_int32), ("head_dim", c_int32),
        ("top_k", c_int32), ("window", c_int32), ("scale", c_float),
        ("kv_stride_b", c_int64), ("kv_stride_h", c_int64), ("kv_stride_t", c_int64), ("kv_v_offset", c_int64),
        ("flags", c_uint32), ("reserved", c_uint32),
    ]


class HsKernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", c_int64), ("total_ms", ctypes.c_double)]


class HsError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libhysparse status {status}: {msg}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Loads libhysparse.so from the package directory (raises if absent)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m token_level_sparse_hs_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.hs_workspace_size.argtypes = [c_int32, POINTER(HsShape), c_int32, POINTER(c_size_t)]
    lib.hs_workspace_size.restype = c_int32
    lib.hs_full_attn_select.argtypes = [POINTER(HsShape), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                        c_void_p, c_size_t, c_void_p]
    lib.hs_full_attn_select.restype = c_int32
    lib.hs_sparse_attn_reuse.argtypes = [POINTER(HsShape), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_size_t, c_void_p]
    lib.hs_sparse_attn_reuse.restype = c_int32
    lib.hs_decode_step.argtypes = [POINTER(HsShape), c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                   c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.hs_decode_step.restype = c_int32
    lib.hs_decode_step_noalloc.argtypes = [POINTER(HsShape), c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                           c_void_p, c_void_p, c_void_p, c_void_p]
    lib.hs_decode_step_noalloc.restype = c_int32
    lib.hs_kv_fp8_size.argtypes = [POINTER(HsShape), POINTER(c_size_t)]
    lib.hs_kv_fp8_size.restype = c_int32
    lib.hs_kv_fp8_convert.argtypes = [POINTER(HsShape), c_void_p, c_void_p, c_void_p, c_void_p]
    lib.hs_kv_fp8_convert.restype = c_int32
    lib.hs_select_diagnostics.argtypes = [POINTER(HsShape), POINTER(c_size_t), POINTER(c_size_t), POINTER(c_size_t)]
    lib.hs_select_diagnostics.restype = c_int32
    lib.hs_kv_bridge.argtypes = [POINTER(HsShape), c_void_p, c_int32, c_void_p, c_void_p, c_void_p]
    lib.hs_kv_bridge.restype = c_int32
    lib.hs_gather_probe.argtypes = [c_void_p, c_int64, c_void_p, c_int64, c_int32, c_void_p, c_void_p]
    lib.hs_gather_probe.restype = c_int32
    lib.hs_status_string.argtypes = [c_int32]
    lib.hs_status_string.restype = ctypes.c_char_p
    lib.hs_last_error.argtypes = []
    lib.hs_last_error.restype = ctypes.c_char_p
    lib.hs_version.argtypes = []
    lib.hs_version.restype = c_int32
    lib.hs_timing_enable.argtypes = [c_int32]
    lib.hs_timing_enable.restype = c_int32
    lib.hs_timing_read.argtypes = [POINTER(HsKernelTime), c_int32, POINTER(c_int32)]
    lib.hs_timing_read.restype = c_int32
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != HS_OK:
        lib = load()
        raise HsError(status, f"{lib.hs_status_string(status).decode()}: {lib.hs_last_error().decode()}")


def ptr(t):
    return None if t is None else c_void_p(t.data_ptr())


def stream_handle(device) -> c_void_p:
    return c_void_p(torch.cuda.current_stream(device).cuda_stream)


def workspace_size(op: int, shape: HsShape, max_seq_len: int = 0) -> int:
    n = c_size_t(0)
    check(load().hs_workspace_size(op, ctypes.byref(shape), max_seq_len, ctypes.byref(n)))
    return n.value


def alloc_workspace(nbytes: int, device) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + nbytes]


def timing_enable(on: bool) -> None:
    check(load().hs_timing_enable(1 if on else 0))


def timing_read() -> dict:
    """{kernel name: (launches, total_ms)} since the last read (waits for the events)."""
    arr = (HsKernelTime * 64)()
    n = c_int32(0)
    check(load().hs_timing_read(arr, 64, ctypes.byref(n)))
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(min(n.value, 64))}

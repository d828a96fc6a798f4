"""ctypes view of the FwPKM C ABI (include/fwpkm.h): structs and symbols.

Argument marshalling only.  The library is built in-tree by
``sparse_weight_memory_amd.build``; if it is missing this module raises --
there is no other implementation to fall back to.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# the checked build (device-side invariant tests; see fwpkm_checked_build)
CHECKED_LIB_PATH = os.path.join(_HERE, "libfwpkm_checked.so")
# FWPKM_LIB_PATH points the binding at another build of the same ABI, such as
# the checked one
LIB_PATH = os.environ.get("FWPKM_LIB_PATH") or os.path.join(_HERE, "libfwpkm.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_ALIAS = -2
ERR_OOM = -3
ERR_HIP = -4
ERR_UNSUPPORTED = -5
ERR_DEVICE_CHECK = -6

SCORE_IDW = 0
SCORE_DOT = 1

MAX_TOPK = 32
MAX_SQRT_SLOTS = 4096
MAX_HALF = 1024
MAX_DIM_V = 2048
MAX_CHUNK = 1024
NOALLOC_SCRATCH_BYTES = 64 << 20

# every symbol the header declares
EXPORTS = (
    "fwpkm_create",
    "fwpkm_workspace_bytes",
    "fwpkm_forward_chunk",
    "fwpkm_forward_chunk_weighted",
    "fwpkm_forward_chunk_noalloc",
    "fwpkm_sequence_workspace_bytes",
    "fwpkm_forward_sequence",
    "fwpkm_destroy",
    "fwpkm_last_error",
    "fwpkm_profile_enable",
    "fwpkm_profile_read",
    "fwpkm_kernel_name",
    "fwpkm_checked_build",
)

NUM_TIMED = 10
KERNEL_NAMES = ("score", "read", "sort", "update", "copy", "addr_stats", "addr_grad", "addr_apply",
                "project", "gate")


class CConfig(ctypes.Structure):
    _fields_ = [
        ("sqrt_slots", ctypes.c_int32),
        ("dim_qk", ctypes.c_int32),
        ("dim_v", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("chunk_size", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("max_batch", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("score_mode", ctypes.c_int32),
        ("addr_weight", ctypes.c_float),
    ]


class CState(ctypes.Structure):
    _fields_ = [
        ("k1", ctypes.c_void_p),
        ("k2", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("batch_stride_k", ctypes.c_int64),
        ("batch_stride_v", ctypes.c_int64),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"FwPKM HIP library not found at {LIB_PATH}; build it with "
            "`python -m sparse_weight_memory_amd.build` (gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.fwpkm_create.argtypes = [ctypes.POINTER(CConfig), ctypes.POINTER(ctypes.c_void_p)]
    lib.fwpkm_create.restype = ctypes.c_int
    lib.fwpkm_workspace_bytes.argtypes = [ctypes.POINTER(CConfig)]
    lib.fwpkm_workspace_bytes.restype = ctypes.c_size_t
    lib.fwpkm_forward_chunk.argtypes = [
        ctypes.c_void_p,                       # handle
        ctypes.c_void_p, ctypes.c_void_p,      # queries, targets
        ctypes.c_int32, ctypes.c_int32,        # batch, tokens
        ctypes.c_float,                        # lr
        ctypes.POINTER(CState), ctypes.POINTER(CState),
        ctypes.c_void_p,                       # retrieved
        ctypes.c_void_p, ctypes.c_void_p,      # out_slots, out_weights
        ctypes.c_void_p,                       # stream
    ]
    lib.fwpkm_forward_chunk.restype = ctypes.c_int
    lib.fwpkm_forward_chunk_weighted.argtypes = [
        ctypes.c_void_p,                       # handle
        ctypes.c_void_p, ctypes.c_void_p,      # queries, targets
        ctypes.c_void_p,                       # token_weights (nullable)
        ctypes.c_int32, ctypes.c_int32,        # batch, tokens
        ctypes.c_float,                        # lr
        ctypes.POINTER(CState), ctypes.POINTER(CState),
        ctypes.c_void_p,                       # retrieved
        ctypes.c_void_p, ctypes.c_void_p,      # out_slots, out_weights
        ctypes.c_void_p,                       # stream
    ]
    lib.fwpkm_forward_chunk_weighted.restype = ctypes.c_int
    lib.fwpkm_forward_chunk_noalloc.argtypes = lib.fwpkm_forward_chunk.argtypes
    lib.fwpkm_forward_chunk_noalloc.restype = ctypes.c_int
    lib.fwpkm_sequence_workspace_bytes.argtypes = [ctypes.POINTER(CConfig), ctypes.c_int32,
                                                   ctypes.c_int32]
    lib.fwpkm_sequence_workspace_bytes.restype = ctypes.c_size_t
    lib.fwpkm_forward_sequence.argtypes = [
        ctypes.c_void_p,                       # handle
        ctypes.c_void_p, ctypes.c_void_p,      # x, w_in
        ctypes.c_void_p, ctypes.c_void_p,      # w_gate, b_gate (nullable)
        ctypes.c_int32, ctypes.c_int32,        # batch, seq
        ctypes.c_float,                        # lr
        ctypes.POINTER(CState), ctypes.POINTER(CState),
        ctypes.c_void_p,                       # out
        ctypes.c_void_p, ctypes.c_void_p,      # out_slots, out_weights
        ctypes.c_void_p, ctypes.c_size_t,      # workspace, workspace_bytes
        ctypes.c_void_p,                       # stream
    ]
    lib.fwpkm_forward_sequence.restype = ctypes.c_int
    lib.fwpkm_destroy.argtypes = [ctypes.c_void_p]
    lib.fwpkm_destroy.restype = None
    lib.fwpkm_last_error.argtypes = []
    lib.fwpkm_last_error.restype = ctypes.c_char_p
    lib.fwpkm_profile_enable.argtypes = [ctypes.c_void_p, ctypes.c_int32]
    lib.fwpkm_profile_enable.restype = ctypes.c_int
    lib.fwpkm_profile_read.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_int64)]
    lib.fwpkm_profile_read.restype = ctypes.c_int
    lib.fwpkm_kernel_name.argtypes = [ctypes.c_int32]
    lib.fwpkm_kernel_name.restype = ctypes.c_char_p
    lib.fwpkm_checked_build.argtypes = []
    lib.fwpkm_checked_build.restype = ctypes.c_int32
    _lib = lib
    return lib


def last_error() -> str:
    return load().fwpkm_last_error().decode()

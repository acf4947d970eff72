"""ctypes loader for libkda.so: the exported C ABI of include/kda.h, nothing more."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# KDA_LIBRARY names another build of the same library (the host-sanitizer build of
# build.py --sanitize-host, for the CPU tests); by default the in-tree libkda.so.
LIB_PATH = os.environ.get("KDA_LIBRARY") or os.path.join(HERE, "libkda.so")

DTYPE_F32 = 0
DTYPE_BF16 = 1
NOALLOC_SCRATCH_BYTES = 256 << 20  # KDA_NOALLOC_SCRATCH_BYTES
STATUS = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARG", 2: "KDA_ERR_UNSUPPORTED", 3: "KDA_ERR_WORKSPACE",
          4: "KDA_ERR_HIP"}
# every symbol include/kda.h declares
EXPORTS = ("kda_chunk_fwd_workspace_size", "kda_chunk_fwd", "kda_chunk_fwd_noalloc",
           "kda_dplr_chunk_fwd_workspace_size", "kda_dplr_chunk_fwd", "kda_decode_step",
           "kda_decode_step_head_gate", "kda_dplr_decode_step",
           "kda_layer_fwd", "kda_layer_decode_step", "kda_chunk_bwd_workspace_size", "kda_chunk_bwd",
           "kda_status_string")


class KdaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_string(status)})")


class Shape(ctypes.Structure):
    """kda_shape_t"""
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int64), ("num_seqs", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int), ("max_seqlen", ctypes.c_int64),
                ("gate_per_head", ctypes.c_int32)]


def shape(batch, seqlen, num_seqs, heads, dk, dv, in_dtype, out_dtype, max_seqlen=0, gate_per_head=0):
    """A kda_shape_t built by field name."""
    return Shape(batch=batch, seqlen=seqlen, num_seqs=num_seqs, heads=heads, dk=dk, dv=dv, in_dtype=in_dtype,
                 out_dtype=out_dtype, max_seqlen=max_seqlen, gate_per_head=gate_per_head)


class Layer(ctypes.Structure):
    """kda_layer_t"""
    _fields_ = [("qk_l2norm", ctypes.c_int32), ("l2_eps", ctypes.c_float), ("gate", ctypes.c_void_p),
                ("out_gate", ctypes.c_void_p), ("norm_weight", ctypes.c_void_p), ("rms_eps", ctypes.c_float)]


_LIB = None


def lib():
    """Load libkda.so; raise loudly if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; "
                          f"g.build()') -- there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.kda_chunk_fwd_workspace_size.restype = sz
    L.kda_chunk_fwd_workspace_size.argtypes = [ctypes.POINTER(Shape)]
    L.kda_chunk_fwd.restype = ctypes.c_int
    L.kda_chunk_fwd.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.kda_chunk_fwd_noalloc.restype = ctypes.c_int
    L.kda_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.kda_dplr_chunk_fwd_workspace_size.restype = sz
    L.kda_dplr_chunk_fwd_workspace_size.argtypes = [ctypes.POINTER(Shape)]
    L.kda_dplr_chunk_fwd.restype = ctypes.c_int
    L.kda_dplr_chunk_fwd.argtypes = [ctypes.POINTER(Shape)] + [vp] * 11 + [sz, vp]
    for name in ("kda_decode_step", "kda_decode_step_head_gate"):
        f = getattr(L, name)
        f.restype = ctypes.c_int
        f.argtypes = [i32, i32, i32, i32, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp]
    L.kda_dplr_decode_step.restype = ctypes.c_int
    L.kda_dplr_decode_step.argtypes = [i32, i32, i32, i32, ctypes.c_int, ctypes.c_int] + [vp] * 9
    L.kda_layer_fwd.restype = ctypes.c_int
    L.kda_layer_fwd.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Layer), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                sz, vp]
    L.kda_layer_decode_step.restype = ctypes.c_int
    L.kda_layer_decode_step.argtypes = [i32, i32, i32, i32, ctypes.c_int, ctypes.c_int, i32,
                                        ctypes.POINTER(Layer), vp, vp, vp, vp, vp, vp, vp]
    L.kda_chunk_bwd_workspace_size.restype = sz
    L.kda_chunk_bwd_workspace_size.argtypes = [ctypes.POINTER(Shape)]
    L.kda_chunk_bwd.restype = ctypes.c_int
    L.kda_chunk_bwd.argtypes = [ctypes.POINTER(Shape)] + [vp] * 16 + [sz, vp]
    L.kda_status_string.restype = ctypes.c_char_p
    L.kda_status_string.argtypes = [ctypes.c_int]
    _LIB = L
    return L


def status_string(st: int) -> str:
    return lib().kda_status_string(int(st)).decode()


def check(st: int, where: str):
    if st != 0:
        raise KdaError(st, where)

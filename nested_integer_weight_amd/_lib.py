"""ctypes view of libmq.so (the C ABI in include/mq.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmq.so")

MQ_F32, MQ_F16, MQ_BF16 = 0, 1, 2
MQ_PREFIX, MQ_ROUND, MQ_ROUND_EXTRA = 0, 1, 2
NPLANES = 5

STATUS = {
    0: "MQ_OK", 1: "MQ_EINVAL", 2: "MQ_EWIDTH", 3: "MQ_ESHAPE", 4: "MQ_EALIGN",
    5: "MQ_ENOPLANE", 6: "MQ_EDTYPE", 7: "MQ_EHIP", 8: "MQ_ERULE", 9: "MQ_ESIZE",
}

# every symbol include/mq.h declares
EXPORTS = (
    "mq_status_str", "mq_plane_bytes", "mq_planes_needed", "mq_pack_parent",
    "mq_linear_workspace_bytes", "mq_linear", "mq_linear_noalloc", "mq_linear_mixed", "mq_slice_codes",
    "mq_dequant", "mq_produce_parent", "mq_linear_mixed_workspace_bytes",
)

# bytes of the static split-k scratch behind mq_linear_noalloc (MQ_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


class MqPacked(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("k", ctypes.c_int32), ("plane", ctypes.c_void_p * NPLANES)]


class MqCall(ctypes.Structure):
    _fields_ = [
        ("x", ctypes.c_void_p), ("x_dtype", ctypes.c_int32), ("m", ctypes.c_int32),
        ("w", ctypes.POINTER(MqPacked)), ("r", ctypes.c_int32), ("rule", ctypes.c_int32),
        ("group", ctypes.c_int32), ("scales", ctypes.c_void_p), ("zeros", ctypes.c_void_p),
        ("y", ctypes.c_void_p),
    ]


class MqError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)}" if what else STATUS.get(status, str(status)))


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m nested_integer_weight_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    P = ctypes.POINTER(MqPacked)
    L.mq_status_str.argtypes = [ctypes.c_int]
    L.mq_status_str.restype = ctypes.c_char_p
    L.mq_plane_bytes.argtypes = [i32, i32, i32]
    L.mq_plane_bytes.restype = sz
    L.mq_planes_needed.argtypes = [i32, i32]
    L.mq_planes_needed.restype = i32
    L.mq_pack_parent.argtypes = [vp, i32, i32, P, vp]
    L.mq_pack_parent.restype = ctypes.c_int
    L.mq_linear_workspace_bytes.argtypes = [i32, i32, i32]
    L.mq_linear_workspace_bytes.restype = sz
    L.mq_linear.argtypes = [vp, i32, i32, P, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    L.mq_linear.restype = ctypes.c_int
    L.mq_linear_noalloc.argtypes = [vp, i32, i32, P, i32, i32, i32, vp, vp, vp, vp]
    L.mq_linear_noalloc.restype = ctypes.c_int
    L.mq_linear_mixed.argtypes = [ctypes.POINTER(MqCall), i32, vp, sz, ctypes.POINTER(i32), vp]
    L.mq_linear_mixed.restype = ctypes.c_int
    L.mq_linear_mixed_workspace_bytes.argtypes = [ctypes.POINTER(MqCall), i32]
    L.mq_linear_mixed_workspace_bytes.restype = sz
    L.mq_slice_codes.argtypes = [P, i32, i32, vp, vp]
    L.mq_slice_codes.restype = ctypes.c_int
    L.mq_dequant.argtypes = [P, i32, i32, i32, vp, vp, i32, vp, vp]
    L.mq_dequant.restype = ctypes.c_int
    L.mq_produce_parent.argtypes = [vp, i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_float), i32,
                                    i32, i32, i32, vp, vp, vp, vp]
    L.mq_produce_parent.restype = ctypes.c_int
    _lib = L
    return L


def check(status: int, what: str = ""):
    if status != 0:
        raise MqError(status, what)

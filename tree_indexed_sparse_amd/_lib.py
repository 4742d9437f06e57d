"""ctypes binding of libzha.so (the C ABI in include/zha.h).

Marshalling only: tensors are checked for device, dtype, shape and contiguity, their
data pointers and torch's current HIP stream are handed to the library, and every step of
the computation runs in the library's gfx950 kernels. There is no fallback: if the
library is not built, importing the binding raises.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libzha.so")

ZHA_MAX_LEVELS = 12
ZHA_N_REF = 16
ZHA_F32, ZHA_BF16 = 0, 1
ZHA_ROUTER_F32, ZHA_ROUTER_MXFP4 = 0, 1
ZHA_NOALLOC_SCRATCH_BYTES = 128 << 20

STATUS = {
    0: "ZHA_OK",
    -1: "ZHA_ERR_INVALID_ARG",
    -2: "ZHA_ERR_SHAPE",
    -3: "ZHA_ERR_DTYPE",
    -4: "ZHA_ERR_CAPACITY",
    -5: "ZHA_ERR_UNSUPPORTED",
    -6: "ZHA_ERR_HIP",
}

EXPORTS = (
    "zha_tree_bytes",
    "zha_build_tree",
    "zha_tree_append",
    "zha_router_bytes",
    "zha_router_quantize",
    "zha_attend_workspace_bytes",
    "zha_attend",
    "zha_attend_causal",
    "zha_attend_noalloc",
    "zha_attend_level_view",
    "zha_attend_level_bits",
    "zha_dense_workspace_bytes",
    "zha_dense_attend",
    "zha_dense_attend_causal",
    "zha_timing_enable",
    "zha_timing_read",
    "zha_last_error",
)

ZHA_K_POOL, ZHA_K_SCORE, ZHA_K_SELECT, ZHA_K_DECODE, ZHA_K_COMPACT, ZHA_K_COMBINE = 0, 2, 3, 4, 5, 6
ZHA_K_DESCENT = 7
ZHA_K_ROUTER = 8


class ZhaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class ZhaTree(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32),
        ("Hkv", ctypes.c_int32),
        ("N", ctypes.c_int32),
        ("N_cap", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("b", ctypes.c_int32),
        ("L", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("level_off", ctypes.c_int64 * (ZHA_MAX_LEVELS + 1)),
        ("pyramid", ctypes.c_void_p),
        ("router", ctypes.c_int32),
        ("router_code_off", ctypes.c_int64 * (ZHA_MAX_LEVELS + 1)),
        ("router_scale_off", ctypes.c_int64 * (ZHA_MAX_LEVELS + 1)),
        ("router_data", ctypes.c_void_p),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load libzha.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python tree_indexed_sparse_amd/build.py` first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    P = ctypes.POINTER
    lib.zha_tree_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.zha_tree_bytes.restype = sz
    lib.zha_build_tree.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, vp, sz,
                                   P(ZhaTree), vp]
    lib.zha_build_tree.restype = i32
    lib.zha_tree_append.argtypes = [P(ZhaTree), vp, vp, i32, vp]
    lib.zha_tree_append.restype = i32
    lib.zha_router_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.zha_router_bytes.restype = sz
    lib.zha_router_quantize.argtypes = [P(ZhaTree), i32, vp, sz, vp]
    lib.zha_router_quantize.restype = i32
    lib.zha_attend_workspace_bytes.argtypes = [P(ZhaTree), i32, i32]
    lib.zha_attend_workspace_bytes.restype = sz
    lib.zha_attend.argtypes = [P(ZhaTree), vp, i32, i32, vp, vp, f32, i32, vp, vp, i64, vp, vp,
                               sz, vp]
    lib.zha_attend.restype = i32
    lib.zha_attend_causal.argtypes = [P(ZhaTree), vp, i32, i32, vp, vp, vp, f32, i32, vp, vp, i64,
                                      vp, vp, sz, vp]
    lib.zha_attend_causal.restype = i32
    lib.zha_attend_noalloc.argtypes = [P(ZhaTree), vp, i32, i32, vp, vp, f32, i32, vp, vp, i64,
                                       vp, vp]
    lib.zha_attend_noalloc.restype = i32
    lib.zha_attend_level_view.argtypes = [P(ZhaTree), i32, i32, i32, P(i64), P(i64), P(i64),
                                          P(i64), P(i64)]
    lib.zha_attend_level_view.restype = i32
    lib.zha_attend_level_bits.argtypes = [P(ZhaTree), i32, i32, i32, P(i64), P(i64), P(i64)]
    lib.zha_attend_level_bits.restype = i32
    lib.zha_dense_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.zha_dense_workspace_bytes.restype = sz
    lib.zha_dense_attend.argtypes = [vp, i32, i32, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp,
                                     sz, vp]
    lib.zha_dense_attend.restype = i32
    lib.zha_dense_attend_causal.argtypes = [vp, i32, i32, vp, vp, vp, i32, i32, i32, i32, i32,
                                            i32, vp, vp, sz, vp]
    lib.zha_dense_attend_causal.restype = i32
    lib.zha_timing_enable.argtypes = [i32]
    lib.zha_timing_enable.restype = i32
    lib.zha_timing_read.argtypes = [i32, i32, P(ctypes.c_double), P(i64)]
    lib.zha_timing_read.restype = i32
    lib.zha_last_error.argtypes = []
    lib.zha_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def check(code: int) -> None:
    if code != 0:
        raise ZhaError(code, load().zha_last_error().decode())

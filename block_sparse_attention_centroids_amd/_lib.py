"""ctypes view of the C ABI in include/vsa.h (libvsa.so, built in-tree)."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libvsa.so")

VSA_OK = 0
VSA_ERR_INVALID_ARG = 1
VSA_ERR_UNSUPPORTED = 2
VSA_ERR_WORKSPACE = 3
VSA_ERR_CAPACITY = 4
VSA_ERR_SHAPE_MISMATCH = 5
VSA_ERR_HIP = 6

VSA_BF16 = 0
VSA_F32 = 1

VSA_TOPK = 0
VSA_TOPP = 1

VSA_EST_MEAN = 0
VSA_EST_DSA = 1
VSA_EST_DSA2 = 2

VSA_HEAD_DYNAMIC = 0
VSA_HEAD_STATIC = 1
VSA_HEAD_DENSE = 2

VSA_PLAN_NOALLOC_MAX_WS = 32 << 20
VSA_CALIB_POOL_BYTES = 4 << 20
VSA_CALIB_MAX_WORKGROUPS = 65536
VSA_CALIB_MAX_ITERS = 100000


class VsaShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("heads", ctypes.c_int32), ("D", ctypes.c_int32),
                ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("W", ctypes.c_int32),
                ("bt", ctypes.c_int32), ("bh", ctypes.c_int32), ("bw", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class VsaIndex(ctypes.Structure):
    _fields_ = [("shape", VsaShape), ("nb", ctypes.c_int32), ("window_t", ctypes.c_int32),
                ("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p),
                ("capacity", ctypes.c_int64), ("equal_heads", ctypes.c_int32)]


class VsaSelect(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("n_value", ctypes.c_int32),
                ("value", ctypes.POINTER(ctypes.c_float)), ("window_t", ctypes.c_int32),
                ("sink", ctypes.c_int32), ("scale", ctypes.c_float), ("estimator", ctypes.c_int32)]


class VsaHeadOption(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("value", ctypes.c_float), ("window_t", ctypes.c_int32)]


class VsaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} (status {status})")


_lib = None

EXPORTS = ("vsa_query", "vsa_plan", "vsa_attn", "vsa_permute", "vsa_unpermute",
           "vsa_centroids", "vsa_centroid_scores", "vsa_sics", "vsa_scheme_workspace",
           "vsa_select_scheme", "vsa_query_select", "vsa_plan_select", "vsa_estimate", "vsa_query_mixed", "vsa_plan_mixed",
           "vsa_plan_noalloc", "vsa_plan_heads", "vsa_attn_heads", "vsa_scheme_means_workspace",
           "vsa_select_scheme_means", "vsa_calib_mfma_bf16", "vsa_status_str")


def load() -> ctypes.CDLL:
    """Load libvsa.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m block_sparse_attention_centroids_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.vsa_query.argtypes = [ctypes.POINTER(VsaShape), ctypes.POINTER(ctypes.c_float), I, I,
                              ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                              ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
    lib.vsa_plan.argtypes = [P, P, ctypes.POINTER(VsaShape), ctypes.POINTER(ctypes.c_float), I, I,
                             ctypes.POINTER(VsaIndex), P, ctypes.c_size_t, P]
    lib.vsa_attn.argtypes = [P, P, P, ctypes.POINTER(VsaIndex), ctypes.c_float, P, P,
                             ctypes.c_size_t, P]
    lib.vsa_permute.argtypes = [P, ctypes.POINTER(VsaShape), P, P]
    lib.vsa_unpermute.argtypes = [P, ctypes.POINTER(VsaShape), P, P]
    lib.vsa_centroids.argtypes = [P, ctypes.POINTER(VsaShape), P, P]
    lib.vsa_centroid_scores.argtypes = [P, P, ctypes.POINTER(VsaShape), P, P]
    lib.vsa_sics.argtypes = [P, ctypes.POINTER(VsaShape), P, P]
    lib.vsa_scheme_workspace.argtypes = [ctypes.POINTER(VsaShape), ctypes.POINTER(ctypes.c_int32), I,
                                         ctypes.POINTER(ctypes.c_size_t)]
    lib.vsa_select_scheme.argtypes = [P, P, ctypes.POINTER(VsaShape), ctypes.POINTER(ctypes.c_int32), I, P, P,
                                      P, ctypes.c_size_t, P]
    lib.vsa_query_select.argtypes = [ctypes.POINTER(VsaShape), ctypes.POINTER(VsaSelect),
                                     ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                                     ctypes.POINTER(ctypes.c_size_t)]
    lib.vsa_plan_select.argtypes = [P, P, ctypes.POINTER(VsaShape), ctypes.POINTER(VsaSelect),
                                    ctypes.POINTER(VsaIndex), P, ctypes.c_size_t, P]
    lib.vsa_estimate.argtypes = [P, P, ctypes.POINTER(VsaShape), I, P, P, ctypes.c_size_t, P]
    lib.vsa_query_mixed.argtypes = [ctypes.POINTER(VsaShape), ctypes.POINTER(VsaHeadOption), I,
                                    ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                                    ctypes.POINTER(ctypes.c_size_t)]
    lib.vsa_plan_mixed.argtypes = [P, P, ctypes.POINTER(VsaShape), ctypes.POINTER(VsaHeadOption), I, P,
                                   ctypes.POINTER(VsaIndex), P, ctypes.c_size_t, P]
    lib.vsa_plan_noalloc.argtypes = [P, P, ctypes.POINTER(VsaShape), ctypes.POINTER(ctypes.c_float), I, I,
                                     ctypes.POINTER(VsaIndex), P]
    lib.vsa_plan_heads.argtypes = [P, P, P, P, ctypes.POINTER(VsaShape), ctypes.POINTER(ctypes.c_int32), I,
                                   ctypes.POINTER(ctypes.c_float), I, I, ctypes.POINTER(VsaIndex), P,
                                   ctypes.c_size_t, P]
    lib.vsa_attn_heads.argtypes = [P, P, P, ctypes.POINTER(VsaIndex), ctypes.POINTER(ctypes.c_int32), I,
                                   ctypes.c_float, P, P, ctypes.c_size_t, P]
    lib.vsa_scheme_means_workspace.argtypes = [ctypes.POINTER(VsaShape), ctypes.POINTER(ctypes.c_int32), I,
                                               ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
    lib.vsa_select_scheme_means.argtypes = [P, P, ctypes.POINTER(VsaShape), ctypes.POINTER(ctypes.c_int32), I, P,
                                            P, P, ctypes.c_size_t, P]
    lib.vsa_calib_mfma_bf16.argtypes = [P, ctypes.c_size_t, P, I, I, P]
    for name in EXPORTS[:-1]:
        getattr(lib, name).restype = ctypes.c_int
    lib.vsa_status_str.argtypes = [ctypes.c_int]
    lib.vsa_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_str(status: int) -> str:
    try:
        return load().vsa_status_str(int(status)).decode()
    except Exception:  # library unavailable: still report the number
        return "status"


def check(status: int, what: str) -> None:
    if status != VSA_OK:
        raise VsaError(status, what)

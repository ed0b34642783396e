"""ctypes declarations of libfusedproj.so (the C ABI in include/fusedproj.h).

The library is loaded from this package directory only; there is no fallback
of any kind: if it is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# FUSEDPROJ_LIBRARY selects another build of the library (the sanitizer build
# the CPU tests make); by default the one built in this directory
LIB_PATH = os.environ.get("FUSEDPROJ_LIBRARY") or os.path.join(PKG, "libfusedproj.so")

FP_F32, FP_F16, FP_BF16, FP_I8, FP_I4, FP_E4M3, FP_MXFP4 = 0, 1, 2, 3, 4, 5, 6
FP_LAYOUT_PACKED, FP_LAYOUT_PACKED_GATE_UP = 0x100, 0x200     # weight layout bits of w_dtype
FP_NORM = {"none": 0, "rms": 1, "layer": 2}
FP_ACT = {"none": 0, "swiglu": 1, "gelu_tanh": 2}
STATUS = ["FP_OK", "FP_E_NULL", "FP_E_SHAPE", "FP_E_DTYPE", "FP_E_ALIGN", "FP_E_ALIAS",
          "FP_E_HIP", "FP_E_WORKSPACE", "FP_E_ARG"]

# every symbol include/fusedproj.h declares
EXPORTS = ["fp_workspace_bytes", "fp_down_workspace_bytes", "fused_add_norm_qkv", "fused_add_norm_qkv_hm", "fused_add_norm_qkv_noalloc", "fused_gateup_act", "fused_down_residual",
           "fused_dequant_i8_bf16", "fused_dequant_i4_bf16", "fused_dequant_mxfp4_bf16", "fused_pack_weight",
           "fused_unpack_weight", "fp_describe_plan", "fp_status_str", "fp_last_error",
           "fp_profile_start", "fp_profile_stop", "fp_tune_install", "fp_tune_count",
           "fp_plan_override_set", "fp_plan_override_get"]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 64), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double)]


class TuneEntry(ctypes.Structure):
    """fp_tune_entry of include/fusedproj.h."""
    _fields_ = [("m_lo", ctypes.c_int64), ("m_hi", ctypes.c_int64), ("hidden", ctypes.c_int64),
                ("n_cols", ctypes.c_int64), ("act_dtype", ctypes.c_int), ("w_dtype", ctypes.c_int),
                ("swiglu", ctypes.c_int32), ("family", ctypes.c_int32), ("rows", ctypes.c_int32),
                ("grid", ctypes.c_int32), ("splits", ctypes.c_int32)]


class PlanOverride(ctypes.Structure):
    """fp_plan_override of include/fusedproj.h."""
    _fields_ = [("splits", ctypes.c_int32), ("stream_nr", ctypes.c_int32), ("stream_target", ctypes.c_int32),
                ("no_stream", ctypes.c_int32), ("no_prefill", ctypes.c_int32), ("fp8_tile", ctypes.c_int32),
                ("no_gemm16", ctypes.c_int32), ("gemm16_stages", ctypes.c_int32), ("no_stream_rows", ctypes.c_int32),
                ("stream_rows_expire", ctypes.c_int32)]


_lib = None


def load(path: str = None):
    """Load (once) and declare the library; ``path`` loads another build without caching it."""
    global _lib
    if path is None:
        if _lib is not None:
            return _lib
        path = LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    vp, i64, f32, ci, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
    lib.fp_workspace_bytes.argtypes = [i64, i64, i64, ci, ci]
    lib.fp_workspace_bytes.restype = sz
    lib.fp_down_workspace_bytes.argtypes = [i64, i64, i64, ci, ci]
    lib.fp_down_workspace_bytes.restype = sz
    lib.fused_add_norm_qkv.argtypes = [vp, vp, vp, vp, vp, ci, f32, vp, vp, vp, vp, vp, vp,
                                       i64, i64, i64, i64, i64, ci, ci, ci, vp, sz, vp]
    lib.fused_add_norm_qkv.restype = ci
    lib.fused_add_norm_qkv_hm.argtypes = [vp, vp, vp, vp, vp, ci, f32, vp, vp, vp, vp, vp, vp,
                                       i64, i64, i64, i64, i64, ci, ci, ci, vp, sz, vp]
    lib.fused_add_norm_qkv_hm.restype = ci
    lib.fused_add_norm_qkv_noalloc.argtypes = [vp, vp, vp, vp, vp, ci, f32, vp, vp, vp, vp, vp, vp,
                                               i64, i64, i64, i64, i64, ci, ci, ci, vp]
    lib.fused_add_norm_qkv_noalloc.restype = ci
    lib.fused_gateup_act.argtypes = [vp, vp, vp, vp, vp, ci, f32, vp, vp, vp, vp,
                                     i64, i64, i64, ci, ci, ci, ci, vp, sz, vp]
    lib.fused_gateup_act.restype = ci
    lib.fused_down_residual.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, ci, ci, ci, vp, sz, vp]
    lib.fused_down_residual.restype = ci
    lib.fused_dequant_i8_bf16.argtypes = [vp, vp, vp, i64, i64, vp]
    lib.fused_dequant_i8_bf16.restype = ci
    lib.fused_dequant_i4_bf16.argtypes = [vp, vp, vp, i64, i64, vp]
    lib.fused_dequant_i4_bf16.restype = ci
    lib.fused_dequant_mxfp4_bf16.argtypes = [vp, vp, vp, i64, i64, vp]
    lib.fused_dequant_mxfp4_bf16.restype = ci
    for fn in (lib.fused_pack_weight, lib.fused_unpack_weight):
        fn.argtypes = [vp, vp, i64, i64, ci, ctypes.c_int32, vp]
        fn.restype = ci
    lib.fp_describe_plan.argtypes = [i64, i64, i64, ci, ci, ci, ctypes.c_char_p, sz]
    lib.fp_describe_plan.restype = ci
    lib.fp_status_str.argtypes = [ci]
    lib.fp_status_str.restype = ctypes.c_char_p
    lib.fp_last_error.argtypes = []
    lib.fp_last_error.restype = ctypes.c_char_p
    lib.fp_profile_start.argtypes = []
    lib.fp_profile_start.restype = ci
    lib.fp_profile_stop.argtypes = [ctypes.POINTER(KernelTime), ci, ctypes.POINTER(ci)]
    lib.fp_profile_stop.restype = ci
    lib.fp_tune_install.argtypes = [ctypes.POINTER(TuneEntry), i64]
    lib.fp_tune_install.restype = ci
    lib.fp_tune_count.argtypes = []
    lib.fp_tune_count.restype = i64
    lib.fp_plan_override_set.argtypes = [ctypes.POINTER(PlanOverride)]
    lib.fp_plan_override_set.restype = ci
    lib.fp_plan_override_get.argtypes = [ctypes.POINTER(PlanOverride)]
    lib.fp_plan_override_get.restype = ci
    if path == LIB_PATH:
        _lib = lib
    return lib

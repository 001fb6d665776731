"""ctypes view of libnarrowcast's C-ABI (include/narrowcast.h).

Structures mirror the header field for field.  ``load()`` opens the in-tree
``libnarrowcast.so`` and fails loudly if it is missing: there is no fallback.
"""

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_int32, c_int64, c_size_t, c_uint32, c_uint64, c_void_p

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libnarrowcast.so")

NC_OK, NC_E_ARG, NC_E_ALIGN, NC_E_SHAPE, NC_E_UNSUPPORTED, NC_E_HIP, NC_E_WORKSPACE, NC_E_SCRATCH = range(8)
NC_STATIC_SCRATCH_BYTES = 8 << 20
NC_F32, NC_BF16 = 0, 1
NC_E4M3, NC_E5M2 = 0, 1
NC_MX_OCP, NC_MX_PLUS1, NC_MX_CEIL = 0, 1, 2
NC_EST_CURRENT, NC_EST_MOST_RECENT, NC_EST_MAX_WINDOW, NC_EST_EMA = 0, 1, 2, 3
NC_MX_ROWS, NC_MX_COLS = 0, 1


class NcTensor(ctypes.Structure):
    _fields_ = [("x", c_void_p), ("codes", c_void_p), ("n", c_int64), ("cols", c_int64),
                ("scales", c_void_p), ("mx_axis", c_int32), ("reserved", c_int32)]


class NcCounts(ctypes.Structure):
    _fields_ = [("n_finite", c_uint64), ("n_clip", c_uint64), ("n_underflow", c_uint64),
                ("n_nonfinite", c_uint64), ("amax_bits", c_uint32), ("reserved", c_uint32)]


class NcStats(ctypes.Structure):
    _fields_ = [(n, c_double) for n in ("sum_e", "sum_abs_e", "sum_e2", "sum_dir_e", "sum_xe", "sum_x2")]


class NcScaleState(ctypes.Structure):
    _fields_ = [("k", c_int32), ("a_ref_bits", c_uint32), ("has_ref", c_int32), ("n_hist", c_int32),
                ("head", c_int32), ("step", c_int32)]


class NcLossScale(ctypes.Structure):
    _fields_ = [("s_log2", c_int32), ("clean_steps", c_int32)]


class NcPolicy(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in ("fmt", "est", "window", "margin", "hysteresis", "interval",
                                       "skip_on_nonfinite", "ls_enable", "ls_growth_interval",
                                       "ls_log2_min", "ls_log2_max")] + [("ema_alpha", ctypes.c_float)]


class NcUpdateTensor(ctypes.Structure):
    _fields_ = [("w", c_void_p), ("d", c_void_p), ("flags", c_void_p), ("n", c_int64)]


class NcSwampCounts(ctypes.Structure):
    _fields_ = [(n, c_uint64) for n in ("n_considered", "n_zero", "n_below", "n_noop", "n_excluded")]


class NcSwampPolicy(ctypes.Structure):
    _fields_ = [("window", c_int32), ("num", c_uint32), ("den", c_uint32), ("reserved", c_int32)]


class NcSwampState(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in ("run", "promoted", "steps", "reserved")]


NC_W_BF16, NC_W_FP16 = 0, 1

EXPORTS = ("nc_amax", "nc_scale_update", "nc_cast_tensor", "nc_cast_tensor_static", "nc_cast_tensor_sr", "nc_cast_mx", "nc_dequant",
           "nc_cast_stats", "nc_workspace_bytes", "nc_status_string", "nc_swamp_workspace_bytes",
           "nc_swamp_watch", "nc_swamp_window")

_lib = None


def load():
    """Open libnarrowcast.so (once) and declare every entry point."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libnarrowcast.so not built at {LIB_PATH}: run "
                           "`python -m scaled_fp8_casting_amd.build` (there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    T = POINTER(NcTensor)
    lib.nc_amax.argtypes = [T, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.nc_scale_update.argtypes = [POINTER(NcPolicy), c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
    lib.nc_cast_tensor.argtypes = [T, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_size_t, c_void_p]
    lib.nc_cast_tensor_static.argtypes = [T, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                          c_void_p]
    lib.nc_cast_tensor_sr.argtypes = [T, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_uint64, c_uint64,
                                      c_void_p, c_void_p, c_size_t, c_void_p]
    lib.nc_cast_mx.argtypes = [T, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                               c_size_t, c_void_p]
    lib.nc_dequant.argtypes = [T, c_int32, c_int32, c_void_p, POINTER(c_void_p), c_int32, c_void_p]
    lib.nc_cast_stats.argtypes = [T, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_size_t, c_void_p]
    U = POINTER(NcUpdateTensor)
    lib.nc_swamp_workspace_bytes.argtypes = [U, c_int32]
    lib.nc_swamp_workspace_bytes.restype = c_size_t
    lib.nc_swamp_watch.argtypes = [U, c_int32, c_int32, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.nc_swamp_window.argtypes = [POINTER(NcSwampPolicy), c_int32, c_void_p, c_void_p, c_void_p]
    lib.nc_workspace_bytes.argtypes = [T, c_int32]
    lib.nc_workspace_bytes.restype = c_size_t
    lib.nc_status_string.argtypes = [c_int32]
    lib.nc_status_string.restype = c_char_p
    for name in ("nc_amax", "nc_scale_update", "nc_cast_tensor", "nc_cast_tensor_static", "nc_cast_tensor_sr", "nc_cast_mx", "nc_dequant",
                 "nc_cast_stats", "nc_swamp_watch", "nc_swamp_window"):
        getattr(lib, name).restype = c_int32
    _lib = lib
    return lib

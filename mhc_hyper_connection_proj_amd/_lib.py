"""ctypes binding of libmhc.so (the C ABI in include/mhc.h).

Argument marshalling only: every step of the mHC path runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory (outputs and
workspaces are allocated with torch.empty) and the current HIP stream.  If
the shared library is missing this module raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmhc.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "mhc.h")

MHC_BF16, MHC_F32 = 0, 1
MHC_KERNEL_NONE, MHC_KERNEL_PROJ_BWD_DXDW = 0, 1  # mhc_kernel_id (mhc_set_kernel_events)
MHC_PROBE_READ, MHC_PROBE_COPY, MHC_PROBE_NONTEMPORAL = 0, 1, 2  # mhc_probe_kind (mhc_bandwidth_probe)
SAVED_STRIDE = 32
STATUS = ["MHC_OK", "MHC_ERR_NULL", "MHC_ERR_SHAPE", "MHC_ERR_UNSUPPORTED", "MHC_ERR_ALIGN",
          "MHC_ERR_ALIAS", "MHC_ERR_WORKSPACE", "MHC_ERR_ARG", "MHC_ERR_HIP"]


class MhcError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS[status] if 0 <= status < len(STATUS) else f"status {status}"
        super().__init__(f"{self.name}: {detail}")


_vp, _i64, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/mhc.h
SIGNATURES = {
    "mhc_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "mhc_last_error": (ctypes.c_char_p, []),
    "mhc_version": (ctypes.c_char_p, []),
    "mhc_saved_stride": (_i32, [_i32]),
    "mhc_set_kernel_events": (ctypes.c_int, [_i32, _vp, _vp]),
    "mhc_bandwidth_probe": (ctypes.c_int, [_vp, _i32, _vp, _vp, _sz]),
    "mhc_proj_rms_h_workspace_size": (_sz, [_i64, _i32, _i64, ctypes.c_int]),
    "mhc_proj_rms_h": (ctypes.c_int, [_vp, _i64, _i32, _i64, ctypes.c_int, _vp, _vp, _vp, _vp, _f32,
                                      _vp, _vp, _vp, _vp, _vp, _sz]),
    "mhc_proj_rms_h_fma": (ctypes.c_int, [_vp, _i64, _i32, _i64, ctypes.c_int, _vp, _vp, _vp, _vp, _f32,
                                          _vp, _vp, _vp, _vp, _vp, _sz]),
    "mhc_proj_rms_h_bwd_workspace_size": (_sz, [_i64, _i32, _i64, ctypes.c_int]),
    "mhc_proj_rms_h_bwd": (ctypes.c_int, [_vp, _i64, _i32, _i64, ctypes.c_int, _vp, _vp, _vp, _vp,
                                          _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _sz]),
    "mhc_sinkhorn_fwd": (ctypes.c_int, [_vp, _i64, _i32, _vp, _vp, _i32, _f32]),
    "mhc_sinkhorn_bwd": (ctypes.c_int, [_vp, _i64, _i32, _vp, _vp, _vp, _i32, _f32]),
    "mhc_h_aggregate_fwd": (ctypes.c_int, [_vp, _i64, _i32, _i64, ctypes.c_int, _vp, _vp, _vp]),
    "mhc_h_aggregate_bwd": (ctypes.c_int, [_vp, _i64, _i32, _i64, ctypes.c_int, _vp, _vp, _vp, _vp,
                                           _i32, _vp]),
    "mhc_h_post_bda_fwd": (ctypes.c_int, [_vp, _i64, _i32, _i64, ctypes.c_int, _vp, _vp, _vp, _vp,
                                          _vp, _vp]),
    "mhc_h_post_bda_bwd_workspace_size": (_sz, [_i64, _i32, _i64, ctypes.c_int, _i32]),
    "mhc_h_post_bda_bwd": (ctypes.c_int, [_vp, _i64, _i32, _i64, ctypes.c_int, _vp, _vp, _vp, _vp,
                                          _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz]),
    "mhc_stream_mix_fwd": (ctypes.c_int, [_vp, _i64, _i32, _i64, ctypes.c_int, _vp, _vp, _vp]),
    "mhc_stream_mix_bwd": (ctypes.c_int, [_vp, _i64, _i32, _i64, ctypes.c_int, _vp, _vp, _vp, _vp, _vp]),
    "mhc_stream_distribute_fwd": (ctypes.c_int, [_vp, _i64, _i32, _i64, ctypes.c_int, _vp, _vp, _vp]),
    "mhc_stream_distribute_bwd": (ctypes.c_int, [_vp, _i64, _i32, _i64, ctypes.c_int, _vp, _vp, _vp, _vp,
                                                 _vp]),
    "mhc_h_aggregate_static_fwd": (ctypes.c_int, [_vp, _i64, _i32, _i64, ctypes.c_int, _vp, _vp, _vp]),
    "mhc_h_aggregate_static_bwd_workspace_size": (_sz, [_i64, _i32, _i64, ctypes.c_int]),
    "mhc_h_aggregate_static_bwd": (ctypes.c_int, [_vp, _i64, _i32, _i64, ctypes.c_int, _vp, _vp, _vp, _vp,
                                                  _i32, _vp, _vp, _sz]),
    "mhc_pre_fwd_workspace_size": (_sz, [_i64, _i32, _i64, ctypes.c_int]),
    "mhc_pre_fwd": (ctypes.c_int, [_vp, _i64, _i32, _i64, ctypes.c_int, _vp, _vp, _vp, _vp, _f32,
                                   _i32, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz]),
    "mhc_pre_fwd_noalloc": (ctypes.c_int, [_vp, _i64, _i32, _i64, ctypes.c_int, _vp, _vp, _vp, _vp, _f32,
                                           _i32, _f32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "mhc_rmsnorm_fwd": (ctypes.c_int, [_vp, _i64, _i64, ctypes.c_int, _vp, _vp, _f32, _vp]),
    "mhc_rmsnorm_bwd_workspace_size": (_sz, [_i64, _i64, ctypes.c_int, _i32]),
    "mhc_rmsnorm_bwd": (ctypes.c_int, [_vp, _i64, _i64, ctypes.c_int, _vp, _vp, _vp, _f32, _vp, _i32, _vp,
                                       _vp, _sz]),
    "mhc_pre_rmsnorm_fwd": (ctypes.c_int, [_vp, _i64, _i32, _i64, ctypes.c_int, _vp, _vp, _vp, _vp, _f32,
                                           _i32, _f32, _vp, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                           _sz]),
    "mhc_pre_bwd_workspace_size": (_sz, [_i64, _i32, _i64, ctypes.c_int]),
    "mhc_pre_bwd": (ctypes.c_int, [_vp, _i64, _i32, _i64, ctypes.c_int, _vp, _vp, _vp, _vp, _vp,
                                   _vp, _vp, _vp, _vp, _vp, _i32, _f32, _vp, _vp, _vp, _i32, _vp,
                                   _vp, _vp, _vp, _vp, _vp, _sz]),
    "mhc_pre_rmsnorm_bwd_workspace_size": (_sz, [_i64, _i32, _i64, ctypes.c_int, _i32]),
    "mhc_pre_rmsnorm_bwd": (ctypes.c_int, [_vp, _i64, _i32, _i64, ctypes.c_int, _vp, _vp, _vp, _f32, _vp, _vp, _vp,
                                           _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _f32, _vp, _vp, _vp, _i32, _vp,
                                           _vp, _vp, _vp, _vp, _vp, _sz]),
}

_lib = None


def header_functions() -> list[str]:
    """Names of the functions include/mhc.h declares."""
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(mhc_[a-z0-9_]+)\s*\(", txt)))


def lib() -> ctypes.CDLL:
    """Load libmhc.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mhc_hyper_connection_proj_amd.build` (no fallback path exists)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(status: int) -> None:
    if status != 0:
        raise MhcError(status, lib().mhc_last_error().decode())


def call(name: str, *args) -> None:
    """Invoke an entry point by name and raise MhcError on a non-OK status."""
    check(getattr(lib(), name)(*args))

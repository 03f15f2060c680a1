"""libmhc: the per-token mHC residual-mixing path as hand-written HIP kernels
for AMD Instinct MI355X (gfx950), behind a C ABI (include/mhc.h).

The binding functions load ``libmhc.so`` on first use and raise if it has not
been built (``python -m mhc_hyper_connection_proj_amd.build``); there is no
CPU or PyTorch fallback.
"""
from .binding import (  # noqa: F401
    mhc_h_aggregate_bwd,
    mhc_h_aggregate_fwd,
    mhc_h_post_bda_bwd,
    mhc_h_post_bda_fwd,
    mhc_pre_bwd,
    mhc_pre_fwd,
    mhc_pre_rmsnorm_bwd,
    mhc_pre_rmsnorm_fwd,
    mhc_proj_rms_h,
    mhc_proj_rms_h_fma,
    mhc_proj_rms_h_bwd,
    mhc_sinkhorn_bwd,
    mhc_sinkhorn_fwd,
)
from ._lib import MhcError  # noqa: F401

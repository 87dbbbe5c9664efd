"""EFLA (Exact Flow Linear Attention) for AMD Instinct MI355X.

The computation lives in libefla.so (HIP kernels for gfx950 behind the C ABI of
include/efla.h); this package only marshals PyTorch tensors into that ABI.
"""
from .efla import (EflaFunction, EflaGatedFunction, efla, efla_bwd, efla_bwd_gated, efla_chunk_ut,
                   efla_decode, efla_decode_gated, efla_fwd, efla_fwd_gated, efla_gated,
                   efla_get_saved_layout, efla_prep, efla_saved_bytes, efla_workspace_bytes,
                   make_problem, profile_enable, profile_read, profile_reset, saved_views)

__all__ = ["EflaFunction", "EflaGatedFunction", "efla", "efla_bwd", "efla_bwd_gated", "efla_chunk_ut",
           "efla_decode", "efla_decode_gated", "efla_fwd", "efla_fwd_gated", "efla_gated",
           "efla_get_saved_layout", "efla_prep", "efla_saved_bytes", "efla_workspace_bytes",
           "make_problem", "profile_enable", "profile_read", "profile_reset", "saved_views"]

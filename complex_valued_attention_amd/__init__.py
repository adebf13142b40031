"""Fused forward pass of complex-valued attention (Born-rule and phase-coherent)
for AMD Instinct gfx950, behind a C ABI (include/cattn.h).

The HIP library is loaded lazily on first use; see :mod:`.cattn`.
"""
from .cattn import born_fwd, pct_fwd, CattnError, LAYOUT_C64, LAYOUT_BF16_PLANES  # noqa: F401

__all__ = ["born_fwd", "pct_fwd", "CattnError", "LAYOUT_C64", "LAYOUT_BF16_PLANES"]

"""MLA decode over a compressed latent KV cache, and GQLA, on MI355X (gfx950).

Every step of the decode path runs in the HIP library ``libmla.so`` built from ``csrc/``;
this package only marshals arguments to its C ABI (``include/mla.h``). The library is
loaded on first use, and using the package without it raises instead of falling back.
"""
from .layout import gqa_cache_shape, latent_cache_shape  # noqa: F401

__all__ = ["gqa_cache_shape", "latent_cache_shape"]

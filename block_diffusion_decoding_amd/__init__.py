"""block-diffusion refinement step on MI355X (gfx950): libbd + Python binding.

``ops`` holds one Python function per C-ABI call of ``include/bd.h``;
``decoder`` drives refinement steps, window advance and commits on one GPU.
The HIP library must be built (``python -m block_diffusion_decoding_amd.build``);
nothing falls back to a CPU implementation.
"""
from ._lib import LIB_PATH, load as load_library  # noqa: F401

__all__ = ["LIB_PATH", "load_library"]

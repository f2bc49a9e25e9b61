"""MI355X (gfx950) hybrid compressed attention (CSA + HCA) for DeepSeek-V4-style layers.

The computation lives in libcsl.so (hand-written HIP kernels behind the C ABI of
include/csl.h); ``ops`` is the torch-facing binding, ``gen`` the seeded synthetic
input generator.
"""
from . import ops  # noqa: F401
from .ops import F32, BF16, KV_PACKED, MXFP4, kv_compress, index_topk, csa_attend, hca_attend  # noqa: F401

__version__ = "0.1.0"

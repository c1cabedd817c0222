"""MI355X (gfx950) forward pass of multi-head self-attention over a 2D patch
grid with relative position encoding: Swin-style per-head bias inside M x M
windows and iRPE contextual terms (key, query and value tables) under the
Product or Cross mapping.

The computation lives in librpe_attn.so (HIP kernels behind the C ABI of
include/rpe_attn.h); this package binds it with ctypes and uses PyTorch only
for device memory and streams.
"""

from .attention import (  # noqa: F401
    PreparedBwd,
    PreparedFwd,
    make_desc,
    prepare_bwd,
    prepare_fwd,
    rpe_attn_axis_index,
    rpe_attn_bucket_map,
    rpe_attn_bwd,
    rpe_attn_bwd_noalloc,
    rpe_attn_cross_to_product,
    rpe_attn_fwd,
    rpe_attn_fwd_plan,
    rpe_attn_num_buckets,
    rpe_attn_undirected_to_product,
    rpe_attn_unit_size,
    rpe_attn_validate,
)
from ._lib import RpeError, load  # noqa: F401

__version__ = "0.2.0"

"""nkv: the paged KV-cache data plane (store, paged prefill, paged decode, prefill over
contiguous K/V for the no-prefix-cache branch, and the fused
q/k norm + rotary + store before them, the residual add + RMSNorm in front of each
block's projections) for MI355X.

``BlockManager`` drives the library's CPU block manager (block allocation, reference
counts, prefix sharing) that writes the index arrays those calls read.

The compute lives in ``libnkv.so`` (HIP kernels for gfx950 behind the C ABI of
``include/nkv.h``); this package is its thin Python binding plus the seeded input
generators (``workloads``) and the algorithmic byte/flop accounting (``accounting``).
The library is loaded on first use and the calls raise if it is not built.
"""

from ._lib import (  # noqa: F401
    BlockManager,
    NkvError,
    load,
    nkv_add_rms_norm,
    nkv_attn_varlen_prefill,
    nkv_paged_attn_decode,
    nkv_paged_attn_decode_noalloc,
    nkv_paged_attn_decode_workspace_size,
    nkv_paged_attn_prefill,
    nkv_qk_norm_rope_store,
    nkv_store_kvcache,
)

__all__ = [
    "BlockManager",
    "NkvError",
    "load",
    "nkv_store_kvcache",
    "nkv_qk_norm_rope_store",
    "nkv_add_rms_norm",
    "nkv_paged_attn_prefill",
    "nkv_attn_varlen_prefill",
    "nkv_paged_attn_decode",
    "nkv_paged_attn_decode_noalloc",
    "nkv_paged_attn_decode_workspace_size",
]

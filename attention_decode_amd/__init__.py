"""MI355X (gfx950) single-step decode attention: split-KV partial passes + LSE merge over
contiguous, paged and block-sparse KV caches, and an MLA variant.

The compute runs in the HIP library libattn_decode.so (C ABI in include/attn_decode.h); this
package is its thin ctypes binding (same entry-point names), the seeded workload generators and
a prepared-step helper. Importing the package does not load the library; the first call does,
and raises if it is not built.
"""
from ._abi import (  # noqa: F401
    AD_BF16, AD_F32, AD_KERNEL_MATRIX, AD_KERNEL_MATRIX16, AD_KERNEL_MLA, AD_KERNEL_VECTOR, AD_KV_FP8_E4M3, AD_KV_INT4, AD_KV_SAME,
    AD_MAX_SPLITS, KERNEL_NAMES, ADError, attn_decode, attn_decode_kernel, attn_decode_last_error,
    attn_decode_launches,
    attn_decode_merge, attn_decode_mla, attn_decode_paged, attn_decode_plan, attn_decode_splitkv,
    attn_decode_workspace_size, lib, make_args, make_paged, make_sparse,
)

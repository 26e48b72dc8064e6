"""Rotated, asymmetric K4/V3 bit-quantized KV cache and fused decode/verify
attention for AMD Instinct MI355X (gfx950).

The method (page "mlx_streaming/core/cache/quant_kv.py"): a seed-fixed
block-diagonal SO(4) rotation of q, k and v; keys quantized to 4-bit and
values to 3-bit group-64 affine codes, bit-packed and appended to a cache that
grows in 256-row steps and can be trimmed; attention over the packed cache
with a causal mask at the cache offset; the inverse rotation of the output;
snapshots of the cache (a device copy of its offset-prefix) and their restore.

Every step runs in the HIP kernels of ``librbq.so`` behind the C ABI declared
in ``include/rbq.h``; ``capi`` binds it with ctypes and ``cache`` wraps it in
a cache object whose buffers are torch tensors.
"""
from .capi import (  # noqa: F401
    RbqError,
    rbq_kv_cache,
    rbq_kv_commit_verified,
    rbq_kv_copy_batch,
    rbq_kv_copy_prefix,
    rbq_kv_grow,
    rbq_kv_quant_append,
    rbq_kv_required_capacity,
    rbq_kv_trim,
    rbq_quant_attn_decode,
    rbq_quant_attn_splits,
    rbq_quant_attn_workspace_bytes,
    rbq_rotation_build,
)
from .cache import (  # noqa: F401
    CacheSnapshot,
    RotatedQuantKVCache,
    build_block_so4,
    commit_tree_row,
    commit_verified_snapshot,
    quaternion_draws,
    restore_caches,
    snapshot_caches,
    tile_caches,
)

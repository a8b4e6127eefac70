"""Paged-KV decode for AMD Instinct MI355X (gfx950).

Hand-written HIP kernels behind a C ABI (``include/pagedkv.h``): the
reshape_and_cache slot scatter, paged-attention decode (direct and split-KV with
a log-sum-exp merge), the two fused into one launch (append form) and the
K8/V4-quantized variants.

The binding (``_binding``) loads ``libpagedkv.so`` on first use of any of the
names below and raises ImportError if the library has not been built; there is
no fallback.  ``workloads`` (seeded synthetic inputs) needs no library.
"""

_EXPORTS = (
    "BLOCK_SIZE", "PKV_BF16", "PKV_F16", "PKV_F32", "PKV_FMT_BF16", "PKV_FMT_F16",
    "PKV_FMT_K8V4", "PagedKVError", "kv_cache_bytes_per_token", "kv_cache_write",
    "kv_cache_write_k8v4", "last_error", "lib", "paged_attention_decode",
    "paged_attention_decode_k8v4", "paged_attention_decode_splitkv",
    "paged_attention_decode_splitkv_k8v4", "splitkv_workspace_size", "version",
    "paged_attention_decode_splitkv_partials", "paged_attention_decode_splitkv_k8v4_partials",
    "paged_attention_decode_splitkv_merge", "paged_attention_decode_append",
    "paged_attention_decode_splitkv_append", "paged_attention_decode_splitkv_append_partials",
    "paged_attention_decode_window", "paged_attention_decode_splitkv_window", "gather_kv_cache",
    "paged_attention_decode_cascade", "cascade_workspace_size",
    "paged_attention_decode_splitkv_sparse_v", "paged_attention_decode_k8v4_append",
    "paged_attention_decode_splitkv_k8v4_append", "paged_attention_decode_window_append",
    "paged_attention_decode_splitkv_window_append", "paged_attention_decode_splitkv_noalloc",
    "NOALLOC_SCRATCH_BYTES",
)

__all__ = list(_EXPORTS)


def __getattr__(name):
    if name in _EXPORTS:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)

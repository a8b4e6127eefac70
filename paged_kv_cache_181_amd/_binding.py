"""ctypes binding of libpagedkv.so: argument marshalling only.

Every call checks shapes, dtypes, devices and contiguity of the torch tensors,
then passes raw device pointers and ``torch.cuda.current_stream().cuda_stream``
to the C ABI declared in ``include/pagedkv.h``.  All computation happens in the
library's HIP kernels; there is no CPU or PyTorch fallback, and a missing
library raises at import time.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# PKV_LIBRARY names another build of the same ABI (the measurement variant
# libpagedkv_qkvalu.so, for an A/B); by default the product library
LIB_PATH = os.environ.get("PKV_LIBRARY") or os.path.join(PKG, "libpagedkv.so")

PKV_F16, PKV_BF16, PKV_F32 = 0, 1, 2
PKV_FMT_F16, PKV_FMT_BF16, PKV_FMT_K8V4 = 0, 1, 3
BLOCK_SIZE = 16

ERRORS = {-1: "PKV_ERR_NULL", -2: "PKV_ERR_SHAPE", -3: "PKV_ERR_UNSUPPORTED",
          -4: "PKV_ERR_WORKSPACE", -5: "PKV_ERR_LAUNCH", -6: "PKV_ERR_ALIGN"}


class PagedKVError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERRORS.get(code, code)}: {message}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m paged_kv_cache_181_amd.build` (hipcc, gfx950)")
    # torch ships its own HIP runtime under the same soname; loading torch first
    # makes the library bind to that one, so the process holds a single runtime
    # (loaded the other way round, the library's calls find no device)
    import torch  # noqa: F401
    return ctypes.CDLL(LIB_PATH)


lib = _load()

_p = ctypes.c_void_p
_i = ctypes.c_int
_i64 = ctypes.c_int64
_f = ctypes.c_float
_sz = ctypes.c_size_t

_ATTN = [_p, _i, _p, _p, _p, _i, _p, _i, _p, _i, _i, _i, _i, _i, _i, _i64, _f]
_ATTN_K8V4 = [_p, _i, _p, _i, _p, _p, _p, _p, _p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _i64, _f]
SIGNATURES = {
    "pkv_last_error": ([], ctypes.c_char_p),
    "pkv_version": ([], _i),
    "kv_cache_write": ([_p, _p, _p, _p, _p, _i64, _i, _i, _i, _i64, _i, _p], _i),
    "paged_attention_decode": (_ATTN + [_p], _i),
    "paged_attention_decode_splitkv_workspace_size": ([_i, _i, _i, _i, _i, _i,
                                                       ctypes.POINTER(_sz)], _i),
    "paged_attention_decode_splitkv": (_ATTN + [_i, _i, _p, _sz, _p], _i),
    "paged_attention_decode_splitkv_noalloc": (_ATTN + [_i, _i, _p], _i),
    "kv_cache_write_k8v4": ([_p, _p, _i, _p, _p, _p, _p, _p, _p, _i64, _i, _i, _i, _i64, _p], _i),
    "paged_attention_decode_k8v4": (_ATTN_K8V4 + [_p], _i),
    "paged_attention_decode_splitkv_k8v4": (_ATTN_K8V4 + [_i, _i, _p, _sz, _p], _i),
    "paged_attention_decode_k8v4_append": (_ATTN_K8V4[:4] + [_p, _p] + _ATTN_K8V4[4:] + [_p], _i),
    "paged_attention_decode_splitkv_k8v4_append": (
        _ATTN_K8V4[:4] + [_p, _p] + _ATTN_K8V4[4:] + [_i, _i, _p, _sz, _p], _i),
    "kv_cache_bytes_per_token": ([_i, _i, _i, _i, ctypes.POINTER(_i64)], _i),
    "paged_attention_decode_splitkv_partials": (_ATTN[2:] + [_i, _i, _p, _sz, _p], _i),
    "paged_attention_decode_splitkv_k8v4_partials": (_ATTN_K8V4[2:] + [_i, _i, _p, _sz, _p], _i),
    "paged_attention_decode_splitkv_merge": ([_p, _i, _i, _i, _i, _i, _i, _i, _p, _sz, _p], _i),
    "paged_attention_decode_append": (_ATTN[:3] + [_p, _p] + _ATTN[3:] + [_p], _i),
    "paged_attention_decode_splitkv_append": (_ATTN[:3] + [_p, _p] + _ATTN[3:]
                                              + [_i, _i, _p, _sz, _p], _i),
    "paged_attention_decode_splitkv_append_partials": ([_p, _p, _p] + _ATTN[3:]
                                                       + [_i, _i, _p, _sz, _p], _i),
    "paged_attention_decode_window": (_ATTN + [_i, _p], _i),
    "gather_kv_cache": ([_p, _p, _i, _p, _i, _p, _i, _i, _p, _p, _i64, _i, _i, _i, _i64, _p], _i),
    "paged_attention_decode_cascade_workspace_size": ([_i, _i, _i, _i, _i, _i, _i,
                                                       ctypes.POINTER(_sz)], _i),
    "paged_attention_decode_cascade": (_ATTN + [_p, _p, _i, _i, _i, _i, _i, _p, _sz, _p], _i),
    "paged_attention_decode_splitkv_sparse_v": (_ATTN + [_f, _p, _i, _i, _p, _sz, _p], _i),
    "paged_attention_decode_splitkv_window": (_ATTN + [_i, _i, _i, _p, _sz, _p], _i),
    "paged_attention_decode_window_append": (_ATTN[:3] + [_p, _p] + _ATTN[3:] + [_i, _p], _i),
    "paged_attention_decode_splitkv_window_append": (_ATTN[:3] + [_p, _p] + _ATTN[3:]
                                                     + [_i, _i, _i, _p, _sz, _p], _i),
}
for _name, (_args, _res) in SIGNATURES.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res


def last_error() -> str:
    return lib.pkv_last_error().decode()


def version() -> int:
    return lib.pkv_version()


def _check(rc: int) -> None:
    if rc != 0:
        raise PagedKVError(rc, last_error())


# ---------------------------------------------------------------- torch glue

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    codes = {torch.float16: PKV_F16, torch.bfloat16: PKV_BF16, torch.float32: PKV_F32}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _dev(*tensors):
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on one device")
    return dev


def _stream(dev):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _expect(cond, msg):
    if not cond:
        raise ValueError(msg)


def kv_cache_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, fmt: int) -> int:
    out = _i64(0)
    _check(lib.kv_cache_bytes_per_token(num_layers, num_kv_heads, head_dim, fmt, ctypes.byref(out)))
    return out.value


def splitkv_workspace_size(batch, q_len, num_q_heads, head_dim, max_context_len,
                           partition_size) -> int:
    out = _sz(0)
    _check(lib.paged_attention_decode_splitkv_workspace_size(
        batch, q_len, num_q_heads, head_dim, max_context_len, partition_size, ctypes.byref(out)))
    return out.value


def kv_cache_write(key, value, key_cache, value_cache, slot_mapping):
    """Scatter key/value ``[T, Hkv, D]`` into caches ``[NB, 16, Hkv, D]`` at
    ``slot_mapping`` (int64 ``[T]``; negative = skip)."""
    torch = _torch()
    dev = _dev(key, value, key_cache, value_cache, slot_mapping)
    _expect(key.dim() == 3 and key.shape == value.shape, "key/value must be [T, Hkv, D]")
    _expect(key_cache.dim() == 4 and key_cache.shape == value_cache.shape,
            "caches must be [NB, 16, Hkv, D]")
    _expect(key_cache.shape[2:] == key.shape[1:], "cache and key disagree on [Hkv, D]")
    _expect(key.dtype == key_cache.dtype == value.dtype == value_cache.dtype, "dtype mismatch")
    _expect(slot_mapping.dtype == torch.int64 and slot_mapping.shape == (key.shape[0],),
            "slot_mapping must be int64 [T]")
    _check(lib.kv_cache_write(_ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
                              _ptr(slot_mapping), key.shape[0], key.shape[1], key.shape[2],
                              key_cache.shape[1], key_cache.shape[0], _dtype_code(key),
                              _stream(dev)))


def kv_cache_write_k8v4(key, value, k_cache, k_scale, v_cache, v_scale, v_zero, slot_mapping):
    """Quantize-on-write of key/value ``[T, Hkv, D]`` into the K8/V4 arrays."""
    torch = _torch()
    dev = _dev(key, value, k_cache, k_scale, v_cache, v_scale, v_zero, slot_mapping)
    T, hkv, d = key.shape
    nb, bs = k_cache.shape[:2]
    _expect(value.shape == key.shape and key.dtype == value.dtype, "key/value mismatch")
    _expect(k_cache.dtype == torch.int8 and k_cache.shape == (nb, bs, hkv, d), "k_cache int8 [NB,16,Hkv,D]")
    _expect(k_scale.dtype == torch.float16 and k_scale.shape == (nb, bs, hkv), "k_scale f16 [NB,16,Hkv]")
    _expect(v_cache.dtype == torch.uint8 and v_cache.shape == (nb, bs, hkv, d // 2), "v_cache u8 [NB,16,Hkv,D/2]")
    for t in (v_scale, v_zero):
        _expect(t.dtype == torch.float16 and t.shape == (nb, bs, hkv, d // 32), "v_scale/v_zero f16 [NB,16,Hkv,D/32]")
    _expect(slot_mapping.dtype == torch.int64 and slot_mapping.shape == (T,), "slot_mapping int64 [T]")
    _check(lib.kv_cache_write_k8v4(_ptr(key), _ptr(value), _dtype_code(key), _ptr(k_cache),
                                   _ptr(k_scale), _ptr(v_cache), _ptr(v_scale), _ptr(v_zero),
                                   _ptr(slot_mapping), T, hkv, d, bs, nb, _stream(dev)))


def _attn_common(out, query, block_tables, context_lens, gqa_factor):
    torch = _torch()
    _expect(query.dim() == 4, "query must be [B, Q, Hq, D]")
    _expect(out.shape == query.shape, "out must match query's shape")
    _expect(block_tables.dtype == torch.int32 and block_tables.dim() == 2
            and block_tables.shape[0] == query.shape[0], "block_tables must be int32 [B, max_blocks]")
    _expect(context_lens.dtype == torch.int32 and context_lens.shape == (query.shape[0],),
            "context_lens must be int32 [B]")
    B, Q, Hq, D = query.shape
    _expect(Hq % gqa_factor == 0, "num_q_heads must be a multiple of gqa_factor")
    return B, Q, Hq, D


def paged_attention_decode(out, query, key_cache, value_cache, block_tables, context_lens,
                           scale, gqa_factor):
    dev = _dev(out, query, key_cache, value_cache, block_tables, context_lens)
    B, Q, Hq, D = _attn_common(out, query, block_tables, context_lens, gqa_factor)
    _expect(key_cache.shape == value_cache.shape and key_cache.shape[2:] == (Hq // gqa_factor, D),
            "caches must be [NB, 16, Hq/G, D]")
    _expect(query.dtype == key_cache.dtype == value_cache.dtype, "query/cache dtype mismatch")
    _check(lib.paged_attention_decode(
        _ptr(out), _dtype_code(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
        _dtype_code(key_cache), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        B, Q, Hq, gqa_factor, D, key_cache.shape[1], key_cache.shape[0], float(scale), _stream(dev)))


def paged_attention_decode_splitkv(out, query, key_cache, value_cache, block_tables, context_lens,
                                   scale, gqa_factor, max_context_len, partition_size, workspace):
    dev = _dev(out, query, key_cache, value_cache, block_tables, context_lens, workspace)
    B, Q, Hq, D = _attn_common(out, query, block_tables, context_lens, gqa_factor)
    _expect(key_cache.shape == value_cache.shape and key_cache.shape[2:] == (Hq // gqa_factor, D),
            "caches must be [NB, 16, Hq/G, D]")
    _expect(query.dtype == key_cache.dtype == value_cache.dtype, "query/cache dtype mismatch")
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.paged_attention_decode_splitkv(
        _ptr(out), _dtype_code(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
        _dtype_code(key_cache), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        B, Q, Hq, gqa_factor, D, key_cache.shape[1], key_cache.shape[0], float(scale),
        int(max_context_len), int(partition_size), _ptr(workspace), nbytes, _stream(dev)))


NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024     # PKV_NOALLOC_SCRATCH_BYTES


def paged_attention_decode_splitkv_noalloc(out, query, key_cache, value_cache, block_tables,
                                           context_lens, scale, gqa_factor, max_context_len,
                                           partition_size):
    """Split-KV decode with the partials in the library's static per-GPU
    scratch (no workspace argument, nothing allocated); calls that overlap in
    time on one GPU race."""
    dev = _dev(out, query, key_cache, value_cache, block_tables, context_lens)
    B, Q, Hq, D = _attn_common(out, query, block_tables, context_lens, gqa_factor)
    _expect(key_cache.shape == value_cache.shape and key_cache.shape[2:] == (Hq // gqa_factor, D),
            "caches must be [NB, 16, Hq/G, D]")
    _expect(query.dtype == key_cache.dtype == value_cache.dtype, "query/cache dtype mismatch")
    _check(lib.paged_attention_decode_splitkv_noalloc(
        _ptr(out), _dtype_code(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
        _dtype_code(key_cache), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        B, Q, Hq, gqa_factor, D, key_cache.shape[1], key_cache.shape[0], float(scale),
        int(max_context_len), int(partition_size), _stream(dev)))


def _append_args(out, query, new_key, new_value, key_cache, value_cache, block_tables,
                 context_lens, gqa_factor):
    B, Q, Hq, D = _attn_common(out, query, block_tables, context_lens, gqa_factor)
    _expect(key_cache.shape == value_cache.shape and key_cache.shape[2:] == (Hq // gqa_factor, D),
            "caches must be [NB, 16, Hq/G, D]")
    _expect(new_key.shape == new_value.shape == (B * Q, Hq // gqa_factor, D),
            "new_key / new_value must be [B*q_len, Hq/G, D]")
    _expect(query.dtype == key_cache.dtype == value_cache.dtype == new_key.dtype == new_value.dtype,
            "query/new rows/cache dtype mismatch")
    return [_ptr(out), _dtype_code(out), _ptr(query), _ptr(new_key), _ptr(new_value),
            _ptr(key_cache), _ptr(value_cache), _dtype_code(key_cache), _ptr(block_tables),
            block_tables.shape[1], _ptr(context_lens), B, Q, Hq, gqa_factor, D,
            key_cache.shape[1], key_cache.shape[0]]


def paged_attention_decode_append(out, query, new_key, new_value, key_cache, value_cache,
                                  block_tables, context_lens, scale, gqa_factor):
    """Slot write of the new rows (at the positions the tables give them) and
    direct decode, in one launch."""
    dev = _dev(out, query, new_key, new_value, key_cache, value_cache, block_tables, context_lens)
    args = _append_args(out, query, new_key, new_value, key_cache, value_cache, block_tables,
                        context_lens, gqa_factor)
    _check(lib.paged_attention_decode_append(*args, float(scale), _stream(dev)))


def paged_attention_decode_splitkv_append(out, query, new_key, new_value, key_cache, value_cache,
                                          block_tables, context_lens, scale, gqa_factor,
                                          max_context_len, partition_size, workspace):
    """Slot write of the new rows and split-KV decode (partition kernel, then
    the merge)."""
    dev = _dev(out, query, new_key, new_value, key_cache, value_cache, block_tables, context_lens,
               workspace)
    args = _append_args(out, query, new_key, new_value, key_cache, value_cache, block_tables,
                        context_lens, gqa_factor)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.paged_attention_decode_splitkv_append(
        *args, float(scale), int(max_context_len), int(partition_size), _ptr(workspace), nbytes,
        _stream(dev)))


def paged_attention_decode_splitkv_append_partials(query, new_key, new_value, key_cache,
                                                   value_cache, block_tables, context_lens, scale,
                                                   gqa_factor, max_context_len, partition_size,
                                                   workspace):
    """Partition-kernel half of the append form (finish with
    paged_attention_decode_splitkv_merge)."""
    dev = _dev(query, new_key, new_value, key_cache, value_cache, block_tables, context_lens,
               workspace)
    args = _append_args(query, query, new_key, new_value, key_cache, value_cache, block_tables,
                        context_lens, gqa_factor)        # (no output: query stands in for its shape)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.paged_attention_decode_splitkv_append_partials(
        *args[2:], float(scale), int(max_context_len), int(partition_size), _ptr(workspace),
        nbytes, _stream(dev)))


def paged_attention_decode_window(out, query, key_cache, value_cache, block_tables, context_lens,
                                  scale, gqa_factor, sliding_window):
    """Direct decode over each row's ``sliding_window`` most recent positions."""
    dev = _dev(out, query, key_cache, value_cache, block_tables, context_lens)
    B, Q, Hq, D = _attn_common(out, query, block_tables, context_lens, gqa_factor)
    _expect(key_cache.shape == value_cache.shape and key_cache.shape[2:] == (Hq // gqa_factor, D),
            "caches must be [NB, 16, Hq/G, D]")
    _expect(query.dtype == key_cache.dtype == value_cache.dtype, "query/cache dtype mismatch")
    _check(lib.paged_attention_decode_window(
        _ptr(out), _dtype_code(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
        _dtype_code(key_cache), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        B, Q, Hq, gqa_factor, D, key_cache.shape[1], key_cache.shape[0], float(scale),
        int(sliding_window), _stream(dev)))


def paged_attention_decode_splitkv_window(out, query, key_cache, value_cache, block_tables,
                                          context_lens, scale, gqa_factor, sliding_window,
                                          max_context_len, partition_size, workspace):
    """Split-KV decode over each row's ``sliding_window`` most recent positions."""
    dev = _dev(out, query, key_cache, value_cache, block_tables, context_lens, workspace)
    B, Q, Hq, D = _attn_common(out, query, block_tables, context_lens, gqa_factor)
    _expect(key_cache.shape == value_cache.shape and key_cache.shape[2:] == (Hq // gqa_factor, D),
            "caches must be [NB, 16, Hq/G, D]")
    _expect(query.dtype == key_cache.dtype == value_cache.dtype, "query/cache dtype mismatch")
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.paged_attention_decode_splitkv_window(
        _ptr(out), _dtype_code(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
        _dtype_code(key_cache), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        B, Q, Hq, gqa_factor, D, key_cache.shape[1], key_cache.shape[0], float(scale),
        int(sliding_window), int(max_context_len), int(partition_size), _ptr(workspace), nbytes,
        _stream(dev)))


def paged_attention_decode_window_append(out, query, new_key, new_value, key_cache, value_cache,
                                         block_tables, context_lens, scale, gqa_factor,
                                         sliding_window):
    """Slot write of the new rows and direct decode over each row's
    ``sliding_window`` most recent positions, in one launch."""
    dev = _dev(out, query, new_key, new_value, key_cache, value_cache, block_tables, context_lens)
    args = _append_args(out, query, new_key, new_value, key_cache, value_cache, block_tables,
                        context_lens, gqa_factor)
    _check(lib.paged_attention_decode_window_append(*args, float(scale), int(sliding_window),
                                                    _stream(dev)))


def paged_attention_decode_splitkv_window_append(out, query, new_key, new_value, key_cache,
                                                 value_cache, block_tables, context_lens, scale,
                                                 gqa_factor, sliding_window, max_context_len,
                                                 partition_size, workspace):
    """Slot write of the new rows and windowed split-KV decode (partition
    kernel, then the merge)."""
    dev = _dev(out, query, new_key, new_value, key_cache, value_cache, block_tables, context_lens,
               workspace)
    args = _append_args(out, query, new_key, new_value, key_cache, value_cache, block_tables,
                        context_lens, gqa_factor)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.paged_attention_decode_splitkv_window_append(
        *args, float(scale), int(sliding_window), int(max_context_len), int(partition_size),
        _ptr(workspace), nbytes, _stream(dev)))


def gather_kv_cache(key_cache, value_cache, block_tables, cu_seq_lens, max_seq_len, key_out,
                    value_out):
    """Copy each sequence's cached rows into packed [total_tokens, Hkv, D]
    outputs: sequence b fills rows cu_seq_lens[b] .. cu_seq_lens[b+1] - 1."""
    torch = _torch()
    dev = _dev(key_cache, value_cache, block_tables, cu_seq_lens, key_out, value_out)
    _expect(key_cache.dim() == 4 and key_cache.shape == value_cache.shape,
            "caches must be [NB, 16, Hkv, D]")
    _expect(block_tables.dtype == torch.int32 and block_tables.dim() == 2,
            "block_tables must be int32 [B, max_blocks]")
    _expect(cu_seq_lens.dtype == torch.int32 and cu_seq_lens.shape == (block_tables.shape[0] + 1,),
            "cu_seq_lens must be int32 [B + 1]")
    _expect(key_out.shape == value_out.shape and key_out.shape[1:] == key_cache.shape[2:],
            "outputs must be [total_tokens, Hkv, D]")
    _expect(key_out.dtype == value_out.dtype == key_cache.dtype == value_cache.dtype,
            "output/cache dtype mismatch")
    _check(lib.gather_kv_cache(
        _ptr(key_cache), _ptr(value_cache), _dtype_code(key_cache), _ptr(block_tables),
        block_tables.shape[1], _ptr(cu_seq_lens), block_tables.shape[0], int(max_seq_len),
        _ptr(key_out), _ptr(value_out), key_out.shape[0], key_cache.shape[2], key_cache.shape[3],
        key_cache.shape[1], key_cache.shape[0], _stream(dev)))


def cascade_workspace_size(batch, q_len, num_q_heads, head_dim, max_context_len, max_prefix_len,
                           partition_size) -> int:
    n = _sz(0)
    _check(lib.paged_attention_decode_cascade_workspace_size(
        batch, q_len, num_q_heads, head_dim, max_context_len, max_prefix_len, partition_size,
        ctypes.byref(n)))
    return n.value


def paged_attention_decode_cascade(out, query, key_cache, value_cache, block_tables, context_lens,
                                   scale, gqa_factor, group_members, group_prefix_blocks,
                                   max_prefix_len, max_context_len, partition_size, workspace):
    """Split-KV decode reading each group's shared prefix once (prefix pass,
    suffix pass, merge).  group_members: int32 [groups, group_size];
    group_prefix_blocks: int32 [groups]."""
    torch = _torch()
    dev = _dev(out, query, key_cache, value_cache, block_tables, context_lens, group_members,
               group_prefix_blocks, workspace)
    B, Q, Hq, D = _attn_common(out, query, block_tables, context_lens, gqa_factor)
    _expect(key_cache.shape == value_cache.shape and key_cache.shape[2:] == (Hq // gqa_factor, D),
            "caches must be [NB, 16, Hq/G, D]")
    _expect(query.dtype == key_cache.dtype == value_cache.dtype, "query/cache dtype mismatch")
    _expect(group_members.dtype == torch.int32 and group_members.dim() == 2,
            "group_members must be int32 [groups, group_size]")
    _expect(group_prefix_blocks.dtype == torch.int32
            and group_prefix_blocks.shape == (group_members.shape[0],),
            "group_prefix_blocks must be int32 [groups]")
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.paged_attention_decode_cascade(
        _ptr(out), _dtype_code(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
        _dtype_code(key_cache), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        B, Q, Hq, gqa_factor, D, key_cache.shape[1], key_cache.shape[0], float(scale),
        _ptr(group_members), _ptr(group_prefix_blocks), group_members.shape[0],
        group_members.shape[1], int(max_prefix_len), int(max_context_len), int(partition_size),
        _ptr(workspace), nbytes, _stream(dev)))


def paged_attention_decode_splitkv_sparse_v(out, query, key_cache, value_cache, block_tables,
                                            context_lens, scale, gqa_factor, v_threshold,
                                            max_context_len, partition_size, workspace,
                                            v_rows_read=None):
    """Approximate split-KV decode that reads a V row only if some query row
    weighs it at least ``v_threshold`` of its running maximum.  ``v_rows_read``
    (int64 [1], optional) accumulates the number of V rows read."""
    torch = _torch()
    dev = _dev(out, query, key_cache, value_cache, block_tables, context_lens, workspace,
               v_rows_read)
    B, Q, Hq, D = _attn_common(out, query, block_tables, context_lens, gqa_factor)
    _expect(key_cache.shape == value_cache.shape and key_cache.shape[2:] == (Hq // gqa_factor, D),
            "caches must be [NB, 16, Hq/G, D]")
    _expect(query.dtype == key_cache.dtype == value_cache.dtype, "query/cache dtype mismatch")
    _expect(v_rows_read is None or (v_rows_read.dtype == torch.int64 and v_rows_read.numel() == 1),
            "v_rows_read must be an int64 tensor of one element")
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.paged_attention_decode_splitkv_sparse_v(
        _ptr(out), _dtype_code(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
        _dtype_code(key_cache), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        B, Q, Hq, gqa_factor, D, key_cache.shape[1], key_cache.shape[0], float(scale),
        float(v_threshold), _ptr(v_rows_read), int(max_context_len), int(partition_size),
        _ptr(workspace), nbytes, _stream(dev)))


def _k8v4_check(query, gqa_factor, k_cache, k_scale, v_cache, v_scale, v_zero):
    torch = _torch()
    B, Q, Hq, D = query.shape
    nb, bs, hkv = k_cache.shape[:3]
    _expect(hkv * gqa_factor == Hq, "k_cache heads must be Hq / gqa_factor")
    _expect(k_cache.dtype == torch.int8 and k_cache.shape == (nb, bs, hkv, D), "k_cache int8 [NB,16,Hkv,D]")
    _expect(k_scale.dtype == torch.float16 and k_scale.shape == (nb, bs, hkv), "k_scale f16 [NB,16,Hkv]")
    _expect(v_cache.dtype == torch.uint8 and v_cache.shape == (nb, bs, hkv, D // 2), "v_cache u8 [NB,16,Hkv,D/2]")
    for t in (v_scale, v_zero):
        _expect(t.dtype == torch.float16 and t.shape == (nb, bs, hkv, D // 32), "v_scale/v_zero f16 [NB,16,Hkv,D/32]")
    return nb, bs


def paged_attention_decode_k8v4(out, query, k_cache, k_scale, v_cache, v_scale, v_zero,
                                block_tables, context_lens, scale, gqa_factor):
    dev = _dev(out, query, k_cache, k_scale, v_cache, v_scale, v_zero, block_tables, context_lens)
    B, Q, Hq, D = _attn_common(out, query, block_tables, context_lens, gqa_factor)
    nb, bs = _k8v4_check(query, gqa_factor, k_cache, k_scale, v_cache, v_scale, v_zero)
    _check(lib.paged_attention_decode_k8v4(
        _ptr(out), _dtype_code(out), _ptr(query), _dtype_code(query), _ptr(k_cache), _ptr(k_scale),
        _ptr(v_cache), _ptr(v_scale), _ptr(v_zero), _ptr(block_tables), block_tables.shape[1],
        _ptr(context_lens), B, Q, Hq, gqa_factor, D, bs, nb, float(scale), _stream(dev)))


def paged_attention_decode_splitkv_k8v4(out, query, k_cache, k_scale, v_cache, v_scale, v_zero,
                                        block_tables, context_lens, scale, gqa_factor,
                                        max_context_len, partition_size, workspace):
    dev = _dev(out, query, k_cache, k_scale, v_cache, v_scale, v_zero, block_tables, context_lens,
               workspace)
    B, Q, Hq, D = _attn_common(out, query, block_tables, context_lens, gqa_factor)
    nb, bs = _k8v4_check(query, gqa_factor, k_cache, k_scale, v_cache, v_scale, v_zero)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.paged_attention_decode_splitkv_k8v4(
        _ptr(out), _dtype_code(out), _ptr(query), _dtype_code(query), _ptr(k_cache), _ptr(k_scale),
        _ptr(v_cache), _ptr(v_scale), _ptr(v_zero), _ptr(block_tables), block_tables.shape[1],
        _ptr(context_lens), B, Q, Hq, gqa_factor, D, bs, nb, float(scale), int(max_context_len),
        int(partition_size), _ptr(workspace), nbytes, _stream(dev)))


def _k8v4_append_check(query, new_key, new_value, k_cache):
    B, Q, Hq, D = query.shape
    hkv = k_cache.shape[2]
    for t in (new_key, new_value):
        _expect(t.shape == (B * Q, hkv, D) and t.dtype == query.dtype and t.is_contiguous(),
                "new_key / new_value must be [batch * q_len, Hkv, D] of the query dtype")


def paged_attention_decode_k8v4_append(out, query, new_key, new_value, k_cache, k_scale, v_cache,
                                       v_scale, v_zero, block_tables, context_lens, scale,
                                       gqa_factor):
    """Quantize-on-write of the new rows and K8/V4 decode, one launch."""
    dev = _dev(out, query, new_key, new_value, k_cache, k_scale, v_cache, v_scale, v_zero,
               block_tables, context_lens)
    B, Q, Hq, D = _attn_common(out, query, block_tables, context_lens, gqa_factor)
    nb, bs = _k8v4_check(query, gqa_factor, k_cache, k_scale, v_cache, v_scale, v_zero)
    _k8v4_append_check(query, new_key, new_value, k_cache)
    _check(lib.paged_attention_decode_k8v4_append(
        _ptr(out), _dtype_code(out), _ptr(query), _dtype_code(query), _ptr(new_key),
        _ptr(new_value), _ptr(k_cache), _ptr(k_scale), _ptr(v_cache), _ptr(v_scale), _ptr(v_zero),
        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), B, Q, Hq, gqa_factor, D,
        bs, nb, float(scale), _stream(dev)))


def paged_attention_decode_splitkv_k8v4_append(out, query, new_key, new_value, k_cache, k_scale,
                                               v_cache, v_scale, v_zero, block_tables,
                                               context_lens, scale, gqa_factor, max_context_len,
                                               partition_size, workspace):
    """Quantize-on-write of the new rows and split-KV K8/V4 decode (partition
    kernel, then the merge)."""
    dev = _dev(out, query, new_key, new_value, k_cache, k_scale, v_cache, v_scale, v_zero,
               block_tables, context_lens, workspace)
    B, Q, Hq, D = _attn_common(out, query, block_tables, context_lens, gqa_factor)
    nb, bs = _k8v4_check(query, gqa_factor, k_cache, k_scale, v_cache, v_scale, v_zero)
    _k8v4_append_check(query, new_key, new_value, k_cache)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.paged_attention_decode_splitkv_k8v4_append(
        _ptr(out), _dtype_code(out), _ptr(query), _dtype_code(query), _ptr(new_key),
        _ptr(new_value), _ptr(k_cache), _ptr(k_scale), _ptr(v_cache), _ptr(v_scale), _ptr(v_zero),
        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), B, Q, Hq, gqa_factor, D,
        bs, nb, float(scale), int(max_context_len), int(partition_size), _ptr(workspace), nbytes,
        _stream(dev)))


def paged_attention_decode_splitkv_partials(query, key_cache, value_cache, block_tables,
                                            context_lens, scale, gqa_factor, max_context_len,
                                            partition_size, workspace):
    """Partition kernel only: per-partition (o, m, l) into ``workspace``."""
    dev = _dev(query, key_cache, value_cache, block_tables, context_lens, workspace)
    B, Q, Hq, D = _attn_common(query, query, block_tables, context_lens, gqa_factor)
    _expect(key_cache.shape == value_cache.shape and key_cache.shape[2:] == (Hq // gqa_factor, D),
            "caches must be [NB, 16, Hq/G, D]")
    _expect(query.dtype == key_cache.dtype == value_cache.dtype, "query/cache dtype mismatch")
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.paged_attention_decode_splitkv_partials(
        _ptr(query), _ptr(key_cache), _ptr(value_cache), _dtype_code(key_cache),
        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), B, Q, Hq, gqa_factor, D,
        key_cache.shape[1], key_cache.shape[0], float(scale), int(max_context_len),
        int(partition_size), _ptr(workspace), nbytes, _stream(dev)))


def paged_attention_decode_splitkv_k8v4_partials(query, k_cache, k_scale, v_cache, v_scale, v_zero,
                                                 block_tables, context_lens, scale, gqa_factor,
                                                 max_context_len, partition_size, workspace):
    dev = _dev(query, k_cache, k_scale, v_cache, v_scale, v_zero, block_tables, context_lens,
               workspace)
    B, Q, Hq, D = _attn_common(query, query, block_tables, context_lens, gqa_factor)
    nb, bs = _k8v4_check(query, gqa_factor, k_cache, k_scale, v_cache, v_scale, v_zero)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.paged_attention_decode_splitkv_k8v4_partials(
        _ptr(query), _dtype_code(query), _ptr(k_cache), _ptr(k_scale), _ptr(v_cache),
        _ptr(v_scale), _ptr(v_zero), _ptr(block_tables), block_tables.shape[1],
        _ptr(context_lens), B, Q, Hq, gqa_factor, D, bs, nb, float(scale), int(max_context_len),
        int(partition_size), _ptr(workspace), nbytes, _stream(dev)))


def paged_attention_decode_splitkv_merge(out, max_context_len, partition_size, workspace):
    """Log-sum-exp merge of the partials in ``workspace`` into ``out`` [B, Q, Hq, D]."""
    dev = _dev(out, workspace)
    _expect(out.dim() == 4, "out must be [B, Q, Hq, D]")
    B, Q, Hq, D = out.shape
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.paged_attention_decode_splitkv_merge(
        _ptr(out), _dtype_code(out), B, Q, Hq, D, int(max_context_len), int(partition_size),
        _ptr(workspace), nbytes, _stream(dev)))

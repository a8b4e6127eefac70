// C ABI of the paged-KV decode library (declared in include/pagedkv.h).
//
// Every entry point validates its arguments on the host first (no HIP call is
// made before validation passes), then enqueues kernels on the caller's stream.
// Nothing is allocated, freed or synchronised here.

#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "../../include/pagedkv.h"
#include "pkv_common.h"
#include "pkv_launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return PKV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int launch_result(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PKV_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

int check_cache_geometry(int num_kv_heads, int head_dim, int block_size, int64_t num_blocks) {
  if (num_kv_heads <= 0) return fail(PKV_ERR_SHAPE, "num_kv_heads must be positive");
  if (num_blocks < 0) return fail(PKV_ERR_SHAPE, "num_blocks must be non-negative");
  if (block_size != 16) return fail(PKV_ERR_UNSUPPORTED, "block_size must be 16 (got %d)", block_size);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  return PKV_OK;
}

// Shared validation of the attention calls; fills the kernel arguments.
int check_attention(void* out, int out_dtype, const void* query, const void* k_cache,
                    const void* v_cache, const int32_t* block_tables, int max_blocks,
                    const int32_t* context_lens, int batch, int q_len, int num_q_heads,
                    int gqa_factor, int head_dim, int block_size, int64_t num_blocks, float scale,
                    pkv::AttnArgs& a, bool need_out = true) {
  if (batch < 0 || q_len <= 0 || num_q_heads <= 0 || gqa_factor <= 0 || max_blocks < 0)
    return fail(PKV_ERR_SHAPE, "batch >= 0, q_len > 0, num_q_heads > 0, gqa_factor > 0, "
                               "max_blocks_per_seq >= 0 required");
  if (num_q_heads % gqa_factor != 0)
    return fail(PKV_ERR_UNSUPPORTED, "num_q_heads (%d) must be a multiple of gqa_factor (%d)",
                num_q_heads, gqa_factor);
  const int hkv = num_q_heads / gqa_factor;
  int rc = check_cache_geometry(hkv, head_dim, block_size, num_blocks);
  if (rc) return rc;
  if ((int64_t)gqa_factor * q_len > 16)
    return fail(PKV_ERR_UNSUPPORTED, "gqa_factor * q_len must be <= 16 (got %d)",
                gqa_factor * q_len);
  if (need_out && out_dtype != PKV_F16 && out_dtype != PKV_BF16 && out_dtype != PKV_F32)
    return fail(PKV_ERR_UNSUPPORTED, "out_dtype must be PKV_F16, PKV_BF16 or PKV_F32");
  if (!std::isfinite(scale)) return fail(PKV_ERR_SHAPE, "scale must be finite");
  if (batch > 65535 || hkv > 65535) return fail(PKV_ERR_UNSUPPORTED, "batch or KV heads too large");
  if (max_blocks > (1 << 26)) return fail(PKV_ERR_UNSUPPORTED, "max_blocks_per_seq above 2^26");
  if (batch == 0) return PKV_OK;
  if ((need_out && !out) || !query || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PKV_ERR_NULL, "a required pointer is NULL");
  if (!aligned16(query) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_ERR_ALIGN, "query and caches must be 16-byte aligned");
  if (num_blocks == 0 || max_blocks == 0)
    return fail(PKV_ERR_SHAPE, "num_blocks and max_blocks_per_seq must be positive when batch > 0");
  a = pkv::AttnArgs{};
  a.out = out;
  a.out_dtype = out_dtype;
  a.q = query;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.max_blocks = max_blocks;
  a.batch = batch;
  a.q_len = q_len;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = hkv;
  a.gqa = gqa_factor;
  a.num_blocks = num_blocks;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.part_blocks = max_blocks;
  a.num_parts = 1;
  return PKV_OK;
}

// partition_size 0 (where `balanced` allows it) asks for the balanced split:
// parts = 0 and bytes = its workspace, (runs + batch) * num_q_heads * q_len
// partial rows of head_dim + 2 floats.
int split_geometry(int batch, int q_len, int num_q_heads, int head_dim, int max_context_len,
                   int partition_size, int64_t& parts, size_t& bytes, bool balanced = false) {
  if (batch < 0 || q_len <= 0 || num_q_heads <= 0 || max_context_len < 0)
    return fail(PKV_ERR_SHAPE, "invalid split-KV sizes");
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  if (partition_size == 0 && balanced) {
    const int runs = pkv::flat_runs_for(num_q_heads);
    if (runs < 8)
      return fail(PKV_ERR_UNSUPPORTED, "balanced split: num_q_heads must be at most %d",
                  pkv::kFlatQueryWaves / 8);
    if (batch > 65535)
      return fail(PKV_ERR_UNSUPPORTED, "balanced split: batch must be at most 65535 (got %d)",
                  batch);
    parts = 0;
    bytes = (size_t)((int64_t)(runs + batch) * num_q_heads * q_len * (head_dim + 2) * 4);
    return PKV_OK;
  }
  if (partition_size <= 0 || partition_size % 16 != 0)
    return fail(PKV_ERR_UNSUPPORTED, "partition_size must be a positive multiple of 16 (got %d)%s",
                partition_size, partition_size == 0 ? "; 0 (balanced split) is not supported here"
                                                    : "");
  parts = ((int64_t)max_context_len + partition_size - 1) / partition_size;
  if (parts < 1) parts = 1;
  if (parts > 65535) return fail(PKV_ERR_UNSUPPORTED, "too many partitions (%lld)", (long long)parts);
  const int64_t rows = (int64_t)batch * q_len * num_q_heads;
  bytes = (size_t)(rows * parts * (head_dim + 2) * 4);
  return PKV_OK;
}

int setup_split(pkv::AttnArgs& a, int head_dim, int max_context_len, int partition_size,
                void* workspace, size_t workspace_bytes, bool balanced = false) {
  int64_t parts = 0;
  size_t need = 0;
  int rc = split_geometry(a.batch, a.q_len, a.num_q_heads, head_dim, max_context_len,
                          partition_size, parts, need, balanced);
  if (rc) return rc;
  if (!workspace) return fail(PKV_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned16(workspace)) return fail(PKV_ERR_ALIGN, "workspace must be 16-byte aligned");
  if (workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "workspace too small: %zu bytes given, %zu needed",
                workspace_bytes, need);
  if (parts == 0) {                       // balanced split
    // flattened block positions are 32-bit in the kernels
    if ((int64_t)a.batch * a.max_blocks > 0x7fffffffLL)
      return fail(PKV_ERR_UNSUPPORTED, "balanced split: batch * max_blocks_per_seq above 2^31");
    // the merge runs one 512-thread workgroup per (sequence, KV head)
    if ((int64_t)a.batch * a.num_kv_heads * 512 > 0xffffffffLL)
      return fail(PKV_ERR_UNSUPPORTED, "balanced split: batch * num_kv_heads above 2^23");
    const int runs = pkv::flat_runs_for(a.num_q_heads);
    const int64_t rows = (int64_t)(runs + a.batch) * a.num_q_heads * a.q_len;
    a.flat_runs = runs;
    a.num_parts = 1;
    a.ws_parts = 0;
    a.part_base = 0;
    a.part_blocks = a.max_blocks;
    a.ws_o = (float*)workspace;
    a.ws_m = a.ws_o + rows * head_dim;
    a.ws_l = a.ws_m + rows;
    return PKV_OK;
  }
  const int64_t rows = (int64_t)a.batch * a.q_len * a.num_q_heads;
  a.num_parts = (int)parts;
  a.ws_parts = (int)parts;
  a.part_base = 0;
  a.part_blocks = partition_size / 16;
  a.ws_o = (float*)workspace;
  a.ws_m = a.ws_o + rows * parts * head_dim;
  a.ws_l = a.ws_m + rows * parts;
  return PKV_OK;
}

int check_k8v4_pointers(const void* k_scale, const void* v_scale, const void* v_zero) {
  if (!k_scale || !v_scale || !v_zero) return fail(PKV_ERR_NULL, "K8/V4 scale arrays are NULL");
  if ((reinterpret_cast<uintptr_t>(k_scale) & 1u) || (reinterpret_cast<uintptr_t>(v_scale) & 7u) ||
      (reinterpret_cast<uintptr_t>(v_zero) & 7u))
    return fail(PKV_ERR_ALIGN, "k_scale must be 2-byte and v_scale/v_zero 8-byte aligned");
  return PKV_OK;
}

// Split-KV partials of paged_attention_decode_splitkv_noalloc: one static
// device array per GPU the library runs on, held until the process ends.  Its
// name is only a host-side handle; kernels get its device address, looked up
// once per device (with that device current) and kept per device.
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PKV_ERR_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(PKV_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(PKV_ERR_LAUNCH, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_err; }

int pkv_version(void) { return 100; }

int kv_cache_bytes_per_token(int num_layers, int num_kv_heads, int head_dim, int kv_format,
                             int64_t* out_bytes) {
  if (!out_bytes) return fail(PKV_ERR_NULL, "out_bytes is NULL");
  if (num_layers < 0 || num_kv_heads < 0 || head_dim < 0)
    return fail(PKV_ERR_SHAPE, "sizes must be non-negative");
  const int64_t lh = (int64_t)num_layers * num_kv_heads;
  if (kv_format == PKV_FMT_F16 || kv_format == PKV_FMT_BF16) {
    *out_bytes = 2 * lh * head_dim * 2;
  } else if (kv_format == PKV_FMT_K8V4) {
    if (head_dim % 32) return fail(PKV_ERR_UNSUPPORTED, "K8/V4 needs head_dim % 32 == 0");
    *out_bytes = lh * (head_dim + 2 + head_dim / 2 + 4 * (head_dim / 32));
  } else {
    return fail(PKV_ERR_UNSUPPORTED, "unknown kv_format %d", kv_format);
  }
  return ok();
}

int kv_cache_write(const void* key, const void* value, void* key_cache, void* value_cache,
                   const int64_t* slot_mapping, int64_t num_tokens, int num_kv_heads,
                   int head_dim, int block_size, int64_t num_blocks, int dtype, void* stream) {
  if (num_tokens < 0) return fail(PKV_ERR_SHAPE, "num_tokens must be non-negative");
  int rc = check_cache_geometry(num_kv_heads, head_dim, block_size, num_blocks);
  if (rc) return rc;
  if (dtype != PKV_F16 && dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "dtype must be PKV_F16 or PKV_BF16");
  if (num_tokens > 0x7fffffff) return fail(PKV_ERR_UNSUPPORTED, "too many tokens");
  if (num_tokens == 0 || num_blocks == 0) return ok();
  if (!key || !value || !key_cache || !value_cache || !slot_mapping)
    return fail(PKV_ERR_NULL, "a required pointer is NULL");
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache))
    return fail(PKV_ERR_ALIGN, "key, value and caches must be 16-byte aligned");
  return launch_result(pkv::launch_kv_write(key, value, key_cache, value_cache, slot_mapping,
                                            num_tokens, num_kv_heads, head_dim, num_blocks,
                                            (hipStream_t)stream),
                       "kv_cache_write");
}

int gather_kv_cache(const void* key_cache, const void* value_cache, int dtype,
                    const int32_t* block_tables, int max_blocks_per_seq,
                    const int32_t* cu_seq_lens, int batch, int max_seq_len, void* key_out,
                    void* value_out, int64_t total_tokens, int num_kv_heads, int head_dim,
                    int block_size, int64_t num_blocks, void* stream) {
  int rc = check_cache_geometry(num_kv_heads, head_dim, block_size, num_blocks);
  if (rc) return rc;
  if (dtype != PKV_F16 && dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "dtype must be PKV_F16 or PKV_BF16");
  if (batch < 0 || max_blocks_per_seq < 0 || max_seq_len < 0 || total_tokens < 0)
    return fail(PKV_ERR_SHAPE, "batch, max_blocks_per_seq, max_seq_len and total_tokens must "
                               "be non-negative");
  if (batch > 65535) return fail(PKV_ERR_UNSUPPORTED, "batch too large");
  if (max_blocks_per_seq > (1 << 26))
    return fail(PKV_ERR_UNSUPPORTED, "max_blocks_per_seq above 2^26");
  if (batch == 0 || total_tokens == 0 || max_seq_len == 0 || max_blocks_per_seq == 0)
    return ok();
  if (!key_cache || !value_cache || !block_tables || !cu_seq_lens || !key_out || !value_out)
    return fail(PKV_ERR_NULL, "a required pointer is NULL");
  if (!aligned16(key_cache) || !aligned16(value_cache) || !aligned16(key_out) ||
      !aligned16(value_out))
    return fail(PKV_ERR_ALIGN, "caches and outputs must be 16-byte aligned");
  return launch_result(pkv::launch_gather(key_cache, value_cache, block_tables,
                                          max_blocks_per_seq, cu_seq_lens, batch, max_seq_len,
                                          total_tokens, num_kv_heads, head_dim, num_blocks,
                                          key_out, value_out, (hipStream_t)stream),
                       "gather_kv_cache");
}

int kv_cache_write_k8v4(const void* key, const void* value, int in_dtype, int8_t* k_cache,
                        void* k_scale, uint8_t* v_cache, void* v_scale, void* v_zero,
                        const int64_t* slot_mapping, int64_t num_tokens, int num_kv_heads,
                        int head_dim, int block_size, int64_t num_blocks, void* stream) {
  if (num_tokens < 0) return fail(PKV_ERR_SHAPE, "num_tokens must be non-negative");
  int rc = check_cache_geometry(num_kv_heads, head_dim, block_size, num_blocks);
  if (rc) return rc;
  if (in_dtype != PKV_F16 && in_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "in_dtype must be PKV_F16 or PKV_BF16");
  if (num_tokens * num_kv_heads > 0x7fffffffLL * 4)
    return fail(PKV_ERR_UNSUPPORTED, "too many tokens");
  if (num_tokens == 0 || num_blocks == 0) return ok();
  if (!key || !value || !k_cache || !v_cache || !slot_mapping)
    return fail(PKV_ERR_NULL, "a required pointer is NULL");
  rc = check_k8v4_pointers(k_scale, v_scale, v_zero);
  if (rc) return rc;
  return launch_result(pkv::launch_kv_write_k8v4(key, value, in_dtype, k_cache, k_scale, v_cache,
                                                 v_scale, v_zero, slot_mapping, num_tokens,
                                                 num_kv_heads, head_dim, num_blocks,
                                                 (hipStream_t)stream),
                       "kv_cache_write_k8v4");
}

int paged_attention_decode(void* out, int out_dtype, const void* query, const void* key_cache,
                           const void* value_cache, int kv_dtype, const int32_t* block_tables,
                           int max_blocks_per_seq, const int32_t* context_lens, int batch,
                           int q_len, int num_q_heads, int gqa_factor, int head_dim,
                           int block_size, int64_t num_blocks, float scale, void* stream) {
  if (kv_dtype != PKV_F16 && kv_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "kv_dtype must be PKV_F16 or PKV_BF16");
  pkv::AttnArgs a{};
  int rc = check_attention(out, out_dtype, query, key_cache, value_cache, block_tables,
                           max_blocks_per_seq, context_lens, batch, q_len, num_q_heads, gqa_factor,
                           head_dim, block_size, num_blocks, scale, a);
  if (rc) return rc;
  if (batch == 0) return ok();
  return launch_result(pkv::launch_attention(a, kv_dtype, kv_dtype, head_dim, (hipStream_t)stream),
                       "paged_attention_decode");
}

int paged_attention_decode_splitkv_workspace_size(int batch, int q_len, int num_q_heads,
                                                  int head_dim, int max_context_len,
                                                  int partition_size, size_t* out_bytes) {
  if (!out_bytes) return fail(PKV_ERR_NULL, "out_bytes is NULL");
  int64_t parts = 0;
  size_t bytes = 0;
  int rc = split_geometry(batch, q_len, num_q_heads, head_dim, max_context_len, partition_size,
                          parts, bytes, true);
  if (rc) return rc;
  *out_bytes = bytes;
  return ok();
}

int paged_attention_decode_splitkv(void* out, int out_dtype, const void* query,
                                   const void* key_cache, const void* value_cache, int kv_dtype,
                                   const int32_t* block_tables, int max_blocks_per_seq,
                                   const int32_t* context_lens, int batch, int q_len,
                                   int num_q_heads, int gqa_factor, int head_dim, int block_size,
                                   int64_t num_blocks, float scale, int max_context_len,
                                   int partition_size, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (kv_dtype != PKV_F16 && kv_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "kv_dtype must be PKV_F16 or PKV_BF16");
  pkv::AttnArgs a{};
  int rc = check_attention(out, out_dtype, query, key_cache, value_cache, block_tables,
                           max_blocks_per_seq, context_lens, batch, q_len, num_q_heads, gqa_factor,
                           head_dim, block_size, num_blocks, scale, a);
  if (rc) return rc;
  if (batch == 0) return ok();
  rc = setup_split(a, head_dim, max_context_len, partition_size, workspace, workspace_bytes, true);
  if (rc) return rc;
  return launch_result(pkv::launch_attention(a, kv_dtype, kv_dtype, head_dim, (hipStream_t)stream),
                       "paged_attention_decode_splitkv");
}

int paged_attention_decode_splitkv_noalloc(void* out, int out_dtype, const void* query,
                                           const void* key_cache, const void* value_cache,
                                           int kv_dtype, const int32_t* block_tables,
                                           int max_blocks_per_seq, const int32_t* context_lens,
                                           int batch, int q_len, int num_q_heads, int gqa_factor,
                                           int head_dim, int block_size, int64_t num_blocks,
                                           float scale, int max_context_len, int partition_size,
                                           void* stream) {
  if (kv_dtype != PKV_F16 && kv_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "kv_dtype must be PKV_F16 or PKV_BF16");
  pkv::AttnArgs a{};
  int rc = check_attention(out, out_dtype, query, key_cache, value_cache, block_tables,
                           max_blocks_per_seq, context_lens, batch, q_len, num_q_heads, gqa_factor,
                           head_dim, block_size, num_blocks, scale, a);
  if (rc) return rc;
  if (batch == 0) return ok();
  int64_t parts = 0;
  size_t need = 0;
  rc = split_geometry(batch, q_len, num_q_heads, head_dim, max_context_len, partition_size, parts,
                      need, true);
  if (rc) return rc;
  if (need > (size_t)PKV_NOALLOC_SCRATCH_BYTES)
    return fail(PKV_ERR_WORKSPACE,
                "the partials need %zu bytes, more than the %zu-byte static scratch holds "
                "(use paged_attention_decode_splitkv with a workspace)",
                need, (size_t)PKV_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc) return rc;
  rc = setup_split(a, head_dim, max_context_len, partition_size, ws, PKV_NOALLOC_SCRATCH_BYTES, true);
  if (rc) return rc;
  return launch_result(pkv::launch_attention(a, kv_dtype, kv_dtype, head_dim, (hipStream_t)stream),
                       "paged_attention_decode_splitkv_noalloc");
}

int paged_attention_decode_window(void* out, int out_dtype, const void* query,
                                  const void* key_cache, const void* value_cache, int kv_dtype,
                                  const int32_t* block_tables, int max_blocks_per_seq,
                                  const int32_t* context_lens, int batch, int q_len,
                                  int num_q_heads, int gqa_factor, int head_dim, int block_size,
                                  int64_t num_blocks, float scale, int sliding_window,
                                  void* stream) {
  if (kv_dtype != PKV_F16 && kv_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "kv_dtype must be PKV_F16 or PKV_BF16");
  if (sliding_window < 0) return fail(PKV_ERR_SHAPE, "sliding_window must be >= 0");
  pkv::AttnArgs a{};
  int rc = check_attention(out, out_dtype, query, key_cache, value_cache, block_tables,
                           max_blocks_per_seq, context_lens, batch, q_len, num_q_heads, gqa_factor,
                           head_dim, block_size, num_blocks, scale, a);
  if (rc) return rc;
  if (batch == 0) return ok();
  a.window = sliding_window;
  return launch_result(pkv::launch_attention(a, kv_dtype, kv_dtype, head_dim, (hipStream_t)stream),
                       "paged_attention_decode_window");
}

int paged_attention_decode_splitkv_window(void* out, int out_dtype, const void* query,
                                          const void* key_cache, const void* value_cache,
                                          int kv_dtype, const int32_t* block_tables,
                                          int max_blocks_per_seq, const int32_t* context_lens,
                                          int batch, int q_len, int num_q_heads, int gqa_factor,
                                          int head_dim, int block_size, int64_t num_blocks,
                                          float scale, int sliding_window, int max_context_len,
                                          int partition_size, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  if (kv_dtype != PKV_F16 && kv_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "kv_dtype must be PKV_F16 or PKV_BF16");
  if (sliding_window < 0) return fail(PKV_ERR_SHAPE, "sliding_window must be >= 0");
  pkv::AttnArgs a{};
  int rc = check_attention(out, out_dtype, query, key_cache, value_cache, block_tables,
                           max_blocks_per_seq, context_lens, batch, q_len, num_q_heads, gqa_factor,
                           head_dim, block_size, num_blocks, scale, a);
  if (rc) return rc;
  if (batch == 0) return ok();
  // partitions are counted from the first block of each sequence's window, so
  // the grid and the workspace only need to span the window
  const int span = sliding_window > 0
                       ? (int)std::min<int64_t>(max_context_len, (int64_t)sliding_window + q_len + 15)
                       : max_context_len;
  rc = setup_split(a, head_dim, span, partition_size, workspace, workspace_bytes);
  if (rc) return rc;
  a.window = sliding_window;
  return launch_result(pkv::launch_attention(a, kv_dtype, kv_dtype, head_dim, (hipStream_t)stream),
                       "paged_attention_decode_splitkv_window");
}

int paged_attention_decode_window_append(void* out, int out_dtype, const void* query,
                                         const void* new_key, const void* new_value,
                                         void* key_cache, void* value_cache, int kv_dtype,
                                         const int32_t* block_tables, int max_blocks_per_seq,
                                         const int32_t* context_lens, int batch, int q_len,
                                         int num_q_heads, int gqa_factor, int head_dim,
                                         int block_size, int64_t num_blocks, float scale,
                                         int sliding_window, void* stream) {
  if (kv_dtype != PKV_F16 && kv_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "kv_dtype must be PKV_F16 or PKV_BF16");
  if (sliding_window < 0) return fail(PKV_ERR_SHAPE, "sliding_window must be >= 0");
  pkv::AttnArgs a{};
  int rc = check_attention(out, out_dtype, query, key_cache, value_cache, block_tables,
                           max_blocks_per_seq, context_lens, batch, q_len, num_q_heads, gqa_factor,
                           head_dim, block_size, num_blocks, scale, a);
  if (rc) return rc;
  if (batch == 0) return ok();
  if (!new_key || !new_value) return fail(PKV_ERR_NULL, "new_key / new_value is NULL");
  if (!aligned16(new_key) || !aligned16(new_value))
    return fail(PKV_ERR_ALIGN, "new_key and new_value must be 16-byte aligned");
  a.window = sliding_window;
  a.new_k = new_key;
  a.new_v = new_value;
  return launch_result(pkv::launch_attention(a, kv_dtype, kv_dtype, head_dim, (hipStream_t)stream),
                       "paged_attention_decode_window_append");
}

int paged_attention_decode_splitkv_window_append(
    void* out, int out_dtype, const void* query, const void* new_key, const void* new_value,
    void* key_cache, void* value_cache, int kv_dtype, const int32_t* block_tables,
    int max_blocks_per_seq, const int32_t* context_lens, int batch, int q_len, int num_q_heads,
    int gqa_factor, int head_dim, int block_size, int64_t num_blocks, float scale,
    int sliding_window, int max_context_len, int partition_size, void* workspace,
    size_t workspace_bytes, void* stream) {
  if (kv_dtype != PKV_F16 && kv_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "kv_dtype must be PKV_F16 or PKV_BF16");
  if (sliding_window < 0) return fail(PKV_ERR_SHAPE, "sliding_window must be >= 0");
  pkv::AttnArgs a{};
  int rc = check_attention(out, out_dtype, query, key_cache, value_cache, block_tables,
                           max_blocks_per_seq, context_lens, batch, q_len, num_q_heads, gqa_factor,
                           head_dim, block_size, num_blocks, scale, a);
  if (rc) return rc;
  if (batch == 0) return ok();
  if (!new_key || !new_value) return fail(PKV_ERR_NULL, "new_key / new_value is NULL");
  if (!aligned16(new_key) || !aligned16(new_value))
    return fail(PKV_ERR_ALIGN, "new_key and new_value must be 16-byte aligned");
  const int span = sliding_window > 0
                       ? (int)std::min<int64_t>(max_context_len, (int64_t)sliding_window + q_len + 15)
                       : max_context_len;
  rc = setup_split(a, head_dim, span, partition_size, workspace, workspace_bytes);
  if (rc) return rc;
  a.window = sliding_window;
  a.new_k = new_key;
  a.new_v = new_value;
  return launch_result(pkv::launch_attention(a, kv_dtype, kv_dtype, head_dim, (hipStream_t)stream),
                       "paged_attention_decode_splitkv_window_append");
}

// Cascade workspace: the prefix pass's partials ([rows][p_pre] slots, rows =
// batch * q_len * num_q_heads), then the balanced suffix pass's partials,
// then each sequence's suffix length and first suffix table entry (int32),
// every region starting on a 256-byte boundary.
struct CascadeLayout {
  int64_t p_pre = 0;
  size_t pre_bytes = 0, flat_bytes = 0, total = 0;
};

static size_t round256(size_t n) { return (n + 255) / 256 * 256; }

static int cascade_layout(int batch, int q_len, int num_q_heads, int head_dim,
                          int max_context_len, int max_prefix_len, int partition_size,
                          CascadeLayout& c) {
  if (max_prefix_len < 0) return fail(PKV_ERR_SHAPE, "max_prefix_len must be >= 0");
  int rc = split_geometry(batch, q_len, num_q_heads, head_dim, max_prefix_len, partition_size,
                          c.p_pre, c.pre_bytes);
  if (rc) return rc;
  int64_t parts = 0;
  rc = split_geometry(batch, q_len, num_q_heads, head_dim, max_context_len, 0, parts,
                      c.flat_bytes, true);
  if (rc) return rc;
  c.total = round256(c.pre_bytes) + round256(c.flat_bytes) + (size_t)batch * 2 * 4;
  return PKV_OK;
}

int paged_attention_decode_cascade_workspace_size(int batch, int q_len, int num_q_heads,
                                                  int head_dim, int max_context_len,
                                                  int max_prefix_len, int partition_size,
                                                  size_t* out_bytes) {
  if (!out_bytes) return fail(PKV_ERR_NULL, "out_bytes is NULL");
  CascadeLayout c;
  int rc = cascade_layout(batch, q_len, num_q_heads, head_dim, max_context_len, max_prefix_len,
                          partition_size, c);
  if (rc) return rc;
  *out_bytes = c.total;
  return ok();
}

int paged_attention_decode_cascade(void* out, int out_dtype, const void* query,
                                   const void* key_cache, const void* value_cache, int kv_dtype,
                                   const int32_t* block_tables, int max_blocks_per_seq,
                                   const int32_t* context_lens, int batch, int q_len,
                                   int num_q_heads, int gqa_factor, int head_dim, int block_size,
                                   int64_t num_blocks, float scale, const int32_t* group_members,
                                   const int32_t* group_prefix_blocks, int num_groups,
                                   int group_size, int max_prefix_len, int max_context_len,
                                   int partition_size, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (kv_dtype != PKV_F16 && kv_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "kv_dtype must be PKV_F16 or PKV_BF16");
  if (num_groups < 0 || group_size < 0 || max_prefix_len < 0)
    return fail(PKV_ERR_SHAPE, "num_groups, group_size and max_prefix_len must be >= 0");
  if (num_groups > 65535) return fail(PKV_ERR_UNSUPPORTED, "too many groups");
  if (num_groups > 0 && ((int64_t)group_size * gqa_factor * q_len > 16 || group_size == 0))
    return fail(PKV_ERR_UNSUPPORTED,
                "group_size * gqa_factor * q_len must be between 1 and 16 (got %lld)",
                (long long)group_size * gqa_factor * q_len);
  pkv::AttnArgs a{};
  int rc = check_attention(out, out_dtype, query, key_cache, value_cache, block_tables,
                           max_blocks_per_seq, context_lens, batch, q_len, num_q_heads, gqa_factor,
                           head_dim, block_size, num_blocks, scale, a);
  if (rc) return rc;
  if (batch == 0) return ok();
  if (num_groups > 0 && (!group_members || !group_prefix_blocks))
    return fail(PKV_ERR_NULL, "group arrays are NULL");
  CascadeLayout c;
  rc = cascade_layout(batch, q_len, num_q_heads, head_dim, max_context_len, max_prefix_len,
                      partition_size, c);
  if (rc) return rc;
  if (!workspace) return fail(PKV_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned16(workspace)) return fail(PKV_ERR_ALIGN, "workspace must be 16-byte aligned");
  if (workspace_bytes < c.total)
    return fail(PKV_ERR_WORKSPACE, "workspace too small: %zu bytes given, %zu needed",
                workspace_bytes, c.total);
  char* base = (char*)workspace;
  char* flat_ws = base + round256(c.pre_bytes);
  int32_t* suf_len = (int32_t*)(flat_ws + round256(c.flat_bytes));
  int32_t* suf_off = suf_len + batch;
  a.grp_members = group_members;
  a.grp_prefix = group_prefix_blocks;
  a.num_groups = num_groups;
  a.group_size = group_size;
  // the suffix pass: a balanced split over every sequence's positions past
  // its group's prefix (checked before anything is launched)
  pkv::AttnArgs suf = a;
  rc = setup_split(suf, head_dim, max_context_len, 0, flat_ws, c.flat_bytes, true);
  if (rc) return rc;
  suf.context_lens = suf_len;
  suf.tbl_off = suf_off;
  const int64_t rows = (int64_t)batch * q_len * num_q_heads;
  hipError_t e = hipSuccess;
  // 1. the shared prefixes, once per group, into their own partial slots
  if (num_groups > 0) {
    pkv::AttnArgs pre = a;
    pre.mode = 1;
    pre.num_parts = (int)c.p_pre;
    pre.ws_parts = (int)c.p_pre;
    pre.part_base = 0;
    pre.part_blocks = partition_size / 16;
    pre.ws_o = (float*)base;
    pre.ws_m = pre.ws_o + rows * c.p_pre * head_dim;
    pre.ws_l = pre.ws_m + rows * c.p_pre;
    e = pkv::launch_attention(pre, kv_dtype, kv_dtype, head_dim, (hipStream_t)stream,
                              pkv::STAGE_PARTIALS);
    if (e != hipSuccess) return launch_result(e, "paged_attention_decode_cascade (prefix)");
    suf.pre_o = pre.ws_o;
    suf.pre_m = pre.ws_m;
    suf.pre_l = pre.ws_l;
    suf.pre_parts = (int)c.p_pre;
  }
  // 2. each sequence's suffix length and first suffix table entry
  e = pkv::launch_cascade_suffix_prep(a, suf_len, suf_off, (hipStream_t)stream);
  if (e != hipSuccess) return launch_result(e, "paged_attention_decode_cascade (suffixes)");
  // 3. the balanced suffix pass and the merge of both passes' partials
  return launch_result(pkv::launch_attention(suf, kv_dtype, kv_dtype, head_dim,
                                             (hipStream_t)stream),
                       "paged_attention_decode_cascade");
}

int paged_attention_decode_splitkv_sparse_v(
    void* out, int out_dtype, const void* query, const void* key_cache, const void* value_cache,
    int kv_dtype, const int32_t* block_tables, int max_blocks_per_seq,
    const int32_t* context_lens, int batch, int q_len, int num_q_heads, int gqa_factor,
    int head_dim, int block_size, int64_t num_blocks, float scale, float v_threshold,
    unsigned long long* v_rows_read, int max_context_len, int partition_size, void* workspace,
    size_t workspace_bytes, void* stream) {
  if (kv_dtype != PKV_F16 && kv_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "kv_dtype must be PKV_F16 or PKV_BF16");
  if (!(v_threshold >= 0.f && v_threshold < 1.f))
    return fail(PKV_ERR_SHAPE, "v_threshold must be in [0, 1)");
  pkv::AttnArgs a{};
  int rc = check_attention(out, out_dtype, query, key_cache, value_cache, block_tables,
                           max_blocks_per_seq, context_lens, batch, q_len, num_q_heads, gqa_factor,
                           head_dim, block_size, num_blocks, scale, a);
  if (rc) return rc;
  if ((int64_t)gqa_factor * q_len > 4)
    return fail(PKV_ERR_UNSUPPORTED, "sparse-V needs gqa_factor * q_len <= 4");
  if (batch == 0) return ok();
  rc = setup_split(a, head_dim, max_context_len, partition_size, workspace, workspace_bytes);
  if (rc) return rc;
  a.v_log2_threshold = v_threshold > 0.f ? std::log2(v_threshold) : -INFINITY;
  a.v_rows_read = v_rows_read;
  return launch_result(pkv::launch_sparse_v(a, kv_dtype, head_dim, (hipStream_t)stream),
                       "paged_attention_decode_splitkv_sparse_v");
}

int paged_attention_decode_append(void* out, int out_dtype, const void* query,
                                  const void* new_key, const void* new_value, void* key_cache,
                                  void* value_cache, int kv_dtype, const int32_t* block_tables,
                                  int max_blocks_per_seq, const int32_t* context_lens, int batch,
                                  int q_len, int num_q_heads, int gqa_factor, int head_dim,
                                  int block_size, int64_t num_blocks, float scale, void* stream) {
  if (kv_dtype != PKV_F16 && kv_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "kv_dtype must be PKV_F16 or PKV_BF16");
  pkv::AttnArgs a{};
  int rc = check_attention(out, out_dtype, query, key_cache, value_cache, block_tables,
                           max_blocks_per_seq, context_lens, batch, q_len, num_q_heads, gqa_factor,
                           head_dim, block_size, num_blocks, scale, a);
  if (rc) return rc;
  if (batch == 0) return ok();
  if (!new_key || !new_value) return fail(PKV_ERR_NULL, "new_key / new_value is NULL");
  if (!aligned16(new_key) || !aligned16(new_value))
    return fail(PKV_ERR_ALIGN, "new_key and new_value must be 16-byte aligned");
  a.new_k = new_key;
  a.new_v = new_value;
  return launch_result(pkv::launch_attention(a, kv_dtype, kv_dtype, head_dim, (hipStream_t)stream),
                       "paged_attention_decode_append");
}

int paged_attention_decode_splitkv_append(void* out, int out_dtype, const void* query,
                                          const void* new_key, const void* new_value,
                                          void* key_cache, void* value_cache, int kv_dtype,
                                          const int32_t* block_tables, int max_blocks_per_seq,
                                          const int32_t* context_lens, int batch, int q_len,
                                          int num_q_heads, int gqa_factor, int head_dim,
                                          int block_size, int64_t num_blocks, float scale,
                                          int max_context_len, int partition_size,
                                          void* workspace, size_t workspace_bytes, void* stream) {
  if (kv_dtype != PKV_F16 && kv_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "kv_dtype must be PKV_F16 or PKV_BF16");
  pkv::AttnArgs a{};
  int rc = check_attention(out, out_dtype, query, key_cache, value_cache, block_tables,
                           max_blocks_per_seq, context_lens, batch, q_len, num_q_heads, gqa_factor,
                           head_dim, block_size, num_blocks, scale, a);
  if (rc) return rc;
  if (batch == 0) return ok();
  if (!new_key || !new_value) return fail(PKV_ERR_NULL, "new_key / new_value is NULL");
  if (!aligned16(new_key) || !aligned16(new_value))
    return fail(PKV_ERR_ALIGN, "new_key and new_value must be 16-byte aligned");
  rc = setup_split(a, head_dim, max_context_len, partition_size, workspace, workspace_bytes, true);
  if (rc) return rc;
  a.new_k = new_key;
  a.new_v = new_value;
  return launch_result(pkv::launch_attention(a, kv_dtype, kv_dtype, head_dim, (hipStream_t)stream),
                       "paged_attention_decode_splitkv_append");
}

int paged_attention_decode_k8v4(void* out, int out_dtype, const void* query, int q_dtype,
                                const int8_t* k_cache, const void* k_scale,
                                const uint8_t* v_cache, const void* v_scale, const void* v_zero,
                                const int32_t* block_tables, int max_blocks_per_seq,
                                const int32_t* context_lens, int batch, int q_len,
                                int num_q_heads, int gqa_factor, int head_dim, int block_size,
                                int64_t num_blocks, float scale, void* stream) {
  if (q_dtype != PKV_F16 && q_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "q_dtype must be PKV_F16 or PKV_BF16");
  pkv::AttnArgs a{};
  int rc = check_attention(out, out_dtype, query, k_cache, v_cache, block_tables,
                           max_blocks_per_seq, context_lens, batch, q_len, num_q_heads, gqa_factor,
                           head_dim, block_size, num_blocks, scale, a);
  if (rc) return rc;
  if (batch == 0) return ok();
  rc = check_k8v4_pointers(k_scale, v_scale, v_zero);
  if (rc) return rc;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.v_zero = v_zero;
  return launch_result(pkv::launch_attention(a, PKV_FMT_K8V4, q_dtype, head_dim,
                                             (hipStream_t)stream),
                       "paged_attention_decode_k8v4");
}

int paged_attention_decode_splitkv_k8v4(void* out, int out_dtype, const void* query, int q_dtype,
                                        const int8_t* k_cache, const void* k_scale,
                                        const uint8_t* v_cache, const void* v_scale,
                                        const void* v_zero, const int32_t* block_tables,
                                        int max_blocks_per_seq, const int32_t* context_lens,
                                        int batch, int q_len, int num_q_heads, int gqa_factor,
                                        int head_dim, int block_size, int64_t num_blocks,
                                        float scale, int max_context_len, int partition_size,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  if (q_dtype != PKV_F16 && q_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "q_dtype must be PKV_F16 or PKV_BF16");
  pkv::AttnArgs a{};
  int rc = check_attention(out, out_dtype, query, k_cache, v_cache, block_tables,
                           max_blocks_per_seq, context_lens, batch, q_len, num_q_heads, gqa_factor,
                           head_dim, block_size, num_blocks, scale, a);
  if (rc) return rc;
  if (batch == 0) return ok();
  rc = check_k8v4_pointers(k_scale, v_scale, v_zero);
  if (rc) return rc;
  rc = setup_split(a, head_dim, max_context_len, partition_size, workspace, workspace_bytes);
  if (rc) return rc;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.v_zero = v_zero;
  return launch_result(pkv::launch_attention(a, PKV_FMT_K8V4, q_dtype, head_dim,
                                             (hipStream_t)stream),
                       "paged_attention_decode_splitkv_k8v4");
}

int paged_attention_decode_k8v4_append(void* out, int out_dtype, const void* query, int q_dtype,
                                       const void* new_key, const void* new_value,
                                       int8_t* k_cache, void* k_scale, uint8_t* v_cache,
                                       void* v_scale, void* v_zero, const int32_t* block_tables,
                                       int max_blocks_per_seq, const int32_t* context_lens,
                                       int batch, int q_len, int num_q_heads, int gqa_factor,
                                       int head_dim, int block_size, int64_t num_blocks,
                                       float scale, void* stream) {
  if (q_dtype != PKV_F16 && q_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "q_dtype must be PKV_F16 or PKV_BF16");
  pkv::AttnArgs a{};
  int rc = check_attention(out, out_dtype, query, k_cache, v_cache, block_tables,
                           max_blocks_per_seq, context_lens, batch, q_len, num_q_heads, gqa_factor,
                           head_dim, block_size, num_blocks, scale, a);
  if (rc) return rc;
  if (batch == 0) return ok();
  rc = check_k8v4_pointers(k_scale, v_scale, v_zero);
  if (rc) return rc;
  if (!new_key || !new_value) return fail(PKV_ERR_NULL, "new_key / new_value is NULL");
  if (!aligned16(new_key) || !aligned16(new_value))
    return fail(PKV_ERR_ALIGN, "new_key and new_value must be 16-byte aligned");
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.v_zero = v_zero;
  a.new_k = new_key;
  a.new_v = new_value;
  return launch_result(pkv::launch_attention(a, PKV_FMT_K8V4, q_dtype, head_dim,
                                             (hipStream_t)stream),
                       "paged_attention_decode_k8v4_append");
}

int paged_attention_decode_splitkv_k8v4_append(
    void* out, int out_dtype, const void* query, int q_dtype, const void* new_key,
    const void* new_value, int8_t* k_cache, void* k_scale, uint8_t* v_cache, void* v_scale,
    void* v_zero, const int32_t* block_tables, int max_blocks_per_seq,
    const int32_t* context_lens, int batch, int q_len, int num_q_heads, int gqa_factor,
    int head_dim, int block_size, int64_t num_blocks, float scale, int max_context_len,
    int partition_size, void* workspace, size_t workspace_bytes, void* stream) {
  if (q_dtype != PKV_F16 && q_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "q_dtype must be PKV_F16 or PKV_BF16");
  pkv::AttnArgs a{};
  int rc = check_attention(out, out_dtype, query, k_cache, v_cache, block_tables,
                           max_blocks_per_seq, context_lens, batch, q_len, num_q_heads, gqa_factor,
                           head_dim, block_size, num_blocks, scale, a);
  if (rc) return rc;
  if (batch == 0) return ok();
  rc = check_k8v4_pointers(k_scale, v_scale, v_zero);
  if (rc) return rc;
  if (!new_key || !new_value) return fail(PKV_ERR_NULL, "new_key / new_value is NULL");
  if (!aligned16(new_key) || !aligned16(new_value))
    return fail(PKV_ERR_ALIGN, "new_key and new_value must be 16-byte aligned");
  rc = setup_split(a, head_dim, max_context_len, partition_size, workspace, workspace_bytes);
  if (rc) return rc;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.v_zero = v_zero;
  a.new_k = new_key;
  a.new_v = new_value;
  return launch_result(pkv::launch_attention(a, PKV_FMT_K8V4, q_dtype, head_dim,
                                             (hipStream_t)stream),
                       "paged_attention_decode_splitkv_k8v4_append");
}

int paged_attention_decode_splitkv_partials(const void* query, const void* key_cache,
                                            const void* value_cache, int kv_dtype,
                                            const int32_t* block_tables, int max_blocks_per_seq,
                                            const int32_t* context_lens, int batch, int q_len,
                                            int num_q_heads, int gqa_factor, int head_dim,
                                            int block_size, int64_t num_blocks, float scale,
                                            int max_context_len, int partition_size,
                                            void* workspace, size_t workspace_bytes,
                                            void* stream) {
  if (kv_dtype != PKV_F16 && kv_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "kv_dtype must be PKV_F16 or PKV_BF16");
  pkv::AttnArgs a{};
  int rc = check_attention(nullptr, PKV_F32, query, key_cache, value_cache, block_tables,
                           max_blocks_per_seq, context_lens, batch, q_len, num_q_heads, gqa_factor,
                           head_dim, block_size, num_blocks, scale, a, false);
  if (rc) return rc;
  if (batch == 0) return ok();
  rc = setup_split(a, head_dim, max_context_len, partition_size, workspace, workspace_bytes);
  if (rc) return rc;
  return launch_result(pkv::launch_attention(a, kv_dtype, kv_dtype, head_dim, (hipStream_t)stream,
                                             pkv::STAGE_PARTIALS),
                       "paged_attention_decode_splitkv_partials");
}

int paged_attention_decode_splitkv_append_partials(
    const void* query, const void* new_key, const void* new_value, void* key_cache,
    void* value_cache, int kv_dtype, const int32_t* block_tables, int max_blocks_per_seq,
    const int32_t* context_lens, int batch, int q_len, int num_q_heads, int gqa_factor,
    int head_dim, int block_size, int64_t num_blocks, float scale, int max_context_len,
    int partition_size, void* workspace, size_t workspace_bytes, void* stream) {
  if (kv_dtype != PKV_F16 && kv_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "kv_dtype must be PKV_F16 or PKV_BF16");
  pkv::AttnArgs a{};
  int rc = check_attention(nullptr, PKV_F32, query, key_cache, value_cache, block_tables,
                           max_blocks_per_seq, context_lens, batch, q_len, num_q_heads, gqa_factor,
                           head_dim, block_size, num_blocks, scale, a, false);
  if (rc) return rc;
  if (batch == 0) return ok();
  if (!new_key || !new_value) return fail(PKV_ERR_NULL, "new_key / new_value is NULL");
  if (!aligned16(new_key) || !aligned16(new_value))
    return fail(PKV_ERR_ALIGN, "new_key and new_value must be 16-byte aligned");
  rc = setup_split(a, head_dim, max_context_len, partition_size, workspace, workspace_bytes);
  if (rc) return rc;
  a.new_k = new_key;
  a.new_v = new_value;
  return launch_result(pkv::launch_attention(a, kv_dtype, kv_dtype, head_dim, (hipStream_t)stream,
                                             pkv::STAGE_PARTIALS),
                       "paged_attention_decode_splitkv_append_partials");
}

int paged_attention_decode_splitkv_k8v4_partials(
    const void* query, int q_dtype, const int8_t* k_cache, const void* k_scale,
    const uint8_t* v_cache, const void* v_scale, const void* v_zero, const int32_t* block_tables,
    int max_blocks_per_seq, const int32_t* context_lens, int batch, int q_len, int num_q_heads,
    int gqa_factor, int head_dim, int block_size, int64_t num_blocks, float scale,
    int max_context_len, int partition_size, void* workspace, size_t workspace_bytes,
    void* stream) {
  if (q_dtype != PKV_F16 && q_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "q_dtype must be PKV_F16 or PKV_BF16");
  pkv::AttnArgs a{};
  int rc = check_attention(nullptr, PKV_F32, query, k_cache, v_cache, block_tables,
                           max_blocks_per_seq, context_lens, batch, q_len, num_q_heads, gqa_factor,
                           head_dim, block_size, num_blocks, scale, a, false);
  if (rc) return rc;
  if (batch == 0) return ok();
  rc = check_k8v4_pointers(k_scale, v_scale, v_zero);
  if (rc) return rc;
  rc = setup_split(a, head_dim, max_context_len, partition_size, workspace, workspace_bytes);
  if (rc) return rc;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.v_zero = v_zero;
  return launch_result(pkv::launch_attention(a, PKV_FMT_K8V4, q_dtype, head_dim,
                                             (hipStream_t)stream, pkv::STAGE_PARTIALS),
                       "paged_attention_decode_splitkv_k8v4_partials");
}

int paged_attention_decode_splitkv_merge(void* out, int out_dtype, int batch, int q_len,
                                         int num_q_heads, int head_dim, int max_context_len,
                                         int partition_size, const void* workspace,
                                         size_t workspace_bytes, void* stream) {
  if (batch < 0 || q_len <= 0 || num_q_heads <= 0)
    return fail(PKV_ERR_SHAPE, "batch >= 0, q_len > 0, num_q_heads > 0 required");
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  if (out_dtype != PKV_F16 && out_dtype != PKV_BF16 && out_dtype != PKV_F32)
    return fail(PKV_ERR_UNSUPPORTED, "out_dtype must be PKV_F16, PKV_BF16 or PKV_F32");
  if (batch > 65535) return fail(PKV_ERR_UNSUPPORTED, "batch too large");
  int64_t parts = 0;
  size_t need = 0;
  int rc = split_geometry(batch, q_len, num_q_heads, head_dim, max_context_len, partition_size,
                          parts, need);
  if (rc) return rc;
  if (batch == 0) return ok();
  if (!out) return fail(PKV_ERR_NULL, "out is NULL");
  if (!workspace) return fail(PKV_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned16(workspace)) return fail(PKV_ERR_ALIGN, "workspace must be 16-byte aligned");
  if (workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "workspace too small: %zu bytes given, %zu needed",
                workspace_bytes, need);
  pkv::AttnArgs a{};
  a.out = out;
  a.out_dtype = out_dtype;
  a.batch = batch;
  a.q_len = q_len;
  a.num_q_heads = num_q_heads;
  const int64_t rows = (int64_t)batch * q_len * num_q_heads;
  a.num_parts = (int)parts;
  a.ws_parts = (int)parts;
  a.part_blocks = partition_size / 16;
  a.ws_o = (float*)workspace;
  a.ws_m = a.ws_o + rows * parts * head_dim;
  a.ws_l = a.ws_m + rows * parts;
  return launch_result(pkv::launch_attention(a, PKV_FMT_F16, PKV_F16, head_dim,
                                             (hipStream_t)stream, pkv::STAGE_MERGE),
                       "paged_attention_decode_splitkv_merge");
}

}  // extern "C"

// gather_kv_cache: the paged cache of each sequence copied out into packed
// contiguous rows, the inverse of the slot scatter ("The KV Cache"
// (metalworking), layout paragraph: the gather_kv_cache kernel beside
// reshape_and_cache).  Sequence b's positions 0 .. L_b - 1 go to output rows
// cu_seq_lens[b] .. cu_seq_lens[b+1] - 1 of [total_tokens, Hkv, D].
//
// A cache block holds the 16 rows of all KV heads contiguously, and so do 16
// consecutive output rows, so each (block, sequence) pair is one contiguous
// copy of up to 16 * Hkv * D elements: one workgroup per pair, 16-byte vector
// loads, several in flight per thread before the stores.  HBM-bound: every
// byte is read once and written once, so both sides use non-temporal
// accesses (the copy is streamed past the caches instead of filling them:
// 105 against 120 us for the Llama-3-8B-shaped batch, 512 threads against
// 256 included).

#include "pkv_common.h"
#include "pkv_launch.h"

namespace pkv {

constexpr int kGatherThreads = 512;
constexpr int kGatherUnroll = 4;

__global__ __launch_bounds__(kGatherThreads) void gather_kernel(
    const u4* __restrict__ key_cache, const u4* __restrict__ value_cache,
    const int32_t* __restrict__ block_tables, int max_blocks, const int32_t* __restrict__ cu,
    int64_t total_tokens, int64_t num_blocks, int row_vecs, u4* __restrict__ key_out,
    u4* __restrict__ value_out) {
  const int i = blockIdx.x, b = blockIdx.y;
  const int64_t first = cu[b];
  const int L = min(max(cu[b + 1] - cu[b], 0), max_blocks * kBlock);
  if (i * kBlock >= L) return;
  const int rows = min(kBlock, L - i * kBlock);
  const int pb = block_tables[(int64_t)b * max_blocks + i];
  const bool ok = pb >= 0 && (int64_t)pb < num_blocks;     // else the rows are zeros
  const int64_t row0 = first + (int64_t)i * kBlock;        // output row of position 16 i
  // output rows kept inside [0, total_tokens)
  const int64_t lo = max<int64_t>(0, -row0) * row_vecs;
  const int64_t hi = min<int64_t>(rows, total_tokens - row0) * row_vecs;
  if (hi <= lo) return;
  const u4* ks = key_cache + (ok ? (int64_t)pb * kBlock * row_vecs : 0);
  const u4* vs = value_cache + (ok ? (int64_t)pb * kBlock * row_vecs : 0);
  u4* kd = key_out + row0 * row_vecs;
  u4* vd = value_out + row0 * row_vecs;
  const u4 zero = u4{0u, 0u, 0u, 0u};
  for (int64_t base = lo + threadIdx.x; base < hi; base += kGatherThreads * kGatherUnroll) {
    u4 tk[kGatherUnroll], tv[kGatherUnroll];
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int64_t v = base + u * kGatherThreads;
      tk[u] = ok && v < hi ? __builtin_nontemporal_load(&ks[v]) : zero;
      tv[u] = ok && v < hi ? __builtin_nontemporal_load(&vs[v]) : zero;
    }
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int64_t v = base + u * kGatherThreads;
      if (v < hi) {
        __builtin_nontemporal_store(tk[u], &kd[v]);
        __builtin_nontemporal_store(tv[u], &vd[v]);
      }
    }
  }
}

hipError_t launch_gather(const void* key_cache, const void* value_cache,
                         const int32_t* block_tables, int max_blocks, const int32_t* cu_seq_lens,
                         int batch, int max_seq_len, int64_t total_tokens, int num_kv_heads,
                         int head_dim, int64_t num_blocks, void* key_out, void* value_out,
                         hipStream_t stream) {
  const int row_vecs = num_kv_heads * head_dim * 2 / 16;
  const int len = min(max_seq_len, max_blocks * kBlock);
  const unsigned gx = (unsigned)((len + kBlock - 1) / kBlock);
  if (gx == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_kernel, dim3(gx, (unsigned)batch), dim3(kGatherThreads), 0, stream,
                     (const u4*)key_cache, (const u4*)value_cache, block_tables, max_blocks,
                     cu_seq_lens, total_tokens, num_blocks, row_vecs, (u4*)key_out,
                     (u4*)value_out);
  return hipGetLastError();
}

}  // namespace pkv

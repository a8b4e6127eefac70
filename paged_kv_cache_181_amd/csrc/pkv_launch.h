// Host-side launchers of the HIP kernels (internal; the public ABI is pagedkv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

hipError_t launch_kv_write(const void* key, const void* value, void* key_cache, void* value_cache,
                           const int64_t* slots, int64_t num_tokens, int num_kv_heads,
                           int head_dim, int64_t num_blocks, hipStream_t stream);

hipError_t launch_kv_write_k8v4(const void* key, const void* value, int in_dtype, int8_t* k_cache,
                                void* k_scale, uint8_t* v_cache, void* v_scale, void* v_zero,
                                const int64_t* slots, int64_t num_tokens, int num_kv_heads,
                                int head_dim, int64_t num_blocks, hipStream_t stream);

// Packed copy of each sequence's cached rows (gather_kv_cache).  Only sequences
// with cu_seq_lens[b+1] - cu_seq_lens[b] <= max_seq_len are copied in full.
hipError_t launch_gather(const void* key_cache, const void* value_cache,
                         const int32_t* block_tables, int max_blocks, const int32_t* cu_seq_lens,
                         int batch, int max_seq_len, int64_t total_tokens, int num_kv_heads,
                         int head_dim, int64_t num_blocks, void* key_out, void* value_out,
                         hipStream_t stream);

// Everything the attention kernels need; filled by the ABI layer after validation.
struct AttnArgs {
  void* out;
  int out_dtype;                 // OutT
  const void* q;                 // [B, Q, Hq, D] 16-bit
  const void* k_cache;           // [NB, 16, Hkv, D] (16-bit or int8 codes)
  const void* v_cache;           // [NB, 16, Hkv, D] 16-bit, or [NB, 16, Hkv, D/2] packed 4-bit
  const void* k_scale;           // K8/V4 only: fp16 [NB, 16, Hkv]
  const void* v_scale;           // K8/V4 only: fp16 [NB, 16, Hkv, D/32]
  const void* v_zero;            // K8/V4 only: fp16 [NB, 16, Hkv, D/32]
  const int32_t* block_tables;   // [B, max_blocks]
  const int32_t* context_lens;   // [B]
  int max_blocks;
  int batch, q_len, num_q_heads, num_kv_heads, gqa;
  int64_t num_blocks;
  float scale_log2;              // softmax scale * log2(e)
  int part_blocks;               // cache blocks per partition
  int num_parts;                 // partitions in the grid (1 = direct form)
  float* ws_o;                   // split form: [B*Q*Hq, P, D] unnormalised partial outputs
  float* ws_m;                   // split form: [B*Q*Hq, P] running max (log2 units)
  float* ws_l;                   // split form: [B*Q*Hq, P] softmax denominators
  const void* new_k;             // append form (16-bit only): [B*Q, Hkv, D] new rows, else NULL
  const void* new_v;             // append form: [B*Q, Hkv, D]
  int window;                    // sliding window in positions (0: the whole context)
  int ws_parts;                  // partition slots per row in the workspace
  int part_base;                 // first slot this launch's partitions write
  int mode;                      // 0 plain, 1 cascade prefix pass
  const int32_t* grp_members;    // cascade: [num_groups, group_size] sequence ids (-1: empty)
  const int32_t* grp_prefix;     // cascade: [num_groups] shared whole blocks
  int num_groups, group_size;
  float v_log2_threshold;        // sparse-V: skip V rows below 2^this of the running max
  unsigned long long* v_rows_read;   // sparse-V: optional device counter of V rows read
  int flat_runs;                 // balanced split: runs (wavefronts) per KV head; 0 = off
  const int32_t* tbl_off;        // balanced split: [B] first table entry of each sequence (NULL: 0)
  const float* pre_o;            // balanced merge: cascade prefix partials [B*Q*Hq, pre_parts, D]
  const float* pre_m;            //   their running maxima [B*Q*Hq, pre_parts]
  const float* pre_l;            //   and denominators; folded in for sequences with tbl_off > 0
  int pre_parts;                 // 0: no prefix partials
};

// Balanced split (partition_size 0): each KV head's flattened blocks are cut
// into flat_runs_for(Hq) equal runs, one per wavefront.  The workspace holds
// (runs + batch) * num_q_heads * q_len partial rows of head_dim + 2 floats.
constexpr int kFlatQueryWaves = 16384;
constexpr int flat_runs_for(int num_q_heads) {
  return num_q_heads > 0 ? (kFlatQueryWaves / num_q_heads) / 8 * 8 : 0;
}

// Cascade with a balanced suffix pass: for each sequence, the blocks of its
// group's shared prefix (the first group whose first slot names a sequence
// and that lists it; 0 outside every group), clamped to its own blocks, into
// suf_off[b], and its length past them into suf_len[b].
hipError_t launch_cascade_suffix_prep(const AttnArgs& a, int32_t* suf_len, int32_t* suf_off,
                                      hipStream_t stream);

// kv_fmt: 0 f16, 1 bf16, 3 k8v4; q_fmt: 0 f16, 1 bf16 (must equal kv_fmt unless k8v4).
// stage: STAGE_ALL launches the partition kernel and, for the split form, the
// merge; STAGE_PARTIALS only the partition kernel; STAGE_MERGE only the merge.
enum { STAGE_ALL = 0, STAGE_PARTIALS = 1, STAGE_MERGE = 2 };
hipError_t launch_attention(const AttnArgs& a, int kv_fmt, int q_fmt, int head_dim,
                            hipStream_t stream, int stage = STAGE_ALL);

// Sparse-V split-KV decode (16-bit caches, G*q_len <= 4): partition kernel
// reading only the V rows some query row needs, then the merge.
hipError_t launch_sparse_v(const AttnArgs& a, int kv_fmt, int head_dim, hipStream_t stream);

}  // namespace pkv

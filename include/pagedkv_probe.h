/*
 * pagedkv_probe.h — read-only measurement probes (libpagedkv_probe.so).
 *
 * Not part of the decode path.  They read memory and compute nothing, to
 * measure how fast the K/V stream of one decode layer can be read at all on
 * this GPU, so that the partition kernel's time can be compared with a
 * ceiling measured on the same machine.  "The KV Cache" (metalworking),
 * arithmetic paragraph: at long context every decoded token streams the
 * whole cache, so decode is bound by how fast that stream can be read.
 *
 * Both probes XOR what they load into one word per wavefront and store it to
 * `sink` (float32, at least grid workgroups x waves entries), so no load can
 * be dropped by the compiler.  Same conventions as pagedkv.h: device pointers,
 * asynchronous on `stream`, 0 or a negative PKV_ERR_* code (text from
 * pkv_probe_last_error()), nothing launched on an error.
 */
#ifndef PAGEDKV_PROBE_H
#define PAGEDKV_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

const char* pkv_probe_last_error(void);

/*
 * pkv_probe_stream_read — plain streaming read of two buffers of
 * `bytes_each` bytes (e.g. one layer's K and V caches).  `workgroups`
 * workgroups of `waves` wavefronts (waves in {4, 8, 16}); workgroup i reads
 * one contiguous slice of 2 * bytes_each / workgroups bytes, its waves taking
 * consecutive 1 KiB chunks (64 lanes x 16 B), `depth` chunks per wave in
 * flight (depth in {1, 2, 4, 8}).  bytes_each must be a multiple of
 * workgroups / 2 * waves * depth KiB, with workgroups even.
 */
int pkv_probe_stream_read(const void* buf0, const void* buf1, size_t bytes_each, int workgroups,
                          int waves, int depth, float* sink, size_t sink_count, void* stream);

/*
 * pkv_probe_paged_read — reads every K and V row of one sequence's
 * `table_blocks` cache blocks (all KV heads) through the block table with the
 * partition kernel's lane addressing (head_dim 128, 16-bit rows: lane l reads
 * 16 B of token l % 16 at byte 16 * (l / 16) + 64 m of the head's row,
 * m = 0..3, for K and for V).  Grid (table_blocks / part_blocks,
 * num_kv_heads / heads_per_wg); a workgroup of `waves` wavefronts takes
 * `heads_per_wg` consecutive KV heads of one partition of `part_blocks`
 * blocks, waves / heads_per_wg waves per head, each wave a contiguous run of
 * the partition's blocks with `depth` blocks in flight (a ring of register
 * sets; each refill waits for the block it replaces, as the attention kernel
 * does).  `lds_bytes` of dynamic LDS per workgroup sets how many workgroups
 * share a CU.  Requires table_blocks % part_blocks == 0,
 * num_kv_heads % heads_per_wg == 0, heads_per_wg in {1, 2, 4, 8},
 * waves in {4, 8, 16} divisible by heads_per_wg, a run of at most 64 blocks,
 * depth in {1, 2, 3, 4} (at most 3 with 16 waves).  A table entry outside
 * [0, num_blocks) is not read.
 */
int pkv_probe_paged_read(const void* k_cache, const void* v_cache, const int32_t* block_table,
                         int table_blocks, int64_t num_blocks, int num_kv_heads, int head_dim,
                         int heads_per_wg, int waves, int part_blocks, int depth, int lds_bytes,
                         float* sink, size_t sink_count, void* stream);

/*
 * pkv_probe_k8v4_read — reads every K code row, V code row, K scale and V
 * scale/zero line of `table_blocks` blocks of a K8/V4 cache (all 8 KV heads,
 * head_dim 128; layouts as paged_attention_decode_k8v4) through the block
 * table, with the K8/V4 head-group form's lane addressing: grid
 * table_blocks / part_blocks workgroups of 8 wavefronts, wave g taking KV head
 * g over the workgroup's `part_blocks` consecutive table entries; lane l
 * (token l % 16, quarter l / 16) issues the attention kernel's six loads per
 * block (two 16 B of the 128-byte K row, 16 B of the 64-byte V row, the 2 B
 * K scale, the 8 B of V scales and the 8 B of V zeros), with `depth` blocks
 * in flight (a ring of register sets).  `lds_bytes` of dynamic LDS per
 * workgroup sets how many share a CU.  Requires num_kv_heads 8, head_dim 128,
 * part_blocks in 1 .. 64 dividing table_blocks, depth in 1 .. 4; sink of at
 * least 8 entries per workgroup.  A table entry outside [0, num_blocks) is
 * not read.
 */
int pkv_probe_k8v4_read(const void* k_codes, const void* v_codes, const void* k_scale,
                        const void* v_scale, const void* v_zero, const int32_t* block_table,
                        int table_blocks, int64_t num_blocks, int num_kv_heads, int head_dim,
                        int part_blocks, int depth, int lds_bytes, float* sink, size_t sink_count,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif

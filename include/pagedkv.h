/*
 * pagedkv.h — C ABI of the paged-KV decode library for AMD Instinct MI355X (gfx950).
 *
 * What it computes
 *   - kv_cache_write*: the slot scatter that stores each step's new K/V rows into
 *     a block-paged cache ("The KV Cache" (metalworking), layout paragraph: the
 *     reshape_and_cache kernel; "How the Paged KV Cache Works in MTPLX",
 *     Physical Layout and Memory Organization: 4-D cache
 *     [num_blocks, block_size, num_kv_heads, head_dim], 16 tokens per block).
 *   - paged_attention_decode*: softmax attention of a block of q_len new query
 *     tokens over the cache of each sequence, resolved through an int32 block
 *     table ("The KV Cache", layout paragraph: fixed-size blocks plus an
 *     indirection table).  Query head h reads KV head h / gqa_factor ("The KV
 *     Cache", arithmetic paragraph, the GQA stride trick).  The split-KV form
 *     partitions each sequence and merges the partitions by log-sum-exp
 *     ("The KV Cache", layout paragraph: split-KV decode kernels for
 *     single-user decode; mlxcel "KV Cache", Paged Decode Storage and Kernels:
 *     a decode split count).
 *   - *_k8v4: the same over a cache holding int8 K (one fp16 scale per token and
 *     KV head) and packed 4-bit V (fp16 scale and zero per 32 elements)
 *     ("The KV Cache", the K/V asymmetry paragraph: K8/V4).
 *
 * Conventions shared by every entry point
 *   - Ownership: the caller allocates and owns every buffer, including the
 *     split-KV workspace.  The library never allocates, frees or synchronises.
 *   - Pointers: device pointers unless stated; all tensors dense, row-major, and
 *     16-byte aligned.  `stream` is a hipStream_t (NULL = the null stream); all
 *     work is enqueued on it, asynchronously, in stream order.
 *   - Errors: every call returns PKV_OK (0) or a negative PKV_ERR_* code.  On an
 *     error nothing is launched and pkv_last_error() (thread-local, static
 *     storage, valid until the next call on that thread) describes it.
 *   - Lengths: context_lens[b] counts the tokens of sequence b after this step's
 *     q_len tokens were written (write first, then attend: "How MTPLX Manages
 *     Memory Using Request-Sized Paged KV Cache", Request-Sized Offset
 *     Tracking).  Query row i of a q_len block sees positions
 *     0 .. context_lens[b] - q_len + i (causal inside the block, as in a
 *     speculative verify block: mlxcel "KV Cache", Matrix-Absorbed MLA Decode).
 *     Rows that see no position produce zeros.
 *   - Device-side values are not range-checked by a host sync.  Instead the
 *     kernels treat them safely: a length is clamped to
 *     [0, max_blocks_per_seq * block_size]; a block-table entry outside
 *     [0, num_blocks) drops its 16 positions from the softmax; a slot that is
 *     negative or >= num_blocks * block_size is not written.  Duplicate slots in
 *     one write call are undefined (the caller never issues them).
 *   - Supported shapes: block_size == 16; head_dim 64 or 128;
 *     num_q_heads % gqa_factor == 0; 1 <= gqa_factor * q_len <= 16.  Anything
 *     else returns PKV_ERR_UNSUPPORTED.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
enum {
  PKV_F16 = 0,   /* IEEE binary16 */
  PKV_BF16 = 1,  /* bfloat16 */
  PKV_F32 = 2    /* float32: only for `out` */
};

/* cache formats for kv_cache_bytes_per_token */
enum {
  PKV_FMT_F16 = 0,
  PKV_FMT_BF16 = 1,
  PKV_FMT_K8V4 = 3
};

/* return codes */
enum {
  PKV_OK = 0,
  PKV_ERR_NULL = -1,         /* a required pointer is NULL */
  PKV_ERR_SHAPE = -2,        /* a size is negative or inconsistent */
  PKV_ERR_UNSUPPORTED = -3,  /* a valid but unsupported configuration */
  PKV_ERR_WORKSPACE = -4,    /* split-KV workspace missing or too small */
  PKV_ERR_LAUNCH = -5,       /* the HIP runtime rejected a launch */
  PKV_ERR_ALIGN = -6         /* a pointer is not 16-byte aligned */
};

/* Text of the last error on this thread ("" after a successful call). */
const char* pkv_last_error(void);

/* Library ABI version (major * 100 + minor). */
int pkv_version(void);

/*
 * kv_cache_write — reshape_and_cache slot scatter for fp16/bf16 caches.
 *   key, value:   [num_tokens, num_kv_heads, head_dim] of `dtype`
 *   key_cache, value_cache: [num_blocks, block_size, num_kv_heads, head_dim] of `dtype`
 *   slot_mapping: int64 [num_tokens]; token t goes to block slot/16, row slot%16.
 *                 Negative or out-of-pool slots are skipped.
 * The copy is bit-exact.  num_tokens == 0 is a no-op.
 */
int kv_cache_write(const void* key, const void* value, void* key_cache, void* value_cache,
                   const int64_t* slot_mapping, int64_t num_tokens, int num_kv_heads,
                   int head_dim, int block_size, int64_t num_blocks, int dtype, void* stream);

/*
 * gather_kv_cache — the inverse of the slot scatter: every sequence's cached
 * rows copied out of the pages into packed contiguous arrays for dense
 * consumers ("The KV Cache" (metalworking), layout paragraph: the
 * gather_kv_cache kernel of the paged kernel family).
 *   key_cache, value_cache: [num_blocks, block_size, num_kv_heads, head_dim]
 *   block_tables:  int32 [batch, max_blocks_per_seq]
 *   cu_seq_lens:   int32 [batch + 1], device; sequence b fills output rows
 *                  cu_seq_lens[b] .. cu_seq_lens[b+1] - 1 with its positions
 *                  0 .. L_b - 1, L_b = cu_seq_lens[b+1] - cu_seq_lens[b]
 *                  (clamped to max_blocks_per_seq * 16 like every length)
 *   max_seq_len:   host bound on every L_b (sizes the grid; positions past
 *                  it are not copied)
 *   key_out, value_out: [total_tokens, num_kv_heads, head_dim], written only
 *                  in the rows the sequences cover (rows outside
 *                  [0, total_tokens) are never written)
 * Position j comes from block block_tables[b][j / 16], row j % 16; if that
 * entry is outside [0, num_blocks) the output row is zero.  A plain copy
 * (bit-exact); dtype (PKV_F16 or PKV_BF16) only fixes the element size.
 */
int gather_kv_cache(const void* key_cache, const void* value_cache, int dtype,
                    const int32_t* block_tables, int max_blocks_per_seq,
                    const int32_t* cu_seq_lens, int batch, int max_seq_len, void* key_out,
                    void* value_out, int64_t total_tokens, int num_kv_heads, int head_dim,
                    int block_size, int64_t num_blocks, void* stream);

/*
 * paged_attention_decode — one workgroup per (sequence, KV head), no workspace.
 *   out:          [batch, q_len, num_q_heads, head_dim] of out_dtype (f16, bf16 or f32)
 *   query:        [batch, q_len, num_q_heads, head_dim] of kv_dtype
 *   key_cache, value_cache: [num_blocks, block_size, num_kv_heads, head_dim] of kv_dtype
 *   block_tables: int32 [batch, max_blocks_per_seq]; only the first
 *                 ceil(len/block_size) entries of a row are read
 *   context_lens: int32 [batch]
 *   num_kv_heads = num_q_heads / gqa_factor.  scale multiplies q.k.
 * Accumulation is fp32; the output is rounded to nearest-even once.
 */
int paged_attention_decode(void* out, int out_dtype, const void* query,
                           const void* key_cache, const void* value_cache, int kv_dtype,
                           const int32_t* block_tables, int max_blocks_per_seq,
                           const int32_t* context_lens, int batch, int q_len, int num_q_heads,
                           int gqa_factor, int head_dim, int block_size, int64_t num_blocks,
                           float scale, void* stream);

/*
 * Workspace bytes for the split-KV calls (host-only arithmetic, no GPU use).
 * partition_size is in tokens and must be a positive multiple of block_size
 * (16), or 0 for the balanced split (below).  max_context_len bounds
 * context_lens for the grid size; a longer sequence is still handled
 * correctly (its last partition runs to its end).
 *   fixed partitions: batch * q_len * num_q_heads * P * (head_dim + 2) * 4,
 *                     P = ceil(max_context_len / partition_size);
 *   balanced split:   (R + batch) * num_q_heads * q_len * (head_dim + 2) * 4,
 *                     R = 16384 / num_q_heads rounded down to a multiple of 8
 *                     (max_context_len plays no part; a call uses at most R
 *                     runs per KV head, see paged_attention_decode_splitkv).
 */
int paged_attention_decode_splitkv_workspace_size(int batch, int q_len, int num_q_heads,
                                                  int head_dim, int max_context_len,
                                                  int partition_size, size_t* out_bytes);

/*
 * paged_attention_decode_splitkv — partition kernel over
 * (partition, KV head, sequence) writing per-partition (o, max, sum) to
 * `workspace` (partitions that start past a sequence's end are marked empty),
 * then a log-sum-exp merge kernel writing `out`.  Same arguments and result as
 * paged_attention_decode (up to fp32 summation order).  The workspace
 * contents on entry do not matter; two calls that overlap in time must not
 * share a workspace.
 *
 * partition_size 0 asks for the balanced split (16-bit caches; also accepted
 * by paged_attention_decode_splitkv_append and
 * paged_attention_decode_splitkv_noalloc, rejected with PKV_ERR_UNSUPPORTED
 * by the other split calls).  For each KV head the batch's blocks are laid
 * end to end in sequence order and cut into equal runs, one per wavefront:
 * as many (a multiple of 8) as give the partition pass one workgroup per
 * compute unit, at most the R of the workspace size.  Every wavefront reads the same
 * number of blocks however ragged the lengths are (mlxcel "KV Cache", Paged
 * Decode Storage and Kernels: the decode split count; here the split follows
 * the batch's total length rather than a fixed partition size).  A run that
 * crosses sequences leaves one partial per sequence; the merge combines each
 * row's partials by log-sum-exp as for fixed partitions.  Requires
 * batch * max_blocks_per_seq < 2^31.
 */
int paged_attention_decode_splitkv(void* out, int out_dtype, const void* query,
                                   const void* key_cache, const void* value_cache, int kv_dtype,
                                   const int32_t* block_tables, int max_blocks_per_seq,
                                   const int32_t* context_lens, int batch, int q_len,
                                   int num_q_heads, int gqa_factor, int head_dim, int block_size,
                                   int64_t num_blocks, float scale, int max_context_len,
                                   int partition_size, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * paged_attention_decode_splitkv_noalloc — paged_attention_decode_splitkv for
 * callers that cannot allocate memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the same arguments without
 * the workspace, the same kernels and the same result bit for bit.  The
 * partials go to a static device array of PKV_NOALLOC_SCRATCH_BYTES bytes
 * inside the library, one per GPU (each GPU holds it until the process ends);
 * its device address is looked up on the first call on each device, and no
 * call allocates or frees anything.
 *   - A call whose partials need more than PKV_NOALLOC_SCRATCH_BYTES
 *     (batch * q_len * num_q_heads * ceil(max_context_len / partition_size)
 *     * (head_dim + 2) * 4 bytes) returns PKV_ERR_WORKSPACE and launches
 *     nothing.
 *   - Every call on one GPU shares that GPU's array: two calls that overlap in
 *     time on one GPU (different streams, or different threads) race and
 *     produce garbage.  Calls in stream order on one stream are safe.  The
 *     array keeps the last call's partials; nothing needs to start at zero.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (16u * 1024u * 1024u)

int paged_attention_decode_splitkv_noalloc(void* out, int out_dtype, const void* query,
                                           const void* key_cache, const void* value_cache,
                                           int kv_dtype, const int32_t* block_tables,
                                           int max_blocks_per_seq, const int32_t* context_lens,
                                           int batch, int q_len, int num_q_heads, int gqa_factor,
                                           int head_dim, int block_size, int64_t num_blocks,
                                           float scale, int max_context_len, int partition_size,
                                           void* stream);

/*
 * The two halves of paged_attention_decode_splitkv as separate launches, for
 * callers that schedule or combine them themselves (e.g. to merge partials of
 * several passes).
 *
 * paged_attention_decode_splitkv_partials launches only the partition kernel.
 * Workspace layout (float32, rows = batch * q_len * num_q_heads in
 * [b][i][h] order, P = ceil(max_context_len / partition_size)):
 *   o[rows][P][head_dim]  unnormalised partial outputs  sum_j 2^(s_j - m) v_j
 *   m[rows][P]            partition max of s_j = scale * q.k_j * log2(e)
 *                         (-inf if the row sees no position in the partition)
 *   l[rows][P]            sum_j 2^(s_j - m)
 * Partition p covers positions [p * partition_size, (p+1) * partition_size),
 * the last one runs to the end of the sequence; a partition that starts at or
 * past a sequence's (clamped) length gets m = -inf, l = 0 and no o.
 *
 * paged_attention_decode_splitkv_merge reads the P partials of every row
 * (skipping those with m = -inf) and writes
 * out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p with M = max_p m_p
 * (zeros where no partition saw a position).
 */
int paged_attention_decode_splitkv_partials(const void* query, const void* key_cache,
                                            const void* value_cache, int kv_dtype,
                                            const int32_t* block_tables, int max_blocks_per_seq,
                                            const int32_t* context_lens, int batch, int q_len,
                                            int num_q_heads, int gqa_factor, int head_dim,
                                            int block_size, int64_t num_blocks, float scale,
                                            int max_context_len, int partition_size,
                                            void* workspace, size_t workspace_bytes, void* stream);

int paged_attention_decode_splitkv_merge(void* out, int out_dtype, int batch, int q_len,
                                         int num_q_heads, int head_dim, int max_context_len,
                                         int partition_size, const void* workspace,
                                         size_t workspace_bytes, void* stream);

/*
 * paged_attention_decode_window / paged_attention_decode_splitkv_window —
 * decode over a sliding window of the context ("How MTPLX Manages Memory
 * Using Request-Sized Paged KV Cache", Sliding-Window Memory Control and the
 * sliding_window argument of its paged attention call: older tokens are
 * masked while their blocks stay allocated; mlxcel "KV Cache",
 * RotatingKVCache).  Query row i of sequence b, at position
 * p = context_lens[b] - q_len + i, sees positions max(0, p - W + 1) .. p,
 * i.e. its W most recent positions (itself included); W = sliding_window,
 * 0 meaning the whole context.  Blocks that hold no position any row may see
 * are not read.  In the split form the partitions of a sequence are counted
 * from the block holding its first visible position, so the grid spans
 * S = min(max_context_len, sliding_window + q_len + 15) positions and the
 * workspace needs paged_attention_decode_splitkv_workspace_size(..., S,
 * partition_size) bytes (partitions with nothing to read are marked empty).
 * Every other argument and the errors are those of
 * paged_attention_decode[_splitkv]; sliding_window < 0 returns PKV_ERR_SHAPE.
 * 16-bit caches only.
 */
int paged_attention_decode_window(void* out, int out_dtype, const void* query,
                                  const void* key_cache, const void* value_cache, int kv_dtype,
                                  const int32_t* block_tables, int max_blocks_per_seq,
                                  const int32_t* context_lens, int batch, int q_len,
                                  int num_q_heads, int gqa_factor, int head_dim, int block_size,
                                  int64_t num_blocks, float scale, int sliding_window,
                                  void* stream);

int paged_attention_decode_splitkv_window(void* out, int out_dtype, const void* query,
                                          const void* key_cache, const void* value_cache,
                                          int kv_dtype, const int32_t* block_tables,
                                          int max_blocks_per_seq, const int32_t* context_lens,
                                          int batch, int q_len, int num_q_heads, int gqa_factor,
                                          int head_dim, int block_size, int64_t num_blocks,
                                          float scale, int sliding_window, int max_context_len,
                                          int partition_size, void* workspace,
                                          size_t workspace_bytes, void* stream);

/*
 * paged_attention_decode_window_append / paged_attention_decode_splitkv_window_append —
 * the windowed decode step with the slot write folded into the attention
 * launch: the result, in `out` and in the caches, is that of
 * paged_attention_decode_append's write followed by
 * paged_attention_decode[_splitkv]_window with the same arguments (the new
 * rows are stored whether or not any window reaches them).  Arguments,
 * workspace (sized for the window's span S) and errors as for those calls.
 * 16-bit caches only.
 */
int paged_attention_decode_window_append(void* out, int out_dtype, const void* query,
                                         const void* new_key, const void* new_value,
                                         void* key_cache, void* value_cache, int kv_dtype,
                                         const int32_t* block_tables, int max_blocks_per_seq,
                                         const int32_t* context_lens, int batch, int q_len,
                                         int num_q_heads, int gqa_factor, int head_dim,
                                         int block_size, int64_t num_blocks, float scale,
                                         int sliding_window, void* stream);

int paged_attention_decode_splitkv_window_append(
    void* out, int out_dtype, const void* query, const void* new_key, const void* new_value,
    void* key_cache, void* value_cache, int kv_dtype, const int32_t* block_tables,
    int max_blocks_per_seq, const int32_t* context_lens, int batch, int q_len, int num_q_heads,
    int gqa_factor, int head_dim, int block_size, int64_t num_blocks, float scale,
    int sliding_window, int max_context_len, int partition_size, void* workspace,
    size_t workspace_bytes, void* stream);

/*
 * paged_attention_decode_cascade — split-KV decode for batches whose
 * sequences share whole-block prefixes in groups (mlxcel "KV Cache", Paged
 * Decode Storage and Kernels: cascade attention for groups that share a
 * sufficiently long whole-page prefix).  The result is that of
 * paged_attention_decode_splitkv (up to fp32 summation order); the shared
 * blocks are read once per group instead of once per member:
 *   1. prefix pass: for group g, the first group_prefix_blocks[g] blocks of
 *      the table of its first member group_members[g][0] are attended by the
 *      query rows of every member at once (the rows are stacked in one tile,
 *      so group_size * gqa_factor * q_len <= 16); each row keeps its own
 *      causal limit;
 *   2. suffix pass: every sequence attends its positions from the end of its
 *      group's prefix (from 0 outside every group), as a balanced split
 *      (paged_attention_decode_splitkv with partition_size 0) over those
 *      suffixes: a small kernel first writes each sequence's suffix length
 *      and first suffix table entry into the workspace;
 *   3. the log-sum-exp merge of both passes' partials.
 *   partition_size applies to the prefix pass (a positive multiple of 16).
 *   group_members: int32 [num_groups, group_size], device; sequence indices,
 *                  -1 for an empty slot.  A sequence appears in at most one
 *                  group; a group whose first slot is -1 is ignored.
 *   group_prefix_blocks: int32 [num_groups], device; the members' first
 *                  group_prefix_blocks[g] table entries must name the same
 *                  blocks (only the first member's are read).
 *   max_prefix_len: host bound on 16 * group_prefix_blocks[g] (grid size).
 * Workspace: paged_attention_decode_cascade_workspace_size bytes: the prefix
 * partials (batch * q_len * num_q_heads rows x P prefix partitions x
 * (head_dim + 2) floats, P = ceil(max_prefix_len / partition_size), at least
 * 1), then the suffix pass's balanced-split workspace (as its
 * paged_attention_decode_splitkv_workspace_size with partition_size 0), then
 * two int32 per sequence, each region rounded up to 256 bytes; contents on
 * entry do not matter.  Requires what the balanced split requires
 * (num_q_heads <= 2048, batch * max_blocks_per_seq < 2^31).  No window, no
 * append form.  16-bit caches only.
 */
int paged_attention_decode_cascade_workspace_size(int batch, int q_len, int num_q_heads,
                                                  int head_dim, int max_context_len,
                                                  int max_prefix_len, int partition_size,
                                                  size_t* out_bytes);

int paged_attention_decode_cascade(void* out, int out_dtype, const void* query,
                                   const void* key_cache, const void* value_cache, int kv_dtype,
                                   const int32_t* block_tables, int max_blocks_per_seq,
                                   const int32_t* context_lens, int batch, int q_len,
                                   int num_q_heads, int gqa_factor, int head_dim, int block_size,
                                   int64_t num_blocks, float scale, const int32_t* group_members,
                                   const int32_t* group_prefix_blocks, int num_groups,
                                   int group_size, int max_prefix_len, int max_context_len,
                                   int partition_size, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * paged_attention_decode_splitkv_sparse_v — APPROXIMATE split-KV decode that
 * skips reading V rows of negligible weight ("The KV Cache" (metalworking),
 * arithmetic paragraph: sparse-V decode at long context is a KV-cache traffic
 * deletion; the skip rule is not given there, this is the library's):
 *   the V row of position j (one KV head) is read only if some query row of
 *   that head has 2^(s_j - m) >= v_threshold, where s is the row's score in
 *   log2 units and m the row's running maximum score including j's block;
 *   skipped positions still count in the softmax sum.
 * Guarantee: a skipped position weighs less than v_threshold times its row's
 * largest weight, so |out - exact| <= sum over such positions of
 * w_j |v_j| / sum_j w_j per element.  v_threshold = 0 reads every row (the
 * exact result).  v_rows_read (device, nullable) is incremented by the
 * number of (block, KV head, token) V rows read.  Same arguments, workspace
 * and errors as paged_attention_decode_splitkv otherwise; v_threshold outside
 * [0, 1) is PKV_ERR_SHAPE; needs gqa_factor * q_len <= 4 and a 16-bit cache.
 * Not recommended on MI355X: the dense split-KV call is faster even where
 * this one reads a tenth of the V rows (32K context, sharply peaked rows:
 * 69 against 32.5 us per layer), because the K -> V dependency adds a
 * workgroup barrier and an exposed V load per round while the dense kernel
 * is bound by load structure and latency, not by bytes.  It is kept as the
 * reading of the pages' traffic deletion, with its proven error bound.
 */
int paged_attention_decode_splitkv_sparse_v(
    void* out, int out_dtype, const void* query, const void* key_cache, const void* value_cache,
    int kv_dtype, const int32_t* block_tables, int max_blocks_per_seq,
    const int32_t* context_lens, int batch, int q_len, int num_q_heads, int gqa_factor,
    int head_dim, int block_size, int64_t num_blocks, float scale, float v_threshold,
    unsigned long long* v_rows_read, int max_context_len, int partition_size, void* workspace,
    size_t workspace_bytes, void* stream);

/*
 * paged_attention_decode_append / paged_attention_decode_splitkv_append —
 * the decode step with the slot write folded into the attention launch
 * (mlxcel "KV Cache", Attention Dispatch and In-Place Decode Writes: the new
 * K/V row is written into the cache in place during decode).  The result, in
 * `out` and in the caches, is that of
 *     kv_cache_write(new_key, new_value, key_cache, value_cache, slots, ...)
 * followed by paged_attention_decode[_splitkv](...) with the same arguments,
 * where the slots are those the block tables give the new positions: token
 * b * q_len + i of new_key / new_value goes to position
 * context_lens[b] - q_len + i of sequence b, i.e. block
 * block_tables[b][pos / 16], row pos % 16.
 *   new_key, new_value: [batch * q_len, num_kv_heads, head_dim] of kv_dtype
 *   key_cache, value_cache: written (the new rows) and read
 * A new token whose position is negative (context_lens[b] < q_len) or whose
 * table entry lies outside [0, num_blocks) is neither stored nor attended.
 * Lengths are clamped to max_blocks_per_seq * 16 first.  Every other argument,
 * the workspace and the errors are those of the unfused calls.  The attention
 * reads the new rows from new_key / new_value, so the launch never reads back
 * what it stores.  Only 16-bit caches (f16, bf16).
 */
int paged_attention_decode_append(void* out, int out_dtype, const void* query,
                                  const void* new_key, const void* new_value, void* key_cache,
                                  void* value_cache, int kv_dtype, const int32_t* block_tables,
                                  int max_blocks_per_seq, const int32_t* context_lens, int batch,
                                  int q_len, int num_q_heads, int gqa_factor, int head_dim,
                                  int block_size, int64_t num_blocks, float scale, void* stream);

int paged_attention_decode_splitkv_append(void* out, int out_dtype, const void* query,
                                          const void* new_key, const void* new_value,
                                          void* key_cache, void* value_cache, int kv_dtype,
                                          const int32_t* block_tables, int max_blocks_per_seq,
                                          const int32_t* context_lens, int batch, int q_len,
                                          int num_q_heads, int gqa_factor, int head_dim,
                                          int block_size, int64_t num_blocks, float scale,
                                          int max_context_len, int partition_size,
                                          void* workspace, size_t workspace_bytes, void* stream);

/* Partition-kernel half of paged_attention_decode_splitkv_append (the new
 * rows are stored and their partial is in the workspace when it completes;
 * finish with paged_attention_decode_splitkv_merge). */
int paged_attention_decode_splitkv_append_partials(
    const void* query, const void* new_key, const void* new_value, void* key_cache,
    void* value_cache, int kv_dtype, const int32_t* block_tables, int max_blocks_per_seq,
    const int32_t* context_lens, int batch, int q_len, int num_q_heads, int gqa_factor,
    int head_dim, int block_size, int64_t num_blocks, float scale, int max_context_len,
    int partition_size, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kv_cache_write_k8v4 — quantize-on-write into a K8/V4 cache.
 *   key, value: [num_tokens, num_kv_heads, head_dim] of in_dtype (f16 or bf16)
 *   k_cache int8   [num_blocks, block_size, num_kv_heads, head_dim]
 *   k_scale fp16   [num_blocks, block_size, num_kv_heads]
 *   v_cache uint8  [num_blocks, block_size, num_kv_heads, head_dim / 2]
 *   v_scale, v_zero fp16 [num_blocks, block_size, num_kv_heads, head_dim / 32]
 * Side tensors are indexed like the cache ("How MTPLX Manages Memory Using
 * Request-Sized Paged KV Cache", Quantization-Aware Memory Layout).
 * K per (token, head), in fp32: amax = max|k|; s = fp16_rne(amax / 127);
 *   code = s == 0 ? 0 : clamp(rint_even(k / s), -127, 127).
 * V per group of 32, in fp32: s = fp16_rne((max - min) / 15); z = fp16_rne(min);
 *   code = s == 0 ? 0 : clamp(rint_even((v - z) / s), 0, 15); element 2i in the
 *   low nibble of byte i, element 2i+1 in the high nibble.
 * Divisions are correctly rounded, so codes and scales are bit-exact.
 */
int kv_cache_write_k8v4(const void* key, const void* value, int in_dtype, int8_t* k_cache,
                        void* k_scale, uint8_t* v_cache, void* v_scale, void* v_zero,
                        const int64_t* slot_mapping, int64_t num_tokens, int num_kv_heads,
                        int head_dim, int block_size, int64_t num_blocks, void* stream);

/*
 * paged_attention_decode_k8v4 — paged_attention_decode over the K8/V4 arrays
 * above, dequantizing in registers (k = code * s; v = code * s + z).
 * query and out as in paged_attention_decode with query of q_dtype (f16/bf16).
 * Range: the V scales enter fp16 products as weight * scale with weights up
 * to 2^8, so every V scale must stay below 65504 / 2^8 (a V group spanning
 * less than about 3800); beyond that the output is not finite.
 */
int paged_attention_decode_k8v4(void* out, int out_dtype, const void* query, int q_dtype,
                                const int8_t* k_cache, const void* k_scale,
                                const uint8_t* v_cache, const void* v_scale, const void* v_zero,
                                const int32_t* block_tables, int max_blocks_per_seq,
                                const int32_t* context_lens, int batch, int q_len,
                                int num_q_heads, int gqa_factor, int head_dim, int block_size,
                                int64_t num_blocks, float scale, void* stream);

/* Split-KV form of paged_attention_decode_k8v4 (workspace as for the fp16 call). */
int paged_attention_decode_splitkv_k8v4(void* out, int out_dtype, const void* query, int q_dtype,
                                        const int8_t* k_cache, const void* k_scale,
                                        const uint8_t* v_cache, const void* v_scale,
                                        const void* v_zero, const int32_t* block_tables,
                                        int max_blocks_per_seq, const int32_t* context_lens,
                                        int batch, int q_len, int num_q_heads, int gqa_factor,
                                        int head_dim, int block_size, int64_t num_blocks,
                                        float scale, int max_context_len, int partition_size,
                                        void* workspace, size_t workspace_bytes, void* stream);

/* Partition-kernel half of paged_attention_decode_splitkv_k8v4 (merge with
 * paged_attention_decode_splitkv_merge). */
int paged_attention_decode_splitkv_k8v4_partials(
    const void* query, int q_dtype, const int8_t* k_cache, const void* k_scale,
    const uint8_t* v_cache, const void* v_scale, const void* v_zero, const int32_t* block_tables,
    int max_blocks_per_seq, const int32_t* context_lens, int batch, int q_len, int num_q_heads,
    int gqa_factor, int head_dim, int block_size, int64_t num_blocks, float scale,
    int max_context_len, int partition_size, void* workspace, size_t workspace_bytes,
    void* stream);

/*
 * paged_attention_decode_k8v4_append / paged_attention_decode_splitkv_k8v4_append —
 * the K8/V4 decode step with the quantize-on-write folded into the attention
 * launch (mlxcel "KV Cache", Attention Dispatch and In-Place Decode Writes; the
 * quantization is that of kv_cache_write_k8v4).  The result, in `out` and in
 * the five cache arrays, is that of
 *     kv_cache_write_k8v4(new_key, new_value, q_dtype, k_cache, ..., slots, ...)
 * followed by paged_attention_decode[_splitkv]_k8v4(...) with the same
 * arguments, the slots being those the block tables give the new positions
 * (as for paged_attention_decode_append): codes and scales bit-exact, the
 * attention over the quantized new rows.
 *   new_key, new_value: [batch * q_len, num_kv_heads, head_dim] of q_dtype
 *   k_cache, k_scale, v_cache, v_scale, v_zero: written (the new rows) and read
 * New tokens whose position is negative or whose table entry lies outside
 * [0, num_blocks) are neither stored nor attended.  Every other argument, the
 * workspace and the errors are those of the unfused calls.
 */
int paged_attention_decode_k8v4_append(void* out, int out_dtype, const void* query, int q_dtype,
                                       const void* new_key, const void* new_value,
                                       int8_t* k_cache, void* k_scale, uint8_t* v_cache,
                                       void* v_scale, void* v_zero, const int32_t* block_tables,
                                       int max_blocks_per_seq, const int32_t* context_lens,
                                       int batch, int q_len, int num_q_heads, int gqa_factor,
                                       int head_dim, int block_size, int64_t num_blocks,
                                       float scale, void* stream);

int paged_attention_decode_splitkv_k8v4_append(
    void* out, int out_dtype, const void* query, int q_dtype, const void* new_key,
    const void* new_value, int8_t* k_cache, void* k_scale, uint8_t* v_cache, void* v_scale,
    void* v_zero, const int32_t* block_tables, int max_blocks_per_seq,
    const int32_t* context_lens, int batch, int q_len, int num_q_heads, int gqa_factor,
    int head_dim, int block_size, int64_t num_blocks, float scale, int max_context_len,
    int partition_size, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Cache bytes one token occupies over all layers (host-only arithmetic).
 * "The KV Cache", arithmetic paragraph: one K and one V vector per KV head per
 * layer; fp16/bf16: 2 * layers * kv_heads * head_dim * 2.  K8/V4:
 * layers * kv_heads * (head_dim + 2 + head_dim/2 + 4 * head_dim/32).
 */
int kv_cache_bytes_per_token(int num_layers, int num_kv_heads, int head_dim, int kv_format,
                             int64_t* out_bytes);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */

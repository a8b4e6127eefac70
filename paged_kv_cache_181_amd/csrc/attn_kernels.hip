// Paged-attention decode kernels for gfx950 (CDNA4).
//
// What is computed (see pagedkv.h for the contract): for every sequence b,
// query token i of a q_len block and query head h, softmax attention over the
// cached positions 0 .. len_b - q_len + i, where position j lives in block
// block_tables[b][j / 16] at row j % 16 ("The KV Cache" (metalworking), layout
// paragraph: fixed-size blocks plus an indirection table) and head h reads KV
// head h / gqa ("The KV Cache", arithmetic paragraph).
//
// Work decomposition
//   grid = (partition, KV head, sequence); a workgroup of NW wavefronts owns the
//   blocks of one partition; wavefront w takes a contiguous run of them.  All
//   G*q_len query rows that share a KV head live in one wavefront, so each K/V
//   byte is read from HBM once.  In the head-pair and head-quad forms a
//   workgroup takes two or four KV heads, an equal share of its wavefronts
//   each (grid = (partition, head group, sequence)); they run when that
//   brings the grid down to one workgroup per CU.  The direct form is the same kernel with one
//   partition per sequence; the split-KV form writes per-partition partials and
//   a second kernel merges them by log-sum-exp.  The same kernel also runs
//   the append form (the new tokens stored into the cache at launch start and
//   attended: patched into the last cache block when they share it, else as
//   one more tile), the
//   sliding window (partitions counted from the window's first block) and the
//   two cascade passes (a group's rows stacked in one tile over its shared
//   prefix; each sequence past its group's prefix).  The approximate sparse-V
//   kernel further down reads V rows selectively.
//
// Per 16-token block, per wavefront (lane l: row l % 16, quarter l / 16):
//   - K rows are loaded straight into the A operand of a 16x16x32 MFMA
//     (lane l holds 8 head dims of token l % 16 per step), giving S^T = K Q^T:
//     lane l ends with the scores of query row l % 16 for tokens 4*(l/16)+r.
//   - Online softmax (running max and sum per row in fp32, exp2 domain); the
//     block max is reduced across the four quarters with two lane exchanges.
//   - The probabilities are already in the B-operand layout of a 16x16x16 MFMA
//     computing O^T = V^T P^T; they are split into a 16-bit high part and a
//     16-bit remainder so the product keeps ~21 bits of each weight.
//   - V rows are staged through LDS (natural [token][dim] layout) and read back
//     transposed as the A operand.  Output lane l holds row l % 16's dims
//     16n + 4*(l/16) + r, so the softmax rescale is one factor per lane.
//   - Loads of the next block are issued before the current block is used.
//   - Positions past the length, past a row's causal limit, before a row's
//     sliding window, or in a block whose table entry is out of range are
//     excluded by selecting -inf scores, and V rows that no row may see are
//     zeroed, so NaN garbage there never propagates.  Blocks wholly before
//     every row's window are not read.
//
// K8/V4 storage: int8 K codes are converted exactly to the MFMA element type and
// the per-token scale multiplies the scores; 4-bit V codes are converted exactly
// and staged like 16-bit V, the per-group scale is folded into the weights
// (sum_t p_t s_tg c_td) and the zero point into a per-group sum (sum_t p_t z_tg).
// The conversions are bit tricks, a few instructions per 8 codes:
//  - K: the offset-binary byte u = c + 128 becomes the fp16 1024 + u by placing
//    it under the exponent byte 0x64 (one byte permute per two codes), or, for
//    bf16 queries, the exact float of u truncated to bf16.  The constant offset
//    (1152 or 128) times the row's query sum starts the score accumulator, so
//    the scores come out exact (one MFMA pass per wave computes it).
//  - V: a nibble masked into fp16 mantissa bits 0..3 under exponent byte 0x64
//    is 1024 + c, in bits 4..7 under 0x54 it is 64 + c; one packed fp16
//    subtract makes it c exactly.  Two masks of a 32-bit word and of the word
//    shifted by 8 give the codes pairwise as (c0,c4), (c1,c5), (c2,c6), (c3,c7),
//    and the V tile is staged in that order; the output dims are put back in
//    order when the partial is written.  The PV products always run in fp16 (codes are
//    small integers; the weights are split hi/lo).

#include <math.h>
#include <atomic>
#include <stddef.h>

#include "pkv_common.h"
#include "pkv_launch.h"

// PKV_QK_VALU=1 builds a measurement variant of the library in which the
// 16-bit partition kernel computes the scores with vector dot products
// instead of MFMA (libpagedkv_qkvalu.so; the MFMA build is the product).
#ifndef PKV_QK_VALU
#define PKV_QK_VALU 0
#endif

namespace pkv {

constexpr float kNegInf = -INFINITY;
constexpr bool kQkOnValu = PKV_QK_VALU != 0;

// Head dims of the K/Q operand held by quarter qd at QK step m (8 consecutive).
template <Fmt KV>
__device__ __forceinline__ int qk_dim(int m, int qd) {
  if constexpr (KV == Fmt::K8V4) return 64 * (m >> 1) + 16 * qd + 8 * (m & 1);
  else return 32 * m + 8 * qd;
}

// Four int8 K codes (one 32-bit word) -> two words of 16-bit MFMA elements
// holding off + c exactly, in dim order: off = 1152 for fp16 queries, 128 for
// bf16 ones.  kK8NegOffset2 is -off in both halves of a word (fp16 0xE480 =
// -1152, bf16 0xC300 = -128): the operand that makes -off * sum(q).
template <Fmt QT> constexpr uint32_t kK8NegOffset2 = QT == Fmt::F16 ? 0xE480E480u : 0xC300C300u;

template <Fmt QT>
__device__ __forceinline__ void k8_codes(uint32_t x, uint32_t& lo, uint32_t& hi) {
  const uint32_t u = x ^ 0x80808080u;                    // bytes c + 128
  if constexpr (QT == Fmt::F16) {
    // {u.b0, 0x64, u.b1, 0x64}: fp16 (0x64 << 8 | u) = 1024 + u
    lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
    hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
  } else {
    // the float of an integer below 256 has 8 significant bits: its upper
    // half is the exact bf16
    const uint32_t f0 = __float_as_uint((float)(u & 0xffu));
    const uint32_t f1 = __float_as_uint((float)((u >> 8) & 0xffu));
    const uint32_t f2 = __float_as_uint((float)((u >> 16) & 0xffu));
    const uint32_t f3 = __float_as_uint((float)(u >> 24));
    lo = __builtin_amdgcn_perm(f1, f0, 0x07060302u);
    hi = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
  }
}

// Eight 4-bit V codes (one 32-bit word, code k in bits 4k..4k+3) -> four words
// of fp16 pairs (c0,c4), (c1,c5), (c2,c6), (c3,c7), exact.  A nibble in
// mantissa bits 0..3 under exponent byte 0x64 is 1024 + c; in bits 4..7 under
// 0x54 it is 64 + c (the unit in the last place there is 1/16).
// The mask and magic constants live in registers (masks in scalar, magics in
// vector registers: one scalar operand per instruction), which lets each
// mask-and-insert be one v_and_or_b32.
struct V4Consts {
  uint32_t m0 = 0x000f000fu, m1 = 0x00f000f0u, e0 = 0x64006400u, e1 = 0x54005400u;
  __device__ __forceinline__ V4Consts() {
    asm volatile("" : "+s"(m0), "+s"(m1), "+v"(e0), "+v"(e1));
  }
};
__device__ __forceinline__ u4 v4_codes(uint32_t w, const V4Consts& c) {
  const uint32_t w8 = w >> 8;
  const h2 o1024 = h2{(_Float16)1024.f, (_Float16)1024.f}, o64 = h2{(_Float16)64.f, (_Float16)64.f};
  const h2 v0 = __builtin_bit_cast(h2, (w & c.m0) | c.e0) - o1024;
  const h2 v1 = __builtin_bit_cast(h2, (w & c.m1) | c.e1) - o64;
  const h2 v2 = __builtin_bit_cast(h2, (w8 & c.m0) | c.e0) - o1024;
  const h2 v3 = __builtin_bit_cast(h2, (w8 & c.m1) | c.e1) - o64;
  return u4{__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1),
            __builtin_bit_cast(uint32_t, v2), __builtin_bit_cast(uint32_t, v3)};
}

// Dim (within its 16-dim tile) of PV output row i of a staged K8/V4 tile:
// position i & 7 of an 8-dim chunk holds dim ((i & 7) >> 1) + 4 * (i & 1).
__device__ __forceinline__ constexpr int v4_dim(int i) {
  return 8 * (i >> 3) + ((i & 7) >> 1) + 4 * (i & 1);
}

// Registers of one block for one lane.
template <Fmt KV, int D> struct BlockRegs;

template <int D> struct BlockRegs<Fmt::F16, D> {
  u4 k[D / 32];
  u4 v[D / 32];
};
template <int D> struct BlockRegs<Fmt::BF16, D> {
  u4 k[D / 32];
  u4 v[D / 32];
};
template <int D> struct BlockRegs<Fmt::K8V4, D> {
  u4 k[D / 64];          // 16 int8 codes per u4
  u4 v;                  // D/8 bytes of packed 4-bit codes (D=64 uses .x,.y)
  uint32_t ks;           // fp16 bits of this lane's token K scale
  u2 vs, vz;             // fp16 bits of the token's V scales / zeros (D/32 groups)
};

// A buffer resource covering `bytes` bytes from `base` (wave-uniform): the
// loads below are a scalar base plus a fixed 32-bit per-lane offset, and any
// access past `bytes` reads 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Keeps a loop-invariant lane offset from being hoisted together with the
// constant added to it, so the constant stays in the load's immediate field
// instead of occupying a register of its own for the whole loop.
__device__ __forceinline__ uint32_t pin(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

template <typename T>
__device__ __forceinline__ T buf_load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (sizeof(T) == 16) {
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
  } else if constexpr (sizeof(T) == 8) {
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
  } else if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
  } else {
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0));
  }
}

// Byte offsets of this lane's data inside one block of one KV head (token rho,
// quarter qd), and the byte size of one block of all KV heads.
template <Fmt KV, int D>
struct LaneOffsets {
  uint32_t k, v, ks, vs;           // K codes/rows, V codes/rows, K scale, V scale/zero
  uint32_t kblk, vblk, ksblk, vsblk;
  __device__ __forceinline__ LaneOffsets(int hkv, int g, int rho, int qd) {
    if constexpr (KV == Fmt::K8V4) {
      k = (uint32_t)((rho * hkv + g) * D + 16 * qd);
      v = (uint32_t)((rho * hkv + g) * (D / 2) + (D == 128 ? 16 : 8) * qd);
      ks = (uint32_t)((rho * hkv + g) * 2);
      vs = (uint32_t)((rho * hkv + g) * (D / 32) * 2);
      kblk = (uint32_t)(kBlock * hkv * D);
      vblk = (uint32_t)(kBlock * hkv * (D / 2));
      ksblk = (uint32_t)(kBlock * hkv * 2);
      vsblk = (uint32_t)(kBlock * hkv * (D / 32) * 2);
    } else {
      k = v = (uint32_t)(((rho * hkv + g) * D + 8 * qd) * 2);
      ks = vs = 0;
      kblk = vblk = (uint32_t)(kBlock * hkv * D * 2);
      ksblk = vsblk = 0;
    }
  }
};

// Loads block pb (wave-uniform) into this lane's registers.  With `live`
// false the loads are still issued (so the code has no branch around them)
// but through zero-length resources: they return zeros and touch no memory.
template <Fmt KV, int D>
__device__ __forceinline__ void load_block(const AttnArgs& a, int64_t pb, bool live,
                                           const LaneOffsets<KV, D>& lo, BlockRegs<KV, D>& br) {
  const uint32_t on = live ? ~0u : 0u;
  if constexpr (KV == Fmt::K8V4) {
    const auto kr = span_rsrc((const char*)a.k_cache + pb * lo.kblk, lo.kblk & on);
    const auto vr = span_rsrc((const char*)a.v_cache + pb * lo.vblk, lo.vblk & on);
    const auto ksr = span_rsrc((const char*)a.k_scale + pb * lo.ksblk, lo.ksblk & on);
    const auto vsr = span_rsrc((const char*)a.v_scale + pb * lo.vsblk, lo.vsblk & on);
    const auto vzr = span_rsrc((const char*)a.v_zero + pb * lo.vsblk, lo.vsblk & on);
    const uint32_t ko = pin(lo.k);
#pragma unroll
    for (int u = 0; u < D / 64; ++u) br.k[u] = buf_load<u4>(kr, ko + 64 * u);
    if constexpr (D == 128) {
      br.v = buf_load<u4>(vr, lo.v);
      br.vs = buf_load<u2>(vsr, lo.vs);
      br.vz = buf_load<u2>(vzr, lo.vs);
    } else {
      const u2 t = buf_load<u2>(vr, lo.v);
      br.v = u4{t.x, t.y, 0u, 0u};
      br.vs = u2{buf_load<uint32_t>(vsr, lo.vs), 0u};
      br.vz = u2{buf_load<uint32_t>(vzr, lo.vs), 0u};
    }
    br.ks = buf_load<uint16_t>(ksr, lo.ks);
  } else {
    const auto kr = span_rsrc((const char*)a.k_cache + pb * lo.kblk, lo.kblk & on);
    const auto vr = span_rsrc((const char*)a.v_cache + pb * lo.vblk, lo.vblk & on);
    const uint32_t ko = pin(lo.k), vo = pin(lo.v);
#pragma unroll
    for (int m = 0; m < D / 32; ++m) br.k[m] = buf_load<u4>(kr, ko + 64 * m);
#pragma unroll
    for (int m = 0; m < D / 32; ++m) br.v[m] = buf_load<u4>(vr, vo + 64 * m);
  }
}

// Workgroup shape: RT query rows per KV head tile (4 when G*q_len <= 4, else
// 16).  The 16-bit 4-row form runs 8 wavefronts at 4 per SIMD (128 registers),
// the K8/V4 4-row form and the 16-bit 16-row form 4 wavefronts at 4 per SIMD
// (the 16-row form's LDS, merge included, stays under 40 KB so that four
// workgroups share a CU), and the K8/V4 16-row form, which holds more per
// lane, 4 wavefronts at 3.
// The K8/V4 head-group form (HP KV heads per workgroup) runs one wavefront
// per head.
template <Fmt KV, int RT, int HP = 1> struct Shape {
  static constexpr bool WIDE = RT == 4 && KV != Fmt::K8V4;
  static constexpr int NW = KV == Fmt::K8V4 && HP > 1 ? HP : WIDE ? 8 : 4;
  static constexpr int WAVES_PER_SIMD = RT == 4 || KV != Fmt::K8V4 ? 4 : 3;
};

template <Fmt KV, int D, int RT, int HP = 1>
struct AttnSmem {
  static constexpr int NW = Shape<KV, RT, HP>::NW;
  static constexpr int GR = D / 32;                        // V groups per row
  static constexpr int VT = 16 * D * 2;                    // one staged V tile (bytes)
  static constexpr int VST = NW * VT;
  // K8/V4: per-token scales; the vector-dot score variant: per-wave scores
  static constexpr int SIDE = KV == Fmt::K8V4 ? NW * 16 * (1 + 2 * GR) * 4
                              : kQkOnValu ? NW * RT * 16 * 4 : 0;
  static constexpr int EP = RT == 16 ? 2 : 1;              // merge passes over the head dims
  static constexpr int MO = NW * RT * (D / EP) * 4;        // merge: per-wave outputs (one pass)
  static constexpr int LOOP = VST + SIDE;
  static constexpr int BYTES = LOOP > MO ? LOOP : MO;
  // append form: the new tokens' tile, parked from the start of the launch to
  // the end of the block loop (lanes of rows rho < RT), after the loop area
  static constexpr int STASH = RT * 4 * (int)sizeof(BlockRegs<KV, D>);
  static constexpr int BYTES_APPEND = LOOP + STASH > MO ? LOOP + STASH : MO;
  // forms with HP > 1 heads per workgroup: a parked tile per head, and more
  // than half of a CU's 160 KB, so that one workgroup runs per CU
  template <int NH> static constexpr int bytes_group() {
    constexpr int used = LOOP + NH * STASH > MO ? LOOP + NH * STASH : MO;
    return used > 82 * 1024 ? used : 82 * 1024;
  }
  static constexpr int QSTR = D + 8;                       // halves per staged query row
  // staged query copies: one per wave (no wave waits on another), or in the
  // 16-row forms one shared copy (keeps their LDS under 40 KB)
  static constexpr int QCOPIES = RT == 16 ? 1 : NW;
};

// Max over lanes l, l^16, l^32, l^48 (the four quarters) without the LDS path.
__device__ __forceinline__ float quarter_max(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float quarter_sum(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Transposing LDS read (gfx950): within each group of 16 lanes, lane j gets
// element j%4 of the 8-byte chunks addressed by lanes 4e + j/4, e = 0..3.
__device__ __forceinline__ u2 lds_read_tr16(const unsigned char* p) {
  typedef short s4v __attribute__((ext_vector_type(4)));
  s4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s4v*)(p));
  return __builtin_bit_cast(u2, v);
}

// The running max of a row only moves when a block's max exceeds it by more
// than this (log2 units), so rescaling the accumulators is rare; weights are
// then at most 2^8, well inside fp16/bf16 range.
constexpr float kRescaleSlack = 8.f;

// HP: KV heads per workgroup.  1: the workgroup's NW waves share one head and
// split its partition into runs.  2, 4 or 8 (16-bit caches, plain mode): waves
// hw*NW/HP .. take head HP*blockIdx.y + hw, each group splitting the same
// partition (with 8, one wave per head walks the whole partition); a token
// row's HP heads (HP * 256 contiguous bytes at D = 128) are then read
// together, and one workgroup runs per CU.
// (The grouped forms run one workgroup per CU, so two waves per SIMD.)
//
// K8/V4 head groups (HP = 8): one wavefront per KV head, each walking the
// whole partition, so a block's K and V rows of all heads (a 1 KiB K row and
// a 512-byte V row per token at D = 128) and its scale lines are read by one
// CU at once, and no merge inside the workgroup is needed; chosen when the
// grid of head groups fills every CU at least once.
template <Fmt KV, Fmt QT, int D, int RT, bool PREFIX, int HP = 1>
__global__ __launch_bounds__((Shape<KV, RT, HP>::NW * kWave),
                             (HP > 1 ? Shape<KV, RT, HP>::NW / 4 : Shape<KV, RT>::WAVES_PER_SIMD))
void attn_partition_kernel(const AttnArgs a) {
  using MM = Mma<QT>;
  using SM = AttnSmem<KV, D, RT, HP>;
  constexpr int NW = SM::NW;
  constexpr int NWH = NW / HP;         // waves per head
  static_assert(HP == 1 || ((HP == 2 || HP == 4 || HP == 8) && !PREFIX && RT == 4 &&
                            (KV != Fmt::K8V4 || HP == 8)),
                "head groups: 16-bit caches in pairs, quads or eights, K8/V4 in eights; "
                "4-row tiles, plain mode");
  constexpr int KS = D / 32;           // QK MFMA steps
  constexpr int NT = D / 16;           // PV output tiles
  constexpr int GR = SM::GR;
  constexpr int QSTR = SM::QSTR;
  __shared__ __align__(16) unsigned char smem[HP > 1 ? SM::template bytes_group<HP>() : SM::BYTES_APPEND];
  __shared__ __align__(16) uint16_t q_s[SM::QCOPIES * RT * QSTR];
  __shared__ float mm_s[NW][16], ml_s[NW][16];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int hw = w / NWH, wh = w % NWH;   // this wave's head within the workgroup, and its run
  const int rho = lane & 15, qd = lane >> 4;
  // Lane rho is token rho of a loaded block and column rho of the score and
  // output tiles.  In K8/V4 4-row tiles column rho computes query row rho % 4
  // and carries the weights scaled by V group rho / 4, so one PV pass serves
  // every group; elsewhere column rho is row rho (copies past the real rows).
  constexpr bool COLG = KV == Fmt::K8V4 && RT == 4;
  const int lrow = COLG ? (rho & 3) : rho;                  // the query row of column rho
  // (partition, KV head, sequence) of this workgroup.  K8/V4 runs on a 1-D
  // grid ordered so that every KV head of one (partition, sequence) lands on
  // the same XCD (workgroups go to the eight XCDs round-robin in dispatch
  // order): a 128-byte line of 4-bit V codes holds two heads' rows and a line
  // of scales or zeros holds every head's, so within one L2 each such line
  // comes from HBM once, not once per XCD that reads it.  Dispatch id
  // 8 * (g + Hkv * (u / 8)) + u % 8 is head g of unit u = p + parts * b; the
  // grid is rounded up to whole groups of eight units.
  int p, g, b;
  if constexpr (KV == Fmt::K8V4 && HP == 1) {
    const int id = (int)blockIdx.x, hk = a.num_kv_heads;
    const int u = (id / (8 * hk)) * 8 + (id & 7);
    if (u >= a.num_parts * a.batch) return;                 // past the last unit (whole group)
    g = (id >> 3) % hk;
    p = u % a.num_parts;
    b = u / a.num_parts;
  } else {
    p = blockIdx.x;
    g = blockIdx.y * HP + hw;
    b = blockIdx.z;
  }
  const int g0 = g - hw;                                    // the workgroup's first head
  const int Q = a.q_len, G = a.gqa, GQ = G * Q, Hq = a.num_q_heads;
  const bool split = a.ws_o != nullptr;
  // Cascade prefix pass over shared whole-block prefixes (PREFIX, mode 1):
  // b is a group; its S members' rows are stacked in the tile (member m's row
  // iq*G + hl at tile row m*GQ + iq*G + hl), so the shared blocks are read
  // once for all of them.  (The suffix pass is a balanced split.)
  const int S = PREFIX ? a.group_size : 1;
  const int GQT = S * GQ;                                   // tile rows that belong to sequences
  // output (= query) row of tile row rr < GQT, or -1 for an empty member slot
  auto orow_head = [&](int rr, int gg) -> int64_t {
    const int m = rr / GQ, rq = rr - m * GQ;
    const int bm = PREFIX ? a.grp_members[(int64_t)b * S + m] : b;
    return bm < 0 ? -1 : ((int64_t)bm * Q + rq / G) * Hq + gg * G + rq % G;
  };
  auto orow_of = [&](int rr) -> int64_t { return orow_head(rr, g); };
  const int64_t wsp = a.ws_parts;                           // partition slots per row

  // ---- loads that do not depend on the sequence length go out first and
  // together: the table entries of this wave's first blocks, this wave's copy
  // of the query rows, and the length.  Wave w owns the contiguous run of
  // `per` blocks starting at bb + wh*per (wh: w counted within its head's
  // waves, so w itself with one head per workgroup; per is first taken from the
  // partition size, so that a full partition's table chunk can be fetched
  // before the length arrives; a shorter partition re-fetches it for its
  // evenly spread runs further down); lane j holds entry
  // j of a 64-entry chunk of the run, picked out later with readlane, so no
  // table load sits between the K/V loads of consecutive blocks.  Nothing
  // waits on another wave before the first K/V loads.
  // the sequence's table row (a group's: its first member's); entries past
  // max_blocks read as 0 (never used)
  const int tab_b = PREFIX ? a.grp_members[(int64_t)b * S] : b;
  const auto btr = span_rsrc(a.block_tables + (int64_t)max(tab_b, 0) * a.max_blocks,
                             (uint32_t)a.max_blocks * 4u);
  const int bb_guess = p * a.part_blocks;       // the partition's first block without a window
  int per = (a.part_blocks + NWH - 1) / NWH;
  int tbl_next;
  {
    const int e = bb_guess + wh * per + lane;
    tbl_next = lane < per ? buf_load<int>(btr, (uint32_t)e * 4u) : 0;
  }
  constexpr int QCW = RT * (D / 8);                         // 16-byte query chunks per wave
  constexpr int QPL = (QCW + kWave - 1) / kWave;            // per lane
  u4 qv[QPL];
#pragma unroll
  for (int u = 0; u < QPL; ++u) {
    const int idx = lane + u * kWave;
    const int r = idx / (D / 8), c8 = idx % (D / 8);
    qv[u] = u4{0u, 0u, 0u, 0u};
    if (idx < QCW && r < GQT) {
      const int64_t qr = orow_of(r);
      if (qr >= 0) qv[u] = *(const u4*)((const uint16_t*)a.q + qr * D + 8 * c8);
    }
  }
  // the length the block loop covers: the sequence's, or a group's shared prefix
  int L = PREFIX ? (tab_b >= 0 ? a.grp_prefix[b] * kBlock : 0) : a.context_lens[b];
  L = min(max(L, 0), a.max_blocks * kBlock);
  // Append form: the q_len new tokens (positions L-Q .. L-1) come from the
  // new K/V rows, not the cache; the partition holding position L-1 attends
  // to them and stores them into the cache.  Cache blocks then cover Lc.
  const bool append = a.new_k != nullptr;
  const int Lc = append ? max(L - Q, 0) : L;                // positions read from the cache
  const int nblk = (Lc + kBlock - 1) / kBlock;
  // Sliding window W: row i (position L-Q+i) sees positions L-Q+i-W+1 ..
  // L-Q+i, so nothing before lo0 (row 0's first position) is read at all,
  // and partitions are counted from lo0's block (the grid covers the window).
  const int W = a.window;
  const int lo0 = W > 0 ? max(L - Q - W + 1, 0) : 0;
  const int sb = lo0 / kBlock;
  const int bb = sb + bb_guess;                             // the partition's first block
  const int p_new = append && L > 0
                        ? min(((L - 1) / kBlock - sb) / a.part_blocks, a.num_parts - 1) : -1;
  const int be = (p == a.num_parts - 1) ? nblk : min(nblk, bb + a.part_blocks);
  const int b0 = bb;                                        // first block of the partition read
  if (split && b0 >= be && p != p_new) {                    // partition with nothing to read:
    // mark it empty (max -inf, sum 0) so the merge can read every partition
    // without first reading the sequence length
    for (int rr = threadIdx.x; rr < HP * GQT; rr += NW * kWave) {
      const int64_t orow = orow_head(rr % GQT, g0 + rr / GQT);
      if (orow < 0) continue;
      const int64_t pi = orow * wsp + a.part_base + p;
      a.ws_m[pi] = kNegInf;
      a.ws_l[pi] = 0.f;
    }
    return;
  }
  if (const int per_fit = (be - b0 + NWH - 1) / NWH; b0 != bb_guess || per_fit != per) {
    // a partition with fewer blocks than the partition size (the direct
    // form, a sequence's last partition), partitions counted from a window's
    // start, or a last partition longer than the others (length past the
    // grid): the runs are spread evenly over the blocks actually read, so no
    // wave idles while another walks a long run; the first table chunk is
    // fetched again for the new runs
    per = per_fit;
    const int e = b0 + wh * per + lane;
    tbl_next = lane < per ? buf_load<int>(btr, (uint32_t)e * 4u) : 0;
  }
  const int w0 = b0 + wh * per;                             // first block of this wave's run
  const int nmine = max(0, min(per, be - w0));

  // the query row this lane owns: lrow = iq * G + hl, or in the prefix pass
  // member lrow / GQ's row (lrow % GQ) (lanes past the rows compute a copy of
  // a real row; their results are never written)
  int row_len = L;                                          // the row's sequence length
  bool row_ok = lrow < GQT;
  if (PREFIX && row_ok) {
    const int bm = a.grp_members[(int64_t)b * S + lrow / GQ];
    row_ok = bm >= 0;
    row_len = row_ok ? min(max(a.context_lens[bm], 0), a.max_blocks * kBlock) : 0;
  }
  const int iq = row_ok ? (lrow % GQ) / G : 0;
  const int nvis = row_ok ? (row_len - Q + iq + 1) : L;     // visible positions of the row
  // every row sees j < full_lim (the prefix pass masks every tile instead)
  const int full_lim = PREFIX ? -(1 << 30) : L - Q + 1;
  const int lo_row = W > 0 && row_ok ? max(L - Q + iq - W + 1, 0) : lo0;   // window start
  const int lo_max = W > 0 ? max(L - W, 0) : 0;             // every row sees j >= lo_max

  // append form: the table entry of each new token's position (lane rho = token)
  int tnew = -1;
  if (p == p_new) {
    const int pos = L - Q + rho;
    if (rho < Q && pos >= 0) tnew = buf_load<int>(btr, (uint32_t)(pos / kBlock) * 4u);
  }

  int tblv = tbl_next;
  if (64 < nmine) {
    const int kk = 64 + lane;
    tbl_next = kk < nmine ? buf_load<int>(btr, (uint32_t)(w0 + kk) * 4u) : 0;
  }
  const LaneOffsets<KV, D> loff(a.num_kv_heads, g, rho, qd);
  // block j of the current chunk of `cnt` (first chunk block c0); returns
  // the mask of its tokens that hold data: none if j >= cnt or its table
  // entry names no pool block, else the tokens before the cache length
  auto fetch = [&](int c0, int j, int cnt, BlockRegs<KV, D>& br) -> uint32_t {
    const int pb = __builtin_amdgcn_readlane(tblv, j & 63);
    const bool ok = j < cnt && pb >= 0 && (int64_t)pb < a.num_blocks;
    load_block<KV, D>(a, ok ? pb : 0, ok, loff, br);
    const int jb = (w0 + c0 + j) * kBlock;                  // the block's first position
    const int left = Lc - jb;                               // cache tokens from it on
    uint32_t m = left >= kBlock ? 0xffffu : (1u << max(left, 0)) - 1u;
    if (lo0 > jb) m &= ~((1u << min(lo0 - jb, kBlock)) - 1u);   // before every window
    return ok ? m : 0u;
  };
  // ---- append form, first half: the last wave of the partition holding
  // position L-1 takes the new tokens (token t at position L-Q+t, rows past
  // q_len read as zeros).  Their rows are requested before the first block's,
  // stored into their cache slots (K8/V4: quantized first, exactly as the
  // quantize-on-write does) while the block loads are in flight, and parked
  // in LDS as one more tile for the end of the block loop.
  // When the new tokens share the sequence's last cache block (that block
  // then holds cache rows too: always so for one new token unless it starts a
  // block), they are patched into that block's registers by the wave that
  // owns it, and no extra tile is needed; otherwise the partition's last wave
  // attends to them as one extra tile after its blocks.
  const int blk_new = (L - 1) / kBlock;                     // the block of position L-1
  const int new_row0 = (L - Q) & (kBlock - 1);              // the first new token's row
  const bool patch = append && L - Q > 0 && new_row0 != 0 && (L - Q) / kBlock == blk_new;
  const bool app_wave = append && p == p_new &&
                        wh == (patch ? (blk_new - b0) / max(per, 1) : NWH - 1);   // wave-uniform
  u4 nkh[D / 32], nvh[D / 32];        // 16-bit: this lane's new-row halves, 8 per u4
  uint32_t nkw[RT], nvw[RT];          // K8/V4: token t's halves of dims lane*E .. +E-1
  constexpr int E = D / kWave;        // K8/V4 quantization: dims per lane and token
  if (app_wave) {
    const uint32_t rows_b = (uint32_t)(Q * a.num_kv_heads * D * 2);
    const int64_t first = (int64_t)b * Q * a.num_kv_heads * D * 2;
    const auto kr = span_rsrc((const char*)a.new_k + first, rows_b);
    const auto vr = span_rsrc((const char*)a.new_v + first, rows_b);
    if constexpr (KV == Fmt::K8V4) {
      // quantized a token at a time with the wave spread over its dims (as the
      // quantize-on-write does), rows t >= q_len read as zeros
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const uint32_t off = (uint32_t)(((t * a.num_kv_heads + g) * D + lane * E) * 2);
        if constexpr (E == 2) {
          nkw[t] = buf_load<uint32_t>(kr, off);
          nvw[t] = buf_load<uint32_t>(vr, off);
        } else {
          nkw[t] = buf_load<uint16_t>(kr, off);
          nvw[t] = buf_load<uint16_t>(vr, off);
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < D / 32; ++m) nkh[m] = buf_load<u4>(kr, loff.k + 64 * m);
#pragma unroll
      for (int m = 0; m < D / 32; ++m) nvh[m] = buf_load<u4>(vr, loff.v + 64 * m);
    }
  }
  BlockRegs<KV, D> r0, r1;
  uint32_t ok0 = fetch(0, 0, min(64, nmine), r0), ok1 = 0u;
  unsigned char* stash = smem + SM::LOOP + hw * SM::STASH;   // this head's parked tile
  const bool tv = tnew >= 0 && (int64_t)tnew < a.num_blocks;   // rho < Q, position >= 0
  if (app_wave) {
    if constexpr (KV != Fmt::K8V4) {
      BlockRegs<KV, D> rn;
      const int pos = L - Q + rho;
      const int64_t row = ((int64_t)tnew * kBlock + (pos & (kBlock - 1))) * a.num_kv_heads + g;
#pragma unroll
      for (int m = 0; m < D / 32; ++m) {
        rn.k[m] = nkh[m];
        rn.v[m] = nvh[m];
      }
      if (tv) {
        char* kd = (char*)a.k_cache + row * (D * 2) + 16 * qd;
        char* vd = (char*)a.v_cache + row * (D * 2) + 16 * qd;
#pragma unroll
        for (int m = 0; m < D / 32; ++m) {
          *(u4*)(kd + 64 * m) = rn.k[m];
          *(u4*)(vd + 64 * m) = rn.v[m];
        }
      }
      if (rho < RT) *(BlockRegs<KV, D>*)(stash + (qd * RT + rho) * sizeof(BlockRegs<KV, D>)) = rn;
    } else {
      // Token by token, lane l quantizing dims l*E .. +E-1 exactly as the
      // quantize-on-write does; the codes and scales go to the cache and into
      // the parked tile, whose lane (token rho, quarter qd) layout is that of
      // a loaded block (K dims 64u + 16qd .. +15, V dims (D/4)qd .. +D/4-1).
      using BR = BlockRegs<KV, D>;
      constexpr int SZ = (int)sizeof(BR), GL = 32 / E;       // GL: lanes per V group
      constexpr int OK_ = (int)offsetof(BR, k), OV = (int)offsetof(BR, v);
      constexpr int OKS = (int)offsetof(BR, ks), OVS = (int)offsetof(BR, vs), OVZ = (int)offsetof(BR, vz);
#pragma unroll
      for (int i = lane; i < RT * 4 * SZ / 16; i += kWave) *(u4*)(stash + 16 * i) = u4{0u, 0u, 0u, 0u};
      wave_lds_fence();
      const int d0 = lane * E;
      auto to_f = [&](uint32_t h) -> float {
        return QT == Fmt::F16 ? f16_bits_to_f32(h & 0xffffu) : bf16_bits_to_f32(h & 0xffffu);
      };
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        if (t >= Q) continue;                                // wave-uniform (no early exit, so the loop unrolls)
        float k[E], v[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          k[e] = to_f(nkw[t] >> (16 * e));
          v[e] = to_f(nvw[t] >> (16 * e));
        }
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(k[e]));
#pragma unroll
        for (int m = 1; m < kWave; m <<= 1) amax = fmaxf(amax, wave_xor(amax, m));
        const uint16_t ks16 = k8_scale_bits(amax);
        const float ks = f16_bits_to_f32(ks16), rks = __builtin_amdgcn_rcpf(ks);
        uint32_t kc = 0u;                                    // E codes, little-endian
#pragma unroll
        for (int e = 0; e < E; ++e) kc |= (uint32_t)(k8_code(k[e], ks, rks) & 0xff) << (8 * e);
        float mn = v[0], mx = v[0];
#pragma unroll
        for (int e = 1; e < E; ++e) { mn = fminf(mn, v[e]); mx = fmaxf(mx, v[e]); }
#pragma unroll
        for (int m = 1; m < GL; m <<= 1) {
          mn = fminf(mn, wave_xor(mn, m));
          mx = fmaxf(mx, wave_xor(mx, m));
        }
        const uint16_t vs16 = v4_scale_bits(mn, mx), vz16 = f32_to_f16_bits(mn);
        const float vs = f16_bits_to_f32(vs16), vz = f16_bits_to_f32(vz16);
        const float rvs = __builtin_amdgcn_rcpf(vs);
        uint32_t vb = v4_code(v[0], vs, rvs, vz);            // this lane's V byte (E == 2) ...
        if constexpr (E == 2) vb |= v4_code(v[1], vs, rvs, vz) << 4;
        else vb |= (uint32_t)__shfl_down((int)vb, 1, kWave) << 4;   // ... or even lanes' (E == 1)
        const bool vlead = E == 2 || (lane & 1) == 0;
        const int gi = d0 / 32;                              // this lane's V group
        // cache slot of token t (its table entry is lane t's)
        const int tn = __builtin_amdgcn_readlane(tnew, t);
        if (tn >= 0 && (int64_t)tn < a.num_blocks) {
          const int64_t row = ((int64_t)tn * kBlock + ((L - Q + t) & (kBlock - 1))) * a.num_kv_heads + g;
          char* kd = (char*)a.k_cache + row * D + d0;
          if constexpr (E == 2) *(uint16_t*)kd = (uint16_t)kc;
          else *(uint8_t*)kd = (uint8_t)kc;
          if (vlead) ((uint8_t*)a.v_cache)[row * (D / 2) + d0 / 2] = (uint8_t)vb;
          if (lane == 0) ((uint16_t*)a.k_scale)[row] = ks16;
          if (lane % GL == 0) {
            ((uint16_t*)a.v_scale)[row * GR + gi] = vs16;
            ((uint16_t*)a.v_zero)[row * GR + gi] = vz16;
          }
        }
        // the parked tile
        unsigned char* ek = stash + (((d0 % 64) / 16) * RT + t) * SZ + OK_ + 16 * (d0 / 64) + d0 % 16;
        if constexpr (E == 2) *(uint16_t*)ek = (uint16_t)kc;
        else *ek = (uint8_t)kc;
        constexpr int NV = D / 4;                            // V dims per quarter
        if (vlead) stash[((d0 / NV) * RT + t) * SZ + OV + (d0 % NV) / 2] = (uint8_t)vb;
        if (lane < 4) *(uint16_t*)(stash + (lane * RT + t) * SZ + OKS) = ks16;
        if (lane % GL == 0) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            *(uint16_t*)(stash + (q4 * RT + t) * SZ + OVS + 2 * gi) = vs16;
            *(uint16_t*)(stash + (q4 * RT + t) * SZ + OVZ + 2 * gi) = vz16;
          }
        }
      }
    }
  }

  // ---- stage the query rows: into this wave's own LDS area, or (one shared
  // copy) by wave 0, the others waiting at a workgroup barrier; either way
  // the first K/V loads are already in flight
  uint16_t* qw = q_s + (SM::QCOPIES == 1 ? 0 : w) * RT * QSTR;
  if (SM::QCOPIES == NW || w == 0) {
#pragma unroll
    for (int u = 0; u < QPL; ++u) {
      const int idx = lane + u * kWave;
      if (idx < QCW) *(u4*)(qw + (idx / (D / 8)) * QSTR + 8 * (idx % (D / 8))) = qv[u];
    }
  }
  if constexpr (SM::QCOPIES == 1) __syncthreads();
  else wave_lds_fence();
  const uint16_t* qrow = qw + (row_ok ? lrow : lrow % GQ) * QSTR;   // this lane's operand row
  // start of every score accumulator: 0, or for K8/V4 -off * (the row's query
  // sum), which cancels the offset the converted K codes carry
  f4 s_init = f4{0.f, 0.f, 0.f, 0.f};
  if constexpr (KV == Fmt::K8V4) {
    constexpr uint32_t n2 = kK8NegOffset2<QT>;
#pragma unroll
    for (int m = 0; m < KS; ++m)
      s_init = MM::qk(u4{n2, n2, n2, n2}, *(const u4*)(qrow + qk_dim<KV>(m, qd)), s_init);
  }

  unsigned char* vst = smem + w * (16 * D * 2);             // this wave's staged V tile
  float* side = (float*)(smem + SM::VST) + w * 16 * (1 + 2 * GR);   // K8/V4 scales
  // byte offset of this lane's 8-byte chunk for the transposing V read:
  // token 4*qd + (rho>>2), dims 4*(rho&3) .. +3 of the 16-dim tile
  const int tr_off = ((((rho & 3) >> 1) * 16) + 4 * qd + (rho >> 2)) * 16 + (rho & 1) * 8;

  float m_run = kNegInf, l_run = 0.f;
  f4 o[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) o[n] = f4{0.f, 0.f, 0.f, 0.f};
  constexpr int NZ = COLG ? 1 : GR;     // zero-point sums: this column's group, or every group
  float zacc[NZ];
#pragma unroll
  for (int gi = 0; gi < NZ; ++gi) zacc[gi] = 0.f;

  const float sl2 = a.scale_log2;
  const V4Consts v4c;                   // (used by K8/V4 only)

  // One tile of 16 tokens at positions j0 .. j0+15; bit t of vmask says
  // whether token t holds data (wave-uniform).
  auto process = [&](int j0, uint32_t vmask, BlockRegs<KV, D>& br) {
    if (app_wave && patch && j0 == blk_new * kBlock) {       // wave-uniform, once
      // the parked new rows replace the block's rows new_row0 .. new_row0+Q-1
      const int t = rho - new_row0;
      if (t >= 0 && t < Q) br = *(const BlockRegs<KV, D>*)(stash + (qd * RT + t) * sizeof(BlockRegs<KV, D>));
      vmask |= ((uint32_t)__builtin_amdgcn_ballot_w64(tv && qd == 0) & ((1u << Q) - 1u)) << new_row0;
    }
    const bool tail = vmask != 0xffffu;                      // some tokens hold no data
    const bool full = !tail && j0 >= lo_max && j0 + kBlock <= full_lim;   // no masking at all
    const bool tok_ok = (vmask >> rho) & 1u;                 // this lane's token (rho) exists

    // ---- stage V in load-lane order: the 16-byte chunk (m, c) of token t at
    // m*1024 + (16c + t)*16, i.e. lane (t, c) of load m writes where it read.
    // Rows past the length are zeroed (their weight is 0, and 0 * NaN is NaN).
    // K8/V4: the decoded codes are finite integers, so rows without data need
    // no zeroing (their weights are exactly 0)
    if constexpr (KV == Fmt::K8V4) {
      constexpr int NC = D / 4;                 // codes held by this lane: dims NC*qd ..
      const uint32_t wd[4] = {br.v.x, br.v.y, br.v.z, br.v.w};
#pragma unroll
      for (int q = 0; q < NC / 8; ++q) {        // 8 codes -> one 16-byte chunk
        const int dim0 = NC * qd + 8 * q;      // first dim of this chunk
        *(u4*)(vst + (dim0 >> 5) * 1024 + (16 * ((dim0 & 31) >> 3) + rho) * 16) = v4_codes(wd[q], v4c);
      }
    } else {
#pragma unroll
      for (int m = 0; m < KS; ++m) {
        u4 vv = br.v[m];
        if (tail && !tok_ok) vv = u4{0u, 0u, 0u, 0u};
        *(u4*)(vst + m * 1024 + lane * 16) = vv;
      }
    }

    // ---- scores S^T = K Q^T
    f4 s = s_init;
    if constexpr (KV == Fmt::K8V4) {
#pragma unroll
      for (int u = 0; u < D / 64; ++u) {
        const u4 c = br.k[u];
        const uint32_t wd[4] = {c.x, c.y, c.z, c.w};
        uint32_t cv[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) k8_codes<QT>(wd[q], cv[2 * q], cv[2 * q + 1]);
        const u4 q0 = *(const u4*)(qrow + qk_dim<KV>(2 * u, qd));
        const u4 q1 = *(const u4*)(qrow + qk_dim<KV>(2 * u + 1, qd));
        s = MM::qk(u4{cv[0], cv[1], cv[2], cv[3]}, q0, s);
        s = MM::qk(u4{cv[4], cv[5], cv[6], cv[7]}, q1, s);
      }
      // per-token K scales and V scale/zero, moved through LDS from the
      // token-owner layout (lane rho) to the score layout (tokens 4*qd + r)
      if (qd == 0) {
        side[rho] = f16_bits_to_f32(br.ks) * sl2;
#pragma unroll
        for (int gi = 0; gi < GR; ++gi) {
          const uint32_t sw = gi < 2 ? br.vs.x : br.vs.y;
          const uint32_t zw = gi < 2 ? br.vz.x : br.vz.y;
          const float sv = f16_bits_to_f32((gi & 1) ? (sw >> 16) : (sw & 0xffff));
          const float zv = f16_bits_to_f32((gi & 1) ? (zw >> 16) : (zw & 0xffff));
          side[16 + rho * 2 * GR + 2 * gi] = tok_ok ? sv : 0.f;
          side[16 + rho * 2 * GR + 2 * gi + 1] = tok_ok ? zv : 0.f;
        }
      }
    } else if constexpr (kQkOnValu) {
      // vector dot products: lane (rho, qd) dots token rho's dims
      // 32 m + 8 qd .. +7 with the same dims of every tile row c, the four
      // quarters are summed with lane swaps, and the scores pass through LDS
      // into the layout the MFMA produces (lane l: row l % 16, tokens
      // 4 (l / 16) + r)
      float* scs = (float*)(smem + SM::VST) + w * RT * 16;
      float part[RT];
#pragma unroll
      for (int c = 0; c < RT; ++c) part[c] = 0.f;
#pragma unroll
      for (int m = 0; m < KS; ++m) {
        const uint32_t kw[4] = {br.k[m].x, br.k[m].y, br.k[m].z, br.k[m].w};
#pragma unroll
        for (int c = 0; c < RT; ++c) {
          if (c >= GQT) continue;                              // wave-uniform
          const u4 q4 = *(const u4*)(qw + c * QSTR + qk_dim<KV>(m, qd));
          const uint32_t qv4[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (QT == Fmt::F16)
              part[c] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, kw[e]),
                                               __builtin_bit_cast(h2, qv4[e]), part[c], false);
            else {
              typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
              part[c] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, kw[e]),
                                                        __builtin_bit_cast(bf2, qv4[e]), part[c],
                                                        false);
            }
          }
        }
      }
#pragma unroll
      for (int c = 0; c < RT; ++c) {
        if (c >= GQT) continue;
        const float tot = quarter_sum(part[c]);
        if (qd == 0) scs[c * 16 + rho] = tot;
      }
      wave_lds_fence();
      s = s + *(const f4*)(scs + (row_ok ? lrow : lrow % GQ) * 16 + 4 * qd);
    } else {
#pragma unroll
      for (int m = 0; m < KS; ++m) {
        const u4 qm = *(const u4*)(qrow + qk_dim<KV>(m, qd));
        s = MM::qk(br.k[m], qm, s);
      }
    }
    wave_lds_fence();

    // ---- online softmax in the exp2 domain (lane: row rho, tokens 4*qd + r)
    float sv[4];
    if constexpr (KV == Fmt::K8V4) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[r] = s[r] * side[4 * qd + r];
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[r] = s[r] * sl2;
    }
    if (!full) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = j0 + 4 * qd + r;
        if (!((vmask >> (4 * qd + r)) & 1u) || j >= nvis || j < lo_row) sv[r] = kNegInf;
      }
    }
    const float mx = quarter_max(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
    const bool grow = mx > m_run + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(grow)) {                 // rare: move the reference max
      // rows that do not grow keep their max (alpha 1: never -inf - -inf);
      // a growing row from -inf gets alpha 0
      const float m_new = grow ? mx : m_run;
      const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;
#pragma unroll
      for (int n = 0; n < NT; ++n) o[n] *= alpha;
      l_run *= alpha;
#pragma unroll
      for (int gi = 0; gi < NZ; ++gi) zacc[gi] *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(sv[r] - m_use);
    l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);

    // ---- O^T += V^T P^T; the V operand comes from one transposing read per tile
    if constexpr (COLG) {
      // this column's group (columns past the groups compute a copy)
      const int gl = min(rho >> 2, GR - 1);
      float pw[4];
      float zs = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float* sd = side + 16 + (4 * qd + r) * 2 * GR + 2 * gl;
        pw[r] = pr[r] * sd[0];
        zs += pr[r] * sd[1];
      }
      zacc[0] += zs;
      u2 phi, plo;
      Mma<Fmt::F16>::split(pw, phi, plo);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const u2 av = lds_read_tr16(vst + tr_off + (n >> 1) * 1024 + (n & 1) * 512);
        o[n] = Mma<Fmt::F16>::pv(av, phi, o[n]);
        o[n] = Mma<Fmt::F16>::pv(av, plo, o[n]);
      }
    } else if constexpr (KV == Fmt::K8V4) {
#pragma unroll
      for (int gi = 0; gi < GR; ++gi) {
        float pw[4];
        float zs = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float* sd = side + 16 + (4 * qd + r) * 2 * GR + 2 * gi;
          pw[r] = pr[r] * sd[0];
          zs += pr[r] * sd[1];
        }
        zacc[gi] += zs;
        u2 phi, plo;
        Mma<Fmt::F16>::split(pw, phi, plo);
#pragma unroll
        for (int nn = 0; nn < 2; ++nn) {
          const int n = 2 * gi + nn;
          const u2 av = lds_read_tr16(vst + tr_off + (n >> 1) * 1024 + (n & 1) * 512);
          o[n] = Mma<Fmt::F16>::pv(av, phi, o[n]);
          o[n] = Mma<Fmt::F16>::pv(av, plo, o[n]);
        }
      }
    } else {
      u2 phi, plo;
      MM::split(pr, phi, plo);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const u2 av = lds_read_tr16(vst + tr_off + (n >> 1) * 1024 + (n & 1) * 512);
        o[n] = MM::pv(av, phi, o[n]);
        o[n] = MM::pv(av, plo, o[n]);
      }
    }
    wave_lds_fence();
  };

  // ---- block loop, in chunks of 64 of this wave's blocks.  Two register
  // sets: the next block's loads are always issued before the current block
  // is consumed, with no branch between them, so the wait before each block
  // covers only that block's loads.  A fetch past the chunk is a no-op load.
  for (int c0 = 0; c0 < nmine; c0 += 64) {
    const int cnt = min(64, nmine - c0);
    if (c0 > 0) {
      tblv = tbl_next;
      if (c0 + 64 < nmine) {                          // next chunk, one chunk ahead
        const int kk = c0 + 64 + lane;
        tbl_next = kk < nmine ? buf_load<int>(btr, (uint32_t)(w0 + kk) * 4u) : 0;
      }
      ok0 = fetch(c0, 0, cnt, r0);
    }
    const int j0 = (w0 + c0) * kBlock;
    for (int k = 0; k < cnt; k += 2) {
      ok1 = fetch(c0, k + 1, cnt, r1);
      process(j0 + k * kBlock, ok0, r0);
      ok0 = fetch(c0, k + 2, cnt, r0);
      if (k + 1 < cnt) process(j0 + (k + 1) * kBlock, ok1, r1);
    }
  }

  // ---- append form, second half: the parked tile of new tokens
  if (app_wave && !patch) {
    BlockRegs<KV, D> rn{};
    if (rho < RT) rn = *(const BlockRegs<KV, D>*)(stash + (qd * RT + rho) * sizeof(BlockRegs<KV, D>));
    const uint32_t vmask = (uint32_t)__builtin_amdgcn_ballot_w64(tv && qd == 0) & 0xffffu;
    process(L - Q, vmask, rn);
  }

  // ---- per-wave totals: the sum is spread over the four quarters
  l_run = quarter_sum(l_run);
  if constexpr (KV == Fmt::K8V4) {
#pragma unroll
    for (int gi = 0; gi < NZ; ++gi) zacc[gi] = quarter_sum(zacc[gi]);
#pragma unroll
    for (int n = 0; n < NT; ++n) o[n] += zacc[COLG ? 0 : n / 2];
  }

  // ---- merge the NW wavefronts of this workgroup (LDS reused), in EP passes
  // over the head dims (the 16-row forms take two, which halves the LDS the
  // merge needs)
  constexpr int EP = SM::EP, DH = D / EP, NTH = NT / EP;
  float* mo = (float*)smem;
  if (qd == 0) {
    mm_s[w][rho] = m_run;
    ml_s[w][rho] = l_run;
  }
#pragma unroll
  for (int e = 0; e < EP; ++e) {
    __syncthreads();                           // the block loop's, or the last pass's, reads done
    if constexpr (COLG) {
      // row lrow's dims of tile n sit in the columns of tile n's V group
      if (lrow < GQT) {
#pragma unroll
        for (int n = 0; n < NTH; ++n) {
          if ((rho >> 2) != (e * NTH + n) / 2) continue;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            mo[(w * RT + lrow) * DH + 16 * n + v4_dim(4 * qd + r)] = o[e * NTH + n][r];
        }
      }
    } else if (rho < RT && rho < GQT) {
#pragma unroll
      for (int n = 0; n < NTH; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * qd + r;            // output row within the tile
          mo[(w * RT + rho) * DH + 16 * n + (KV == Fmt::K8V4 ? v4_dim(i) : i)] = o[e * NTH + n][r];
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < HP * GQT * DH; idx += NW * kWave) {
      const int hh = HP == 1 ? 0 : idx / (GQT * DH);              // head within the workgroup
      const int rem = HP == 1 ? idx : idx - hh * (GQT * DH);
      const int rr = rem / DH, dh = rem % DH, d = e * DH + dh;
      // constant trip counts, so the loops unroll and the LDS reads of all
      // of the head's waves go out together
      float M = kNegInf;
#pragma unroll
      for (int j = 0; j < NWH; ++j) M = fmaxf(M, mm_s[hh * NWH + j][rr]);
      const float Mu = M == kNegInf ? 0.f : M;
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int j = 0; j < NWH; ++j) {
        const int ww = hh * NWH + j;
        const float ew = fast_exp2(mm_s[ww][rr] - Mu);
        num += ew * mo[(ww * RT + rr) * DH + dh];
        den += ew * ml_s[ww][rr];
      }
      const int64_t orow = orow_head(rr, g0 + hh);
      if (orow < 0) continue;
      if (split) {
        const int64_t pi = orow * wsp + a.part_base + p;
        a.ws_o[pi * D + d] = num;
        if (d == 0) {
          a.ws_m[pi] = M;
          a.ws_l[pi] = den;
        }
      } else {
        store_out(a.out, (OutT)a.out_dtype, orow * D + d, den > 0.f ? num / den : 0.f);
      }
    }
  }
}

// ------------------------------------------------------------------------------
// Balanced split-KV (partition_size 0; 16-bit caches, plain and append forms).
//
// For each KV head the batch's blocks are laid end to end: sequence b's blocks
// 0 .. nblk_b - 1 (nblk_b = ceil(L_b / 16), L_b clamped like every length)
// follow those of sequences 0 .. b-1, T blocks in all.  The T blocks are cut
// into S equal runs, one per wavefront (run s covers flattened blocks
// [s * per, (s+1) * per), per = ceil(T / S)), so every wavefront streams the
// same number of blocks however ragged the lengths; with fixed-size
// partitions the longest ones set the launch's end while most CUs sit idle.
// A run may cross sequence boundaries: the wave attends each sequence's piece
// of it (a segment) and writes one partial per segment, to slot s + b of its
// KV head.  No two segments share a slot: walking the flattened blocks, each
// new segment starts a new run, a new sequence, or both, so s + b grows with
// every segment.  The merge kernel finds a row's slots from the same lengths.
// There is no merge inside the workgroup; waves h*NWH .. of a workgroup take
// KV head HP*blockIdx.y + h and runs blockIdx.x*NWH + (w % NWH), so with HP = 2
// the two heads' waves read the same blocks together.
//
// Workspace: o[Hkv][S + B][G*Q][D] (unnormalised), m[..][G*Q], l[..][G*Q],
// tile row r of a slot being query row (i = r / G, head g*G + r % G).

// Built for three waves per SIMD in the 4-row form (up to 168 registers) and
// two in the 16-row form, which holds more per lane.
// wavefronts per workgroup of the balanced kernel, by tile rows
template <int RT> constexpr int kFlatWaves = RT == 4 ? 8 : 4;

template <Fmt KV, int D, int RT, int HP>
__global__ __launch_bounds__((kFlatWaves<RT> * kWave), (RT == 4 ? 3 : 2))
void attn_flat_kernel(const AttnArgs a) {
  using MM = Mma<KV>;
  static_assert(KV != Fmt::K8V4, "balanced split: 16-bit caches");
  constexpr int NW = kFlatWaves<RT>;
  constexpr int NWH = NW / HP;
  constexpr int KS = D / 32, NT = D / 16;
  constexpr int QSTR = D + 8;
  __shared__ __align__(16) unsigned char v_s[NW * 16 * D * 2];
  __shared__ __align__(16) uint16_t q_s[NW * RT * QSTR];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hw = w / NWH;
  const int g = blockIdx.y * HP + hw;                       // KV head
  const int S = a.flat_runs;
  const int s = blockIdx.x * NWH + w % NWH;                 // this wave's run
  const int rho = lane & 15, qd = lane >> 4;
  const int Q = a.q_len, G = a.gqa, GQ = G * Q, Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int B = a.batch;
  const int cap = a.max_blocks * kBlock;
  const bool append = a.new_k != nullptr;

  // ---- lengths, 64 sequences per chunk (lane i: sequence base + i), and
  // the flattened end of each: ends are inclusive prefix sums of nblk; with
  // a.tbl_off, also each sequence's first table entry (a cascade's suffix
  // pass: its lengths count from there)
  auto chunk_lens = [&](int base, int& len, int& end, int carry, int* off) {
    const int b = base + lane;
    int L = b < B ? a.context_lens[b] : 0;
    if (off) *off = a.tbl_off != nullptr && b < B ? min(max(a.tbl_off[b], 0), a.max_blocks) : 0;
    L = min(max(L, 0), cap);
    len = L;
    int v = (L + kBlock - 1) / kBlock;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int t = __shfl_up(v, d, kWave);
      if (lane >= d) v += t;
    }
    end = carry + v;
  };
  int base = 0, len_c = 0, end_c = 0, off_c = 0;
  chunk_lens(0, len_c, end_c, 0, &off_c);
  // (readlane, not a shuffle, so the compiler knows these values are
  // wave-uniform and keeps the segment loop in scalar control flow)
  int T = __builtin_amdgcn_readlane(end_c, kWave - 1);
  for (int bb = kWave; bb < B; bb += kWave) {               // batches past 64 sequences
    int l2, e2;
    chunk_lens(bb, l2, e2, T, nullptr);
    T = __builtin_amdgcn_readlane(e2, kWave - 1);
  }
  const int per = (T + S - 1) / S;
  const int r0 = min(s * per, T), r1 = min(r0 + per, T);
  if (r0 >= r1) return;                                      // nothing left for this run
  // the chunk holding the first sequence that ends past r0 (one exists, since
  // r0 < T; the bound on base only makes the loop's end evident)
  uint64_t past = __builtin_amdgcn_ballot_w64(base + lane < B && end_c > r0);
  while (past == 0) {
    const int carry = __builtin_amdgcn_readlane(end_c, kWave - 1);
    base += kWave;
    if (base >= B) return;
    chunk_lens(base, len_c, end_c, carry, &off_c);
    past = __builtin_amdgcn_ballot_w64(base + lane < B && end_c > r0);
  }
  int b = base + __builtin_ctzll(past);

  const LaneOffsets<KV, D> loff(Hkv, g, rho, qd);
  unsigned char* vst = v_s + w * (16 * D * 2);
  uint16_t* qw = q_s + w * RT * QSTR;
  const uint16_t* qrow = qw + (rho < GQ ? rho : rho % GQ) * QSTR;
  const int tr_off = ((((rho & 3) >> 1) * 16) + 4 * qd + (rho >> 2)) * 16 + (rho & 1) * 8;
  const float sl2 = a.scale_log2;
  const int64_t slot_base = (int64_t)g * (S + B);
  constexpr int QCW = RT * (D / 8);                          // 16-byte query chunks per wave
  constexpr int QPL = (QCW + kWave - 1) / kWave;

  // the lengths chunk holding sequence b (b only grows)
  auto chunk_of = [&]() {
    while (b - base >= kWave) {
      const int carry = __builtin_amdgcn_readlane(end_c, kWave - 1);
      base += kWave;
      chunk_lens(base, len_c, end_c, carry, &off_c);
    }
  };
  for (int pos = r0; pos < r1;) {
    // sequence b covers flattened blocks [end_b - nblk_b, end_b); skip empty ones
    chunk_of();
    int end_b = __builtin_amdgcn_readlane(end_c, b - base);
    while (end_b <= pos) {
      if (++b >= B) return;                                  // (not reached: pos < T)
      chunk_of();
      end_b = __builtin_amdgcn_readlane(end_c, b - base);
    }
    const int L = __builtin_amdgcn_readlane(len_c, b - base);
    const int toff = __builtin_amdgcn_readlane(off_c, b - base);   // 0 without a.tbl_off
    const int start_b = end_b - (L + kBlock - 1) / kBlock;
    const int seg_end = min(r1, end_b);
    const int jb0 = pos - start_b, n = seg_end - pos;        // the segment's blocks of b

    // the segment's table entries (64 per chunk), query rows and new rows
    const auto btr = span_rsrc(a.block_tables + (int64_t)b * a.max_blocks + toff,
                               (uint32_t)(a.max_blocks - toff) * 4u);
    int tbl = lane < n ? buf_load<int>(btr, (uint32_t)(jb0 + lane) * 4u) : 0;
    u4 qv[QPL];
#pragma unroll
    for (int u = 0; u < QPL; ++u) {
      const int idx = lane + u * kWave;
      const int r = idx / (D / 8), c8 = idx % (D / 8);
      qv[u] = u4{0u, 0u, 0u, 0u};
      if (idx < QCW && r < GQ)
        qv[u] = *(const u4*)((const uint16_t*)a.q +
                             (((int64_t)b * Q + r / G) * Hq + g * G + r % G) * D + 8 * c8);
    }
    const uint32_t new_bytes = append ? (uint32_t)(Q * Hkv * D * 2) : 0u;
    const auto nkr = span_rsrc((const char*)a.new_k + (append ? (int64_t)b * Q * Hkv * D * 2 : 0),
                               new_bytes);
    const auto nvr = span_rsrc((const char*)a.new_v + (append ? (int64_t)b * Q * Hkv * D * 2 : 0),
                               new_bytes);
    const int first_new = append ? L - Q : L;                // positions from here on are new rows

    // block j of the current table chunk (first segment block jbase): loads
    // its rows (new tokens' rows from the new K/V input) and returns the mask
    // of its tokens that hold data
    auto fetch = [&](int j, int cnt, int jbase, BlockRegs<KV, D>& br) -> uint32_t {
      const int pb = __builtin_amdgcn_readlane(tbl, j & 63);
      const bool ok = j < cnt && pb >= 0 && (int64_t)pb < a.num_blocks;
      load_block<KV, D>(a, ok ? pb : 0, ok, loff, br);
      const int jb = (jbase + j) * kBlock;
      if (ok && jb + kBlock > first_new) {                    // wave-uniform: new tokens here
        const int t = jb + rho - first_new;
        if (t >= 0 && t < Q) {
          const uint32_t off = (uint32_t)(((t * Hkv + g) * D + 8 * qd) * 2);
#pragma unroll
          for (int m = 0; m < KS; ++m) br.k[m] = buf_load<u4>(nkr, off + 64 * m);
#pragma unroll
          for (int m = 0; m < KS; ++m) br.v[m] = buf_load<u4>(nvr, off + 64 * m);
        }
      }
      const int left = L - jb;
      const uint32_t msk = left >= kBlock ? 0xffffu : (1u << max(left, 0)) - 1u;
      return ok ? msk : 0u;
    };

    // stage the query rows (this wave's copy) behind the first loads
    BlockRegs<KV, D> r0s, r1s;
    const int cnt0 = min(64, n);
    uint32_t ok0 = fetch(0, cnt0, jb0, r0s), ok1 = 0u;
#pragma unroll
    for (int u = 0; u < QPL; ++u) {
      const int idx = lane + u * kWave;
      if (idx < QCW) *(u4*)(qw + (idx / (D / 8)) * QSTR + 8 * (idx % (D / 8))) = qv[u];
    }
    wave_lds_fence();

    const bool row_ok = rho < GQ;
    const int iq = row_ok ? rho / G : 0;
    const int nvis = row_ok ? (L - Q + iq + 1) : L;          // visible positions of the row
    const int full_lim = L - Q + 1;                          // every row sees j < full_lim
    float m_run = kNegInf, l_run = 0.f;
    f4 o[NT];
#pragma unroll
    for (int nn = 0; nn < NT; ++nn) o[nn] = f4{0.f, 0.f, 0.f, 0.f};

    // one tile: the new rows go to their cache slots, V into LDS, S^T = K Q^T,
    // then the online softmax and O^T += V^T P^T, as in the partition kernel
    auto process = [&](int j, int jbase, uint32_t vmask, BlockRegs<KV, D>& br) {
      const int j0 = (jbase + j) * kBlock;
      if (append && vmask != 0u && j0 + kBlock > first_new) { // wave-uniform
        const int t = j0 + rho - first_new;
        if (t >= 0 && t < Q) {
          const int pb = __builtin_amdgcn_readlane(tbl, j & 63);
          const int64_t row = ((int64_t)pb * kBlock + rho) * Hkv + g;
          char* kd = (char*)a.k_cache + row * (D * 2) + 16 * qd;
          char* vd = (char*)a.v_cache + row * (D * 2) + 16 * qd;
#pragma unroll
          for (int m = 0; m < KS; ++m) {
            *(u4*)(kd + 64 * m) = br.k[m];
            *(u4*)(vd + 64 * m) = br.v[m];
          }
        }
      }
      const bool tail = vmask != 0xffffu;
      const bool tok_ok = (vmask >> rho) & 1u;
#pragma unroll
      for (int m = 0; m < KS; ++m) {
        u4 vv = br.v[m];
        if (tail && !tok_ok) vv = u4{0u, 0u, 0u, 0u};         // 0 * NaN is NaN
        *(u4*)(vst + m * 1024 + lane * 16) = vv;
      }
      f4 sc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < KS; ++m) sc = MM::qk(br.k[m], *(const u4*)(qrow + 32 * m + 8 * qd), sc);
      wave_lds_fence();
      float sv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[r] = sc[r] * sl2;
      if (tail || j0 + kBlock > full_lim) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int jj = j0 + 4 * qd + r;
          if (!((vmask >> (4 * qd + r)) & 1u) || jj >= nvis) sv[r] = kNegInf;
        }
      }
      const float mx = quarter_max(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
      const bool grow = mx > m_run + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? mx : m_run;
        const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;
#pragma unroll
        for (int nn = 0; nn < NT; ++nn) o[nn] *= alpha;
        l_run *= alpha;
        m_run = m_new;
      }
      const float m_use = m_run == kNegInf ? 0.f : m_run;
      float pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(sv[r] - m_use);
      l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);
      u2 phi, plo;
      MM::split(pr, phi, plo);
#pragma unroll
      for (int nn = 0; nn < NT; ++nn) {
        const u2 av = lds_read_tr16(vst + tr_off + (nn >> 1) * 1024 + (nn & 1) * 512);
        o[nn] = MM::pv(av, phi, o[nn]);
        o[nn] = MM::pv(av, plo, o[nn]);
      }
      wave_lds_fence();
    };

    // ---- the segment's blocks, 64 table entries at a time; two register
    // sets, the next block's loads issued before the current block is used
    for (int c0 = 0; c0 < n; c0 += 64) {
      const int cnt = min(64, n - c0);
      if (c0 > 0) {
        tbl = lane < cnt ? buf_load<int>(btr, (uint32_t)(jb0 + c0 + lane) * 4u) : 0;
        ok0 = fetch(0, cnt, jb0 + c0, r0s);
      }
      for (int k = 0; k < cnt; k += 2) {
        ok1 = fetch(k + 1, cnt, jb0 + c0, r1s);
        process(k, jb0 + c0, ok0, r0s);
        ok0 = fetch(k + 2, cnt, jb0 + c0, r0s);
        if (k + 1 < cnt) process(k + 1, jb0 + c0, ok1, r1s);
      }
    }

    // ---- this segment's partial, straight from the registers: lane (rho, qd)
    // holds row rho's dims 16 n + 4 qd .. +3
    l_run = quarter_sum(l_run);
    if (row_ok) {
      const int64_t pi = (slot_base + s + b) * GQ + rho;
      float* od = a.ws_o + pi * D + 4 * qd;
#pragma unroll
      for (int nn = 0; nn < NT; ++nn) *(f4*)(od + 16 * nn) = o[nn];
      if (qd == 0) {
        a.ws_m[pi] = m_run;
        a.ws_l[pi] = l_run;
      }
    }
    wave_lds_fence();                  // the next segment rewrites this wave's query rows
    pos = seg_end;
    ++b;
  }
}

// Merge of the balanced split's partials: one workgroup per (sequence b, KV
// head g), covering the G*q_len rows of that pair, which share their slots:
// s + b for the runs s that hold a block of sequence b, found from the same
// lengths as the partition pass.  Thread (item, grp), item = (row, 4-dim
// chunk), folds slots grp, grp + NG, ... into a running (max, sum, acc) with
// their loads in flight together; the NG running states of an item are then
// combined in LDS, as in attn_merge_kernel.  In a cascade (a.pre_parts > 0)
// the rows of a sequence whose suffix starts past its group's shared prefix
// (a.tbl_off[b] > 0) also fold the prefix pass's a.pre_parts partials of
// their output row.
constexpr int kFlatMergeThreads = 512;

template <int D>
__global__ __launch_bounds__(kFlatMergeThreads) void attn_flat_merge_kernel(const AttnArgs a) {
  constexpr int NC = D / 4;                                 // float4 chunks per row
  constexpr int NT = kFlatMergeThreads;
  __shared__ f4 acc_s[NT];
  __shared__ float m_s[NT], den_s[NT];
  __shared__ int geo_s[3];               // the first slot, the slot count, prefix partials

  const int t = threadIdx.x;
  const int Q = a.q_len, Hq = a.num_q_heads, G = a.gqa, GQ = G * Q, B = a.batch;
  const int Hkv = a.num_kv_heads;
  const int b = (int)(blockIdx.x / Hkv), g = (int)(blockIdx.x % Hkv);
  const int S = a.flat_runs;
  const int cap = a.max_blocks * kBlock;
  if (t < kWave) {                       // wave 0: T and the blocks before sequence b
    // a cascade's prefix partials count for b when its suffix starts past a
    // shared prefix (sequences outside every group have none written)
    const int off_b = a.pre_parts > 0 && a.tbl_off != nullptr ? a.tbl_off[b] : 0;
    int tot = 0, before = 0, nb_b = 0;
    for (int base = 0; base < B; base += kWave) {
      const int bi = base + t;
      int L = bi < B ? a.context_lens[bi] : 0;
      L = min(max(L, 0), cap);
      const int nb = (L + kBlock - 1) / kBlock;
      int v = nb, vb = bi < b ? nb : 0, vo = bi == b ? nb : 0;   // vo: sequence b's own
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        v += __shfl_xor(v, d, kWave);
        vb += __shfl_xor(vb, d, kWave);
        vo += __shfl_xor(vo, d, kWave);
      }
      tot += v;
      before += vb;
      nb_b += vo;
    }
    if (t == 0) {
      const int per = (tot + S - 1) / S;
      int first = 0, count = 0;
      if (per > 0 && nb_b > 0) {                           // runs holding a block of b
        first = before / per;
        count = (before + nb_b - 1) / per - first + 1;
      }
      geo_s[0] = first + b;
      geo_s[1] = count;
      geo_s[2] = off_b > 0 ? a.pre_parts : 0;
    }
  }
  __syncthreads();
  const int np = geo_s[1];
  const int ntot = np + geo_s[2];                           // slots, then prefix partials
  const int NI = GQ * NC;                                   // items (at most 16 * 32 = NT)
  const int NG = NT / NI;                                   // thread groups per item
  const int item = t % NI, grp = t / NI;
  const int rr = item / NC, c = item % NC;                  // tile row, chunk
  const int64_t p0 = ((int64_t)g * (S + B) + geo_s[0]) * GQ + rr;   // the row's first partial
  const int64_t orow = ((int64_t)b * Q + rr / G) * Hq + g * G + rr % G;   // output row
  const int64_t pj0 = orow * a.pre_parts;                   // its prefix partials
  float m_t = kNegInf, den = 0.f;
  f4 acc = f4{0.f, 0.f, 0.f, 0.f};
  if (grp < NG) {
    constexpr int U = 8;
    for (int q0 = grp; q0 < ntot; q0 += U * NG) {
      float mp[U], lp[U];
      f4 op[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {      // loads first (clamped index), no branches between
        const int qq = min(q0 + u * NG, ntot - 1);
        const int64_t pi = qq < np ? p0 + (int64_t)qq * GQ : pj0 + (qq - np);
        const float* wm = qq < np ? a.ws_m : a.pre_m;
        const float* wl = qq < np ? a.ws_l : a.pre_l;
        const float* wo = qq < np ? a.ws_o : a.pre_o;
        mp[u] = wm[pi];
        lp[u] = wl[pi];
        op[u] = *(const f4*)(wo + pi * D + 4 * c);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) asm volatile("" : "+v"(mp[u]), "+v"(lp[u]), "+v"(op[u]));
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool use = q0 + u * NG < ntot && mp[u] != kNegInf;
        const float m_new = use ? fmaxf(m_t, mp[u]) : m_t;
        const float e_old = m_t == kNegInf ? 0.f : fast_exp2(m_t - m_new);
        const float e_new = use ? fast_exp2(mp[u] - m_new) : 0.f;
        const f4 o_u = use ? op[u] : f4{0.f, 0.f, 0.f, 0.f};
        const float l_u = use ? lp[u] : 0.f;
        acc = acc * e_old + o_u * e_new;
        den = den * e_old + l_u * e_new;
        m_t = m_new;
      }
    }
  }
  acc_s[t] = acc;
  m_s[t] = m_t;
  den_s[t] = den;
  __syncthreads();
  if (t < NI) {
    float M = kNegInf;
    for (int gg = 0; gg < NG; ++gg) M = fmaxf(M, m_s[gg * NI + t]);
    f4 tot = f4{0.f, 0.f, 0.f, 0.f};
    float dt = 0.f;
    if (M != kNegInf) {
      for (int gg = 0; gg < NG; ++gg) {
        const float mg = m_s[gg * NI + t];
        const float e = mg == kNegInf ? 0.f : fast_exp2(mg - M);
        tot += acc_s[gg * NI + t] * e;
        dt += den_s[gg * NI + t] * e;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      store_out(a.out, (OutT)a.out_dtype, orow * D + 4 * c + r, dt > 0.f ? tot[r] / dt : 0.f);
  }
}

// Cascade with a balanced suffix pass: one thread per sequence finds its
// group (the first group whose first slot names a sequence and that lists
// it), scanning the member slots through LDS 256 at a time, and writes the
// group's prefix blocks, clamped to the sequence's own blocks, and the length
// past them.
__global__ __launch_bounds__(256) void cascade_suffix_prep_kernel(const AttnArgs a,
                                                                  int32_t* suf_len,
                                                                  int32_t* suf_off) {
  __shared__ int mem_s[256];
  const int b = (int)blockIdx.x * 256 + (int)threadIdx.x;
  const int total = a.num_groups * a.group_size;
  // the length first, so that its load overlaps the member scan
  const int L = b < a.batch ? min(max(a.context_lens[b], 0), a.max_blocks * kBlock) : 0;
  int pre = 0;
  bool found = false;
  for (int c0 = 0; c0 < total; c0 += 256) {               // every thread reaches the barriers
    __syncthreads();
    const int idx = c0 + (int)threadIdx.x;
    int m = -1;
    if (idx < total && a.grp_members[(int64_t)(idx / a.group_size) * a.group_size] >= 0)
      m = a.grp_members[idx];
    mem_s[threadIdx.x] = m;
    __syncthreads();
    const int n = min(256, total - c0);
    for (int k = 0; k < n && !found; ++k) {
      if (mem_s[k] == b) {
        pre = a.grp_prefix[(c0 + k) / a.group_size];
        found = true;
      }
    }
  }
  if (b >= a.batch) return;
  pre = min(max(pre, 0), (L + kBlock - 1) / kBlock);
  suf_off[b] = pre;
  suf_len[b] = max(L - pre * kBlock, 0);
}

hipError_t launch_cascade_suffix_prep(const AttnArgs& a, int32_t* suf_len, int32_t* suf_off,
                                      hipStream_t stream) {
  if (a.batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(cascade_suffix_prep_kernel, dim3((unsigned)((a.batch + 255) / 256)),
                     dim3(256), 0, stream, a, suf_len, suf_off);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------
// Sparse-V partition kernel (approximate; 16-bit caches, G*q_len <= 4).
//
// The V row of position j is read only when some query row of the KV head has
// weight 2^(s_j - m) >= threshold, m being that row's running maximum score so
// far (log2 units, this block included).  A running maximum never exceeds the
// final one, so every skipped row weighs less than `threshold` times the
// row's largest weight; skipped positions still count in the softmax sum.
// ("The KV Cache" (metalworking), arithmetic paragraph: sparse-V decode at 32K
// is a KV-cache traffic deletion; the rule itself is this library's reading.)
//
// Rounds: each wavefront loads the K of up to 4 of its blocks at once (3 at
// head_dim 128, for registers), scores them, and the workgroup's waves share
// their row maxima through LDS, so the
// reference maximum is the one over every block the partition has scored so
// far (the whole partition when a round covers it).  Then the V rows some row
// needs are requested for all of the round's blocks together (into the
// registers the K rows used; the offsets of skipped rows are pushed out of the
// buffer's range, so those lanes read zeros and touch no memory), and the PV
// products follow.  V latency is exposed once per round, not once per block.
constexpr uint32_t kOutOfRange = 0x7f000000u;   // past any block, no 32-bit wrap

template <Fmt KV, int D>
__global__ __launch_bounds__((8 * kWave), 4) void attn_sparse_v_kernel(const AttnArgs a) {
  using MM = Mma<KV>;
  using SM = AttnSmem<KV, D, 4>;
  constexpr int NW = 8, RT = 4, GB = D == 128 ? 3 : 4;   // GB: blocks per wave per round
  // table entries per chunk: a whole number of rounds (63 or 64), so the
  // blocks of one round never straddle two chunks
  constexpr int CH = (kWave / GB) * GB;
  constexpr int KS = D / 32;
  constexpr int NT = D / 16;
  constexpr int QSTR = SM::QSTR;
  static_assert(SM::NW == NW, "the 4-row 16-bit shape runs 8 wavefronts");
  __shared__ __align__(16) unsigned char smem[SM::BYTES];
  __shared__ __align__(16) uint16_t q_s[NW * RT * QSTR];
  __shared__ float mm_s[NW][16], ml_s[NW][16];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rho = lane & 15, qd = lane >> 4;
  const int p = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int Q = a.q_len, G = a.gqa, GQ = G * Q, Hq = a.num_q_heads;
  const bool split = a.ws_o != nullptr;
  const int64_t wsp = a.ws_parts;
  const auto btr = span_rsrc(a.block_tables + (int64_t)b * a.max_blocks,
                             (uint32_t)a.max_blocks * 4u);
  const int bb = p * a.part_blocks;
  int per = (a.part_blocks + NW - 1) / NW;
  int tbl_next;
  {
    const int e = bb + w * per + lane;
    tbl_next = lane < per ? buf_load<int>(btr, (uint32_t)e * 4u) : 0;
  }
  constexpr int QCW = RT * (D / 8);
  u4 qv = u4{0u, 0u, 0u, 0u};
  {
    const int r = lane / (D / 8), c8 = lane % (D / 8);
    if (lane < QCW && r < GQ)
      qv = *(const u4*)((const uint16_t*)a.q +
                        (((int64_t)b * Q + r / G) * Hq + g * G + r % G) * D + 8 * c8);
  }
  int L = a.context_lens[b];
  L = min(max(L, 0), a.max_blocks * kBlock);
  const int nblk = (L + kBlock - 1) / kBlock;
  const int be = (p == a.num_parts - 1) ? nblk : min(nblk, bb + a.part_blocks);
  if (split && bb >= be) {
    for (int rr = threadIdx.x; rr < GQ; rr += NW * kWave) {
      const int64_t pi = (((int64_t)b * Q + rr / G) * Hq + g * G + rr % G) * wsp + p;
      a.ws_m[pi] = kNegInf;
      a.ws_l[pi] = 0.f;
    }
    return;
  }
  if (const int per_fit = (be - bb + NW - 1) / NW; per_fit != per) {
    // runs spread evenly over the blocks the partition holds (shorter than
    // the partition size, or a last partition longer than the others);
    // per is workgroup-uniform, so every wave still runs the same rounds
    per = per_fit;
    const int e = bb + w * per + lane;
    tbl_next = lane < per ? buf_load<int>(btr, (uint32_t)e * 4u) : 0;
  }
  const int w0 = bb + w * per;
  const int nmine = max(0, min(per, be - w0));
  const int rounds = (per + GB - 1) / GB;          // the same for every wave of the group
  const bool row_ok = rho < GQ;
  const int iq = row_ok ? rho / G : 0;
  const int nvis = row_ok ? (L - Q + iq + 1) : L;
  const int full_lim = L - Q + 1;

  int tblv = tbl_next;
  if (CH < per) {
    const int kk = CH + lane;
    tbl_next = lane < CH && kk < nmine ? buf_load<int>(btr, (uint32_t)(w0 + kk) * 4u) : 0;
  }
  const LaneOffsets<KV, D> loff(a.num_kv_heads, g, rho, qd);
  const uint32_t kblk = loff.kblk;
  // K of run block j (zeros and no memory traffic past the run or for a table
  // entry outside the pool); returns the mask of tokens with data
  auto fetch_k = [&](int j, u4 (&kr)[KS]) -> uint32_t {
    const int pb = __builtin_amdgcn_readlane(tblv, j % CH);
    const bool ok = j < nmine && pb >= 0 && (int64_t)pb < a.num_blocks;
    const auto kres = span_rsrc((const char*)a.k_cache + (int64_t)(ok ? pb : 0) * kblk,
                                ok ? kblk : 0u);
    const uint32_t ko = pin(loff.k);
#pragma unroll
    for (int m = 0; m < KS; ++m) kr[m] = buf_load<u4>(kres, ko + 64 * m);
    const int left = L - (w0 + j) * kBlock;
    return !ok ? 0u : left >= kBlock ? 0xffffu : (1u << max(left, 0)) - 1u;
  };
  // V of run block j for the tokens in `need` only
  auto fetch_v = [&](int j, uint32_t need, u4 (&vr)[KS]) {
    const int pb = __builtin_amdgcn_readlane(tblv, j % CH);
    const bool ok = need != 0u && pb >= 0 && (int64_t)pb < a.num_blocks;
    const auto vres = span_rsrc((const char*)a.v_cache + (int64_t)(ok ? pb : 0) * kblk,
                                ok ? kblk : 0u);
    const uint32_t vo = ((need >> rho) & 1u) ? pin(loff.v) : kOutOfRange;
#pragma unroll
    for (int m = 0; m < KS; ++m) vr[m] = buf_load<u4>(vres, vo + 64 * m);
  };

  uint16_t* qw = q_s + w * RT * QSTR;
  if (lane < QCW) *(u4*)(qw + (lane / (D / 8)) * QSTR + 8 * (lane % (D / 8))) = qv;
  wave_lds_fence();
  const uint16_t* qrow = qw + (row_ok ? rho : rho % GQ) * QSTR;
  unsigned char* vst = smem + w * (16 * D * 2);
  const int tr_off = ((((rho & 3) >> 1) * 16) + 4 * qd + (rho >> 2)) * 16 + (rho & 1) * 8;

  const float sl2 = a.scale_log2;
  const float lt = a.v_log2_threshold;             // -inf: read every V row
  float m_run = kNegInf, l_run = 0.f;
  f4 o[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) o[n] = f4{0.f, 0.f, 0.f, 0.f};
  uint32_t rows_read = 0;

  for (int rd = 0; rd < rounds; ++rd) {
    const int k0 = rd * GB;
    if (k0 > 0 && k0 % CH == 0) {                  // next chunk of the run
      tblv = tbl_next;
      const int kk = k0 + CH + lane;
      tbl_next = lane < CH && kk < nmine ? buf_load<int>(btr, (uint32_t)(w0 + kk) * 4u) : 0;
    }
    u4 buf[GB][KS];
    uint32_t vm[GB];
#pragma unroll
    for (int u = 0; u < GB; ++u) vm[u] = fetch_k(k0 + u, buf[u]);
    // scores of the round's blocks and this wave's row maximum over them
    float sv[GB][4];
    float mxw = kNegInf;
#pragma unroll
    for (int u = 0; u < GB; ++u) {
      f4 s = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < KS; ++m) {
        const u4 qm = *(const u4*)(qrow + 32 * m + 8 * qd);
        s = MM::qk(buf[u][m], qm, s);
      }
      const int j0 = (w0 + k0 + u) * kBlock;
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[u][r] = s[r] * sl2;
      if (vm[u] != 0xffffu || j0 + kBlock > full_lim) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = j0 + 4 * qd + r;
          if (!((vm[u] >> (4 * qd + r)) & 1u) || j >= nvis) sv[u][r] = kNegInf;
        }
      }
      mxw = fmaxf(mxw, fmaxf(fmaxf(sv[u][0], sv[u][1]), fmaxf(sv[u][2], sv[u][3])));
    }
    mxw = quarter_max(mxw);
    // the workgroup's row maximum over everything scored so far
    if (qd == 0) mm_s[w][rho] = mxw;
    __syncthreads();
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, mm_s[ww][rho]);
    __syncthreads();
    if (M > m_run) {                                 // the reference moves up: rescale
      const float alpha = m_run == kNegInf ? 0.f : fast_exp2(m_run - M);
#pragma unroll
      for (int n = 0; n < NT; ++n) o[n] *= alpha;
      l_run *= alpha;
      m_run = M;
    }
    // the V rows some row of this head needs, for all of the round's blocks
#pragma unroll
    for (int u = 0; u < GB; ++u) {
      uint32_t need = 0u;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool vote = row_ok && sv[u][r] != kNegInf && sv[u][r] >= m_run + lt;
        const uint64_t bal = __builtin_amdgcn_ballot_w64(vote);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if ((bal >> (16 * q)) & 0xffffull) need |= 1u << (4 * q + r);
      }
      rows_read += __builtin_popcount(need);
      fetch_v(k0 + u, need, buf[u]);
    }
    // weights and PV, block by block
    const float m_use = m_run == kNegInf ? 0.f : m_run;
#pragma unroll
    for (int u = 0; u < GB; ++u) {
      float pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(sv[u][r] - m_use);
      l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);
#pragma unroll
      for (int m = 0; m < KS; ++m) *(u4*)(vst + m * 1024 + lane * 16) = buf[u][m];
      wave_lds_fence();
      u2 phi, plo;
      MM::split(pr, phi, plo);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const u2 av = lds_read_tr16(vst + tr_off + (n >> 1) * 1024 + (n & 1) * 512);
        o[n] = MM::pv(av, phi, o[n]);
        o[n] = MM::pv(av, plo, o[n]);
      }
      wave_lds_fence();
    }
  }
  if (a.v_rows_read != nullptr && lane == 0)
    atomicAdd((unsigned long long*)a.v_rows_read, (unsigned long long)rows_read);

  l_run = quarter_sum(l_run);
  __syncthreads();
  float* mo = (float*)smem;
  if (rho < RT && row_ok) {
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) mo[(w * RT + rho) * D + 16 * n + 4 * qd + r] = o[n][r];
  }
  if (qd == 0) {
    mm_s[w][rho] = m_run;
    ml_s[w][rho] = l_run;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < GQ * D; idx += NW * kWave) {
    const int rr = idx / D, d = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, mm_s[ww][rr]);
    const float Mu = M == kNegInf ? 0.f : M;
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float e = fast_exp2(mm_s[ww][rr] - Mu);
      num += e * mo[(ww * RT + rr) * D + d];
      den += e * ml_s[ww][rr];
    }
    const int64_t orow = ((int64_t)b * Q + rr / G) * Hq + g * G + rr % G;
    if (split) {
      const int64_t pi = orow * wsp + p;
      a.ws_o[pi * D + d] = num;
      if (d == 0) {
        a.ws_m[pi] = M;
        a.ws_l[pi] = den;
      }
    } else {
      store_out(a.out, (OutT)a.out_dtype, orow * D + d, den > 0.f ? num / den : 0.f);
    }
  }
}

hipError_t launch_sparse_v(const AttnArgs& a, int kv_fmt, int head_dim, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  const dim3 grid((unsigned)a.num_parts, (unsigned)a.num_kv_heads, (unsigned)a.batch);
  if (kv_fmt == (int)Fmt::F16) {
    if (head_dim == 64)
      hipLaunchKernelGGL((attn_sparse_v_kernel<Fmt::F16, 64>), grid, dim3(8 * kWave), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_sparse_v_kernel<Fmt::F16, 128>), grid, dim3(8 * kWave), 0, stream, a);
  } else {
    if (head_dim == 64)
      hipLaunchKernelGGL((attn_sparse_v_kernel<Fmt::BF16, 64>), grid, dim3(8 * kWave), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_sparse_v_kernel<Fmt::BF16, 128>), grid, dim3(8 * kWave), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.ws_o == nullptr) return e;
  return launch_attention(a, kv_fmt, kv_fmt, head_dim, stream, STAGE_MERGE);
}

// Log-sum-exp merge of the split-KV partials: one workgroup per DC output
// dims of an output row (b, i, h), grid (rows, D / DC).
// out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p, M = max_p m_p.
// Single pass: thread (c, grp) takes partitions grp, grp+NG, ... for the 4
// dims of chunk c, folding each into a running (max, sum, acc) so every load
// can be in flight at once.  The NG running states are then combined in
// parallel: the workgroup's max M, every state rescaled to M by its own
// thread, and a sum over the groups (xor shuffles inside a wavefront, the
// four wavefronts' sums in LDS).  DC < D is for few rows: more workgroups,
// each with fewer partitions per thread, so that one round of loads covers
// many partitions.
template <int D, int DC>
__global__ __launch_bounds__(256) void attn_merge_kernel(const AttnArgs a) {
  static_assert(D % DC == 0 && DC % 4 == 0 && DC / 4 <= kWave && (DC / 4 & (DC / 4 - 1)) == 0,
                "merge slice: a power-of-two count of float4 chunks, at most a wavefront");
  constexpr int NC = DC / 4;             // float4 chunks per workgroup
  constexpr int NG = 256 / NC;           // partition groups
  constexpr int NWV = 256 / kWave;       // wavefronts
  __shared__ f4 acc_s[NWV][NC];
  __shared__ float m_s[NWV], den_s[NWV];

  const int64_t row = blockIdx.x;
  const int col0 = blockIdx.y * DC;
  const int t = threadIdx.x;
  // every partition of the grid holds a partial or an empty marker (max -inf)
  const int np = a.ws_parts;
  const float* wm = a.ws_m + row * np;
  const float* wl = a.ws_l + row * np;
  const float* wo = a.ws_o + row * np * D + col0;

  const int c = t % NC, grp = t / NC;
  float m_t = kNegInf, den = 0.f;
  f4 acc = f4{0.f, 0.f, 0.f, 0.f};
  constexpr int U = 8;                   // partitions whose loads are issued together
  for (int p0 = grp; p0 < np; p0 += U * NG) {
    float mp[U], lp[U];
    f4 op[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {        // loads first (clamped index), no branches between
      const int pp = min(p0 + u * NG, np - 1);
      mp[u] = wm[pp];
      lp[u] = wl[pp];
      op[u] = *(const f4*)(wo + (int64_t)pp * D + 4 * c);
    }
    // every value passes through an empty asm here, so the compiler cannot
    // sink a partition's o and l loads below the test of its m (it did for
    // the first one, which cost a second dependent round trip)
#pragma unroll
    for (int u = 0; u < U; ++u) asm volatile("" : "+v"(mp[u]), "+v"(lp[u]), "+v"(op[u]));
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // -inf: the partition saw nothing and its o was never written (it may
      // hold anything, NaN included), so it is selected away, not weighted by 0
      const bool use = p0 + u * NG < np && mp[u] != kNegInf;
      const float m_new = use ? fmaxf(m_t, mp[u]) : m_t;
      const float e_old = m_t == kNegInf ? 0.f : fast_exp2(m_t - m_new);
      const float e_new = use ? fast_exp2(mp[u] - m_new) : 0.f;
      const f4 o_u = use ? op[u] : f4{0.f, 0.f, 0.f, 0.f};
      const float l_u = use ? lp[u] : 0.f;
      acc = acc * e_old + o_u * e_new;
      den = den * e_old + l_u * e_new;
      m_t = m_new;
    }
  }
  // lanes c, c + NC, ... of a wavefront hold the same chunk of different groups
  const int lane = t % kWave, w = t / kWave;
  float mx = m_t;
#pragma unroll
  for (int d = NC; d < kWave; d <<= 1) mx = fmaxf(mx, __shfl_xor(mx, d, kWave));
  if (lane == 0) m_s[w] = mx;
  __syncthreads();
  float M = m_s[0];
#pragma unroll
  for (int i = 1; i < NWV; ++i) M = fmaxf(M, m_s[i]);
  // a group that saw nothing (and with it M -inf, when no partition saw
  // anything) weighs 0
  const float e = m_t == kNegInf ? 0.f : fast_exp2(m_t - M);
  acc = acc * e;
  den = den * e;
#pragma unroll
  for (int d = NC; d < kWave; d <<= 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] += __shfl_xor(acc[r], d, kWave);
    den += __shfl_xor(den, d, kWave);
  }
  if (lane < NC) acc_s[w][lane] = acc;
  if (lane == 0) den_s[w] = den;
  __syncthreads();
  if (t < NC) {
    f4 tot = acc_s[0][t];
    float dt = den_s[0];
#pragma unroll
    for (int i = 1; i < NWV; ++i) {
      tot += acc_s[i][t];
      dt += den_s[i];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      store_out(a.out, (OutT)a.out_dtype, row * D + col0 + 4 * t + r,
                dt > 0.f ? tot[r] / dt : 0.f);
  }
}

static int device_cu_count();

template <int D>
static hipError_t launch_merge(const AttnArgs& a, hipStream_t stream) {
  const unsigned rows = (unsigned)((int64_t)a.batch * a.q_len * a.num_q_heads);
  // a whole-row workgroup loads 8 partitions per thread in one round; with
  // more partitions than that and rows too few to fill the compute units,
  // 32-dim slices keep it to one round (and spread it over more CUs)
  constexpr int kOneRound = 8 * (256 / (D / 4));
  const int cus = device_cu_count();
  if (a.ws_parts > kOneRound && cus > 0 && (int64_t)rows <= 2 * (int64_t)cus)
    hipLaunchKernelGGL((attn_merge_kernel<D, 32>), dim3(rows, D / 32), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_merge_kernel<D, D>), dim3(rows), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// Compute units of the current device (0 if unknown), read once per device.
static int device_cu_count() {
  // written once per device; calls from several host threads may race to
  // write the same value, hence the relaxed atomics
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = -1;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n > 0 ? n : 0;
}

// Balanced split: grid (runs / waves per head, KV heads / HP), then the merge.
template <Fmt KV, int D>
static hipError_t launch_flat(const AttnArgs& a, hipStream_t stream) {
  if constexpr (KV == Fmt::K8V4) {
    return hipErrorInvalidValue;
  } else {
    const int rows = a.gqa * a.q_len;
    // runs per KV head: as many as give one workgroup per compute unit (the
    // grid is runs * Hkv / NW workgroups, whatever the heads per workgroup),
    // a multiple of 8, at most the a.flat_runs the workspace is sized for.
    // One round of workgroups, and fewer partials for the merge to read.
    AttnArgs f = a;
    const int cus = device_cu_count();
    if (cus > 0) {
      const int nw = rows <= 4 ? kFlatWaves<4> : kFlatWaves<16>;
      const int want = (int)((int64_t)cus * nw / a.num_kv_heads) / 8 * 8;
      f.flat_runs = want < 8 ? 8 : want < a.flat_runs ? want : a.flat_runs;
    }
    // heads per workgroup: all of a workgroup's waves on one run, one head
    // each (a block's token rows of all those heads read by one CU), when the
    // KV heads divide into groups of that size; else pairs, else one head
    if (rows <= 4) {
      constexpr int NW = kFlatWaves<4>;
      const int hp = a.num_kv_heads % NW == 0 ? NW : a.num_kv_heads % 2 == 0 ? 2 : 1;
      const dim3 grid((unsigned)(f.flat_runs / (NW / hp)), (unsigned)(a.num_kv_heads / hp));
      if (hp == NW)
        hipLaunchKernelGGL((attn_flat_kernel<KV, D, 4, NW>), grid, dim3(NW * kWave), 0, stream, f);
      else if (hp == 2)
        hipLaunchKernelGGL((attn_flat_kernel<KV, D, 4, 2>), grid, dim3(NW * kWave), 0, stream, f);
      else
        hipLaunchKernelGGL((attn_flat_kernel<KV, D, 4, 1>), grid, dim3(NW * kWave), 0, stream, f);
    } else {
      constexpr int NW = kFlatWaves<16>;
      const int hp = a.num_kv_heads % NW == 0 ? NW : a.num_kv_heads % 2 == 0 ? 2 : 1;
      const dim3 grid((unsigned)(f.flat_runs / (NW / hp)), (unsigned)(a.num_kv_heads / hp));
      if (hp == NW)
        hipLaunchKernelGGL((attn_flat_kernel<KV, D, 16, NW>), grid, dim3(NW * kWave), 0, stream, f);
      else if (hp == 2)
        hipLaunchKernelGGL((attn_flat_kernel<KV, D, 16, 2>), grid, dim3(NW * kWave), 0, stream, f);
      else
        hipLaunchKernelGGL((attn_flat_kernel<KV, D, 16, 1>), grid, dim3(NW * kWave), 0, stream, f);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned pairs = (unsigned)((int64_t)a.batch * a.num_kv_heads);   // (sequence, KV head)
    hipLaunchKernelGGL((attn_flat_merge_kernel<D>), dim3(pairs), dim3(kFlatMergeThreads), 0,
                       stream, f);
    return hipGetLastError();
  }
}

template <Fmt KV, Fmt QT, int D>
static hipError_t launch_typed(const AttnArgs& a, hipStream_t stream, int stage) {
  if (a.flat_runs > 0) {
    if (stage != STAGE_ALL || a.mode != 0 || a.window != 0) return hipErrorInvalidValue;
    return launch_flat<KV, D>(a, stream);
  }
  if (stage != STAGE_MERGE) {
    const int rows = (a.mode == 1 ? a.group_size : 1) * a.gqa * a.q_len;
    dim3 grid((unsigned)a.num_parts, (unsigned)a.num_kv_heads,
              (unsigned)(a.mode == 1 ? a.num_groups : a.batch));
    if constexpr (KV == Fmt::K8V4) {
      // head groups of eight when their grid fills every CU at least once
      const int64_t hg_wgs = (int64_t)a.num_parts * (a.num_kv_heads / 8) * a.batch;
      const int64_t cus = device_cu_count();
      if (a.mode == 0 && rows <= 4 && a.num_kv_heads % 8 == 0 && cus > 0 && hg_wgs >= cus) {
        const dim3 hgrid((unsigned)a.num_parts, (unsigned)(a.num_kv_heads / 8), (unsigned)a.batch);
        hipLaunchKernelGGL((attn_partition_kernel<KV, QT, D, 4, false, 8>), hgrid,
                           dim3(Shape<KV, 4, 8>::NW * kWave), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || a.ws_o == nullptr || stage == STAGE_PARTIALS) return e;
        return launch_merge<D>(a, stream);
      }
    }
    if constexpr (KV == Fmt::K8V4) {     // 1-D, XCD-grouped order (see the kernel)
      if (a.mode != 0) return hipErrorInvalidValue;
      const int64_t units = (int64_t)a.num_parts * a.batch;
      const int64_t n = 8 * (int64_t)a.num_kv_heads * ((units + 7) / 8);
      // a launch covers fewer than 2^32 work-items per dimension
      if (n * Shape<KV, 4>::NW * kWave > 0xffffffffLL || n * Shape<KV, 16>::NW * kWave > 0xffffffffLL)
        return hipErrorInvalidConfiguration;
      grid = dim3((unsigned)n, 1u, 1u);
    }
    if constexpr (KV != Fmt::K8V4) {
      if (a.mode == 1) {                 // cascade prefix pass: its own instantiation
        if (rows <= 4)
          hipLaunchKernelGGL((attn_partition_kernel<KV, QT, D, 4, true>), grid,
                             dim3(Shape<KV, 4>::NW * kWave), 0, stream, a);
        else
          hipLaunchKernelGGL((attn_partition_kernel<KV, QT, D, 16, true>), grid,
                             dim3(Shape<KV, 16>::NW * kWave), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || stage == STAGE_PARTIALS) return e;
        return launch_merge<D>(a, stream);
      }
    }
    // Head pairs (quads) when the one-head grid needs two (up to four)
    // workgroups per CU and the grouped grid fits in one: the 32K sequence's
    // 512 workgroups become 256 pairs.  A smaller grid keeps one head per
    // workgroup: grouping would leave CUs idle, and one CU alone streams far
    // below its share of HBM.
    int hp = 1;
    if constexpr (KV != Fmt::K8V4) {
      const int64_t wgs = (int64_t)a.num_parts * a.num_kv_heads * a.batch;
      const int64_t cus = device_cu_count();
      // h heads per workgroup (one workgroup per CU) leave about
      // ceil(wgs / (h cus)) * h partitions of work on a CU, the one-head form
      // (two workgroups per CU) ceil(wgs / cus): group only when that is no
      // more, i.e. (h - 1) cus < wgs <= h cus
      auto fits = [&](int h) {
        return a.num_kv_heads % h == 0 && wgs > (int64_t)(h - 1) * cus && wgs <= (int64_t)h * cus;
      };
      if (rows <= 4 && a.mode == 0 && cus > 0) {
        if (fits(2)) hp = 2;
        else if (fits(4)) hp = 4;
        else if (fits(8)) hp = 8;                                     // one wave per head
      }
    }
    if (hp > 1) {
      if constexpr (KV != Fmt::K8V4) {
        const dim3 hgrid((unsigned)a.num_parts, (unsigned)(a.num_kv_heads / hp), (unsigned)a.batch);
        if (hp == 2)
          hipLaunchKernelGGL((attn_partition_kernel<KV, QT, D, 4, false, 2>), hgrid,
                             dim3(Shape<KV, 4>::NW * kWave), 0, stream, a);
        else if (hp == 4)
          hipLaunchKernelGGL((attn_partition_kernel<KV, QT, D, 4, false, 4>), hgrid,
                             dim3(Shape<KV, 4>::NW * kWave), 0, stream, a);
        else
          hipLaunchKernelGGL((attn_partition_kernel<KV, QT, D, 4, false, 8>), hgrid,
                             dim3(Shape<KV, 4>::NW * kWave), 0, stream, a);
      }
    } else if (rows <= 4) {
      hipLaunchKernelGGL((attn_partition_kernel<KV, QT, D, 4, false>), grid,
                         dim3(Shape<KV, 4>::NW * kWave), 0, stream, a);
    } else {
      hipLaunchKernelGGL((attn_partition_kernel<KV, QT, D, 16, false>), grid,
                         dim3(Shape<KV, 16>::NW * kWave), 0, stream, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.ws_o == nullptr || stage == STAGE_PARTIALS) return e;
  }
  return launch_merge<D>(a, stream);
}

template <int D>
static hipError_t launch_d(const AttnArgs& a, int kv_fmt, int q_fmt, hipStream_t stream,
                           int stage) {
  if (stage == STAGE_MERGE) return launch_merge<D>(a, stream);
  if (kv_fmt == (int)Fmt::F16) return launch_typed<Fmt::F16, Fmt::F16, D>(a, stream, stage);
  if (kv_fmt == (int)Fmt::BF16) return launch_typed<Fmt::BF16, Fmt::BF16, D>(a, stream, stage);
  if (q_fmt == (int)Fmt::F16) return launch_typed<Fmt::K8V4, Fmt::F16, D>(a, stream, stage);
  return launch_typed<Fmt::K8V4, Fmt::BF16, D>(a, stream, stage);
}

hipError_t launch_attention(const AttnArgs& a, int kv_fmt, int q_fmt, int head_dim,
                            hipStream_t stream, int stage) {
  if (a.batch == 0) return hipSuccess;
  return head_dim == 64 ? launch_d<64>(a, kv_fmt, q_fmt, stream, stage)
                        : launch_d<128>(a, kv_fmt, q_fmt, stream, stage);
}

}  // namespace pkv

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
//   blocks of one partition; wavefront w takes blocks w, w+NW, ... of it.  All
//   G*q_len query rows that share a KV head live in one wavefront, so each K/V
//   byte is read from HBM once.  The direct form is the same kernel with one
//   partition per sequence; the split-KV form writes per-partition partials and
//   a second kernel merges them by log-sum-exp.
//
// Per 16-token block, per wavefront (lane l: row l % 16, quarter l / 16):
//   - K rows are loaded straight into the A operand of a 16x16x32 MFMA
//     (lane l holds 8 head dims of token l % 16 per step), giving S^T = K Q^T:
//     lane l ends with the scores of query row l % 16 for tokens 4*(l/16)+r.
//   - Online softmax (running max and sum per row in fp32, exp2 domain); the
//     block max is reduced across the four quarters with two lane exchanges.
//   - The probabilities are already in the B-operand layout of a 16x16x16 MFMA
//     computing O^T = V^T P^T; they are split into a 16-bit high part and a
//     16-bit remainder so the product keeps ~22 bits of each weight.
//   - V rows are staged through LDS (natural [token][dim] layout) and read back
//     transposed as the A operand.  Output lane l holds row l % 16's dims
//     16n + 4*(l/16) + r, so the softmax rescale is one factor per lane.
//   - Loads of the next block are issued before the current block is used.
//   - Positions past the length, past a row's causal limit, or in a block whose
//     table entry is out of range are excluded by selecting -inf scores, and V
//     rows past the length are zeroed, so NaN garbage there never propagates.
//
// K8/V4 storage: int8 K codes are converted exactly to the MFMA element type and
// the per-token scale multiplies the scores; 4-bit V codes are converted exactly
// and staged like 16-bit V, the per-group scale is folded into the weights
// (sum_t p_t s_tg c_td) and the zero point into a per-group sum (sum_t p_t z_tg).

#include <math.h>

#include "pkv_common.h"
#include "pkv_launch.h"

namespace pkv {

constexpr int NW = 4;                  // wavefronts per workgroup
constexpr float kNegInf = -INFINITY;

// Head dims of the K/Q operand held by quarter qd at QK step m (8 consecutive).
template <Fmt KV>
__device__ __forceinline__ int qk_dim(int m, int qd) {
  if constexpr (KV == Fmt::K8V4) return 64 * (m >> 1) + 16 * qd + 8 * (m & 1);
  else return 32 * m + 8 * qd;
}

// int8 code -> 16-bit element bits of the MFMA type (exact: |c| <= 127).
template <Fmt QT>
__device__ __forceinline__ uint32_t code_bits(int c) {
  if constexpr (QT == Fmt::F16) return f32_to_f16_bits((float)c);
  else return __float_as_uint((float)c) >> 16;
}

template <Fmt QT>
__device__ __forceinline__ uint32_t pack2_codes(int c0, int c1) {
  return code_bits<QT>(c0) | (code_bits<QT>(c1) << 16);
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

template <Fmt KV, int D>
__device__ __forceinline__ void load_block(const AttnArgs& a, int64_t pb, int g, int rho, int qd,
                                           BlockRegs<KV, D>& br) {
  const int64_t row = (pb * kBlock + rho) * a.num_kv_heads + g;   // (block, token, head)
  if constexpr (KV == Fmt::K8V4) {
    const int8_t* kc = (const int8_t*)a.k_cache + row * D;
#pragma unroll
    for (int u = 0; u < D / 64; ++u) br.k[u] = *(const u4*)(kc + 64 * u + 16 * qd);
    const uint8_t* vc = (const uint8_t*)a.v_cache + row * (D / 2);
    if constexpr (D == 128) {
      br.v = *(const u4*)(vc + 16 * qd);
    } else {
      u2 t = *(const u2*)(vc + 8 * qd);
      br.v = u4{t.x, t.y, 0u, 0u};
    }
    br.ks = ((const uint16_t*)a.k_scale)[row];
    if constexpr (D == 128) {
      br.vs = *(const u2*)((const uint16_t*)a.v_scale + row * 4);
      br.vz = *(const u2*)((const uint16_t*)a.v_zero + row * 4);
    } else {
      br.vs = u2{*(const uint32_t*)((const uint16_t*)a.v_scale + row * 2), 0u};
      br.vz = u2{*(const uint32_t*)((const uint16_t*)a.v_zero + row * 2), 0u};
    }
  } else {
    const uint16_t* kc = (const uint16_t*)a.k_cache + row * D;
    const uint16_t* vc = (const uint16_t*)a.v_cache + row * D;
#pragma unroll
    for (int m = 0; m < D / 32; ++m) br.k[m] = *(const u4*)(kc + 32 * m + 8 * qd);
#pragma unroll
    for (int m = 0; m < D / 32; ++m) br.v[m] = *(const u4*)(vc + 32 * m + 8 * qd);
  }
}

template <Fmt KV, Fmt QT, int D>
struct AttnSmem {
  static constexpr int VSTR = D + 4;                       // halves per staged V row
  static constexpr int GR = D / 32;                        // V groups per row
  static constexpr int VST = NW * 16 * VSTR * 2;           // staged V bytes
  static constexpr int SIDE = KV == Fmt::K8V4 ? NW * 16 * (1 + 2 * GR) * 4 : 0;
  static constexpr int MO = NW * 16 * D * 4;               // merge: per-wave outputs
  static constexpr int BYTES = (VST + SIDE) > MO ? (VST + SIDE) : MO;
};

template <Fmt KV, Fmt QT, int D>
__global__ __launch_bounds__(NW * kWave) void attn_partition_kernel(const AttnArgs a) {
  using MM = Mma<QT>;
  using SM = AttnSmem<KV, QT, D>;
  constexpr int KS = D / 32;           // QK MFMA steps
  constexpr int NT = D / 16;           // PV output tiles
  constexpr int VSTR = SM::VSTR;
  constexpr int GR = SM::GR;
  __shared__ __align__(16) unsigned char smem[SM::BYTES];
  __shared__ float mm_s[NW][16], ml_s[NW][16];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int rho = lane & 15, qd = lane >> 4;
  const int p = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int Q = a.q_len, G = a.gqa, GQ = G * Q, Hq = a.num_q_heads;
  const bool split = a.ws_o != nullptr;

  int L = a.context_lens[b];
  L = min(max(L, 0), a.max_blocks * kBlock);
  const int nblk = (L + kBlock - 1) / kBlock;
  const int bb = p * a.part_blocks;
  if (split && bb >= nblk) return;                          // partition past this sequence
  const int be = (p == a.num_parts - 1) ? nblk : min(nblk, bb + a.part_blocks);

  // the query row this lane owns: rho = iq * G + hl
  const bool row_ok = rho < GQ;
  const int iq = row_ok ? rho / G : 0;
  const int h = g * G + (row_ok ? rho % G : 0);
  const int nvis = row_ok ? (L - Q + iq + 1) : L;           // visible positions of the row
  const int full_lim = L - Q + 1;                           // every row sees j < full_lim

  u4 qop[KS];
  {
    const uint16_t* qp = (const uint16_t*)a.q + (((int64_t)b * Q + iq) * Hq + h) * D;
#pragma unroll
    for (int m = 0; m < KS; ++m)
      qop[m] = row_ok ? *(const u4*)(qp + qk_dim<KV>(m, qd)) : u4{0u, 0u, 0u, 0u};
  }

  uint16_t* vst = (uint16_t*)smem + w * 16 * VSTR;          // this wave's staged V tile
  float* side = (float*)(smem + SM::VST) + w * 16 * (1 + 2 * GR);   // K8/V4 scales

  float m_run = kNegInf, l_run = 0.f;
  f4 o[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) o[n] = f4{0.f, 0.f, 0.f, 0.f};
  float zacc[GR];
#pragma unroll
  for (int gi = 0; gi < GR; ++gi) zacc[gi] = 0.f;

  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks;
  const float sl2 = a.scale_log2;

  // This wave's blocks are bb + w + NW*k, k = 0 .. nmine-1.  Their table
  // entries are read 64 at a time into one VGPR (lane j holds entry j of the
  // chunk) and picked out with readlane, so no table load sits between the
  // K/V loads of consecutive blocks.
  const int nmine = be > bb + w ? (be - bb - w + NW - 1) / NW : 0;
  int tblv = 0;
  auto fetch = [&](int j, BlockRegs<KV, D>& br) -> bool {
    const int pb = __builtin_amdgcn_readlane(tblv, j);
    const bool ok = pb >= 0 && (int64_t)pb < a.num_blocks;
    load_block<KV, D>(a, ok ? pb : 0, g, rho, qd, br);
    return ok;
  };

  auto process = [&](int i, bool ok, BlockRegs<KV, D>& br) {
    const int j0 = i * kBlock;
    const bool tail = !ok || j0 + kBlock > L;                // some tokens past the length
    const bool full = ok && j0 + kBlock <= full_lim;         // no masking needed at all
    const bool tok_ok = ok && j0 + rho < L;                  // this lane's token (rho) exists

    // ---- scores S^T = K Q^T
    f4 s = f4{0.f, 0.f, 0.f, 0.f};
    if constexpr (KV == Fmt::K8V4) {
#pragma unroll
      for (int u = 0; u < D / 64; ++u) {
        const u4 c = br.k[u];
        u4 lo, hi;
        const uint32_t wd[4] = {c.x, c.y, c.z, c.w};
        uint32_t cv[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int x = (int)wd[q];
          cv[2 * q] = pack2_codes<QT>((int8_t)(x & 0xff), (int8_t)((x >> 8) & 0xff));
          cv[2 * q + 1] = pack2_codes<QT>((int8_t)((x >> 16) & 0xff), (int8_t)((x >> 24) & 0xff));
        }
        lo = u4{cv[0], cv[1], cv[2], cv[3]};
        hi = u4{cv[4], cv[5], cv[6], cv[7]};
        s = MM::qk(lo, qop[2 * u], s);
        s = MM::qk(hi, qop[2 * u + 1], s);
      }
      // per-token K scales and V scale/zero, redistributed through LDS from the
      // token-owner layout (lane rho) to the score layout (tokens 4*qd + r)
      if (qd == 0) {
        side[rho] = f16_bits_to_f32(br.ks);
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
    } else {
#pragma unroll
      for (int m = 0; m < KS; ++m) s = MM::qk(br.k[m], qop[m], s);
    }

    // ---- stage V (natural [token][dim] layout), zeroing rows past the length
    if constexpr (KV == Fmt::K8V4) {
      constexpr int NC = D / 4;                 // codes held by this lane: dims NC*qd ..
      const uint32_t wd[4] = {br.v.x, br.v.y, br.v.z, br.v.w};
#pragma unroll
      for (int q = 0; q < NC / 8; ++q) {
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t byte = (wd[q] >> (8 * e)) & 0xffu;
          const int c0 = tok_ok ? (int)(byte & 0xfu) : 0;
          const int c1 = tok_ok ? (int)(byte >> 4) : 0;
          pk[e] = pack2_codes<QT>(c0, c1);
        }
        uint16_t* dst = vst + rho * VSTR + NC * qd + 8 * q;
        *(u2*)(dst) = u2{pk[0], pk[1]};
        *(u2*)(dst + 4) = u2{pk[2], pk[3]};
      }
    } else {
#pragma unroll
      for (int m = 0; m < KS; ++m) {
        u4 vv = br.v[m];
        if (tail && !tok_ok) vv = u4{0u, 0u, 0u, 0u};
        uint16_t* dst = vst + rho * VSTR + 32 * m + 8 * qd;
        *(u2*)(dst) = u2{vv.x, vv.y};
        *(u2*)(dst + 4) = u2{vv.z, vv.w};
      }
    }
    wave_lds_fence();

    // ---- online softmax in the exp2 domain
    float sv[4];
    if constexpr (KV == Fmt::K8V4) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[r] = s[r] * side[4 * qd + r] * sl2;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[r] = s[r] * sl2;
    }
    if (!full) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = j0 + 4 * qd + r;
        if (!ok || j >= nvis) sv[r] = kNegInf;
      }
    }
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = fmaxf(mx, wave_xor(mx, 16));
    mx = fmaxf(mx, wave_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(sv[r] - m_use);
    l_run = l_run * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    m_run = m_new;
#pragma unroll
    for (int n = 0; n < NT; ++n) o[n] *= alpha;

    // ---- O^T += V^T P^T
    if constexpr (KV == Fmt::K8V4) {
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
        zacc[gi] = zacc[gi] * alpha + zs;
        u2 phi, plo;
        MM::split(pw, phi, plo);
#pragma unroll
        for (int nn = 0; nn < 2; ++nn) {
          const int n = 2 * gi + nn;
          const uint16_t* src = vst + (4 * qd) * VSTR + 16 * n + rho;
          const u2 av = u2{(uint32_t)src[0] | ((uint32_t)src[VSTR] << 16),
                           (uint32_t)src[2 * VSTR] | ((uint32_t)src[3 * VSTR] << 16)};
          o[n] = MM::pv(av, phi, o[n]);
          o[n] = MM::pv(av, plo, o[n]);
        }
      }
    } else {
      u2 phi, plo;
      MM::split(pr, phi, plo);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const uint16_t* src = vst + (4 * qd) * VSTR + 16 * n + rho;
        const u2 av = u2{(uint32_t)src[0] | ((uint32_t)src[VSTR] << 16),
                         (uint32_t)src[2 * VSTR] | ((uint32_t)src[3 * VSTR] << 16)};
        o[n] = MM::pv(av, phi, o[n]);
        o[n] = MM::pv(av, plo, o[n]);
      }
    }
    wave_lds_fence();
  };

  // ---- block loop, in chunks of 64 of this wave's blocks.  Two register
  // sets: in the steady state the next block's loads are always issued before
  // the current block is consumed, with no branch between them, so the wait
  // before each block covers only that block's loads.
  for (int c0 = 0; c0 < nmine; c0 += 64) {
    const int cnt = min(64, nmine - c0);
    tblv = lane < cnt ? bt[bb + w + NW * (c0 + lane)] : 0;
    const int i0 = bb + w + NW * c0;
    BlockRegs<KV, D> r0, r1;
    bool ok0 = fetch(0, r0), ok1 = false;
    int k = 0;
    for (int pr = (cnt - 1) >> 1; pr > 0; --pr) {     // branch-free pairs of blocks
      ok1 = fetch(k + 1, r1);
      process(i0 + NW * k, ok0, r0);
      ok0 = fetch(k + 2, r0);
      process(i0 + NW * (k + 1), ok1, r1);
      k += 2;
    }
    if (k + 1 < cnt) {                                // two blocks left
      ok1 = fetch(k + 1, r1);
      process(i0 + NW * k, ok0, r0);
      process(i0 + NW * (k + 1), ok1, r1);
    } else {                                          // one block left
      process(i0 + NW * k, ok0, r0);
    }
  }

  // ---- per-wave totals: the sum is spread over the four quarters
  l_run += wave_xor(l_run, 16);
  l_run += wave_xor(l_run, 32);
  if constexpr (KV == Fmt::K8V4) {
#pragma unroll
    for (int gi = 0; gi < GR; ++gi) {
      zacc[gi] += wave_xor(zacc[gi], 16);
      zacc[gi] += wave_xor(zacc[gi], 32);
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) o[n] += zacc[n / 2];
  }

  // ---- merge the NW wavefronts of this workgroup (LDS reused)
  __syncthreads();
  float* mo = (float*)smem;
  if (row_ok) {
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) mo[(w * 16 + rho) * D + 16 * n + 4 * qd + r] = o[n][r];
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
      num += e * mo[(ww * 16 + rr) * D + d];
      den += e * ml_s[ww][rr];
    }
    const int64_t orow = ((int64_t)b * Q + rr / G) * Hq + g * G + rr % G;
    if (split) {
      const int64_t pi = orow * a.num_parts + p;
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

// Log-sum-exp merge of the split-KV partials: one workgroup per output row
// (b, i, h).  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p, M = max_p m_p.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(const AttnArgs a) {
  constexpr int NC = D / 4;              // float4 chunks per row
  constexpr int NG = 256 / NC;           // partition groups
  __shared__ float red[256];
  __shared__ f4 acc_s[NG][NC];
  __shared__ float den_s[NG];

  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const int b = (int)(row / ((int64_t)a.q_len * a.num_q_heads));
  int L = a.context_lens[b];
  L = min(max(L, 0), a.max_blocks * kBlock);
  const int nblk = (L + kBlock - 1) / kBlock;
  const int np = nblk == 0 ? 0 : min((nblk + a.part_blocks - 1) / a.part_blocks, a.num_parts);
  const float* wm = a.ws_m + row * a.num_parts;
  const float* wl = a.ws_l + row * a.num_parts;
  const float* wo = a.ws_o + row * a.num_parts * D;

  float M = kNegInf;
  for (int pp = t; pp < np; pp += 256) M = fmaxf(M, wm[pp]);
  red[t] = M;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) red[t] = fmaxf(red[t], red[t + s]);
    __syncthreads();
  }
  M = red[0];
  const float Mu = M == kNegInf ? 0.f : M;

  const int c = t % NC, grp = t / NC;
  f4 acc = f4{0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int pp = grp; pp < np; pp += NG) {
    const float e = fast_exp2(wm[pp] - Mu);
    acc += e * *(const f4*)(wo + (int64_t)pp * D + 4 * c);
    den += e * wl[pp];
  }
  acc_s[grp][c] = acc;
  if (c == 0) den_s[grp] = den;
  __syncthreads();
  if (t < NC) {
    f4 tot = f4{0.f, 0.f, 0.f, 0.f};
    float dt = 0.f;
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) {
      tot += acc_s[gg][t];
      dt += den_s[gg];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      store_out(a.out, (OutT)a.out_dtype, row * D + 4 * t + r, dt > 0.f ? tot[r] / dt : 0.f);
  }
}

template <int D>
static hipError_t launch_merge(const AttnArgs& a, hipStream_t stream) {
  const unsigned rows = (unsigned)((int64_t)a.batch * a.q_len * a.num_q_heads);
  hipLaunchKernelGGL((attn_merge_kernel<D>), dim3(rows), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <Fmt KV, Fmt QT, int D>
static hipError_t launch_typed(const AttnArgs& a, hipStream_t stream, int stage) {
  if (stage != STAGE_MERGE) {
    const dim3 grid((unsigned)a.num_parts, (unsigned)a.num_kv_heads, (unsigned)a.batch);
    hipLaunchKernelGGL((attn_partition_kernel<KV, QT, D>), grid, dim3(NW * kWave), 0, stream, a);
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

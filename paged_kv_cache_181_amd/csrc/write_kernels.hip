// Slot-scatter kernels: the reshape_and_cache step that stores each step's new
// K/V rows into the block-paged cache ("The KV Cache" (metalworking), layout
// paragraph; "How the Paged KV Cache Works in MTPLX", Physical Layout and Memory
// Organization: cache [num_blocks, 16, num_kv_heads, head_dim]).
//
// HBM traffic is tiny (one token row per sequence per step), so the kernels are
// latency-bound: one workgroup per token moves the whole [Hkv, D] row with
// 16-byte vector loads/stores.

#include "pkv_common.h"
#include "pkv_launch.h"

namespace pkv {

// One workgroup per token; each thread moves 16-byte chunks of the K and V rows.
__global__ __launch_bounds__(256) void kv_write_kernel(const u4* __restrict__ key,
                                                       const u4* __restrict__ value,
                                                       u4* __restrict__ key_cache,
                                                       u4* __restrict__ value_cache,
                                                       const int64_t* __restrict__ slots,
                                                       int64_t num_slots, int row_vecs,
                                                       int stride) {
  const int64_t t = blockIdx.x;
  int64_t slot = slots[t];
  const u4* ks = key + t * row_vecs;
  const u4* vs = value + t * row_vecs;
  for (int i = threadIdx.x; i < row_vecs; i += stride) {   // stride = the workgroup size
    // the row's loads go out together with the slot's, not after it: the
    // empty asm takes the loaded values and passes the slot through, so
    // nothing that depends on the slot (the check, the destination) is
    // placed above the loads and the two latencies overlap
    const u4 kk = ks[i], vv = vs[i];
    asm volatile("" : "+s"(slot) : "v"(kk), "v"(vv));
    if (slot < 0 || slot >= num_slots) break;            // skipped token
    key_cache[slot * row_vecs + i] = kk;
    value_cache[slot * row_vecs + i] = vv;
  }
}

hipError_t launch_kv_write(const void* key, const void* value, void* key_cache, void* value_cache,
                           const int64_t* slots, int64_t num_tokens, int num_kv_heads,
                           int head_dim, int64_t num_blocks, hipStream_t stream) {
  const int row_vecs = num_kv_heads * head_dim * 2 / 16;
  const int threads = row_vecs >= 256 ? 256 : ((row_vecs + 63) / 64) * 64;
  hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)num_tokens), dim3(threads), 0, stream,
                     (const u4*)key, (const u4*)value, (u4*)key_cache, (u4*)value_cache, slots,
                     num_blocks * kBlock, row_vecs, threads);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------
// K8/V4 quantize-on-write.  One wavefront per (token, KV head).  All integer
// decisions are taken in fp32 with correctly rounded division and
// round-to-nearest-even, exactly as stated in pagedkv.h:
//   K: s = fp16(amax / 127); code = clamp(rint(k / s), -127, 127) (0 if s == 0)
//   V: per 32 elements s = fp16((max - min) / 15), z = fp16(min);
//      code = clamp(rint((v - z) / s), 0, 15) (0 if s == 0); two codes per byte.
// ("How MTPLX Manages Memory with KV Caching Strategies", VllmMetalPagedKVCache:
// a symmetric quantizer on the write path; "The KV Cache", K/V asymmetry: K8/V4.)

template <Fmt IN, int D>
__global__ __launch_bounds__(256) void kv_write_k8v4_kernel(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
    int8_t* __restrict__ k_cache, uint16_t* __restrict__ k_scale, uint8_t* __restrict__ v_cache,
    uint16_t* __restrict__ v_scale, uint16_t* __restrict__ v_zero,
    const int64_t* __restrict__ slots, int64_t num_tokens, int hkv, int64_t num_slots) {
  constexpr int E = D / kWave;           // elements per lane: 1 (D=64) or 2 (D=128)
  const int lane = threadIdx.x & 63;
  const int64_t unit = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x >> 6);
  if (unit >= num_tokens * hkv) return;
  const int64_t t = unit / hkv;
  const int h = (int)(unit % hkv);
  const int64_t slot = slots[t];

  // this lane's elements: d = lane * E + e (loaded together with the slot)
  float k[E], v[E];
  const int64_t src = (t * hkv + h) * D + lane * E;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    k[e] = IN == Fmt::F16 ? f16_bits_to_f32(key[src + e]) : bf16_bits_to_f32(key[src + e]);
    v[e] = IN == Fmt::F16 ? f16_bits_to_f32(value[src + e]) : bf16_bits_to_f32(value[src + e]);
    asm volatile("" ::"v"(k[e]), "v"(v[e]));                // keeps the loads above the check
  }
  if (slot < 0 || slot >= num_slots) return;                // skipped token

  // ---- K: symmetric int8, one scale per (token, head)
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(k[e]));
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) amax = fmaxf(amax, wave_xor(amax, m));
  const uint16_t ks16 = k8_scale_bits(amax);
  const float ks = f16_bits_to_f32(ks16);
  const int64_t dst_row = slot * hkv + h;            // (block, row, head) flattened
  const float rks = __builtin_amdgcn_rcpf(ks);
#pragma unroll
  for (int e = 0; e < E; ++e) k_cache[dst_row * D + lane * E + e] = (int8_t)k8_code(k[e], ks, rks);
  if (lane == 0) k_scale[dst_row] = ks16;

  // ---- V: asymmetric 4-bit per group of 32 (32 / E lanes per group)
  constexpr int GL = 32 / E;                          // lanes per group: 32 or 16
  float mn = v[0], mx = v[0];
#pragma unroll
  for (int e = 1; e < E; ++e) { mn = fminf(mn, v[e]); mx = fmaxf(mx, v[e]); }
#pragma unroll
  for (int m = 1; m < GL; m <<= 1) {
    mn = fminf(mn, wave_xor(mn, m));
    mx = fmaxf(mx, wave_xor(mx, m));
  }
  const uint16_t vs16 = v4_scale_bits(mn, mx);
  const uint16_t vz16 = f32_to_f16_bits(mn);
  const float vs = f16_bits_to_f32(vs16), vz = f16_bits_to_f32(vz16);
  uint32_t code[E];
  const float rvs = __builtin_amdgcn_rcpf(vs);
#pragma unroll
  for (int e = 0; e < E; ++e) code[e] = v4_code(v[e], vs, rvs, vz);
  if constexpr (E == 2) {
    v_cache[dst_row * (D / 2) + lane] = (uint8_t)(code[0] | (code[1] << 4));
  } else {
    const uint32_t hi = (uint32_t)__shfl_down((int)code[0], 1, kWave);
    if ((lane & 1) == 0) v_cache[dst_row * (D / 2) + lane / 2] = (uint8_t)(code[0] | (hi << 4));
  }
  if ((lane % GL) == 0) {
    const int grp = lane / GL;
    v_scale[dst_row * (D / 32) + grp] = vs16;
    v_zero[dst_row * (D / 32) + grp] = vz16;
  }
}

hipError_t launch_kv_write_k8v4(const void* key, const void* value, int in_dtype, int8_t* k_cache,
                                void* k_scale, uint8_t* v_cache, void* v_scale, void* v_zero,
                                const int64_t* slots, int64_t num_tokens, int num_kv_heads,
                                int head_dim, int64_t num_blocks, hipStream_t stream) {
  const int64_t units = num_tokens * num_kv_heads;
  const dim3 grid((unsigned)((units + 3) / 4)), block(256);
  const int64_t ns = num_blocks * kBlock;
#define PKV_K8V4_LAUNCH(IN, D)                                                               \
  hipLaunchKernelGGL((kv_write_k8v4_kernel<IN, D>), grid, block, 0, stream,                 \
                     (const uint16_t*)key, (const uint16_t*)value, k_cache, (uint16_t*)k_scale, \
                     v_cache, (uint16_t*)v_scale, (uint16_t*)v_zero, slots, num_tokens,      \
                     num_kv_heads, ns)
  const bool f16 = in_dtype == (int)Fmt::F16;
  if (head_dim == 64) {
    if (f16) PKV_K8V4_LAUNCH(Fmt::F16, 64); else PKV_K8V4_LAUNCH(Fmt::BF16, 64);
  } else {
    if (f16) PKV_K8V4_LAUNCH(Fmt::F16, 128); else PKV_K8V4_LAUNCH(Fmt::BF16, 128);
  }
#undef PKV_K8V4_LAUNCH
  return hipGetLastError();
}

}  // namespace pkv

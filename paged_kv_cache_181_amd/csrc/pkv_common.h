// Internal helpers shared by the HIP kernels of the paged-KV library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kBlock = 16;     // tokens per cache block
constexpr int kWave = 64;      // CDNA wavefront width

enum class Fmt : int { F16 = 0, BF16 = 1, K8V4 = 3 };
enum class OutT : int { F16 = 0, BF16 = 1, F32 = 2 };

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float32 -> bfloat16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)x;   // v_cvt_f16_f32, round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// ---------------------------------------------------------------- K8/V4 quantization
//
// The arithmetic of the quantize-on-write, in one place for every kernel that
// stores K8/V4 rows ("How MTPLX Manages Memory Using Request-Sized Paged KV
// Cache", Quantization-Aware Memory Layout; the formulas are this library's
// reading): K per (token, head) symmetric int8 with an fp16 scale, V per group
// of 32 dims asymmetric 4-bit with fp16 scale and zero.  fp32 throughout, the
// divisions correctly rounded, ties of the rounding to even.

// fp16 bits of the K scale of a row whose largest magnitude is amax
__device__ __forceinline__ uint16_t k8_scale_bits(float amax) {
  return f32_to_f16_bits(__fdiv_rn(amax, 127.0f));
}
// rint(fdiv_rn(x, s)) (ties to even), with rs = the hardware reciprocal of s.
// x * rs is within 1.5 units in the last place of x / s, far below 2^-13 for
// the quotients met here (|x / s| < 300), so when it lies farther than 2^-13
// from a half-integer it rounds to the same integer as the correctly rounded
// quotient; otherwise the exact division decides.
__device__ __forceinline__ float rint_div(float x, float s, float rs) {
  const float q = x * rs;
  float c = rintf(q);
  if (fabsf(q - c) > 0.5f - 0x1p-13f) c = rintf(__fdiv_rn(x, s));
  return c;
}
// the code of k under the (fp16-exact) scale s (rs: its reciprocal, as above)
__device__ __forceinline__ int k8_code(float k, float s, float rs) {
  float c = 0.f;
  if (s != 0.f) c = fminf(fmaxf(rint_div(k, s, rs), -127.f), 127.f);
  return (int)c;
}
// fp16 bits of the V scale of a group spanning [mn, mx] (the zero is fp16(mn))
__device__ __forceinline__ uint16_t v4_scale_bits(float mn, float mx) {
  return f32_to_f16_bits(__fdiv_rn(mx - mn, 15.0f));
}
// the code of v under the (fp16-exact) scale s and zero z
__device__ __forceinline__ uint32_t v4_code(float v, float s, float rs, float z) {
  float c = 0.f;
  if (s != 0.f) c = fminf(fmaxf(rint_div(v - z, s, rs), 0.f), 15.f);
  return (uint32_t)c;
}

// ---------------------------------------------------------------- MFMA wrappers
//
// S^T = K . Q^T uses the 16x16x32 form (K tile rows = 16 tokens, reduction over
// 32 head dims per step).  O^T = V^T . P^T uses the 16x16x16 form (reduction
// over the 16 tokens of a block).  Lane l holds row (l % 16) of the A operand
// and column (l % 16) of the B operand; the result lane l holds rows
// 4*(l/16) .. 4*(l/16)+3 of column l % 16.

template <Fmt T> struct Mma;

template <> struct Mma<Fmt::F16> {
  static __device__ __forceinline__ f4 qk(u4 a, u4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a),
                                                  __builtin_bit_cast(h8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f4 pv(u2 a, u2 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4, a),
                                                 __builtin_bit_cast(h4, b), c, 0, 0, 0);
  }
  // p -> (hi, lo): hi = f16 of p rounded toward zero (one packed conversion
  // per pair), lo = f16_rne(p - hi), written straight into its half; the
  // difference is exact in fp32, so hi + lo carries ~21 bits of p.
  static __device__ __forceinline__ void split(const float p[4], u2& hi, u2& lo) {
    const h2 h01 = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(p[0], p[1]));
    const h2 h23 = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(p[2], p[3]));
    const h2 l01 = h2{(_Float16)(p[0] - (float)h01.x), (_Float16)(p[1] - (float)h01.y)};
    const h2 l23 = h2{(_Float16)(p[2] - (float)h23.x), (_Float16)(p[3] - (float)h23.y)};
    hi = u2{__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)};
    lo = u2{__builtin_bit_cast(uint32_t, l01), __builtin_bit_cast(uint32_t, l23)};
  }
};

template <> struct Mma<Fmt::BF16> {
  static __device__ __forceinline__ f4 qk(u4 a, u4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a),
                                                   __builtin_bit_cast(b8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f4 pv(u2 a, u2 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, a),
                                                     __builtin_bit_cast(s4, b), c, 0, 0, 0);
  }
  // hi = p truncated to bf16 (exact remainder), lo = bf16_rne(p - hi).
  static __device__ __forceinline__ void split(const float p[4], u2& hi, u2& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint32_t u = __float_as_uint(p[r]) & 0xffff0000u;
      h[r] = u >> 16;
      l[r] = f32_to_bf16_bits(p[r] - __uint_as_float(u));
    }
    hi = u2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
    lo = u2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
  }
};

// ---------------------------------------------------------------- wave helpers

__device__ __forceinline__ float wave_xor(float v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Keeps the compiler from reordering this wave's LDS accesses across a
// cross-lane exchange through LDS.  The hardware executes the LDS instructions
// of one wavefront in issue order, so no wait is needed, and none is emitted
// (a memory fence here would also wait for the global loads in flight).
__device__ __forceinline__ void wave_lds_fence() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ void store_out(void* out, OutT t, int64_t idx, float v) {
  if (t == OutT::F32) {
    reinterpret_cast<float*>(out)[idx] = v;
  } else if (t == OutT::F16) {
    reinterpret_cast<uint16_t*>(out)[idx] = f32_to_f16_bits(v);
  } else {
    reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16_bits(v);
  }
}

}  // namespace pkv

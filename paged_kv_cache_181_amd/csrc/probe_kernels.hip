// Read-only measurement probes (declared in include/pagedkv_probe.h): how fast
// one decode layer's K/V stream can be read on this GPU, as a plain streaming
// read and with the partition kernel's own paged lane addressing.  They load
// and XOR, nothing else.

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/pagedkv.h"
#include "../../include/pagedkv_probe.h"

namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
constexpr int kWave = 64;

thread_local char g_err[256] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int launched(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  g_err[0] = '\0';
  return PKV_OK;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

__device__ __forceinline__ uint32_t fold(u4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// ---------------------------------------------------------------- streaming read
//
// Workgroup i reads slice i of buffer (i < half ? buf0 : buf1).  Per round a
// wave reads DEPTH consecutive 1 KiB chunks; the next round's loads are issued
// before the current round's data is folded, so between DEPTH and 2 * DEPTH
// chunks per wave are in flight.
template <int NW, int DEPTH>
__global__ __launch_bounds__(NW * kWave) void stream_read_kernel(const char* buf0, const char* buf1,
                                                                 uint32_t slice, float* sink) {
  const int half = gridDim.x / 2;
  const int i = blockIdx.x;
  const char* base = (i < half ? buf0 : buf1) + (size_t)(i % half) * slice;
  const auto r = rsrc(base, slice);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  constexpr uint32_t kRound = NW * DEPTH * 1024;          // bytes per round of the workgroup
  const uint32_t rounds = slice / kRound;
  const uint32_t lo = (uint32_t)(w * DEPTH * 1024 + lane * 16);
  uint32_t acc = 0;
  u4 cur[DEPTH], nxt[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) cur[d] = load16(r, lo + d * 1024);
  for (uint32_t k = 0; k < rounds; ++k) {
    const uint32_t o = (k + 1) * kRound + lo;             // past the slice: reads zeros
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) nxt[d] = load16(r, o + d * 1024);
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) acc ^= fold(cur[d]);
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) cur[d] = nxt[d];
  }
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) acc ^= fold(cur[d]);
  for (int m = 1; m < kWave; m <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, kWave);
  if (lane == 0) sink[(size_t)blockIdx.x * NW + w] = __uint_as_float(acc);
}

// ---------------------------------------------------------------- paged read
//
// The partition kernel's addressing at head_dim 128 with 16-bit rows: lane l
// of a wave reads token rho = l % 16 and bytes 16 * (l / 16) + 64 m of the
// head's 256-byte row, m = 0..3, in K and in V.  A ring of DEPTH register
// sets: the loads of block j + DEPTH - 1 are issued before block j is folded.
struct PagedArgs {
  const char* k;
  const char* v;
  const int32_t* table;
  int64_t num_blocks;
  int hkv, part_blocks;
  float* sink;
};

template <int HP, int NW, int DEPTH>
__global__ __launch_bounds__(NW * kWave) void paged_read_kernel(PagedArgs a) {
  // (the launch's dynamic LDS only sets how many workgroups share a CU)
  constexpr int NWH = NW / HP;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hw = w / NWH, wh = w % NWH;
  const int g = blockIdx.y * HP + hw;
  const int per = a.part_blocks / NWH;
  const int w0 = blockIdx.x * a.part_blocks + wh * per;
  const int tbl = lane < per ? a.table[w0 + lane] : -1;
  const int rho = lane & 15, qd = lane >> 4;
  const uint32_t blk = (uint32_t)(16 * a.hkv * 128 * 2);  // bytes of one block, all heads
  const uint32_t lo = (uint32_t)(((rho * a.hkv + g) * 128 + 8 * qd) * 2);
  uint32_t acc = 0;
  u4 kr[DEPTH][4], vr[DEPTH][4];
  auto load = [&](int j, u4 (&kk)[4], u4 (&vv)[4]) {
    const int pb = __builtin_amdgcn_readlane(tbl, j & 63);
    const bool ok = j < per && pb >= 0 && (int64_t)pb < a.num_blocks;
    const int64_t base = (int64_t)(ok ? pb : 0) * blk;
    const auto rk = rsrc(a.k + base, ok ? blk : 0u);
    const auto rv = rsrc(a.v + base, ok ? blk : 0u);
#pragma unroll
    for (int m = 0; m < 4; ++m) kk[m] = load16(rk, lo + 64 * m);
#pragma unroll
    for (int m = 0; m < 4; ++m) vv[m] = load16(rv, lo + 64 * m);
  };
#pragma unroll
  for (int d = 0; d < DEPTH - 1; ++d) load(d, kr[d], vr[d]);
  for (int j0 = 0; j0 < per; j0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int j = j0 + d;
      const int fill = (d + DEPTH - 1) % DEPTH;           // the set of block j + DEPTH - 1
      load(j + DEPTH - 1, kr[fill], vr[fill]);
#pragma unroll
      for (int m = 0; m < 4; ++m) acc ^= fold(kr[d][m]) ^ fold(vr[d][m]);
    }
  }
  for (int m = 1; m < kWave; m <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, kWave);
  if (lane == 0)
    a.sink[((size_t)blockIdx.y * gridDim.x + blockIdx.x) * NW + w] = __uint_as_float(acc);
}

template <int HP, int NW>
void launch_paged_depth(const PagedArgs& a, dim3 grid, int depth, int lds, hipStream_t s) {
  const dim3 blk(NW * kWave);
  switch (depth) {
    case 1: hipLaunchKernelGGL((paged_read_kernel<HP, NW, 1>), grid, blk, lds, s, a); break;
    case 2: hipLaunchKernelGGL((paged_read_kernel<HP, NW, 2>), grid, blk, lds, s, a); break;
    case 3: hipLaunchKernelGGL((paged_read_kernel<HP, NW, 3>), grid, blk, lds, s, a); break;
    default:
      // four register sets at 16 waves per workgroup would not fit in the
      // registers (the entry point rejects it)
      if constexpr (NW < 16) hipLaunchKernelGGL((paged_read_kernel<HP, NW, 4>), grid, blk, lds, s, a);
      break;
  }
}

template <int HP>
void launch_paged_hp(const PagedArgs& a, dim3 grid, int waves, int depth, int lds, hipStream_t s) {
  if constexpr (HP <= 4) {
    if (waves == 4) { launch_paged_depth<HP, 4>(a, grid, depth, lds, s); return; }
  }
  if (waves == 8) { launch_paged_depth<HP, 8>(a, grid, depth, lds, s); return; }
  launch_paged_depth<HP, 16>(a, grid, depth, lds, s);
}

// ---------------------------------------------------------------- K8/V4 paged read
//
// The K8/V4 head-group form's addressing at head_dim 128: one wave per KV head,
// each walking every block of its workgroup's partition.  Lane l (token
// rho = l % 16, quarter qd = l / 16) loads 16 B at 16 qd and at 64 + 16 qd of
// token rho's 128-byte K code row, 16 B at 16 qd of its 64-byte V code row, the
// token's K scale (2 B) and its four V scales and four V zeros (8 B each), six
// loads per block as the attention kernel issues them.  A ring of DEPTH
// register sets as in paged_read_kernel.
struct K8Args {
  const char *k, *v, *ks, *vs, *vz;
  const int32_t* table;
  int64_t num_blocks;
  int hkv, part_blocks;
  float* sink;
};

struct K8Set {
  u4 k0, k1, v;
  uint32_t ks;
  uint32_t vs0, vs1, vz0, vz1;
};

template <int DEPTH>
__global__ __launch_bounds__(8 * kWave) void k8v4_read_kernel(K8Args a) {
  // (the launch's dynamic LDS only sets how many workgroups share a CU)
  const int lane = threadIdx.x & 63;
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // KV head
  const int per = a.part_blocks;
  const int w0 = blockIdx.x * per;
  const int tbl = lane < per ? a.table[w0 + lane] : -1;
  const int rho = lane & 15, qd = lane >> 4;
  const int row = rho * a.hkv + g;                                   // (token, head) row
  const uint32_t kblk = (uint32_t)(16 * a.hkv * 128), vblk = (uint32_t)(16 * a.hkv * 64);
  const uint32_t ksblk = (uint32_t)(16 * a.hkv * 2), vsblk = (uint32_t)(16 * a.hkv * 8);
  const uint32_t ko = (uint32_t)(row * 128 + 16 * qd), vo = (uint32_t)(row * 64 + 16 * qd);
  const uint32_t kso = (uint32_t)(row * 2), vso = (uint32_t)(row * 8);
  uint32_t acc = 0;
  K8Set set[DEPTH];
  auto load = [&](int j, K8Set& r) {
    const int pb = __builtin_amdgcn_readlane(tbl, j & 63);
    const bool ok = j < per && pb >= 0 && (int64_t)pb < a.num_blocks;
    const int64_t b = ok ? pb : 0;
    const auto rk = rsrc(a.k + b * kblk, ok ? kblk : 0u);
    const auto rv = rsrc(a.v + b * vblk, ok ? vblk : 0u);
    const auto rks = rsrc(a.ks + b * ksblk, ok ? ksblk : 0u);
    const auto rvs = rsrc(a.vs + b * vsblk, ok ? vsblk : 0u);
    const auto rvz = rsrc(a.vz + b * vsblk, ok ? vsblk : 0u);
    r.k0 = load16(rk, ko);
    r.k1 = load16(rk, ko + 64);
    r.v = load16(rv, vo);
    r.ks = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rks, (int)kso, 0, 0);
    const auto s2 = __builtin_amdgcn_raw_buffer_load_b64(rvs, (int)vso, 0, 0);
    const auto z2 = __builtin_amdgcn_raw_buffer_load_b64(rvz, (int)vso, 0, 0);
    r.vs0 = (uint32_t)s2[0];
    r.vs1 = (uint32_t)s2[1];
    r.vz0 = (uint32_t)z2[0];
    r.vz1 = (uint32_t)z2[1];
  };
#pragma unroll
  for (int d = 0; d < DEPTH - 1; ++d) load(d, set[d]);
  for (int j0 = 0; j0 < per; j0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int fill = (d + DEPTH - 1) % DEPTH;           // the set of block j0 + d + DEPTH - 1
      load(j0 + d + DEPTH - 1, set[fill]);
      const K8Set& r = set[d];
      acc ^= fold(r.k0) ^ fold(r.k1) ^ fold(r.v) ^ r.ks ^ r.vs0 ^ r.vs1 ^ r.vz0 ^ r.vz1;
    }
  }
  for (int m = 1; m < kWave; m <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, kWave);
  if (lane == 0) a.sink[(size_t)blockIdx.x * 8 + g] = __uint_as_float(acc);
}

template <int NW>
void launch_stream_nw(const char* b0, const char* b1, uint32_t slice, float* sink, int wgs,
                      int depth, hipStream_t s) {
  const dim3 grid((unsigned)wgs), blk(NW * kWave);
  switch (depth) {
    case 1: hipLaunchKernelGGL((stream_read_kernel<NW, 1>), grid, blk, 0, s, b0, b1, slice, sink); break;
    case 2: hipLaunchKernelGGL((stream_read_kernel<NW, 2>), grid, blk, 0, s, b0, b1, slice, sink); break;
    case 4: hipLaunchKernelGGL((stream_read_kernel<NW, 4>), grid, blk, 0, s, b0, b1, slice, sink); break;
    default: hipLaunchKernelGGL((stream_read_kernel<NW, 8>), grid, blk, 0, s, b0, b1, slice, sink); break;
  }
}

}  // namespace

extern "C" {

const char* pkv_probe_last_error(void) { return g_err; }

int pkv_probe_stream_read(const void* buf0, const void* buf1, size_t bytes_each, int workgroups,
                          int waves, int depth, float* sink, size_t sink_count, void* stream) {
  if (!buf0 || !buf1 || !sink) return fail(PKV_ERR_NULL, "a required pointer is NULL");
  if (waves != 4 && waves != 8 && waves != 16) return fail(PKV_ERR_UNSUPPORTED, "waves: 4, 8 or 16");
  if (depth != 1 && depth != 2 && depth != 4 && depth != 8)
    return fail(PKV_ERR_UNSUPPORTED, "depth: 1, 2, 4 or 8");
  if (workgroups < 2 || workgroups % 2 || workgroups > 65536)
    return fail(PKV_ERR_SHAPE, "workgroups must be even, 2 .. 65536");
  const size_t half = (size_t)workgroups / 2;
  const size_t round = (size_t)waves * depth * 1024;
  if (bytes_each == 0 || bytes_each % (half * round) || bytes_each / half > 0x7fffffffu)
    return fail(PKV_ERR_SHAPE, "bytes_each must be a positive multiple of workgroups/2 * waves * "
                               "depth KiB, with slices under 2 GiB");
  if (sink_count < (size_t)workgroups * waves) return fail(PKV_ERR_SHAPE, "sink too small");
  const uint32_t slice = (uint32_t)(bytes_each / half);
  const char* b0 = (const char*)buf0;
  const char* b1 = (const char*)buf1;
  hipStream_t s = (hipStream_t)stream;
  if (waves == 4) launch_stream_nw<4>(b0, b1, slice, sink, workgroups, depth, s);
  else if (waves == 8) launch_stream_nw<8>(b0, b1, slice, sink, workgroups, depth, s);
  else launch_stream_nw<16>(b0, b1, slice, sink, workgroups, depth, s);
  return launched("pkv_probe_stream_read");
}

int pkv_probe_paged_read(const void* k_cache, const void* v_cache, const int32_t* block_table,
                         int table_blocks, int64_t num_blocks, int num_kv_heads, int head_dim,
                         int heads_per_wg, int waves, int part_blocks, int depth, int lds_bytes,
                         float* sink, size_t sink_count, void* stream) {
  if (!k_cache || !v_cache || !block_table || !sink)
    return fail(PKV_ERR_NULL, "a required pointer is NULL");
  if (head_dim != 128) return fail(PKV_ERR_UNSUPPORTED, "head_dim must be 128");
  if (heads_per_wg != 1 && heads_per_wg != 2 && heads_per_wg != 4 && heads_per_wg != 8)
    return fail(PKV_ERR_UNSUPPORTED, "heads_per_wg: 1, 2, 4 or 8");
  if ((waves != 4 && waves != 8 && waves != 16) || waves % heads_per_wg)
    return fail(PKV_ERR_UNSUPPORTED, "waves: 4, 8 or 16, a multiple of heads_per_wg");
  if (depth < 1 || depth > (waves == 16 ? 3 : 4))
    return fail(PKV_ERR_UNSUPPORTED, "depth: 1 .. 4 (1 .. 3 at 16 waves)");
  if (num_kv_heads <= 0 || num_kv_heads % heads_per_wg || num_kv_heads > 64)
    return fail(PKV_ERR_SHAPE, "num_kv_heads must be a multiple of heads_per_wg, at most 64");
  if (table_blocks <= 0 || part_blocks <= 0 || table_blocks % part_blocks)
    return fail(PKV_ERR_SHAPE, "table_blocks must be a positive multiple of part_blocks");
  const int nwh = waves / heads_per_wg;
  if (part_blocks % nwh || part_blocks / nwh > 64)
    return fail(PKV_ERR_SHAPE, "part_blocks must split into runs of at most 64 blocks per wave");
  if (num_blocks <= 0 || num_blocks * 16 * num_kv_heads * 256 > ((int64_t)1 << 40))
    return fail(PKV_ERR_SHAPE, "num_blocks out of range");
  if (lds_bytes < 0 || lds_bytes > 160 * 1024) return fail(PKV_ERR_SHAPE, "lds_bytes: 0 .. 160 KiB");
  const dim3 grid((unsigned)(table_blocks / part_blocks), (unsigned)(num_kv_heads / heads_per_wg));
  if (sink_count < (size_t)grid.x * grid.y * waves) return fail(PKV_ERR_SHAPE, "sink too small");
  PagedArgs a{(const char*)k_cache, (const char*)v_cache, block_table, num_blocks, num_kv_heads,
              part_blocks, sink};
  hipStream_t s = (hipStream_t)stream;
  switch (heads_per_wg) {
    case 1: launch_paged_hp<1>(a, grid, waves, depth, lds_bytes, s); break;
    case 2: launch_paged_hp<2>(a, grid, waves, depth, lds_bytes, s); break;
    case 4: launch_paged_hp<4>(a, grid, waves, depth, lds_bytes, s); break;
    default: launch_paged_hp<8>(a, grid, waves, depth, lds_bytes, s); break;
  }
  return launched("pkv_probe_paged_read");
}

int pkv_probe_k8v4_read(const void* k_codes, const void* v_codes, const void* k_scale,
                        const void* v_scale, const void* v_zero, const int32_t* block_table,
                        int table_blocks, int64_t num_blocks, int num_kv_heads, int head_dim,
                        int part_blocks, int depth, int lds_bytes, float* sink, size_t sink_count,
                        void* stream) {
  if (!k_codes || !v_codes || !k_scale || !v_scale || !v_zero || !block_table || !sink)
    return fail(PKV_ERR_NULL, "a required pointer is NULL");
  if (head_dim != 128) return fail(PKV_ERR_UNSUPPORTED, "head_dim must be 128");
  if (num_kv_heads != 8) return fail(PKV_ERR_UNSUPPORTED, "num_kv_heads must be 8");
  if (depth < 1 || depth > 4) return fail(PKV_ERR_UNSUPPORTED, "depth: 1 .. 4");
  if (table_blocks <= 0 || part_blocks <= 0 || part_blocks > 64 || table_blocks % part_blocks)
    return fail(PKV_ERR_SHAPE, "table_blocks must be a positive multiple of part_blocks (1 .. 64)");
  if (num_blocks <= 0 || num_blocks * 16 * num_kv_heads * 128 > ((int64_t)1 << 40))
    return fail(PKV_ERR_SHAPE, "num_blocks out of range");
  if (lds_bytes < 0 || lds_bytes > 160 * 1024) return fail(PKV_ERR_SHAPE, "lds_bytes: 0 .. 160 KiB");
  const dim3 grid((unsigned)(table_blocks / part_blocks)), blk(8 * kWave);
  if (sink_count < (size_t)grid.x * 8) return fail(PKV_ERR_SHAPE, "sink too small");
  K8Args a{(const char*)k_codes, (const char*)v_codes, (const char*)k_scale, (const char*)v_scale,
           (const char*)v_zero, block_table, num_blocks, num_kv_heads, part_blocks, sink};
  hipStream_t s = (hipStream_t)stream;
  switch (depth) {
    case 1: hipLaunchKernelGGL((k8v4_read_kernel<1>), grid, blk, lds_bytes, s, a); break;
    case 2: hipLaunchKernelGGL((k8v4_read_kernel<2>), grid, blk, lds_bytes, s, a); break;
    case 3: hipLaunchKernelGGL((k8v4_read_kernel<3>), grid, blk, lds_bytes, s, a); break;
    default: hipLaunchKernelGGL((k8v4_read_kernel<4>), grid, blk, lds_bytes, s, a); break;
  }
  return launched("pkv_probe_k8v4_read");
}

}  // extern "C"

// Shared device helpers of the JSSA HIP library (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jssa {

constexpr int kWave = 64;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kPage = 16;

// Device-side view of a GQA cache descriptor (passed by value to kernels).
struct GqaDev {
  int B, Hq, Hkv, G, d, r, max_seq;
  int page_size, num_pages, max_pages;
  const int32_t* page_table;
  const int32_t* seq_lens;
};

__device__ __forceinline__ int seq_len(const GqaDev& g, int b) {
  if (!g.seq_lens) return g.max_seq;
  int t = g.seq_lens[b];
  return t < 0 ? 0 : (t > g.max_seq ? g.max_seq : t);
}

// Element offset of row (b, j, t) in a cache of row width `w`, or -1 when the
// token has no valid page.
__device__ __forceinline__ int64_t row_off(const GqaDev& g, int b, int j, int t, int w) {
  if (g.page_size == 0) return ((int64_t(b) * g.Hkv + j) * g.max_seq + t) * w;
  int pg = g.page_table[int64_t(b) * g.max_pages + (t >> 4)];
  if (pg < 0 || pg >= g.num_pages) return -1;
  return ((int64_t(pg) * g.Hkv + j) * kPage + (t & (kPage - 1))) * w;
}

// bf16 <-> fp32. A bf16 is the upper half of an fp32.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  return uint16_t((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Correctly rounded fp64 -> bf16 (nearest, ties to even) by bit arithmetic:
// round the fp64 significand at bit 45 and re-bias the exponent (1023 -> 127);
// magnitudes below 2^-126 become bf16 subnormals with quantum 2^-133.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  uint64_t u = uint64_t(__double_as_longlong(x));
  uint32_t sign = uint32_t(u >> 48) & 0x8000u;
  uint64_t a = u & 0x7fffffffffffffffull;
  if ((a >> 52) >= 897) {
    uint64_t r = (a + 0x00000fffffffffffull + ((a >> 45) & 1ull)) >> 45;
    int64_t rb = int64_t(r) - (int64_t(896) << 7);
    if (rb > 0x7f80) rb = 0x7f80;
    return uint16_t(sign | uint32_t(rb));
  }
  double m = __builtin_rint(__builtin_fabs(x) * 0x1p133);
  return uint16_t(sign | uint32_t(m));
}

// Cross-lane moves inside 16-lane rows (DPP).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
// Sum over the 16 lanes of a row; every lane receives the total.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<0xb1>(x);   // quad_perm [1,0,3,2]
  x += dpp_mov<0x4e>(x);   // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);  // row_half_mirror
  x += dpp_mov<0x140>(x);  // row_mirror
  return x;
}

// Reductions over the 64 lanes of a wave (every lane active), returned
// wave-uniform: DPP moves inside each 16-lane row, then the four rows'
// results read out of lanes 0, 16, 32 and 48.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return uint32_t(__builtin_amdgcn_mov_dpp(int(x), CTRL, 0xf, 0xf, false));
}
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t x, Op op) {
  x = op(x, dpp_u32<0xb1>(x));
  x = op(x, dpp_u32<0x4e>(x));
  x = op(x, dpp_u32<0x141>(x));
  x = op(x, dpp_u32<0x140>(x));
  const uint32_t a = uint32_t(__builtin_amdgcn_readlane(int(x), 0)), b = uint32_t(__builtin_amdgcn_readlane(int(x), 16));
  const uint32_t c = uint32_t(__builtin_amdgcn_readlane(int(x), 32)), d = uint32_t(__builtin_amdgcn_readlane(int(x), 48));
  return op(op(a, b), op(c, d));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  return wave_reduce_u32(x, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  return wave_reduce_u32(x, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
  return wave_reduce_u32(x, [](uint32_t a, uint32_t b) { return a + b; });
}

__device__ __forceinline__ float xor_max(float x, int m) { return fmaxf(x, __shfl_xor(x, m, kWave)); }

// Max and sum over the four 16-lane rows of a wave of a value that is
// uniform inside each row: four read-lanes, no LDS round trip. The sum is
// added as the xor-16 then xor-32 butterfly adds it, (row0 + row1) + (row2 +
// row3), so the result is bit-identical to it.
__device__ __forceinline__ float rows_max(float x) {
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ float rows_sum(float x) {
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return (r0 + r1) + (r2 + r3);
}
__device__ __forceinline__ float xor_sum(float x, int m) { return x + __shfl_xor(x, m, kWave); }

// Order-preserving map fp32 -> uint32 (larger score -> larger key); -0 == +0.
// Key 0 means "no token": -inf (the score of a position past the sequence
// or behind an invalid page) maps to it, as does the all-ones NaN that
// staging uses for such positions, so neither is ever selected. Finite
// scores map to keys >= 0x00800000.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0;
  const uint32_t key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return u == 0xff800000u ? 0u : key;
}

// Ordering fence for data exchanged through LDS between lanes of one wave.
__device__ __forceinline__ void wave_lds_sync() {
  // Fences limited to LDS ("local"): they order the wave's LDS accesses
  // without waiting for its global loads in flight.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (kWave - 1);
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace jssa

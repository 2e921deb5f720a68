// Projected key cache: Kp[t] = bf16_rne(K[t] . P_j), accumulated in fp64.
//
// JSSA scores candidates in a low-dimensional subspace shared by queries and
// keys (ai4snews digest, Synopsis). Keeping the keys' r-dim projection in the
// cache lets the score stage read 2r bytes per token instead of 2d. The
// projection runs once per appended token (decode) or once over a whole cache
// (set-up). fp64 accumulation makes every stored element the correctly
// rounded value of the exact product: each bf16 x fp32 product is exact in
// fp64 and 128 of them sum with ~2^-46 relative error, far below bf16's
// half-ulp.
#include "internal.hpp"

namespace jssa {
namespace {

constexpr int kTok = 64;     // tokens per block: 16 per wave
constexpr int kD = 128;      // head width
typedef double f64x4 __attribute__((ext_vector_type(4)));

// Kp tile (16 tokens x 16 columns) of one wave as fp64 matrix products:
// v_mfma_f64_16x16x4f64 takes A[m][k] from lane 16k + m, B[k][n] from lane
// 16k + n, and leaves D[k' + 4i][n] in register i of lane 16k' + n. The 128
// dims are split over the four k lanes as 32 steps: at step s, lane group
// kq covers dim 32*kq + s (the same dim order for A and B), so a lane's A
// values are its token's 32 consecutive dims, loaded as 64 contiguous bytes.
// Every product (bf16 x fp32) is exact in fp64 and the fp64 sums of 128 of
// them carry ~2^-46 relative error, far below half a bf16 ulp.
template <int R>
__global__ __launch_bounds__(256) void project_kernel(GqaDev g, const uint16_t* __restrict__ src,
                                                      const int32_t* __restrict__ pos, int n_tok,
                                                      int append, uint16_t* __restrict__ K,
                                                      uint16_t* __restrict__ V,
                                                      const uint16_t* __restrict__ vsrc,
                                                      const float* __restrict__ P,
                                                      uint16_t* __restrict__ Kp) {
  static_assert(R % 16 == 0, "columns in tiles of 16");
  __shared__ __attribute__((aligned(16))) float Ps[kD * R];

  const int b = blockIdx.z, j = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int m = lane & 15, kq = lane >> 4;
  const int Tb = seq_len(g, b);
  const int base = append ? pos[b] : 0;
  const int tok0 = blockIdx.x * kTok + 16 * w;         // first token (of the n_tok) of this wave

  for (int e = tid * 4; e < kD * R; e += 256 * 4)
    *reinterpret_cast<f32x4*>(Ps + e) = *reinterpret_cast<const f32x4*>(P + int64_t(j) * kD * R + e);

  // destination slot of token tok0 + r (r < 16), or -1
  auto slot = [&](int r) -> int {
    const int i = tok0 + r, t = base + i;
    const bool ok = i < n_tok && t >= 0 && t < g.max_seq && (append || t < Tb);
    return ok && row_off(g, b, j, t, kD) >= 0 ? t : -1;
  };
  // A operand source: dims 32*kq .. 32*kq+31 of token tok0 + m (zero if none)
  u32x4 kv[4] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
  {
    const int t = slot(m);
    if (t >= 0) {
      const int64_t off = row_off(g, b, j, t, kD) + 32 * kq;
      if (append) {
        const int64_t s = ((int64_t(b) * g.Hkv + j) * n_tok + tok0 + m) * kD + 32 * kq;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          kv[q] = reinterpret_cast<const u32x4*>(src + s)[q];
          reinterpret_cast<u32x4*>(K + off)[q] = kv[q];
          reinterpret_cast<u32x4*>(V + off)[q] = reinterpret_cast<const u32x4*>(vsrc + s)[q];
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) kv[q] = reinterpret_cast<const u32x4*>(src + off)[q];
      }
    }
  }
  __syncthreads();                                     // Ps complete

  int dst[4];                                          // tokens of this lane's D rows kq + 4i
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = slot(kq + 4 * i);
#pragma unroll 1
  for (int ct = 0; ct < R / 16; ++ct) {
    const float* pcol = Ps + (32 * kq) * R + 16 * ct + m;   // B: P[32*kq + s][16*ct + m]
    f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      const uint32_t wd = kv[s >> 3][(s >> 1) & 3];
      const double a = double(__uint_as_float((s & 1) ? (wd & 0xffff0000u) : (wd << 16)));
      const double bb = double(pcol[s * R]);
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bb, acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (dst[i] < 0) continue;
      Kp[row_off(g, b, j, dst[i], R) + 16 * ct + m] = f64_to_bf16_rne(acc[i]);
    }
  }
}

}  // namespace

hipError_t launch_project(const GqaDev& g, const uint16_t* src, int64_t, const int32_t* pos,
                          int n_tok, bool append, uint16_t* K, uint16_t* V, const uint16_t* v_src,
                          const float* P, uint16_t* Kp, hipStream_t st) {
  dim3 grid((n_tok + kTok - 1) / kTok, g.Hkv, g.B);
  switch (g.r) {
#define JSSA_CASE(R)                                                                          \
  case R:                                                                                     \
    hipLaunchKernelGGL(project_kernel<R>, grid, dim3(256), 0, st, g, src, pos, n_tok,         \
                       append ? 1 : 0, K, V, v_src, P, Kp);                                   \
    break;
    JSSA_CASE(16) JSSA_CASE(32) JSSA_CASE(48) JSSA_CASE(64) JSSA_CASE(128)
#undef JSSA_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace jssa

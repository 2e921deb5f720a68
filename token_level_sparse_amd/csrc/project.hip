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

constexpr int kTok = 64;     // tokens per block
constexpr int kD = 128;      // head width
constexpr int kKS = kTok + 4;  // row stride of the transposed key tile (16-byte aligned rows)

// Threads of a block: one per 4-token x 4-column output tile.
constexpr int project_threads(int r) { return (kTok / 4) * (r / 4); }

// A block projects kTok tokens of one (sequence, KV head). The tokens' keys
// are staged transposed (Kt[i][t], fp32: bf16 widens exactly) and P_j as
// fp32, so a thread computing 4 tokens x 4 columns reads 4 keys and 4
// weights of dim i with two 16-byte LDS reads per 16 fp64 FMAs. Every output
// is the same fp64 FMA chain over i = 0..127 as a plain dot product.
template <int R>
__global__ __launch_bounds__(project_threads(R)) void project_kernel(GqaDev g, const uint16_t* __restrict__ src,
                                                      const int32_t* __restrict__ pos, int n_tok,
                                                      int append, uint16_t* __restrict__ K,
                                                      uint16_t* __restrict__ V,
                                                      const uint16_t* __restrict__ vsrc,
                                                      const float* __restrict__ P,
                                                      uint16_t* __restrict__ Kp) {
  static_assert(R % 4 == 0, "columns in groups of 4");
  constexpr int kPT = project_threads(R);
  __shared__ __attribute__((aligned(16))) float Ps[kD * R];
  __shared__ __attribute__((aligned(16))) float Kt[kD * kKS];
  __shared__ int dst_row[kTok];       // destination token slot, or -1

  const int b = blockIdx.z, j = blockIdx.y;
  const int i0 = blockIdx.x * kTok;
  const int tid = threadIdx.x;
  const int Tb = seq_len(g, b);
  const int base = append ? pos[b] : 0;

  for (int e = tid * 4; e < kD * R; e += kPT * 4)
    *reinterpret_cast<f32x4*>(Ps + e) = *reinterpret_cast<const f32x4*>(P + int64_t(j) * kD * R + e);

  // 16 lanes per key row, 16 bytes (dims 8l .. 8l+7) per lane.
  for (int rr = tid >> 4; rr < kTok; rr += kPT / 16) {
    const int i = i0 + rr;
    const int t = base + i;
    bool ok = i < n_tok && t >= 0 && t < g.max_seq && (append || t < Tb);
    int64_t off = ok ? row_off(g, b, j, t, kD) : -1;
    if (off < 0) ok = false;
    const int lane = tid & 15;
    u32x4 kv = u32x4{0u, 0u, 0u, 0u};
    if (ok) {
      if (append) {
        const int64_t s = ((int64_t(b) * g.Hkv + j) * n_tok + i) * kD;
        kv = reinterpret_cast<const u32x4*>(src + s)[lane];
        const u32x4 vv = reinterpret_cast<const u32x4*>(vsrc + s)[lane];
        reinterpret_cast<u32x4*>(K + off)[lane] = kv;
        reinterpret_cast<u32x4*>(V + off)[lane] = vv;
      } else {
        kv = reinterpret_cast<const u32x4*>(src + off)[lane];
      }
    }
    const uint32_t w[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      Kt[(8 * lane + 2 * h) * kKS + rr] = __uint_as_float(w[h] << 16);
      Kt[(8 * lane + 2 * h + 1) * kKS + rr] = __uint_as_float(w[h] & 0xffff0000u);
    }
    if (lane == 0) dst_row[rr] = ok ? t : -1;
  }
  __syncthreads();

  constexpr int CG = R / 4;                       // column groups
  {
    const int tg = tid / CG, cg = tid - (tid / CG) * CG;
    double acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[a][c] = 0.0;
#pragma unroll 8
    for (int i = 0; i < kD; ++i) {
      const f32x4 kk = *reinterpret_cast<const f32x4*>(Kt + i * kKS + 4 * tg);
      const f32x4 pp = *reinterpret_cast<const f32x4*>(Ps + i * R + 4 * cg);
      const double kd[4] = {double(kk.x), double(kk.y), double(kk.z), double(kk.w)};
      const double pd[4] = {double(pp.x), double(pp.y), double(pp.z), double(pp.w)};
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[a][c] = __builtin_fma(kd[a], pd[c], acc[a][c]);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int t = dst_row[4 * tg + a];
      if (t < 0) continue;
      const int64_t off = row_off(g, b, j, t, R);
      if (off < 0) continue;
      const uint32_t lo = uint32_t(f64_to_bf16_rne(acc[a][0])) | (uint32_t(f64_to_bf16_rne(acc[a][1])) << 16);
      const uint32_t hi = uint32_t(f64_to_bf16_rne(acc[a][2])) | (uint32_t(f64_to_bf16_rne(acc[a][3])) << 16);
      *reinterpret_cast<uint2*>(Kp + off + 4 * cg) = uint2{lo, hi};
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
    hipLaunchKernelGGL(project_kernel<R>, grid, dim3(project_threads(R)), 0, st, g, src, pos, n_tok, \
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

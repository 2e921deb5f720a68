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

template <int R>
__global__ __launch_bounds__(256) void project_kernel(GqaDev g, const uint16_t* __restrict__ src,
                                                      const int32_t* __restrict__ pos, int n_tok,
                                                      int append, uint16_t* __restrict__ K,
                                                      uint16_t* __restrict__ V,
                                                      const uint16_t* __restrict__ vsrc,
                                                      const float* __restrict__ P,
                                                      uint16_t* __restrict__ Kp) {
  __shared__ float Ps[kD * R];
  __shared__ uint16_t Ks[kTok * kD];
  __shared__ int64_t dst_row[kTok];   // destination row index (token slot) or -1

  const int b = blockIdx.z, j = blockIdx.y;
  const int i0 = blockIdx.x * kTok;
  const int tid = threadIdx.x;
  const int Tb = seq_len(g, b);
  const int base = append ? pos[b] : 0;

  for (int e = tid; e < kD * R; e += 256) Ps[e] = P[int64_t(j) * kD * R + e];

  // 16 lanes per row, 16 bytes per lane.
  for (int rr = tid >> 4; rr < kTok; rr += 16) {
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
    reinterpret_cast<u32x4*>(Ks + rr * kD)[lane] = kv;
    if (lane == 0) dst_row[rr] = ok ? t : -1;
  }
  __syncthreads();

  for (int o = tid; o < kTok * R; o += 256) {
    const int ti = o / R, c = o - (o / R) * R;
    const int64_t t = dst_row[ti];
    if (t < 0) continue;
    double acc = 0.0;
#pragma unroll 16
    for (int i = 0; i < kD; ++i)
      acc = __builtin_fma(double(bf(Ks[ti * kD + i])), double(Ps[i * R + c]), acc);
    const int64_t off = row_off(g, b, j, int(t), R);
    if (off >= 0) Kp[off + c] = f64_to_bf16_rne(acc);
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
    hipLaunchKernelGGL(project_kernel<R>, grid, dim3(256), 0, st, g, src, pos, n_tok,        \
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

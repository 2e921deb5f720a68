// Subspace score stream: scores[b,j,t] = qp(b,j) . Kp[b,j,t,:].
//
// JSSA ranks candidate tokens in a low-dimensional space that holds queries
// and keys together (ai4snews digest, Synopsis and Interpretation). A KV
// head's score sums its G query heads' scores; by linearity that is one dot of
// qp = P_j^T (sum_h q_h) with the stored projected key, so the stream reads
// 2r bytes per token and does r FMAs.
//
// HBM-bound streaming kernel. Each wave reads a tile of 64 tokens' projected
// keys as 64*r/8 contiguous 16-byte pieces, one coalesced dwordx4 load per
// piece column (1 KB per wave instruction), so every load instruction covers
// whole cache lines. Lane l of load m holds piece m*64+l; its 8-element
// partial dot goes through LDS and lane t then sums the r/8 partials of token
// t and writes one fp32 score (a coalesced 256-byte store per wave). The next
// tile's loads are issued before the current tile is reduced.
#include "internal.hpp"

namespace jssa {
namespace {

constexpr int kD = 128;
constexpr int kWaves = 4;

template <int R>
struct ScoreShape {
  static constexpr int PP = R / 8;                 // 16-byte pieces per token
  static constexpr int M = PP;                     // loads per lane per 64-token tile
  static constexpr bool kUniformSlice = (64 % PP) == 0;
};

template <int R>
__global__ __launch_bounds__(256) void score_kernel(GqaDev g, const uint16_t* __restrict__ q,
                                                    const float* __restrict__ P,
                                                    const uint16_t* __restrict__ Kp,
                                                    float* __restrict__ scores, int tiles_per_wave) {
  using S = ScoreShape<R>;
  __shared__ float qbar[kD];
  __shared__ float qpart[256];
  __shared__ float qp[R];
  __shared__ float part[kWaves][64 * S::M];

  const int b = blockIdx.z, j = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int Tb = seq_len(g, b);

  // ---- prologue: qp = P_j^T sum_{h in group} q_h (fp32)
  if (tid < kD) {
    const uint16_t* qg = q + (int64_t(b) * g.Hq + int64_t(j) * g.G) * kD + tid;
    float s = 0.f;
    for (int h = 0; h < g.G; ++h) s += bf(qg[h * kD]);
    qbar[tid] = s;
  }
  __syncthreads();
  {
    constexpr int NS = 256 / R;          // i-slices per output column
    const int c = tid % R, sl = tid / R;
    if (sl < NS) {
      const float* Pj = P + int64_t(j) * kD * R;
      float s = 0.f;
      for (int i = sl; i < kD; i += NS) s = __builtin_fmaf(Pj[i * R + c], qbar[i], s);
      qpart[sl * R + c] = s;
    }
    __syncthreads();
    if (tid < R) {
      float s = 0.f;
      for (int k = 0; k < NS; ++k) s += qpart[k * R + tid];
      qp[tid] = s;
    }
    __syncthreads();
  }

  // per-load qp slices held in registers
  constexpr int NSL = S::kUniformSlice ? 1 : S::M;
  float qr[NSL][8];
#pragma unroll
  for (int m = 0; m < NSL; ++m) {
    const int sl = (m * 64 + lane) % S::PP;
#pragma unroll
    for (int e = 0; e < 8; ++e) qr[m][e] = qp[sl * 8 + e];
  }

  const int chunk = kWaves * 64 * tiles_per_wave;
  const int t_begin = blockIdx.x * chunk;
  float* srow = scores + (int64_t(b) * g.Hkv + j) * g.max_seq;
  const bool paged = g.page_size != 0;

  auto load_tile = [&](int tile, u32x4 (&buf)[S::M]) {
    const int t0 = t_begin + (tile * kWaves + w) * 64;
#pragma unroll
    for (int m = 0; m < S::M; ++m) {
      const int p = m * 64 + lane;
      const int t = t0 + p / S::PP;
      const int pc = p % S::PP;
      buf[m] = u32x4{0u, 0u, 0u, 0u};
      if (t < Tb) {
        if (!paged) {
          const u32x4* base = reinterpret_cast<const u32x4*>(
              Kp + ((int64_t(b) * g.Hkv + j) * g.max_seq + t0) * R);
          buf[m] = __builtin_nontemporal_load(base + p);
        } else {
          const int64_t off = row_off(g, b, j, t, R);
          if (off >= 0) buf[m] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Kp + off) + pc);
        }
      }
    }
  };

  u32x4 cur[S::M];
  load_tile(0, cur);
  for (int tile = 0; tile < tiles_per_wave; ++tile) {
    const int t0 = t_begin + (tile * kWaves + w) * 64;
    u32x4 nxt[S::M];
    if (tile + 1 < tiles_per_wave) load_tile(tile + 1, nxt);
#pragma unroll
    for (int m = 0; m < S::M; ++m) {
      const float* qs = qr[S::kUniformSlice ? 0 : m];
      const u32x4 v = cur[m];
      float a = 0.f;
      a = __builtin_fmaf(qs[0], bf_lo(v.x), a);
      a = __builtin_fmaf(qs[1], bf_hi(v.x), a);
      a = __builtin_fmaf(qs[2], bf_lo(v.y), a);
      a = __builtin_fmaf(qs[3], bf_hi(v.y), a);
      a = __builtin_fmaf(qs[4], bf_lo(v.z), a);
      a = __builtin_fmaf(qs[5], bf_hi(v.z), a);
      a = __builtin_fmaf(qs[6], bf_lo(v.w), a);
      a = __builtin_fmaf(qs[7], bf_hi(v.w), a);
      part[w][m * 64 + lane] = a;
    }
    wave_lds_sync();
    float s = 0.f;
#pragma unroll
    for (int pc = 0; pc < S::PP; ++pc) s += part[w][lane * S::PP + pc];
    wave_lds_sync();
    const int t = t0 + lane;
    if (t < g.max_seq) srow[t] = (t < Tb) ? s : -__builtin_inff();
    if (tile + 1 < tiles_per_wave) {
#pragma unroll
      for (int m = 0; m < S::M; ++m) cur[m] = nxt[m];
    }
  }
}

}  // namespace

hipError_t launch_score(const GqaDev& g, const uint16_t* q, const float* P, const uint16_t* Kp,
                        float* scores, hipStream_t st) {
  // Aim for about 8 blocks of 4 waves per CU over the whole grid; at least 4
  // tiles per wave so the prologue is amortised.
  const int64_t units = int64_t(g.B) * g.Hkv;
  const int64_t tiles_total = (g.max_seq + 63) / 64;
  int64_t want_blocks = 2048;
  int64_t tpw = (units * tiles_total + want_blocks * kWaves - 1) / (want_blocks * kWaves);
  if (tpw < 4) tpw = 4;
  if (tpw > 64) tpw = 64;
  const int64_t chunk = kWaves * 64 * tpw;
  dim3 grid(unsigned((g.max_seq + chunk - 1) / chunk), g.Hkv, g.B);
  switch (g.r) {
#define JSSA_CASE(R)                                                                             \
  case R:                                                                                        \
    hipLaunchKernelGGL(score_kernel<R>, grid, dim3(256), 0, st, g, q, P, Kp, scores, int(tpw)); \
    break;
    JSSA_CASE(16) JSSA_CASE(32) JSSA_CASE(48) JSSA_CASE(64) JSSA_CASE(128)
#undef JSSA_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace jssa

// Log-sum-exp combine of split partials, and the gather ablation copy.
//
// Combine: split-K decode produces per-split (o_s, lse_s); the exact softmax
// over the union of the splits weights each o_s by exp(lse_s - max lse).
// Gather: the common token-sparse implementation copies the selected K/V rows
// into a contiguous buffer and then runs a dense kernel; JSSA's digest
// (Interpretation) reports that this copy is comparable to the reduced
// attention itself. It is built here only to measure that ablation.
#include "internal.hpp"

namespace jssa {
namespace {

// A row (b, h) is handled by tpr = dv/4 threads (4 outputs each) times SG
// split groups: group sg weights splits sg, sg + SG, ..., with up to 8 of
// its loads in flight at a time, and the groups' sums are added in LDS in
// group order (deterministic). Several rows share a 256-thread block when
// tpr * SG < 256. Every thread first reads all S log-sum-exps of its row for
// the maximum (the same addresses across the row's threads).
__global__ __launch_bounds__(256) void combine_kernel(int rows, int S, int dv, int SG,
                                                      const float* __restrict__ part_o,
                                                      const float* __restrict__ part_lse,
                                                      void* __restrict__ out, int out_bf16,
                                                      float* __restrict__ lse_out) {
  __shared__ f32x4 red_o[256];
  __shared__ float red_l[256];
  const int tpr = dv / 4, tprow = tpr * SG;
  const int rpb = 256 / tprow;
  const int slot = threadIdx.x / tprow;                 // row of the block
  const int sg = (threadIdx.x / tpr) % SG, c4 = threadIdx.x % tpr;
  const int bh = blockIdx.x * rpb + slot;
  const bool live = slot < rpb && bh < rows;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f, M = -__builtin_inff();
  if (live) {
    const float* pl = part_lse + int64_t(bh) * S;
    for (int s0 = 0; s0 < S; s0 += 8) {
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = s0 + i < S ? pl[s0 + i] : -__builtin_inff();
#pragma unroll
      for (int i = 0; i < 8; ++i) M = fmaxf(M, x[i]);
    }
    if (M != -__builtin_inff()) {
      const f32x4* po = reinterpret_cast<const f32x4*>(part_o + int64_t(bh) * S * dv) + c4;
      for (int s0 = sg; s0 < S; s0 += 8 * SG) {
        f32x4 v[8];
        float wgt[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int s = s0 + i * SG;
          wgt[i] = s < S ? __expf(pl[s] - M) : 0.f;
          v[i] = (s < S && wgt[i] != 0.f) ? po[int64_t(s) * tpr] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          L += wgt[i];
          acc += wgt[i] * v[i];
        }
      }
    }
  }
  if (SG > 1) {                                         // block-uniform
    red_o[threadIdx.x] = acc;
    red_l[threadIdx.x] = L;
    __syncthreads();
    if (!live || sg != 0) return;
    const int r0 = slot * tprow;
    acc = red_o[r0 + c4];
    L = red_l[r0];
    for (int x = 1; x < SG; ++x) {
      acc += red_o[r0 + x * tpr + c4];
      L += red_l[r0 + x * tpr];
    }
  } else if (!live) {
    return;
  }
  if (L > 0.f) acc *= 1.f / L;
  if (out_bf16) {
    uint16_t* o = static_cast<uint16_t*>(out) + int64_t(bh) * dv + c4 * 4;
    u32x2 pk = {uint32_t(f32_to_bf16_rne(acc.x)) | (uint32_t(f32_to_bf16_rne(acc.y)) << 16),
                uint32_t(f32_to_bf16_rne(acc.z)) | (uint32_t(f32_to_bf16_rne(acc.w)) << 16)};
    *reinterpret_cast<u32x2*>(o) = pk;
  } else {
    reinterpret_cast<f32x4*>(static_cast<float*>(out) + int64_t(bh) * dv)[c4] = acc;
  }
  if (lse_out && c4 == 0) lse_out[bh] = L > 0.f ? M + __logf(L) : -__builtin_inff();
}

// One 16-lane group per selected row; 16 rows per 256-thread block.
__global__ __launch_bounds__(256) void gather_kernel(GqaDev g, const uint16_t* __restrict__ K,
                                                     const uint16_t* __restrict__ V,
                                                     const int32_t* __restrict__ idx, int k,
                                                     uint16_t* __restrict__ Kg,
                                                     uint16_t* __restrict__ Vg,
                                                     int32_t* __restrict__ lens_out) {
  const int b = blockIdx.z, j = blockIdx.y;
  const int i = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const int Tb = seq_len(g, b);
  if (lens_out && j == 0 && blockIdx.x == 0 && threadIdx.x == 0) lens_out[b] = min(k, Tb);
  if (i >= k) return;
  const int t = idx[(int64_t(b) * g.Hkv + j) * k + i];
  int64_t off = -1;
  if (t >= 0 && t < Tb) off = row_off(g, b, j, t, 128);
  u32x4 kv = u32x4{0u, 0u, 0u, 0u}, vv = u32x4{0u, 0u, 0u, 0u};
  if (off >= 0) {
    kv = reinterpret_cast<const u32x4*>(K + off)[sub];
    vv = reinterpret_cast<const u32x4*>(V + off)[sub];
  }
  const int64_t d = ((int64_t(b) * g.Hkv + j) * k + i) * 128;
  reinterpret_cast<u32x4*>(Kg + d)[sub] = kv;
  reinterpret_cast<u32x4*>(Vg + d)[sub] = vv;
}

}  // namespace

hipError_t launch_combine(int B, int H, int S, int dv, const float* part_o, const float* part_lse,
                          void* out, bool out_bf16, float* lse, hipStream_t st) {
  const int rows = B * H;
  const int tpr = dv / 4;
  if (tpr > 256 || tpr < 1 || S < 1) return hipErrorInvalidValue;
  // split groups per row: up to 8, as many as fit the block and the splits
  int SG = 256 / tpr;
  SG = SG < 8 ? SG : 8;
  SG = SG < S ? SG : S;
  const int rpb = 256 / (tpr * SG);
  hipLaunchKernelGGL(combine_kernel, dim3((rows + rpb - 1) / rpb), dim3(256), 0, st, rows, S, dv, SG, part_o,
                     part_lse, out, out_bf16 ? 1 : 0, lse);
  return hipGetLastError();
}

hipError_t launch_gather(const GqaDev& g, const uint16_t* K, const uint16_t* V, const int32_t* idx,
                         int k, uint16_t* Kg, uint16_t* Vg, int32_t* lens_out, hipStream_t st) {
  dim3 grid((k + 15) / 16, g.Hkv, g.B);
  hipLaunchKernelGGL(gather_kernel, grid, dim3(256), 0, st, g, K, V, idx, k, Kg, Vg, lens_out);
  return hipGetLastError();
}

}  // namespace jssa

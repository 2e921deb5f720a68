// Split-K decode attention over (a) the selected token set, read in place
// through its indices, and (b) every cached token (dense baseline).
//
// JSSA executes attention on the per-KV-head selected tokens with a
// gather-free kernel: the rows are read where they lie in the standard GQA
// cache through scattered indices instead of being copied to a contiguous
// buffer first (ai4snews digest, Interpretation; JSSA abstract). The full-KV
// variant is the baseline the method's decode speedup is measured against.
//
// Layout of the work: a block handles one (sequence b, KV head j, query-head
// group, split s). Inside a wave, 16 lanes cover one 128-dim row (16 bytes
// each), so one dwordx4 load instruction fetches 4 rows = 1 KB. A wave issues
// the K and V loads of STEPS x 4 rows before consuming any of them, computes
// all GT query heads' logits from each K row (one load serves the whole GQA
// group), and keeps an online softmax (running max m, sum l, output o) in
// fp32 in the log2 domain. Multi-wave blocks merge their waves in LDS.
// Outputs are per-split partials (o, lse); jssa_combine merges the splits.
#include "internal.hpp"
#include "attn_core.hpp"

namespace jssa {
namespace {

template <int GT, int STEPS, int NW, bool DENSE, bool PAGED>
__global__ __launch_bounds__(NW * 64) void attn_kernel(GqaDev g, const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ K,
                                                       const uint16_t* __restrict__ V,
                                                       const int32_t* __restrict__ idx, int k,
                                                       int S, float scale, float* __restrict__ part_o,
                                                       float* __restrict__ part_lse) {
  const int s = blockIdx.x;
  const int ngroups = (g.G + GT - 1) / GT;
  const int j = blockIdx.y / ngroups, hg = blockIdx.y % ngroups;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int Tb = seq_len(g, b);
  const int h0 = j * g.G + hg * GT;             // first global query head of this block
  const int nh = min(GT, g.G - hg * GT);        // valid heads in the group

  // rows [r0, r1) of this split
  int r0, r1;
  if (DENSE) {
    const int cs = (Tb + S - 1) / S;
    r0 = min(s * cs, Tb);
    r1 = min(r0 + cs, Tb);
  } else {
    const int cs = (k + S - 1) / S;
    r0 = min(s * cs, k);
    r1 = min(r0 + cs, k);
  }
  const int32_t* irow = DENSE ? nullptr : idx + (int64_t(b) * g.Hkv + j) * k;

  bf16x2 qv[GT][4];
  attn_load_q<GT>(qv, q, int64_t(b) * g.Hq + h0, nh, lane & 15);
  const float qs = scale * kAttnLog2e;
  AttnAcc<GT> A;
  attn_init(A);
  constexpr int RB = STEPS * 4;                 // rows per wave batch
  for (int base = r0 + w * RB; base < r1; base += NW * RB) {
    if constexpr (DENSE)
      attn_batch<GT, STEPS, PAGED>(g, b, j, Tb, K, V, qv, qs, base, r1, [](int rr) { return rr; }, A);
    else
      attn_batch<GT, STEPS, PAGED>(g, b, j, Tb, K, V, qv, qs, base, r1, [&](int rr) { return irow[rr]; }, A);
  }
  attn_wave_reduce(A);
  auto od = [&](int h) { return part_o + ((int64_t(b) * g.Hq + h0 + h) * S + s) * kAttnD; };
  auto ld = [&](int h) { return part_lse + (int64_t(b) * g.Hq + h0 + h) * S + s; };
  if constexpr (NW > 1) {
    __shared__ AttnMergeSmem<GT, NW> msm;
    attn_block_merge_store(A, msm, nh, od, ld);
  } else {
    attn_store(A, nh, od, ld);
  }
}

template <int GT, int STEPS, int NW, bool DENSE>
hipError_t launch_attn_t(const GqaDev& g, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                         const int32_t* idx, int k, int S, float scale, float* po, float* pl,
                         hipStream_t st) {
  const int ngroups = (g.G + GT - 1) / GT;
  dim3 grid(S, g.Hkv * ngroups, g.B);
  if (g.page_size)
    hipLaunchKernelGGL((attn_kernel<GT, STEPS, NW, DENSE, true>), grid, dim3(NW * 64), 0, st, g, q, K, V,
                       idx, k, S, scale, po, pl);
  else
    hipLaunchKernelGGL((attn_kernel<GT, STEPS, NW, DENSE, false>), grid, dim3(NW * 64), 0, st, g, q, K, V,
                       idx, k, S, scale, po, pl);
  return hipGetLastError();
}

template <bool DENSE, int NW>
hipError_t launch_attn_g(const GqaDev& g, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                         const int32_t* idx, int k, int S, float scale, float* po, float* pl,
                         hipStream_t st) {
  switch (g.G) {
    case 1: return launch_attn_t<1, 8, NW, DENSE>(g, q, K, V, idx, k, S, scale, po, pl, st);
    case 2: return launch_attn_t<2, 8, NW, DENSE>(g, q, K, V, idx, k, S, scale, po, pl, st);
    case 3: case 6: case 9: case 12: case 15:
      return launch_attn_t<3, 8, NW, DENSE>(g, q, K, V, idx, k, S, scale, po, pl, st);
    case 5: case 10:
      return launch_attn_t<5, 8, NW, DENSE>(g, q, K, V, idx, k, S, scale, po, pl, st);
    default:   // 4, 8, 16 and 7, 11, 13, 14: groups of up to 4 heads
      return launch_attn_t<4, 8, NW, DENSE>(g, q, K, V, idx, k, S, scale, po, pl, st);
  }
}

}  // namespace

hipError_t launch_indexed(const GqaDev& g, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                          const int32_t* idx, int k, int S, float scale, float* part_o,
                          float* part_lse, hipStream_t st) {
  // one wave per 32 rows of a split, up to 8 waves merged in LDS
  const int rows = (k + S - 1) / S;
  if (rows > 128) return launch_attn_g<false, 8>(g, q, K, V, idx, k, S, scale, part_o, part_lse, st);
  if (rows > 64) return launch_attn_g<false, 4>(g, q, K, V, idx, k, S, scale, part_o, part_lse, st);
  if (rows > 32) return launch_attn_g<false, 2>(g, q, K, V, idx, k, S, scale, part_o, part_lse, st);
  return launch_attn_g<false, 1>(g, q, K, V, idx, k, S, scale, part_o, part_lse, st);
}

hipError_t launch_dense(const GqaDev& g, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                        int S, float scale, float* part_o, float* part_lse, hipStream_t st) {
  return launch_attn_g<true, 4>(g, q, K, V, nullptr, 0, S, scale, part_o, part_lse, st);
}

}  // namespace jssa

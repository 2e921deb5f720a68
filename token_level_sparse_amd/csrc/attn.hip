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

namespace jssa {
namespace {

constexpr int kD = 128;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2e = 1.4426950408889634f;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Reinterpret one dword (two packed bf16) as a bf16 pair. Takes the dword by
// value: bit-casting a vector-element lvalue (v.y) directly reads element 0.
__device__ __forceinline__ bf16x2 as_pair(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

template <int GT, int STEPS, int NW, bool DENSE>
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
  const int gi = lane >> 4, sub = lane & 15;
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

  // query slice (dims sub*8..+8) of each head as bf16 pairs; logits use
  // v_dot2_f32_bf16 (exact bf16 products, fp32 sums) and are scaled into the
  // log2 domain after the row reduction
  bf16x2 qv[GT][4];
  const float qs = scale * kLog2e;
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (h < nh) v = *reinterpret_cast<const u32x4*>(q + (int64_t(b) * g.Hq + h0 + h) * kD + sub * 8);
    qv[h][0] = as_pair(v.x);
    qv[h][1] = as_pair(v.y);
    qv[h][2] = as_pair(v.z);
    qv[h][3] = as_pair(v.w);
  }

  float m[GT], l[GT], o[GT][8];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    m[h] = -__builtin_inff();
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
  }

  constexpr int RB = STEPS * 4;                 // rows per wave batch
  for (int base = r0 + w * RB; base < r1; base += NW * RB) {
    // Every load of the batch is issued without a data-dependent branch (a
    // load under one would be waited for before the next is issued): the
    // batch's indices, then (paged) their page ids, then the K and V rows.
    // Rows past the split or with no valid token read a valid row (token 0,
    // or page 0) and are masked out.
    u32x4 kr[STEPS], vr[STEPS];
    bool ok[STEPS];
    int tt[STEPS];
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int rr = base + st * 4 + gi;
      tt[st] = DENSE ? rr : irow[rr < r1 ? rr : r1 - 1];
    }
    int pg[STEPS];                              // page ids (paged cache), also loaded together
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int rr = base + st * 4 + gi;
      ok[st] = rr < r1 && tt[st] >= 0 && tt[st] < Tb;
      tt[st] = ok[st] ? tt[st] : 0;
      pg[st] = g.page_size ? g.page_table[int64_t(b) * g.max_pages + (tt[st] >> 4)] : 0;
    }
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      int64_t off;
      if (g.page_size) {
        ok[st] = ok[st] && pg[st] >= 0 && pg[st] < g.num_pages;
        off = ((int64_t(ok[st] ? pg[st] : 0) * g.Hkv + j) * kPage + (tt[st] & (kPage - 1))) * kD;
      } else {
        off = ((int64_t(b) * g.Hkv + j) * g.max_seq + tt[st]) * kD;
      }
      kr[st] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(K + off) + sub);
      vr[st] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(V + off) + sub);
    }
    float lg[STEPS][GT];
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const u32x4 v = kr[st];
      const bf16x2 k0 = as_pair(v.x), k1 = as_pair(v.y), k2 = as_pair(v.z), k3 = as_pair(v.w);
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        float a = __builtin_amdgcn_fdot2_f32_bf16(qv[h][0], k0, 0.f, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(qv[h][1], k1, a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(qv[h][2], k2, a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(qv[h][3], k3, a, false);
        a = row16_sum(a) * qs;
        lg[st][h] = ok[st] ? a : -__builtin_inff();
      }
    }
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      float mb = lg[0][h];
#pragma unroll
      for (int st = 1; st < STEPS; ++st) mb = fmaxf(mb, lg[st][h]);
      mb = xor_max(mb, 16);
      mb = xor_max(mb, 32);
      const float mn = fmaxf(m[h], mb);
      if (mn == -__builtin_inff()) continue;      // nothing valid yet (wave-uniform)
      const float alpha = __builtin_amdgcn_exp2f(m[h] - mn);
      m[h] = mn;
      float ls = 0.f;
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = o[h][e] * alpha;
#pragma unroll
      for (int st = 0; st < STEPS; ++st) {
        const float p = __builtin_amdgcn_exp2f(lg[st][h] - mn);
        ls += p;
        const u32x4 v = vr[st];
        acc[0] = __builtin_fmaf(p, bf_lo(v.x), acc[0]);
        acc[1] = __builtin_fmaf(p, bf_hi(v.x), acc[1]);
        acc[2] = __builtin_fmaf(p, bf_lo(v.y), acc[2]);
        acc[3] = __builtin_fmaf(p, bf_hi(v.y), acc[3]);
        acc[4] = __builtin_fmaf(p, bf_lo(v.z), acc[4]);
        acc[5] = __builtin_fmaf(p, bf_hi(v.z), acc[5]);
        acc[6] = __builtin_fmaf(p, bf_lo(v.w), acc[6]);
        acc[7] = __builtin_fmaf(p, bf_hi(v.w), acc[7]);
      }
      l[h] = l[h] * alpha + ls;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] = acc[e];
    }
  }

  // reduce the four 16-lane row groups of the wave
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    l[h] = xor_sum(xor_sum(l[h], 16), 32);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = xor_sum(xor_sum(o[h][e], 16), 32);
  }

  if constexpr (NW > 1) {
    __shared__ float sm_m[NW][GT], sm_l[NW][GT];
    __shared__ float sm_o[NW][GT][kD];
    if (lane < 16) {
#pragma unroll
      for (int h = 0; h < GT; ++h) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sm_o[w][h][sub * 8 + e] = o[h][e];
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < GT; ++h) { sm_m[w][h] = m[h]; sm_l[w][h] = l[h]; }
    }
    __syncthreads();
    if (w != 0) return;
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      float M = -__builtin_inff();
#pragma unroll
      for (int x = 0; x < NW; ++x) M = fmaxf(M, sm_m[x][h]);
      float L = 0.f, acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (M != -__builtin_inff()) {
#pragma unroll
        for (int x = 0; x < NW; ++x) {
          const float f = __builtin_amdgcn_exp2f(sm_m[x][h] - M);
          L += sm_l[x][h] * f;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += sm_o[x][h][sub * 8 + e] * f;
        }
      }
      m[h] = M;
      l[h] = L;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] = acc[e];
    }
  }

  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      if (h >= nh) break;
      const int64_t ob = ((int64_t(b) * g.Hq + h0 + h) * S + s);
      const float inv = l[h] > 0.f ? 1.f / l[h] : 0.f;
      f32x4 a = {o[h][0] * inv, o[h][1] * inv, o[h][2] * inv, o[h][3] * inv};
      f32x4 c = {o[h][4] * inv, o[h][5] * inv, o[h][6] * inv, o[h][7] * inv};
      f32x4* dst = reinterpret_cast<f32x4*>(part_o + ob * kD + sub * 8);
      dst[0] = a;
      dst[1] = c;
      if (sub == 0)
        part_lse[ob] = l[h] > 0.f ? (m[h] + __builtin_log2f(l[h])) * kLn2 : -__builtin_inff();
    }
  }
}

template <int GT, int STEPS, int NW, bool DENSE>
hipError_t launch_attn_t(const GqaDev& g, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                         const int32_t* idx, int k, int S, float scale, float* po, float* pl,
                         hipStream_t st) {
  const int ngroups = (g.G + GT - 1) / GT;
  dim3 grid(S, g.Hkv * ngroups, g.B);
  hipLaunchKernelGGL((attn_kernel<GT, STEPS, NW, DENSE>), grid, dim3(NW * 64), 0, st, g, q, K, V,
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

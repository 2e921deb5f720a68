// Building blocks of decode attention over rows of the GQA cache, shared by
// the split-K attention kernels and the fused select + attend kernel.
//
// Lane layout: inside a wave, 16 lanes (a row group, gi = lane/16) cover one
// 128-dim row, 16 bytes (dims sub*8 .. sub*8+7, sub = lane%16) each, so one
// dwordx4 load instruction fetches 4 rows = 1 KB. A batch is STEPS such
// loads of K and of V (4*STEPS rows), all issued before any is used. Every
// K row serves the GT query heads of its GQA group. The online softmax
// (running max m, sum l, output o) is fp32 in the log2 domain; m is kept
// uniform over the wave, l and o are per row group until attn_wave_reduce.
#pragma once
#include "common.hpp"

namespace jssa {

constexpr int kAttnD = 128;
constexpr float kAttnLn2 = 0.6931471805599453f;
constexpr float kAttnLog2e = 1.4426950408889634f;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Reinterpret one dword (two packed bf16) as a bf16 pair. Takes the dword by
// value: bit-casting a vector-element lvalue (v.y) directly reads element 0.
__device__ __forceinline__ bf16x2 as_pair(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

template <int GT>
struct AttnAcc {
  float m[GT], l[GT], o[GT][8];
};

template <int GT>
__device__ __forceinline__ void attn_init(AttnAcc<GT>& A) {
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    A.m[h] = -__builtin_inff();
    A.l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) A.o[h][e] = 0.f;
  }
}

// Query slice (dims sub*8..+8) of heads qrow0 .. qrow0+nh-1 (rows of q
// [.,128]) as bf16 pairs; heads past nh (>= 1) are zero. Logits use
// v_dot2_f32_bf16 (exact bf16 products, fp32 sums). The loads are
// unconditional (heads past nh re-read row qrow0 and are zeroed after), so
// none of them sits under a branch: a value merged from a branch would make
// the compiler wait for every load in flight at that point.
template <int GT>
__device__ __forceinline__ void attn_load_q(bf16x2 (&qv)[GT][4], const uint16_t* q, int64_t qrow0, int nh,
                                            int sub) {
  u32x4 v[GT];
#pragma unroll
  for (int h = 0; h < GT; ++h) v[h] = *reinterpret_cast<const u32x4*>(q + (qrow0 + (h < nh ? h : 0)) * kAttnD + sub * 8);
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    const u32x4 x = h < nh ? v[h] : u32x4{0u, 0u, 0u, 0u};
    qv[h][0] = as_pair(x.x);
    qv[h][1] = as_pair(x.y);
    qv[h][2] = as_pair(x.z);
    qv[h][3] = as_pair(x.w);
  }
}

// One batch of rows rr = base + st*4 + gi (st < STEPS) of the list [.., r1):
// tok(rr) gives the token of list row rr (called with rr < r1 only); tokens
// outside [0, Tb) or without a valid page are skipped. qs = scale * log2(e).
//
// Every load of the batch is issued without a data-dependent branch (a load
// under one would be waited for before the next is issued): the batch's
// tokens, then (PAGED: a paged cache, page_size 16) their page ids, then the
// K and V rows. Skipped rows read a valid row (token 0, or page 0) and are
// masked out.
template <int GT, int STEPS, bool PAGED, class TokFn>
__device__ __forceinline__ void attn_batch(const GqaDev& g, int b, int j, int Tb, const uint16_t* __restrict__ K,
                                           const uint16_t* __restrict__ V, const bf16x2 (&qv)[GT][4], float qs,
                                           int base, int r1, TokFn tok, AttnAcc<GT>& A) {
  const int lane = threadIdx.x & 63, gi = lane >> 4, sub = lane & 15;
  u32x4 kr[STEPS], vr[STEPS];
  bool ok[STEPS];
  int tt[STEPS];
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int rr = base + st * 4 + gi;
    tt[st] = tok(rr < r1 ? rr : r1 - 1);
  }
  int pg[STEPS];
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int rr = base + st * 4 + gi;
    ok[st] = rr < r1 && tt[st] >= 0 && tt[st] < Tb;
    tt[st] = ok[st] ? tt[st] : 0;
    if constexpr (PAGED) pg[st] = g.page_table[int64_t(b) * g.max_pages + (tt[st] >> 4)];
  }
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    int64_t off;
    if constexpr (PAGED) {
      ok[st] = ok[st] && pg[st] >= 0 && pg[st] < g.num_pages;
      off = ((int64_t(ok[st] ? pg[st] : 0) * g.Hkv + j) * kPage + (tt[st] & (kPage - 1))) * kAttnD;
    } else {
      off = ((int64_t(b) * g.Hkv + j) * g.max_seq + tt[st]) * kAttnD;
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
    mb = rows_max(mb);                          // (lg is uniform inside each 16-lane row)
    const float mn = fmaxf(A.m[h], mb);
    if (mn == -__builtin_inff()) continue;      // nothing valid yet (wave-uniform)
    const float alpha = __builtin_amdgcn_exp2f(A.m[h] - mn);
    A.m[h] = mn;
    float ls = 0.f;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = A.o[h][e] * alpha;
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
    A.l[h] = A.l[h] * alpha + ls;
#pragma unroll
    for (int e = 0; e < 8; ++e) A.o[h][e] = acc[e];
  }
}

// Sum l and o over the wave's four row groups (m is already wave-uniform).
template <int GT>
__device__ __forceinline__ void attn_wave_reduce(AttnAcc<GT>& A) {
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    A.l[h] = rows_sum(A.l[h]);                  // (l is uniform inside each 16-lane row)
#pragma unroll
    for (int e = 0; e < 8; ++e) A.o[h][e] = xor_sum(xor_sum(A.o[h][e], 16), 32);
  }
}

template <int GT, int NW>
struct __attribute__((aligned(16))) AttnMergeSmem {
  float m[NW][GT], l[NW][GT];
  float o[NW][GT][kAttnD];                      // at a 16-byte offset (8 NW GT bytes before it, NW >= 2)
};

// Merge the NW waves' (reduced) states through LDS and store the normalised
// outputs and lse of the block's first nh heads. The merge is spread over
// the block: thread i < nh * 32 takes head i / 32, dims 4 (i % 32) .. +3,
// and adds the waves in order 0 .. NW-1, each weighted by exp2(m_w - M)
// with M the largest m_w; then o / L and lse = (M + log2 L) ln 2. (With one
// wave walking every head and every wave's state in turn instead, blocks
// of 8 waves took 1.3 us more for 2 heads and 3.6 us more for 5.) Every
// thread of the block must call it.
template <int GT, int NW, class ODst, class LDst>
__device__ __forceinline__ void attn_block_merge_store(const AttnAcc<GT>& A, AttnMergeSmem<GT, NW>& sm, int nh,
                                                       ODst o_dst, LDst lse_dst) {
  static_assert(__builtin_offsetof(AttnMergeSmem<GT, NW>, o) % 16 == 0, "16-byte reads of the merged outputs");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, sub = lane & 15;
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.o[w][h][sub * 8 + e] = A.o[h][e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      sm.m[w][h] = A.m[h];
      sm.l[w][h] = A.l[h];
    }
  }
  __syncthreads();
  for (int i = tid; i < nh * 32; i += NW * 64) {
    const int h = i / 32, d = 4 * (i % 32);
    float M = -__builtin_inff();
#pragma unroll
    for (int x = 0; x < NW; ++x) M = fmaxf(M, sm.m[x][h]);
    float L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (M != -__builtin_inff()) {
#pragma unroll
      for (int x = 0; x < NW; ++x) {
        const float f = __builtin_amdgcn_exp2f(sm.m[x][h] - M);
        L += sm.l[x][h] * f;
        const f32x4 o = *reinterpret_cast<const f32x4*>(&sm.o[x][h][d]);
        acc.x += o.x * f;
        acc.y += o.y * f;
        acc.z += o.z * f;
        acc.w += o.w * f;
      }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    *reinterpret_cast<f32x4*>(o_dst(h) + d) = f32x4{acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
    if (d == 0) *lse_dst(h) = L > 0.f ? (M + __builtin_log2f(L)) * kAttnLn2 : -__builtin_inff();
  }
}

// Normalised output and lse of head h (h < nh) from lanes 0..15 of a wave
// holding a reduced state: o_dst(h) -> float* row of 128, lse_dst(h) -> float*.
template <int GT, class ODst, class LDst>
__device__ __forceinline__ void attn_store(const AttnAcc<GT>& A, int nh, ODst o_dst, LDst lse_dst) {
  const int lane = threadIdx.x & 63, sub = lane & 15;
  if (lane >= 16) return;
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    if (h >= nh) break;
    const float inv = A.l[h] > 0.f ? 1.f / A.l[h] : 0.f;
    f32x4 a = {A.o[h][0] * inv, A.o[h][1] * inv, A.o[h][2] * inv, A.o[h][3] * inv};
    f32x4 c = {A.o[h][4] * inv, A.o[h][5] * inv, A.o[h][6] * inv, A.o[h][7] * inv};
    f32x4* dst = reinterpret_cast<f32x4*>(o_dst(h) + sub * 8);
    dst[0] = a;
    dst[1] = c;
    if (sub == 0)
      *lse_dst(h) = A.l[h] > 0.f ? (A.m[h] + __builtin_log2f(A.l[h])) * kAttnLn2 : -__builtin_inff();
  }
}

}  // namespace jssa

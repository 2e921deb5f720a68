// A row's final top-k selection fused with the attention of its query heads
// over the selected tokens, read in place (one split).
//
// JSSA runs attention on each KV head's own selected tokens and reads them
// where they lie in the GQA cache, through their indices (ai4snews digest,
// Interpretation; JSSA abstract, Abstract). Here the selected indices go
// from the selection straight into the attention through LDS, without a
// round trip through memory or a second launch.
//
// One 512-thread block per (row, share of the row's query heads). The
// kernel is a chain of dependent latencies, so it is written for a short
// chain:
//  - every load it needs up front goes out at once: the segment summaries,
//    the candidates (segment s is read by NT/nseg threads at fixed slots,
//    16 per thread, which the launch guarantees covers a segment's
//    capacity), the pseudo-max slots of the top-delta rule, and the query
//    rows of the block's first head group;
//  - the row's candidate count and the bracket [lo, hi] of its k-th key
//    come from the segment summaries (wave reductions in DPP, one barrier);
//  - the threshold is found with 4096-bin histogram levels over the
//    bracket; both histograms of the first two levels are cleared up front,
//    and a bin of at most 64 keys is finished by one wave;
//  - block scans are DPP scans inside 16-lane rows, read-lane adds across
//    rows and one LDS exchange across waves (alternating buffers, so no
//    trailing barrier);
//  - the taken tokens (key above the threshold, and the lowest-indexed
//    ones equal to it) are placed in list order, which is ascending token
//    order, into LDS and, by the row's first block, into idx.
#include "internal.hpp"
#include "select.hpp"
#include "attn_core.hpp"

namespace jssa {
namespace {

constexpr int kNT = 512;
constexpr int kNW = kNT / 64;
constexpr int kEF = 16;                 // candidate slots per thread
constexpr int kBins = 4096;
constexpr int kBinsPT = kBins / kNT;    // bins per thread in a scan
constexpr int kSmallBin = 64;           // a bin this small is finished by one wave
constexpr int kMaxSel = 512;            // selected tokens held in LDS

// (wave_incl_scan, the DPP wave scan, comes from select.hpp)

template <int GT>
struct FaSmem {
  uint32_t hist[2][kBins];
  int wsum[2][kNW];
  uint32_t red[6][kNW];
  int res[2];
  uint32_t bin[kSmallBin];
  int nbin;
  int32_t sel[kMaxSel];
  AttnMergeSmem<GT, kNW> msm;
};

// Exclusive scan of v over the block (thread order); total in *tot. Uses
// wsum[par]: consecutive scans must alternate par (each scan's barrier then
// orders the previous reads of the other buffer).
template <int GT>
__device__ __forceinline__ int block_excl_scan(int v, FaSmem<GT>& sm, int par, int* tot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int inc = wave_incl_scan(v);
  if (lane == 63) sm.wsum[par][w] = inc;
  __syncthreads();
  int pre = 0, t = 0;
#pragma unroll
  for (int i = 0; i < kNW; ++i) {
    const int s = sm.wsum[par][i];
    pre += i < w ? s : 0;
    t += s;
  }
  *tot = t;
  return inc - v + pre;
}

struct FaArgs {
  GqaDev g;
  const uint16_t* q;
  const uint16_t* K;
  const uint16_t* V;
  float scale;
  float* out;
  float* lse;
  int32_t* idx;
  int k;
  int hs, hpb;                          // blocks per row, heads per block
  CandSegs segs;
  DeltaArgs dl;
};

template <int GT, bool PAGED>
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(2, 2))) void select_attend_kernel(FaArgs a) {
  __shared__ FaSmem<GT> sm;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const GqaDev& g = a.g;
  // A row's hs blocks sit 8 launch positions apart (one XCD, shared L2).
  int row, hsplit;
  {
    const int hs = a.hs, lin = blockIdx.x;
    if (hs > 1 && (gridDim.x / hs) % 8 == 0) {          // lin = (q*hs + hsplit)*8 + row % 8
      row = (lin / (8 * hs)) * 8 + lin % 8;
      hsplit = (lin / 8) % hs;
    } else {
      row = lin / hs;
      hsplit = lin % hs;
    }
  }
  const int b = row / g.Hkv, j = row % g.Hkv;
  const int Tb = seq_len(g, b);
  const int k = a.k, need = min(k, Tb);
  const CandSegs& segs = a.segs;
  const int nseg = segs.nseg;
  const int64_t seg0 = int64_t(row) * nseg;
  const uint32_t* gkey = segs.key + seg0 * segs.cap;
  const int32_t* gidx = segs.idx + seg0 * segs.cap;
  const SegInfo* ginfo = segs.info + seg0;
  const int hb0 = hsplit * a.hpb, hb1 = min(g.G, hb0 + a.hpb);   // this block's heads (of the group)

  // ---- loads, all issued before any is used
  const int TPS = kNT / nseg;                           // >= 1, TPS * kEF >= cap (launch condition)
  const int dseg = tid / TPS, dj = (tid % TPS) * kEF;
  const bool has_seg = dseg < nseg;
  const int ds = has_seg ? dseg : 0;
  const u32x4 dinfo = *reinterpret_cast<const u32x4*>(ginfo + ds);
  uint32_t rkey[kEF];
  int32_t ridx[kEF];
  {
    const int64_t o = int64_t(ds) * segs.cap;
#pragma unroll
    for (int e = 0; e < kEF; e += 4) {
      const int j0 = dj + e < segs.cap ? dj + e : segs.cap - 4;   // in the segment's slots
      const u32x4 kv = *reinterpret_cast<const u32x4*>(gkey + o + j0);
      const u32x4 iv = *reinterpret_cast<const u32x4*>(gidx + o + j0);
      rkey[e] = kv.x; rkey[e + 1] = kv.y; rkey[e + 2] = kv.z; rkey[e + 3] = kv.w;
      ridx[e] = int32_t(iv.x); ridx[e + 1] = int32_t(iv.y); ridx[e + 2] = int32_t(iv.z); ridx[e + 3] = int32_t(iv.w);
    }
  }
  // (unconditional load: without the top-delta rule it re-reads a segment
  // summary word, and the value is dropped)
  const bool delta = a.dl.pmax != nullptr;
  const uint32_t* pmp = delta ? a.dl.pmax + int64_t(row) * a.dl.nseg0 + (tid < a.dl.nseg0 ? tid : 0)
                              : reinterpret_cast<const uint32_t*>(ginfo);
  uint32_t pm = *pmp;
  pm = delta && tid < a.dl.nseg0 ? pm : 0u;
  bf16x2 qv[GT][4];                                     // the first head group's query rows
  attn_load_q<GT>(qv, a.q, int64_t(b) * g.Hq + j * g.G + hb0, min(GT, hb1 - hb0), lane & 15);
  // both histograms of the first two levels, cleared while the loads fly
#pragma unroll
  for (int i = 0; i < 2 * kBins / kNT; i += 4)
    *reinterpret_cast<u32x4*>(&sm.hist[0][0] + (tid * (2 * kBins / kNT) + i)) = u32x4{0u, 0u, 0u, 0u};
  if (tid == 0) sm.nbin = 0;

  // ---- the row's candidate count and the bracket of its k-th key
  const bool lead = has_seg && dj == 0;                 // one thread per segment
  const uint32_t cnt_s = dinfo.x;
  {
    const uint32_t n_ = wave_sum_u32(lead ? cnt_s : 0u);
    const uint32_t f_ = wave_max_u32(lead ? dinfo.y : 0u);
    const uint32_t t_ = wave_max_u32(lead ? dinfo.z : 0u);
    const uint32_t u_ = wave_min_u32(lead ? dinfo.w : 0xffffffffu);
    const uint32_t p_ = wave_max_u32(pm);
    if (lane == 0) {
      sm.red[0][wv] = n_;
      sm.red[1][wv] = f_;
      sm.red[2][wv] = t_;
      sm.red[3][wv] = u_;
      sm.red[4][wv] = p_;
    }
  }
  __syncthreads();
  int n = 0;
  uint32_t lo = 0u, hi = 0u, lbot = 0xffffffffu;
  pm = 0u;
#pragma unroll
  for (int i = 0; i < kNW; ++i) {
    n += int(sm.red[0][i]);
    lo = sm.red[1][i] > lo ? sm.red[1][i] : lo;
    hi = sm.red[2][i] > hi ? sm.red[2][i] : hi;
    lbot = sm.red[3][i] < lbot ? sm.red[3][i] : lbot;
    pm = sm.red[4][i] > pm ? sm.red[4][i] : pm;
  }
  lo = lbot > lo ? lbot : lo;                           // at or below the need-th largest key
  uint32_t thr_key = 0u;                                // top-delta filter (0: none)
  if (a.dl.pmax && pm != 0u) thr_key = score_key(key_score(pm) - a.dl.thr_off);
  {
    const int c = has_seg ? int(cnt_s) : 0;
#pragma unroll
    for (int e = 0; e < kEF; ++e)
      if (dj + e >= c) ridx[e] = -1;
  }

  // ---- threshold: take key > tkey, and the first trem candidates (lowest
  // token indices) whose key equals tkey
  uint32_t tkey = 0u;
  int trem = 0x7fffffff;
  int par = 0;
  if (n > need && need > 0) {                           // block-uniform
    uint32_t blo = lo, bhi = hi;
    int rem = need;
    for (int level = 0;; ++level) {
      uint32_t* hist = sm.hist[level & 1];
      const uint32_t range = bhi - blo;
      const int sh = range < uint32_t(kBins) ? 0 : (32 - __builtin_clz(range)) - 12;
      if (level >= 2) {                                 // (rare) a third level reuses the first histogram
        for (int i = tid; i < kBins; i += kNT) hist[i] = 0u;
        if (tid == 0) sm.nbin = 0;
        __syncthreads();
      }
#pragma unroll
      for (int e = 0; e < kEF; ++e)
        if (ridx[e] >= 0 && rkey[e] >= blo && rkey[e] <= bhi) atomicAdd(&hist[(rkey[e] - blo) >> sh], 1u);
      __syncthreads();
      // the bin D holding the rem-th largest key: this thread's bins, from the top down
      uint32_t hb[kBinsPT];
      {
        const int top = kBins - 1 - tid * kBinsPT;       // bins top .. top - kBinsPT + 1
        const u32x4 x0 = *reinterpret_cast<const u32x4*>(hist + top - 7);
        const u32x4 x1 = *reinterpret_cast<const u32x4*>(hist + top - 3);
        hb[0] = x1.w; hb[1] = x1.z; hb[2] = x1.y; hb[3] = x1.x;
        hb[4] = x0.w; hb[5] = x0.z; hb[6] = x0.y; hb[7] = x0.x;
      }
      int mine = 0;
#pragma unroll
      for (int i = 0; i < kBinsPT; ++i) mine += int(hb[i]);
      int tot;
      int before = block_excl_scan(mine, sm, par, &tot);
      par ^= 1;
#pragma unroll
      for (int i = 0; i < kBinsPT; ++i) {
        if (before < rem && before + int(hb[i]) >= rem) {
          sm.res[0] = kBins - 1 - tid * kBinsPT - i;
          sm.res[1] = before;
        }
        before += int(hb[i]);
      }
      __syncthreads();
      const uint32_t D = uint32_t(sm.res[0]);
      rem -= sm.res[1];
      const int cnt = int(hist[D]);
      const uint32_t bl = blo + (D << sh);               // D < 2^12, sh <= 20: no overflow
      if (cnt == rem) {                                 // the whole bin is taken
        tkey = bl;
        break;
      }
      if (sh == 0) {                                    // a single key value, tied
        tkey = bl;
        trem = rem;
        break;
      }
      if (cnt <= kSmallBin) {                           // few keys: one wave ranks them exactly
#pragma unroll
        for (int e = 0; e < kEF; ++e)
          if (ridx[e] >= 0 && rkey[e] >= blo && rkey[e] <= bhi && ((rkey[e] - blo) >> sh) == D)
            sm.bin[atomicAdd(&sm.nbin, 1)] = rkey[e];
        __syncthreads();
        if (wv == 0) {
          const uint32_t mk = lane < cnt ? sm.bin[lane] : 0u;
          int gt = 0, eq = 0;                          // keys of the bin above / equal to this lane's
          for (int i = 0; i < cnt; ++i) {
            const uint32_t x = uint32_t(__builtin_amdgcn_readlane(int(mk), i));
            gt += x > mk ? 1 : 0;
            eq += x == mk ? 1 : 0;
          }
          // the rem-th largest key v of the bin: gt < rem <= gt + eq; take
          // the rem - gt first of the keys equal to v (all of them: no ranking)
          if (lane < cnt && gt < rem && rem <= gt + eq) {
            sm.res[0] = int(mk);
            sm.res[1] = rem - gt == eq ? 0x7fffffff : rem - gt;
          }
        }
        __syncthreads();
        tkey = uint32_t(sm.res[0]);
        trem = sm.res[1];
        break;
      }
      const uint32_t wid = (1u << sh) - 1u;
      blo = bl;
      bhi = bhi - bl > wid ? bl + wid : bhi;
    }
  }

  // ---- emit in list order (ascending token order)
  int tr = 0;
  if (trem != 0x7fffffff) {                             // tied candidates ranked only when some are left out
    int nt = 0;
#pragma unroll
    for (int e = 0; e < kEF; ++e) nt += (ridx[e] >= 0 && rkey[e] == tkey) ? 1 : 0;
    int tt;
    tr = block_excl_scan(nt, sm, par, &tt);
    par ^= 1;
  }
  uint32_t take = 0u;
#pragma unroll
  for (int e = 0; e < kEF; ++e) {
    bool t = false;
    if (ridx[e] >= 0) {
      if (rkey[e] > tkey) t = true;
      else if (rkey[e] == tkey) t = tr++ < trem;
    }
    t = t && rkey[e] >= thr_key;
    take |= t ? 1u << e : 0u;
  }
  int cnt_sel;
  int at = block_excl_scan(__builtin_popcount(take), sm, par, &cnt_sel);
#pragma unroll
  for (int e = 0; e < kEF; ++e)
    if (take >> e & 1u) sm.sel[at++] = ridx[e];
  __syncthreads();                                      // sel complete

  // ---- attention of the block's heads over the selected rows
  constexpr int STEPS = 8, RB = STEPS * 4;
  const float qs = a.scale * kAttnLog2e;
  for (int hl = hb0; hl < hb1; hl += GT) {
    const int h0 = j * g.G + hl, nh = min(GT, hb1 - hl);
    if (hl != hb0) attn_load_q<GT>(qv, a.q, int64_t(b) * g.Hq + h0, nh, lane & 15);
    AttnAcc<GT> A;
    attn_init(A);
    for (int base = wv * RB; base < cnt_sel; base += kNW * RB)
      attn_batch<GT, STEPS, PAGED>(g, b, j, Tb, a.K, a.V, qv, qs, base, cnt_sel, [&](int rr) { return sm.sel[rr]; }, A);
    attn_wave_reduce(A);
    attn_block_merge_store(A, sm.msm, nh, [&](int h) { return a.out + (int64_t(b) * g.Hq + h0 + h) * kAttnD; },
                           [&](int h) { return a.lse + int64_t(b) * g.Hq + h0 + h; });
    if (hl + GT < hb1) __syncthreads();                 // msm is reused by the next head group
  }
  // The indices leave last, coalesced from LDS: a store issued before the
  // attention's row loads would hold up their completion (a wave's memory
  // operations complete in issue order).
  if (hsplit == 0) {
    int32_t* dst = a.idx + int64_t(row) * k;
    for (int i = tid; i < k; i += kNT) dst[i] = i < cnt_sel ? sm.sel[i] : -1;
    if (a.dl.counts && tid == 0) a.dl.counts[row] = cnt_sel;
  }
}

}  // namespace

bool select_attend_fused(const CandSegs& segs, int k, int G) {
  return segs.nseg >= 1 && segs.nseg <= kNT && (kNT / segs.nseg) * kEF >= segs.cap && segs.cap % 4 == 0 &&
         k <= kMaxSel && G <= 16;
}

hipError_t launch_select_attend(const GqaDev& g, int k, CandSegs segs, const uint16_t* q, const uint16_t* K,
                                const uint16_t* V, float scale, int32_t* idx, float* out, float* lse,
                                hipStream_t st, DeltaArgs dl) {
  if (!select_attend_fused(segs, k, g.G)) return hipErrorInvalidValue;
  const int rows = g.B * g.Hkv;
  // Spread the row's query heads over hs blocks until the launch covers the
  // CUs (256 blocks); the selection is repeated per block, the attention
  // (the larger part) is split.
  int hs = 1;
  while (rows * hs < 256 && hs < g.G) ++hs;
  const int hpb = (g.G + hs - 1) / hs;
  hs = (g.G + hpb - 1) / hpb;
  const FaArgs fa{g, q, K, V, scale, out, lse, idx, k, hs, hpb, segs, dl};
  // query heads per pass over the selected rows: all of the block's heads
  // when they are 1, 2 or 5 (or 10, 15), else 4 at a time
  const int gt = hpb <= 2 ? hpb : (hpb % 5 == 0 ? 5 : 4);
#define JSSA_SA(GT)                                                                                      \
  do {                                                                                                   \
    if (g.page_size)                                                                                     \
      hipLaunchKernelGGL((select_attend_kernel<GT, true>), dim3(rows * hs), dim3(kNT), 0, st, fa);        \
    else                                                                                                 \
      hipLaunchKernelGGL((select_attend_kernel<GT, false>), dim3(rows * hs), dim3(kNT), 0, st, fa);       \
  } while (0)
  switch (gt) {
    case 1: JSSA_SA(1); break;
    case 2: JSSA_SA(2); break;
    case 5: JSSA_SA(5); break;
    default: JSSA_SA(4); break;
  }
#undef JSSA_SA
  return hipGetLastError();
}

}  // namespace jssa

// Block-level building blocks of the top-k selection (shared by the
// standalone top-k and the fused score + select kernel).
//
// Keys are order-preserving uint32 images of fp32 scores (score_key). A
// chunk keeps every token whose key is at or above a threshold at or below
// the chunk's own k-th largest key (found with at most two LDS histogram
// levels): any token below it has at least k better tokens in the same chunk
// and cannot be among the row's k best. The kept tokens and their keys go to
// the chunk's segment of a workspace; a per-row final pass resolves the exact
// threshold.
#pragma once
#include "common.hpp"

namespace jssa {

constexpr int kSelBins = 2048;

// Summary of one candidate segment, written by its producer beside the list
// (one 16-byte store) and read by the row's final pass together with the
// candidates, so that the final pass needs no reduction over the candidates
// to bracket the row's k-th key.
struct SegInfo {
  int32_t cnt;     // candidates in the segment (at most cap)
  uint32_t floor;  // a key with at least k of the segment's candidates at or above it; 0: none known
  uint32_t top;    // at or above every candidate key (0 when empty)
  uint32_t bot;    // at or below every candidate key (0xffffffff when empty)
};

// Segmented candidate lists: segment (row, s) holds info[row*nseg+s].cnt
// entries at key/idx + (row*nseg+s)*cap, in ascending token order.
struct CandSegs {
  SegInfo* info;
  uint32_t* key;
  int32_t* idx;
  int nseg, cap;
};

// Slots per segment for a budget k: a chunk keeps at most this many
// candidates (at most 2k through the top-two bound, else k plus the slack of
// the histogram select; a chunk whose kept set would exceed it resolves its
// k-th key exactly and keeps exactly k). Never more than the chunk length.
__host__ __device__ inline int seg_cap(int k, int chunk_len) {
  int c = 2 * k > k + 64 ? 2 * k : k + 64;
  c = (c + 3) & ~3;
  return c < chunk_len ? c : chunk_len;
}

__device__ __forceinline__ void write_info(const CandSegs& out, int64_t seg, int cnt, uint32_t floor, uint32_t top,
                                           uint32_t bot) {
  *reinterpret_cast<u32x4*>(out.info + seg) = u32x4{uint32_t(cnt), floor, top, bot};
}

template <int NT>
struct ScanSmem {
  int sc[NT / 64];
};

// Inclusive scan over the 64 lanes of a wave: DPP shifts inside each 16-lane
// row (no LDS round trip), then the totals of the rows before, read out of
// lanes 15, 31 and 47.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// Inclusive scan over the NT threads of the block; total in *tot.
template <int NT>
__device__ __forceinline__ int block_scan(int v, ScanSmem<NT>& s, int* tot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_incl_scan(v);
  if (lane == 63) s.sc[w] = v;
  __syncthreads();
  int pre = 0, t = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const int x = s.sc[i];
    pre += i < w ? x : 0;
    t += x;
  }
  __syncthreads();
  *tot = t;
  return v + pre;
}

// Over a histogram of NT*BPT bins, the bin D such that fewer than `need`
// counted items come before D in scan order and at least `need` come before
// or in D. desc scans from the top bin down (largest keys first), otherwise
// from bin 0 up. Result: res[0] = D, res[1] = items before D. Every thread
// must call it; res is valid after the call.
template <int NT, int BPT>
__device__ __forceinline__ void pick_bin(const uint32_t* h, int need, bool desc, ScanSmem<NT>& s,
                                         int* res) {
  const int tid = threadIdx.x;
  int loc[BPT];
  int mine = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    const int pos = tid * BPT + i;
    loc[i] = int(h[desc ? (NT * BPT - 1 - pos) : pos]);
    mine += loc[i];
  }
  int tot;
  int before = block_scan<NT>(mine, s, &tot) - mine;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    if (before < need && before + loc[i] >= need) {
      const int pos = tid * BPT + i;
      res[0] = desc ? (NT * BPT - 1 - pos) : pos;
      res[1] = before;
    }
    before += loc[i];
  }
  __syncthreads();
}

template <int NT, int E>
struct ChunkSmem {
  uint32_t hist[kSelBins];
  ScanSmem<NT> scan;
  uint32_t red[5][NT / 64];
  int res[2];
};

// Extra candidates a chunk may keep in its threshold bin before a second,
// finer histogram level pays for itself (they only cost the final pass work;
// callers whose final pass is the bottleneck pass a smaller slack).
constexpr int kSelSlack = 32;

// Chunk-local selection. Each thread holds E keys; key e of thread tid is
// token base + tid*E + e, a real token iff it is below `lim`. n = number of
// real tokens in the block (block-uniform). Writes the kept (key, index)
// pairs to segment `seg`, in ascending token order, and its count; every
// real token whose key is at or above the chunk's k-th largest key is kept.
//
// The histogram is adaptive: its 2048 bins split [lo, hi] linearly in key
// space, so one level usually brackets the k-th key to a few candidates. lo
// is the best of the cheap lower bounds on the chunk's k-th key that apply:
//  - in a full chunk with k <= NT, the smallest per-thread maximum (each of
//    the NT threads holds a key at or above it);
//  - in a full chunk with k <= 2*64*NW, the smallest over the NW waves of the
//    wave's r-th largest per-thread second maximum, r = ceil(k / (2*NW)):
//    each wave then has r threads holding two keys at or above it;
//  - otherwise the smallest real key.
template <int NT, int E>
__device__ void chunk_select(const uint32_t (&key)[E], int base, int lim, int n, int k, ChunkSmem<NT, E>& sm,
                             CandSegs out, int64_t seg, int slack = kSelSlack) {
  static_assert(E <= 32, "one mask bit per key");
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // key 0 (no token: past the row, behind an invalid page, or a dropped
  // tile of a screened chunk) takes no part in the bounds or the
  // histograms; thousands of them in one bin would serialize its atomics.
  // Every caller gives positions at or past lim the key 0 as well. The
  // candidates (real tokens with a key) are one bit each of cmask, built
  // without branches: per-key branches would cost exec-mask changes and
  // spilled lane masks for every key.
  const int nreal = lim - (base + tid * E);      // keys e < nreal are real tokens
  uint32_t cmask = 0u;
  uint32_t m1 = 0u, m2 = 0u, tmin = 0xffffffffu;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool c = e < nreal && key[e] != 0u;
    cmask |= c ? (1u << e) : 0u;
    const uint32_t x = c ? key[e] : 0u;          // (0: no effect on m1, m2)
    m2 = x > m1 ? m1 : (x > m2 ? x : m2);
    m1 = x > m1 ? x : m1;
    tmin = c && x < tmin ? x : tmin;
  }
  auto cand = [&](int e) { return ((cmask >> e) & 1u) != 0u; };
  uint32_t nc = uint32_t(__builtin_popcount(cmask));
  const bool keep_all = n <= k;
  const bool full = n == NT * E;
  uint32_t thr = 0;                          // keep real keys >= thr
  uint32_t bound2 = 0u;                      // the wave's r-th largest m2 (0: not usable)
  const int r = (k + 2 * NW - 1) / (2 * NW);
  if (!keep_all && full && r <= 64) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = bound2 | (1u << bit);
      if (__popcll(__ballot(m2 >= c)) >= r) bound2 = c;
    }
  }
  // (DPP inside rows, read-lanes across them: no LDS round trips)
  const uint32_t mx = wave_max_u32(m1), mnmx = wave_min_u32(m1), mn = wave_min_u32(tmin);
  nc = wave_sum_u32(nc);
  if (lane == 0) {
    sm.red[0][wv] = mx;
    sm.red[1][wv] = mnmx;
    sm.red[2][wv] = mn;
    sm.red[3][wv] = bound2;
    sm.red[4][wv] = nc;
  }
  if (!keep_all)
    for (int i = tid; i < kSelBins; i += NT) sm.hist[i] = 0u;
  __syncthreads();
  uint32_t hi = sm.red[0][0], lo_full = sm.red[1][0], lo_any = sm.red[2][0], lo2 = sm.red[3][0];
  uint32_t ncand = sm.red[4][0];
#pragma unroll
  for (int i = 1; i < NW; ++i) {
    hi = sm.red[0][i] > hi ? sm.red[0][i] : hi;
    lo_full = sm.red[1][i] < lo_full ? sm.red[1][i] : lo_full;
    lo_any = sm.red[2][i] < lo_any ? sm.red[2][i] : lo_any;
    lo2 = sm.red[3][i] < lo2 ? sm.red[3][i] : lo2;
    ncand += sm.red[4][i];
  }
  // at most k candidates (absent tokens and keys under a row floor do not
  // count): every one of them is kept, no threshold to find
  if (!keep_all && int(ncand) > k) {
    uint32_t lo = lo_any;
    if (full && k <= NT) lo = lo_full > lo ? lo_full : lo;
    if (full && r <= 64) lo = lo2 > lo ? lo2 : lo;
    const uint32_t range = hi - lo;
    const int sh0 = range < uint32_t(kSelBins) ? 0 : (32 - __builtin_clz(range)) - 11;
    // fewer than k candidates (a screened chunk): no bin reaches k, and the
    // threshold stays lo, the smallest candidate key, so all of them stay
    if (tid == 0) {
      sm.res[0] = 0;
      sm.res[1] = 0;
    }
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (cand(e) && key[e] >= lo) atomicAdd(&sm.hist[(key[e] - lo) >> sh0], 1u);
    __syncthreads();
    pick_bin<NT, kSelBins / NT>(sm.hist, k, true, sm.scan, sm.res);
    const uint32_t d0 = uint32_t(sm.res[0]);
    const int need = k - sm.res[1];
    const int cnt0 = int(sm.hist[d0]);
    thr = lo + (d0 << sh0);
    __syncthreads();
    if (sh0 > 0 && cnt0 - need > slack) {              // block-uniform
      const int sh1 = sh0 > 11 ? sh0 - 11 : 0;
      for (int i = tid; i < kSelBins; i += NT) sm.hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (cand(e) && key[e] >= thr && ((key[e] - lo) >> sh0) == d0)
          atomicAdd(&sm.hist[(key[e] - thr) >> sh1], 1u);
      __syncthreads();
      pick_bin<NT, kSelBins / NT>(sm.hist, need, true, sm.scan, sm.res);
      thr += uint32_t(sm.res[0]) << sh1;
      __syncthreads();                                 // (the histogram is reused below)
    }
  }
  // The kept set: every candidate at or above thr, one bit per key.
  uint32_t take = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) take |= (cand(e) && key[e] >= thr) ? (1u << e) : 0u;
  int tot;
  int at = block_scan<NT>(__builtin_popcount(take), sm.scan, &tot) - __builtin_popcount(take);
  uint32_t floor = 0u, bot = thr > lo_any ? thr : lo_any;
  if (tot > out.cap) {
    // More than the segment holds (long runs of equal or nearly equal keys):
    // resolve the chunk's k-th key K exactly, by further histogram levels
    // over the bracket [thr, hi] that holds it, and keep exactly k tokens:
    // every key above K and the lowest-indexed tokens equal to K. Tokens of
    // the chunk outside these are outranked by k of its own tokens and
    // cannot be among the row's k best. (tot > cap >= k: K >= thr.)
    uint32_t elo = thr, ehi = hi;                       // 32-bit bracket: keys compare as 32-bit
    int rem = k, trem = 0x7fffffff;
    uint32_t tkey = thr;
    for (;;) {
      const uint32_t range = ehi - elo;
      const int sh = range < uint32_t(kSelBins) ? 0 : (32 - __builtin_clz(range)) - 11;
      for (int i = tid; i < kSelBins; i += NT) sm.hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int e = 0; e < E; ++e)                       // (elo >= 1: key 0, no token, is never counted)
        if (key[e] >= elo && key[e] <= ehi) atomicAdd(&sm.hist[(key[e] - elo) >> sh], 1u);
      __syncthreads();
      pick_bin<NT, kSelBins / NT>(sm.hist, rem, true, sm.scan, sm.res);
      const uint32_t D = uint32_t(sm.res[0]);
      rem -= sm.res[1];
      const int cnt = int(sm.hist[D]);
      __syncthreads();
      const uint32_t blo = elo + (D << sh);                  // D < 2^11, sh <= 21: no overflow
      if (cnt == rem) { tkey = blo; break; }                 // the whole bin is taken
      if (sh == 0) { tkey = blo; trem = rem; break; }        // one key value, tied
      const uint32_t wid = (1u << sh) - 1u;
      elo = blo;
      ehi = ehi - blo > wid ? blo + wid : ehi;
    }
    int nt = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) nt += key[e] == tkey ? 1 : 0;   // (tkey >= 1)
    int ttot;
    int tr = block_scan<NT>(nt, sm.scan, &ttot) - nt;       // ties before this thread's, in token order
    take = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      bool t = key[e] > tkey;
      if (key[e] == tkey) t = tr++ < trem;
      take |= t ? (1u << e) : 0u;
    }
    at = block_scan<NT>(__builtin_popcount(take), sm.scan, &tot) - __builtin_popcount(take);
    floor = tkey;
    bot = tkey;
  } else if (tot >= k) {
    floor = bot;                                        // >= k candidates at or above thr and lo_any
  }
  // Compaction in token order: a thread's tokens are consecutive, so one
  // block scan of the per-thread counts places every kept key. The kept
  // pairs are gathered in LDS (over the histogram, which is no longer read)
  // and leave as coalesced stores; more than fit go out directly.
  uint32_t* okey = out.key + seg * out.cap;
  int32_t* oidx = out.idx + seg * out.cap;
  constexpr int kStaged = kSelBins / 2;
  const bool staged = tot <= kStaged;                  // block-uniform
  uint32_t* skey = sm.hist;
  int32_t* sidx = reinterpret_cast<int32_t*>(sm.hist + kStaged);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if ((take >> e) & 1u) {
      if (staged) {
        skey[at] = key[e];
        sidx[at] = base + tid * E + e;
      } else {
        okey[at] = key[e];
        oidx[at] = base + tid * E + e;
      }
      ++at;
    }
  }
  if (staged) {
    __syncthreads();
    for (int i = tid; i < tot; i += NT) {
      okey[i] = skey[i];
      oidx[i] = sidx[i];
    }
  }
  if (tid == 0) write_info(out, seg, tot, floor, hi, tot > 0 ? bot : 0xffffffffu);
}

constexpr int kTop2Bins = 256;

template <int NT>
struct Top2Smem {
  uint32_t hist[kTop2Bins];
  ScanSmem<NT> scan;
  uint32_t red[2][NT / 64];
  int res[2];
};

// Chunk-local selection for a full chunk (every one of the NT*E tokens real)
// with k <= NT, whose keys also stay readable in LDS: key e of thread tid is
// score_key(stage[e * SS + tid]), token base + tid*E + e. Same contract as
// chunk_select, with a cheaper threshold.
//
// Let M be the multiset of every thread's two largest keys (2*NT values).
// Any c with at least k values of M at or above it is at or below the
// chunk's k-th largest key, since the values of M are distinct tokens'
// keys. c is taken as the lower edge of the bin, in a linear histogram of M
// over [min M, max M], that holds M's k-th largest value: two LDS atomics
// per thread instead of a pass over all keys. Tokens above the chunk's k-th
// key that M misses (a thread's third best and lower) are the only ones that
// make c looser than the exact k-th key, and there are few: for Gaussian
// scores, k = 256 and 8192 tokens, about 295 keys are kept on average.
//
// The kept keys are marked in a per-thread bit mask; a thread then visits
// only its set bits, re-reading each key from LDS, instead of running a
// divergent branch for every key.
//
// The bound assumes the chunk's best tokens are spread over many threads.
// When they cluster (neighbouring tokens alike: a thread's 32 consecutive
// tokens all near the top), M misses most of them and c falls far below the
// k-th key. Then more than 2k keys pass; the function writes nothing and
// returns false (block-uniform), and the caller runs chunk_select on the
// same keys instead.
template <int NT, int E>
__device__ bool chunk_select_top2(const uint32_t (&key)[E], int base, int k, Top2Smem<NT>& sm,
                                  const float* stage, int SS, CandSegs out, int64_t seg) {
  static_assert(E <= 32, "one mask bit per key");
  static_assert(kTop2Bins == NT, "one histogram bin per thread");
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint32_t m1 = 0u, m2 = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t x = key[e];
    const uint32_t y = x < m1 ? x : m1;
    m2 = y > m2 ? y : m2;
    m1 = x > m1 ? x : m1;
  }
  uint32_t hi = wave_max_u32(m1), lo = wave_min_u32(m2);   // (DPP: no LDS round trips)
  if (lane == 0) {
    sm.red[0][wv] = hi;
    sm.red[1][wv] = lo;
  }
  sm.hist[tid] = 0u;
  __syncthreads();
  hi = sm.red[0][0];
  lo = sm.red[1][0];
#pragma unroll
  for (int i = 1; i < NW; ++i) {
    hi = sm.red[0][i] > hi ? sm.red[0][i] : hi;
    lo = sm.red[1][i] < lo ? sm.red[1][i] : lo;
  }
  const uint32_t range = hi - lo;                 // M lies in [lo, hi]
  const int sh = range < uint32_t(kTop2Bins) ? 0 : (32 - __builtin_clz(range)) - 8;
  atomicAdd(&sm.hist[(m1 - lo) >> sh], 1u);
  atomicAdd(&sm.hist[(m2 - lo) >> sh], 1u);
  __syncthreads();
  pick_bin<NT, 1>(sm.hist, k, true, sm.scan, sm.res);
  const uint32_t c = lo + (uint32_t(sm.res[0]) << sh);

  uint32_t mask = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) mask |= (key[e] >= c && key[e] != 0u) ? (1u << e) : 0u;   // key 0: no token
  const int mine = __builtin_popcount(mask);
  int tot;
  int at = block_scan<NT>(mine, sm.scan, &tot) - mine;
  if (tot > 2 * k) return false;
  uint32_t* okey = out.key + seg * out.cap;
  int32_t* oidx = out.idx + seg * out.cap;
  while (mask) {
    const int e = __builtin_ctz(mask);
    mask &= mask - 1u;
    okey[at] = score_key(stage[e * SS + tid]);
    oidx[at] = base + tid * E + e;
    ++at;
  }
  // at least k keys of M (distinct tokens) are at or above c, and all are kept
  if (tid == 0) write_info(out, seg, tot, c, hi, tot > 0 ? c : 0xffffffffu);
  return true;
}

// Top-delta filter of a row's final selection (Faster Than Flash review on
// evolve.pub, Summary and FAQ: a token stays when its log-weight is no more
// than delta below a stand-in for the maximum taken over the first and the
// most recent tokens). pmax[row * nseg0 + s]
// is the largest score key of the row's sink or local tokens in segment s
// (0: none there); the row's pseudo-max m is their maximum, and a selected
// token stays only if its score is >= m - thr_off (thr_off = delta * G /
// scale: the group-mean logit within delta of the pseudo-max's). Tokens
// with a -inf score (no valid page) never stay. Because the kept set is an
// upper set of scores, filtering the top-k selection gives exactly the
// top-k of the kept set. counts[row] receives the number kept. pmax ==
// nullptr: no filter.
struct DeltaArgs {
  const uint32_t* pmax;
  int nseg0;
  float thr_off;
  int32_t* counts;
};

// Inverse of score_key.
__device__ __forceinline__ float key_score(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
  return __uint_as_float(u);
}

// Per-row final selection over candidate segments (merging groups of
// segments first when a row's list is long). merge_ws: merge_workspace_bytes.
size_t merge_workspace_bytes(int rows, int nseg, int k);
hipError_t launch_select_final(int rows, int H, int max_seq, const int32_t* seq_lens, int k, CandSegs segs,
                               int32_t* idx, void* merge_ws, hipStream_t st, DeltaArgs dl = DeltaArgs{});
// Final selection fused with the attention of each row's query heads over the
// selected tokens (one split; final_attend.hip), when select_attend_fused
// holds: every segment fits the fused kernel's direct layout, k <= 512 and
// G <= 16.
bool select_attend_fused(const CandSegs& segs, int k, int G);
hipError_t launch_select_attend(const GqaDev& g, int k, CandSegs segs, const uint16_t* q, const uint16_t* K,
                                const uint16_t* V, float scale, int32_t* idx, float* out, float* lse,
                                hipStream_t st, DeltaArgs dl = DeltaArgs{});

}  // namespace jssa

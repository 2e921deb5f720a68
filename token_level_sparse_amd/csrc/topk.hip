// Per-(sequence, head) top-k with lowest-index ties.
//
// JSSA keeps a distinct selected token set for each KV head (JSSA abstract;
// ai4snews digest, Synopsis). The result is the first min(k, T_b) tokens of
// the total order (score descending, index ascending), listed ascending.
//
// Radix selection over order-preserving uint32 keys, two kernels, no global
// atomics (same-address atomics serialise across the XCDs):
//  chunk   one 256-thread block per 8192 scores of a row (32 per thread)
//          keeps every token at or above a bound on the chunk's own k-th key
//          (chunk_select_top2 for full chunks with k <= 256, else
//          chunk_select: a token below that key cannot be in the row's top-k)
//          and writes them to the chunk's workspace segment.
//  final   one block per row loads the row's candidate list (its segments
//          in order, which is ascending token order) into registers, finds
//          the exact threshold key with adaptive LDS histogram levels (each
//          splits the current key bracket into 4096 linear bins), and writes
//          the taken tokens in list order: every key above the threshold,
//          and the lowest-index tokens of a tied threshold key.
// Every decision depends only on keys and indices, so the result does not
// depend on scheduling. Rows whose candidate count exceeds the register
// capacity re-read their segments at each level (slower, same result).
#include "internal.hpp"
#include "select.hpp"
#include "attn_core.hpp"

namespace jssa {
namespace {

constexpr int kCT = 256;              // threads of the chunk kernel
constexpr int kCE = 32;               // scores per thread
constexpr int kChunk = kCT * kCE;     // 8192
constexpr int kFinBits = 12;
constexpr int kFinBins = 1 << kFinBits;
constexpr int kMaxSeg = 4096;

__device__ __forceinline__ int row_len(int max_seq, const int32_t* seq_lens, int b) {
  int t = seq_lens ? seq_lens[b] : max_seq;
  return t < 0 ? 0 : (t > max_seq ? max_seq : t);
}

// ---------------------------------------------------------------------------
// chunk pass over a score buffer
// ---------------------------------------------------------------------------
// A token past the row's end is staged as this NaN, whose score_key is 0,
// the key of no token.
constexpr uint32_t kNoTokenBits = 0xffffffffu;

__global__ __launch_bounds__(kCT) void chunk_kernel(int H, int max_seq, const int32_t* __restrict__ seq_lens,
                                                    const float* __restrict__ scores, int k, CandSegs segs) {
  // The chunk's scores go through LDS: loaded 16 bytes per lane (coalesced),
  // staged so that thread i then reads its kCE consecutive tokens
  // o = i*kCE + e at e*SS + i (token o sits at (o % kCE)*SS + o / kCE; the
  // pad makes the writes and those reads hit distinct banks).
  constexpr int SS = kCT + (kCE <= 64 ? 64 / kCE : 1);
  constexpr int kStageBytes = kCE * SS * 4;
  constexpr int kBufBytes =
      kStageBytes > int(sizeof(ChunkSmem<kCT, kCE>)) ? kStageBytes : int(sizeof(ChunkSmem<kCT, kCE>));
  __shared__ __attribute__((aligned(16))) char sbuf[kBufBytes];   // staged scores, then selection scratch
  __shared__ Top2Smem<kCT> tsm;
  // launch position x holds chunk (x + row) mod gridDim.x, which spreads each
  // chunk index over the XCDs (blocks go to them round-robin by position;
  // with ragged rows the late chunks are the empty ones)
  const int tid = threadIdx.x, row = blockIdx.y;
  const int chunk = int((blockIdx.x + unsigned(row) % 8u) % gridDim.x);
  const int Tb = row_len(max_seq, seq_lens, row / H);
  const int start = chunk * kChunk;
  int n = Tb - start;
  n = n < 0 ? 0 : (n > kChunk ? kChunk : n);
  const float* src = scores + int64_t(row) * max_seq + start;
  const int64_t seg = int64_t(row) * segs.nseg + chunk;
  if (n == 0) {
    if (tid == 0) segs.cnt[seg] = 0;
    return;
  }
  float* stage = reinterpret_cast<float*>(sbuf);
  auto sidx = [](int o) { return (o % kCE) * SS + o / kCE; };
  const float none = __uint_as_float(kNoTokenBits);
  // All loads are issued together; positions past the row's end read a
  // readable position and are staged as no token.
  if ((max_seq & 3) == 0) {                      // 16-byte aligned rows (block-uniform)
    const int lim = max_seq - start < kChunk ? max_seq - start : kChunk;   // readable, a multiple of 4, >= 4
    f32x4 v[kCE / 4];
#pragma unroll
    for (int i = 0; i < kCE / 4; ++i) {
      const int o = (i * kCT + tid) * 4;
      v[i] = *reinterpret_cast<const f32x4*>(src + (o < lim ? o : lim - 4));
    }
#pragma unroll
    for (int i = 0; i < kCE / 4; ++i) {
      const int o = (i * kCT + tid) * 4;
      stage[sidx(o)] = o < n ? v[i].x : none;
      stage[sidx(o + 1)] = o + 1 < n ? v[i].y : none;
      stage[sidx(o + 2)] = o + 2 < n ? v[i].z : none;
      stage[sidx(o + 3)] = o + 3 < n ? v[i].w : none;
    }
  } else {
    float v[kCE];
#pragma unroll
    for (int i = 0; i < kCE; ++i) {
      const int o = i * kCT + tid;
      v[i] = src[o < n ? o : n - 1];
    }
#pragma unroll
    for (int i = 0; i < kCE; ++i) {
      const int o = i * kCT + tid;
      stage[sidx(o)] = o < n ? v[i] : none;
    }
  }
  __syncthreads();
  uint32_t key[kCE];
#pragma unroll
  for (int e = 0; e < kCE; ++e) key[e] = score_key(stage[e * SS + tid]);   // token tid*kCE + e
  // the top-two bound first (block-uniform; it leaves the stage intact),
  // the histogram select when it does not apply or keeps too many
  const bool done = n == kChunk && k <= kCT && chunk_select_top2<kCT, kCE>(key, start, k, tsm, stage, SS, segs, seg);
  if (!done) {
    __syncthreads();                             // the stage is reused below
    ChunkSmem<kCT, kCE>& csm = *reinterpret_cast<ChunkSmem<kCT, kCE>*>(sbuf);
    chunk_select<kCT, kCE>(key, start, start + n, n, k, csm, segs, seg);
  }
}

// Wide chunks, for rows too few to fill the GPU with 8192-token chunks and
// budgets large enough that those chunks' lists would need a merge level
// (e.g. one latent head per sequence, k = 2048): one 1024-thread block per
// 32768 scores of a row, 32 consecutive scores per thread, the histogram
// select. Four such chunks of a 128K row keep few enough candidates for the
// final pass to read them directly.
constexpr int kWT = 1024;
constexpr int kWideChunk = kWT * kCE;   // 32768

__global__ __launch_bounds__(kWT) void chunk_wide_kernel(int H, int max_seq, const int32_t* __restrict__ seq_lens,
                                                         const float* __restrict__ scores, int k, CandSegs segs) {
  __shared__ ChunkSmem<kWT, kCE> sm;
  const int tid = threadIdx.x, row = blockIdx.y;
  const int chunk = int((blockIdx.x + unsigned(row) % 8u) % gridDim.x);   // spread over the XCDs, as above
  const int Tb = row_len(max_seq, seq_lens, row / H);
  const int start = chunk * kWideChunk;
  int n = Tb - start;
  n = n < 0 ? 0 : (n > kWideChunk ? kWideChunk : n);
  const float* src = scores + int64_t(row) * max_seq + start;
  const int64_t seg = int64_t(row) * segs.nseg + chunk;
  if (n == 0) {
    if (tid == 0) segs.cnt[seg] = 0;
    return;
  }
  // Thread i takes scores i*kCE .. i*kCE+kCE-1, all loads issued together;
  // positions past the row's end read a readable position and are masked.
  float v[kCE];
  const int p0 = tid * kCE;
  if ((max_seq & 3) == 0) {                      // 16-byte aligned rows (block-uniform)
    const int lim = max_seq - start < kWideChunk ? max_seq - start : kWideChunk;   // a multiple of 4, >= 4
#pragma unroll
    for (int i = 0; i < kCE / 4; ++i) {
      const int o = p0 + 4 * i;
      const f32x4 x = *reinterpret_cast<const f32x4*>(src + (o < lim ? o : lim - 4));
      v[4 * i] = x.x;
      v[4 * i + 1] = x.y;
      v[4 * i + 2] = x.z;
      v[4 * i + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < kCE; ++e) v[e] = src[p0 + e < n ? p0 + e : n - 1];
  }
  uint32_t key[kCE];
#pragma unroll
  for (int e = 0; e < kCE; ++e) key[e] = p0 + e < n ? score_key(v[e]) : 0u;
  chunk_select<kWT, kCE>(key, start, start + n, n, k, sm, segs, seg);
}

// ---------------------------------------------------------------------------
// final pass
// ---------------------------------------------------------------------------
constexpr int kBinList = 64;   // a bin this small is finished by one wave
template <int NT>
struct FinalSmem {
  uint32_t hist[kFinBins];
  int offs[kMaxSeg + 1];
  ScanSmem<NT> scan;
  uint32_t red[2][NT / 64];
  int res[2];
  uint32_t bin[kBinList];
  int nbin;
};

// One block per (row, group of gs consecutive segments). MERGE = false: the
// group is the whole row (gs = nseg) and the block writes the row's selected
// indices. MERGE = true: the block writes its group's first min(k, n)
// candidates of the (key desc, index asc) order, as (key, index) pairs in
// token order, to segment (row, group) of `outs`: a smaller candidate list
// for the next level that still holds the row's top k.
// With GT > 0 (final mode only) the block then runs the attention of the
// row's query heads over the selected tokens, read in place, and writes the
// normalised outputs and log-sum-exps (split-K with one split): the indices
// never make a round trip through memory before the attention reads them.
// hs blocks share a row: each makes the same (deterministic) selection and
// attends for its own heads hpb*h .. hpb*h+hpb-1 of the row's group; only
// the first writes the indices. A row's blocks are 8 launch positions apart,
// so they land on one XCD and share its L2 for the candidates and K/V rows.
struct AttendArgs {
  GqaDev g;
  const uint16_t* q;
  const uint16_t* K;
  const uint16_t* V;
  float scale;
  float* out;
  float* lse;
  int hs, hpb;                                          // blocks per row, heads per block
};
constexpr int kAttendMaxK = 512;

template <int NT, int EF, bool MERGE, int GT = 0>
__global__ __launch_bounds__(NT) void final_kernel(int H, int max_seq, const int32_t* __restrict__ seq_lens, int k,
                                                   CandSegs segs, int gs, int32_t* __restrict__ out, CandSegs outs,
                                                   AttendArgs at = AttendArgs{}, DeltaArgs dl = DeltaArgs{}) {
  static_assert(GT == 0 || !MERGE, "attention follows the row's final selection only");
  constexpr int NW = NT / 64;
  __shared__ FinalSmem<NT> sm;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ng = (segs.nseg + gs - 1) / gs;
  int row = blockIdx.x / ng, grp = blockIdx.x % ng;
  int hsplit = 0;                                       // this block's head share (GT > 0)
  if constexpr (GT > 0) {
    const int hs = at.hs, lin = blockIdx.x;
    if (hs > 1 && (gridDim.x / hs) % 8 == 0) {          // lin = (q*hs + hsplit)*8 + row % 8
      row = (lin / (8 * hs)) * 8 + lin % 8;
      hsplit = (lin / 8) % hs;
    } else {
      row = lin / hs;
      hsplit = lin % hs;
    }
    grp = 0;
  }
  const int Tb = row_len(max_seq, seq_lens, row / H);
  const int need_all = MERGE ? k : min(k, Tb);
  const int s0 = grp * gs;
  const int nseg = min(gs, segs.nseg - s0);             // segments in this block's list
  const int64_t seg0 = int64_t(row) * segs.nseg + s0;
  const uint32_t* gkey = segs.key + seg0 * segs.cap;
  const int32_t* gidx = segs.idx + seg0 * segs.cap;

  // Direct layout: segment s is read by TPS = NT/nseg threads, EF slots each,
  // at fixed positions, so these loads go out together with the segment
  // counts instead of after them. Thread order is then list order. Used when
  // every segment fits its TPS*EF slots; otherwise the list is re-read below
  // by list position.
  static_assert(EF % 4 == 0, "direct slots are read 16 bytes at a time");
  const int TPS = NT / nseg;
  const bool try_direct = TPS > 0 && TPS * EF <= segs.cap && segs.cap % 4 == 0;   // block-uniform
  const int dseg = TPS > 0 ? tid / TPS : nseg;
  const int dj = TPS > 0 ? (tid % TPS) * EF : 0;
  uint32_t rkey[EF];
  int32_t ridx[EF];
  if (try_direct) {
    const int64_t o = int64_t(dseg < nseg ? dseg : 0) * segs.cap + dj;
#pragma unroll
    for (int e = 0; e < EF; e += 4) {
      const u32x4 kv = *reinterpret_cast<const u32x4*>(gkey + o + e);
      const u32x4 iv = *reinterpret_cast<const u32x4*>(gidx + o + e);
      rkey[e] = kv.x; rkey[e + 1] = kv.y; rkey[e + 2] = kv.z; rkey[e + 3] = kv.w;
      ridx[e] = int32_t(iv.x); ridx[e + 1] = int32_t(iv.y); ridx[e + 2] = int32_t(iv.z); ridx[e + 3] = int32_t(iv.w);
    }
  }

  // segment offsets: each thread scans SPT consecutive segments
  constexpr int SPT = kMaxSeg / NT;
  int c[SPT];
  int mine = 0;
#pragma unroll
  for (int x = 0; x < SPT; ++x) {
    const int s = tid * SPT + x;
    c[x] = segs.cnt[seg0 + (s < nseg ? s : nseg - 1)];
  }
#pragma unroll
  for (int x = 0; x < SPT; ++x) {
    c[x] = tid * SPT + x < nseg ? c[x] : 0;
    mine += c[x];
  }
  // top-delta (final level only): the row's pseudo-max and the key a kept
  // token must reach (0: no filter)
  uint32_t thr_key = 0u;
  if constexpr (!MERGE) {
    if (dl.pmax) {                                      // block-uniform
      __shared__ uint32_t pred[NW];
      uint32_t pm = 0u;
      for (int s = tid; s < dl.nseg0; s += NT) {
        const uint32_t v = dl.pmax[int64_t(row) * dl.nseg0 + s];
        pm = v > pm ? v : pm;
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = uint32_t(__shfl_xor(int(pm), o, 64));
        pm = y > pm ? y : pm;
      }
      if (lane == 0) pred[wv] = pm;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < NW; ++i) pm = pred[i] > pm ? pred[i] : pm;
      if (pm != 0u) thr_key = score_key(key_score(pm) - dl.thr_off);
      const uint32_t neg_inf = score_key(-__builtin_inff());
      thr_key = thr_key > neg_inf ? thr_key : neg_inf + 1u;      // -inf scores: no valid page
    }
  }
  int n;
  int run = block_scan<NT>(mine, sm.scan, &n) - mine;
#pragma unroll
  for (int x = 0; x < SPT; ++x) {
    const int s = tid * SPT + x;
    if (s < nseg) sm.offs[s] = run;
    run += c[x];
  }
  if (tid == 0) sm.offs[nseg] = n;
  bool over = false;
#pragma unroll
  for (int x = 0; x < SPT; ++x) over = over || c[x] > TPS * EF;
  const bool direct = !__syncthreads_or(over) && try_direct;   // (the barrier also orders the offs writes)
  // The row's candidate list is its segments one after the other: ascending
  // token order (segments cover ascending token ranges, each in token order).
  auto locate = [&](int i) -> int {      // segment holding list position i < n
    int lo = 0, hi = nseg - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sm.offs[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  // list positions i0 .. i0+EF-1 (idx -1 past the end). Addresses first,
  // then every load at once; positions past the end re-read entry n - 1.
  auto offsets = [&](int i0, int32_t (&o)[EF]) {   // row-relative offsets of positions i0..
    int s = locate(i0 < n ? i0 : n - 1);
#pragma unroll
    for (int e = 0; e < EF; ++e) {
      const int i = i0 + e < n ? i0 + e : n - 1;
      while (i >= sm.offs[s + 1]) ++s;
      o[e] = s * segs.cap + (i - sm.offs[s]);
    }
  };
  auto fetch = [&](int i0, uint32_t (&ck)[EF], int32_t (&ci)[EF]) {
    int32_t o[EF];
    offsets(i0, o);
#pragma unroll
    for (int e = 0; e < EF; ++e) {
      ck[e] = gkey[o[e]];
      ci[e] = gidx[o[e]];
    }
#pragma unroll
    for (int e = 0; e < EF; ++e)
      if (i0 + e >= n) ci[e] = -1;
  };

  // candidates live in registers when they fit (block-uniform choice): in
  // the direct layout, or else each thread holding EF consecutive list
  // positions
  constexpr int kRegCap = NT * EF;
  const bool reg = direct || n <= kRegCap;
  if (direct) {
    const int cnt = dseg < nseg ? sm.offs[dseg + 1] - sm.offs[dseg] : 0;
#pragma unroll
    for (int e = 0; e < EF; ++e)
      if (dj + e >= cnt) ridx[e] = -1;
  } else if (reg && n > 0) {
    fetch(tid * EF, rkey, ridx);
  } else {
#pragma unroll
    for (int e = 0; e < EF; ++e) {
      rkey[e] = 0u;
      ridx[e] = -1;
    }
  }
  auto for_each_key = [&](auto&& fn) {
    if (reg) {
#pragma unroll
      for (int e = 0; e < EF; ++e)
        if (ridx[e] >= 0) fn(rkey[e]);
    } else {                             // page by page, as held in registers
      for (int p0 = 0; p0 < n; p0 += kRegCap) {
        const int i0 = p0 + tid * EF;
        int32_t o[EF];
        offsets(i0, o);
#pragma unroll
        for (int e = 0; e < EF; ++e) rkey[e] = gkey[o[e]];   // the register list is free here
#pragma unroll
        for (int e = 0; e < EF; ++e)
          if (i0 + e < n) fn(rkey[e]);
      }
    }
  };

  // Selection rule: take key > tkey, and the first trem candidates (in list
  // order, i.e. lowest token indices) whose key equals tkey.
  uint32_t tkey = 0u;
  int trem = 0x7fffffff;
  if (n > need_all && need_all > 0) {
    uint32_t mx = 0u, mn = 0xffffffffu;
    for_each_key([&](uint32_t key) {
      mx = key > mx ? key : mx;
      mn = key < mn ? key : mn;
    });
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t a = uint32_t(__shfl_xor(int(mx), o, 64));
      const uint32_t c = uint32_t(__shfl_xor(int(mn), o, 64));
      mx = a > mx ? a : mx;
      mn = c < mn ? c : mn;
    }
    if (lane == 0) {
      sm.red[0][wv] = mx;
      sm.red[1][wv] = mn;
    }
    __syncthreads();
    uint64_t hi = 0, lo = 0xffffffffull;
    for (int i = 0; i < NW; ++i) {
      hi = sm.red[0][i] > hi ? sm.red[0][i] : hi;
      lo = sm.red[1][i] < lo ? sm.red[1][i] : lo;
    }
    // Adaptive levels: kFinBins linear bins over the current bracket
    // [lo, hi] of keys; the bin holding the rem-th largest key becomes the
    // next bracket. Every level narrows the bracket by 2^12, so at most three
    // levels reach a single key value.
    int rem = need_all;
    for (;;) {
      const uint64_t range = hi - lo;
      const int sh = range < uint64_t(kFinBins) ? 0 : (64 - __builtin_clzll(range)) - kFinBits;
      for (int i = tid; i < kFinBins; i += NT) sm.hist[i] = 0u;
      if (tid == 0) sm.nbin = 0;
      __syncthreads();
      for_each_key([&](uint32_t key) {
        if (key >= lo && key <= hi) atomicAdd(&sm.hist[(key - lo) >> sh], 1u);
      });
      __syncthreads();
      pick_bin<NT, kFinBins / NT>(sm.hist, rem, true, sm.scan, sm.res);
      const uint64_t D = uint64_t(sm.res[0]);
      rem -= sm.res[1];
      const int cnt = int(sm.hist[D]);
      __syncthreads();
      const uint64_t blo = lo + (D << sh);
      if (cnt == rem) {                  // the whole bin is taken
        tkey = uint32_t(blo);
        break;
      }
      if (sh == 0) {                     // a single key value, tied
        tkey = uint32_t(blo);
        trem = rem;
        break;
      }
      if (cnt <= kBinList) {             // few keys in the bin: one wave ranks them exactly
        for_each_key([&](uint32_t key) {
          if (key >= lo && key <= hi && ((key - lo) >> sh) == D) sm.bin[atomicAdd(&sm.nbin, 1)] = key;
        });
        __syncthreads();
        if (wv == 0) {
          const uint32_t mine = lane < cnt ? sm.bin[lane] : 0u;
          int gt = 0, eq = 0;                      // keys of the bin above / equal to this lane's
          for (int i = 0; i < cnt; ++i) {
            const uint32_t x = uint32_t(__builtin_amdgcn_readlane(int(mine), i));
            gt += x > mine ? 1 : 0;
            eq += x == mine ? 1 : 0;
          }
          // the rem-th largest key v of the bin: gt < rem <= gt + eq; take
          // the rem - gt first of the keys equal to v (all of them: no ranking)
          if (lane < cnt && gt < rem && rem <= gt + eq) {
            sm.res[0] = int(mine);
            sm.res[1] = rem - gt == eq ? 0x7fffffff : rem - gt;
          }
        }
        __syncthreads();
        tkey = uint32_t(sm.res[0]);
        trem = sm.res[1];
        break;
      }
      const uint64_t bhi = blo + (uint64_t(1) << sh) - 1;
      lo = blo;
      hi = bhi < hi ? bhi : hi;
    }
  }

  // Output in list order, which is ascending token order: two block scans
  // per page of candidates, one ranking the tied candidates and one placing
  // the taken ones.
  int32_t* dst = MERGE ? outs.idx + (int64_t(row) * ng + grp) * outs.cap : out + int64_t(row) * k;
  const bool write_idx = MERGE || hsplit == 0;
  uint32_t* dkey = MERGE ? outs.key + (int64_t(row) * ng + grp) * outs.cap : nullptr;
  int tie_base = 0, out_base = 0;
  __shared__ int32_t sel[GT > 0 ? kAttendMaxK : 1];   // the selected tokens, for the attention
  auto emit = [&](const uint32_t (&ck)[EF], const int32_t (&ci)[EF]) {
    int tt = 0, tr = 0;
    if (trem != 0x7fffffff) {                         // tied candidates are ranked only when some are left out
      int nt = 0;
#pragma unroll
      for (int e = 0; e < EF; ++e) nt += (ci[e] >= 0 && ck[e] == tkey) ? 1 : 0;
      tr = block_scan<NT>(nt, sm.scan, &tt) - nt + tie_base;
    }
    static_assert(EF <= 32, "taken flags are one bit each");
    uint32_t take = 0u;
#pragma unroll
    for (int e = 0; e < EF; ++e) {
      bool t = false;
      if (ci[e] >= 0) {
        if (ck[e] > tkey) t = true;
        else if (ck[e] == tkey) t = tr++ < trem;
      }
      t = t && ck[e] >= thr_key;                        // top-delta filter (thr_key 0: none)
      take |= t ? 1u << e : 0u;
    }
    const int ns = __popc(take);
    int st;
    int at = block_scan<NT>(ns, sm.scan, &st) - ns + out_base;
#pragma unroll
    for (int e = 0; e < EF; ++e)
      if (take >> e & 1u) {
        if constexpr (MERGE) dkey[at] = ck[e];
        if constexpr (GT > 0) sel[at] = ci[e];
        if (write_idx) dst[at] = ci[e];
        ++at;
      }
    tie_base += tt;
    out_base += st;
  };
  if (n == 0) {
  } else if (reg) {
    emit(rkey, ridx);
  } else {
    for (int p0 = 0; p0 < n; p0 += kRegCap) {
      fetch(p0 + tid * EF, rkey, ridx);
      emit(rkey, ridx);
    }
  }
  if constexpr (MERGE) {
    if (tid == 0) outs.cnt[int64_t(row) * ng + grp] = out_base;
  } else {
    if (write_idx)
      for (int i = out_base + tid; i < k; i += NT) dst[i] = -1;
    if (dl.counts && write_idx && tid == 0) dl.counts[row] = out_base;
  }
  if constexpr (GT > 0) {
    constexpr int STEPS = 8, RB = STEPS * 4;
    const GqaDev& g = at.g;
    const int b = row / H, j = row % H, w = tid >> 6;
    const int cnt = out_base;                           // selected tokens (<= kAttendMaxK)
    const float qs = at.scale * kAttnLog2e;
    __shared__ AttnMergeSmem<GT, NW> msm;
    __syncthreads();                                    // sel complete
    const int hb0 = hsplit * at.hpb, hb1 = min(g.G, hb0 + at.hpb);   // heads of this block
    for (int hl = hb0; hl < hb1; hl += GT) {
      const int h0 = j * g.G + hl, nh = min(GT, hb1 - hl);
      bf16x2 qv[GT][4];
      attn_load_q<GT>(qv, at.q, int64_t(b) * g.Hq + h0, nh, lane & 15);
      AttnAcc<GT> A;
      attn_init(A);
      for (int base = w * RB; base < cnt; base += NW * RB)
        attn_batch<GT, STEPS>(g, b, j, Tb, at.K, at.V, qv, qs, base, cnt, [&](int rr) { return sel[rr]; }, A);
      attn_wave_reduce(A);
      attn_block_merge(A, msm);
      if (w == 0)
        attn_store(A, nh, [&](int h) { return at.out + (int64_t(b) * g.Hq + h0 + h) * kAttnD; },
                   [&](int h) { return at.lse + int64_t(b) * g.Hq + h0 + h; });
      __syncthreads();                                  // msm is reused by the next head group
    }
  }
}

int chunks_of(int max_seq) { return (max_seq + kChunk - 1) / kChunk; }

}  // namespace

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

CandSegs carve_segs(void* base, int rows, int nseg, int cap, size_t* total) {
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) { char* q = p ? p + off : nullptr; off += align256(bytes); return q; };
  CandSegs w;
  w.cnt = reinterpret_cast<int32_t*>(take(size_t(rows) * nseg * 4));
  w.key = reinterpret_cast<uint32_t*>(take(size_t(rows) * nseg * cap * 4));
  w.idx = reinterpret_cast<int32_t*>(take(size_t(rows) * nseg * cap * 4));
  w.nseg = nseg;
  w.cap = cap;
  if (total) *total = off;
  return w;
}

// A row's list goes straight to the final pass when it fits the final
// block's registers at the small configuration; otherwise groups of segments
// are first merged down to k candidates each, level after level.
namespace {
constexpr int kFinalDirect = 8192;
int merge_group(int k) { return max(2, kFinalDirect / k); }
bool needs_merge(int nseg, int k) { return nseg > 1 && int64_t(nseg) * k > kFinalDirect; }
}  // namespace

size_t merge_workspace_bytes(int rows, int nseg, int k) {
  if (!needs_merge(nseg, k)) return 0;
  const int ng = (nseg + merge_group(k) - 1) / merge_group(k);
  size_t one = 0;
  carve_segs(nullptr, rows, ng, k, &one);
  return 2 * one;                                      // two alternating levels
}

hipError_t launch_select_final(int rows, int H, int max_seq, const int32_t* seq_lens, int k, CandSegs segs,
                               int32_t* idx, void* merge_ws, hipStream_t st, DeltaArgs dl) {
  if (segs.nseg > kMaxSeg) return hipErrorInvalidValue;
  CandSegs cur = segs;
  if (needs_merge(segs.nseg, k)) {
    const int gs = merge_group(k);
    size_t one = 0;
    carve_segs(nullptr, rows, (segs.nseg + gs - 1) / gs, k, &one);
    int level = 0;
    while (needs_merge(cur.nseg, k)) {
      const int ng = (cur.nseg + gs - 1) / gs;
      CandSegs nxt = carve_segs(static_cast<char*>(merge_ws) + (level & 1) * one, rows, ng, k, nullptr);
      // a group holds about gs * k <= 8192 candidates (+ ties): 12288 in registers
      hipLaunchKernelGGL((final_kernel<1024, 12, true>), dim3(rows * ng), dim3(1024), 0, st, H, max_seq,
                         seq_lens, k, cur, gs, nullptr, nxt);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      cur = nxt;
      ++level;
    }
  }
  // candidates per row ~ nseg * (k + a few): up to 8192 held in registers by
  // 1024 threads x 8, more by 1024 x 12; rows with more than 12288 (ties)
  // are streamed from memory page by page
  if (int64_t(cur.nseg) * k <= kFinalDirect)
    hipLaunchKernelGGL((final_kernel<1024, 8, false>), dim3(rows), dim3(1024), 0, st, H, max_seq, seq_lens, k,
                       cur, cur.nseg, idx, CandSegs{}, AttendArgs{}, dl);
  else
    hipLaunchKernelGGL((final_kernel<1024, 12, false>), dim3(rows), dim3(1024), 0, st, H, max_seq, seq_lens, k,
                       cur, cur.nseg, idx, CandSegs{}, AttendArgs{}, dl);
  return hipGetLastError();
}

bool select_attend_fused(int nseg, int k, int G) {
  return !needs_merge(nseg, k) && k <= kAttendMaxK && G <= 16;
}

hipError_t launch_select_attend(const GqaDev& g, int k, CandSegs segs, const uint16_t* q, const uint16_t* K,
                                const uint16_t* V, float scale, int32_t* idx, float* out, float* lse,
                                hipStream_t st, DeltaArgs dl) {
  if (segs.nseg > kMaxSeg || !select_attend_fused(segs.nseg, k, g.G)) return hipErrorInvalidValue;
  const int rows = g.B * g.Hkv;
  // Spread the row's query heads over hs blocks until the launch covers the
  // CUs (256 blocks); the selection is repeated per block, the attention
  // (the larger part) is split.
  int hs = 1;
  while (rows * hs < 256 && hs < g.G) ++hs;
  const int hpb = (g.G + hs - 1) / hs;
  hs = (g.G + hpb - 1) / hpb;
  const AttendArgs aa{g, q, K, V, scale, out, lse, hs, hpb};
  // query heads per pass over the selected rows: all of the block's heads
  // when they are 1, 2 or 5 (or 10, 15), else 4 at a time
  const int gt = hpb <= 2 ? hpb : (hpb % 5 == 0 ? 5 : 4);
#define JSSA_FA(GT)                                                                                      \
  hipLaunchKernelGGL((final_kernel<512, 16, false, GT>), dim3(rows * hs), dim3(512), 0, st, g.Hkv,         \
                     g.max_seq, g.seq_lens, k, segs, segs.nseg, idx, CandSegs{}, aa, dl)
  switch (gt) {
    case 1: JSSA_FA(1); break;
    case 2: JSSA_FA(2); break;
    case 5: JSSA_FA(5); break;
    default: JSSA_FA(4); break;
  }
#undef JSSA_FA
  return hipGetLastError();
}

namespace {
// Wide chunks when the 8192-token grid is small (fewer blocks than CUs) and
// its lists would need merging, but the wide lists would not.
bool use_wide(int rows, int max_seq, int k) {
  const int nchunks = chunks_of(max_seq), nwide = (max_seq + kWideChunk - 1) / kWideChunk;
  return int64_t(rows) * nchunks < 256 && needs_merge(nchunks, k) && !needs_merge(nwide, k);
}
}  // namespace

size_t topk_workspace_bytes(int rows, int max_seq, int k) {
  size_t total = 0;
  carve_segs(nullptr, rows, chunks_of(max_seq), kChunk, &total);
  total += merge_workspace_bytes(rows, chunks_of(max_seq), k);
  if (use_wide(rows, max_seq, k)) {
    size_t wide = 0;
    carve_segs(nullptr, rows, (max_seq + kWideChunk - 1) / kWideChunk, kWideChunk, &wide);
    total = wide > total ? wide : total;
  }
  return total;
}

hipError_t launch_topk(int B, int H, int max_seq, const int32_t* seq_lens, const float* scores, int k,
                       int32_t* idx, void* wsp, hipStream_t st) {
  const int rows = B * H;
  const int nchunks = chunks_of(max_seq);
  if (use_wide(rows, max_seq, k)) {               // (the workspace size covers this layout)
    const int nwide = (max_seq + kWideChunk - 1) / kWideChunk;
    CandSegs segs = carve_segs(wsp, rows, nwide, kWideChunk, nullptr);
    hipLaunchKernelGGL(chunk_wide_kernel, dim3(nwide, rows), dim3(kWT), 0, st, H, max_seq, seq_lens, scores, k,
                       segs);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // about nwide * k candidates plus ties: the 12-per-thread final holds them
    hipLaunchKernelGGL((final_kernel<1024, 12, false>), dim3(rows), dim3(1024), 0, st, H, max_seq, seq_lens, k,
                       segs, segs.nseg, idx, CandSegs{}, AttendArgs{}, DeltaArgs{});
    return hipGetLastError();
  }
  size_t main_bytes = 0;
  CandSegs segs = carve_segs(wsp, rows, nchunks, kChunk, &main_bytes);
  hipLaunchKernelGGL(chunk_kernel, dim3(nchunks, rows), dim3(kCT), 0, st, H, max_seq, seq_lens, scores, k, segs);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_select_final(rows, H, max_seq, seq_lens, k, segs, idx, static_cast<char*>(wsp) + main_bytes, st);
}

}  // namespace jssa

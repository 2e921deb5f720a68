// Per-(sequence, head) top-k with lowest-index ties.
//
// Each KV head gets its own selection (JSSA abstract; ai4snews digest,
// Synopsis). The result is the first min(k, n) existing tokens of the total
// order (score descending, index ascending), listed ascending; a -inf score
// marks a position without a token (past T_b, or behind an invalid page).
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
    if (tid == 0) write_info(segs, seg, 0, 0u, 0u, 0xffffffffu);
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
    if (tid == 0) write_info(segs, seg, 0, 0u, 0u, 0xffffffffu);
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
  uint32_t red[6][NT / 64];
  int res[2];
  uint32_t bin[kBinList];
  int nbin;
};

// Exact top-k of one score row straight from its scores, for rows whose
// candidate lists were not enough: the row's tokens are its positions below
// T_b with a score above -inf (key 0: a position behind an invalid page
// holds no token). A count, then three radix levels over the order-
// preserving keys (bits 31..20, 19..8, 7..0; each a histogram of the keys
// that match the levels above), then the taken tokens in token order, tiles
// of NT with block scans (ties, lowest index first). Slow (the row is read
// five times), and only run when a row's lists do not hold its top k.
template <int NT>
__device__ void lists_fallback(const float* __restrict__ srow, int Tb, int k, int32_t* __restrict__ dst,
                               uint32_t* hist, ScanSmem<NT>& scan, int* res) {
  const int tid = threadIdx.x;
  int nt0 = 0;
  for (int t = tid; t < Tb; t += NT) nt0 += score_key(srow[t]) != 0u ? 1 : 0;
  int ntok;
  block_scan<NT>(nt0, scan, &ntok);
  const int need = min(k, ntok);
  uint32_t tkey = 1u, prefix = 0u, pmask = 0u;        // (tkey 1: every token, no ties to rank)
  int trem = 0x7fffffff;
  if (need < ntok) {
    int rem = need;
    constexpr int kShift[3] = {20, 8, 0};
    constexpr uint32_t kMask[3] = {0xfffu, 0xfffu, 0xffu};
    for (int lv = 0; lv < 3; ++lv) {
      const int sh = kShift[lv];
      for (int i = tid; i < kFinBins; i += NT) hist[i] = 0u;
      __syncthreads();
      for (int t = tid; t < Tb; t += NT) {
        const uint32_t key = score_key(srow[t]);
        if (key != 0u && (key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & kMask[lv]], 1u);
      }
      __syncthreads();
      pick_bin<NT, kFinBins / NT>(hist, rem, true, scan, res);
      const uint32_t D = uint32_t(res[0]);
      rem -= res[1];
      const int cnt = int(hist[D]);
      __syncthreads();
      prefix |= D << sh;
      pmask |= kMask[lv] << sh;
      tkey = prefix > 1u ? prefix : 1u;  // the lowest key of the bin (a token's key is at least 1)
      if (cnt == rem) break;             // the whole bin is taken: every key >= tkey
      if (lv == 2) trem = rem;           // one key value, tied
    }
  }
  int tie_base = 0, out_base = 0;
  for (int t0 = 0; t0 < Tb; t0 += NT) {
    const int t = t0 + tid;
    const uint32_t key = t < Tb ? score_key(srow[t]) : 0u;
    const bool real = key != 0u;
    int tt = 0, tr = 0;
    if (trem != 0x7fffffff) {
      const int nt = real && key == tkey ? 1 : 0;
      tr = block_scan<NT>(nt, scan, &tt) - nt + tie_base;
    }
    const bool take = real && (key > tkey || (key == tkey && tr < trem));
    int st;
    const int at = block_scan<NT>(take ? 1 : 0, scan, &st) - (take ? 1 : 0) + out_base;
    if (take) dst[at] = t;
    tie_base += tt;
    out_base += st;
  }
  for (int i = out_base + tid; i < k; i += NT) dst[i] = -1;
}

// LISTS (final level only): each segment holds the top candidates of one
// chunk of `lists.chunk_len` tokens of the score row `lists.scores`, a list
// that need not contain the row's top k. A chunk that dropped real tokens
// keeps every key above its segment's bot, so the union holds the row's top
// k when every such chunk's bot is below the row's k-th key; the block checks
// that once the k-th key is known, and otherwise selects the row again from
// its scores (lists_fallback). Either way the result is exact.
struct ListArgs {
  const float* scores;
  int chunk_len;
};

template <int NT, int EF, bool MERGE, bool LISTS = false>
__global__ __launch_bounds__(NT) void final_kernel(int H, int max_seq, const int32_t* __restrict__ seq_lens, int k,
                                                   CandSegs segs, int gs, int32_t* __restrict__ out, CandSegs outs,
                                                   DeltaArgs dl = DeltaArgs{}, ListArgs lists = ListArgs{}) {
  constexpr int NW = NT / 64;
  __shared__ FinalSmem<NT> sm;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ng = (segs.nseg + gs - 1) / gs;
  const int row = blockIdx.x / ng, grp = blockIdx.x % ng;
  const int Tb = row_len(max_seq, seq_lens, row / H);
  const int need_all = MERGE ? k : min(k, Tb);
  const int s0 = grp * gs;
  const int nseg = min(gs, segs.nseg - s0);             // segments in this block's list
  const int64_t seg0 = int64_t(row) * segs.nseg + s0;
  const uint32_t* gkey = segs.key + seg0 * segs.cap;
  const int32_t* gidx = segs.idx + seg0 * segs.cap;
  const SegInfo* ginfo = segs.info + seg0;

  // Direct layout: segment s is read by TPS = NT/nseg threads, EF slots each
  // (slots past the segment's capacity are not read), at fixed positions, so
  // these loads go out together with the segment summaries instead of after
  // them; thread order is then list order. Used when every segment's count
  // fits its threads' slots (always when TPS*EF >= cap); otherwise the list
  // is re-read below by list position.
  static_assert(EF % 4 == 0, "direct slots are read 16 bytes at a time");
  const int TPS = NT / nseg;
  const bool try_direct = TPS > 0 && segs.cap % 4 == 0;      // block-uniform
  const int dslots = TPS > 0 ? min(TPS * EF, segs.cap) : 0;  // direct slots per segment
  const int dseg = TPS > 0 ? tid / TPS : nseg;
  const int dj = TPS > 0 ? (tid % TPS) * EF : 0;
  uint32_t rkey[EF];
  int32_t ridx[EF];
  int dcnt = 0;                                         // candidates of this thread's direct segment
  if (try_direct) {
    const int ds = dseg < nseg ? dseg : 0;
    dcnt = ginfo[ds].cnt;
    const int64_t o = int64_t(ds) * segs.cap;
#pragma unroll
    for (int e = 0; e < EF; e += 4) {
      const int j0 = dj + e < segs.cap ? dj + e : segs.cap - 4;   // in the segment's slots
      const u32x4 kv = *reinterpret_cast<const u32x4*>(gkey + o + j0);
      const u32x4 iv = *reinterpret_cast<const u32x4*>(gidx + o + j0);
      rkey[e] = kv.x; rkey[e + 1] = kv.y; rkey[e + 2] = kv.z; rkey[e + 3] = kv.w;
      ridx[e] = int32_t(iv.x); ridx[e + 1] = int32_t(iv.y); ridx[e + 2] = int32_t(iv.z); ridx[e + 3] = int32_t(iv.w);
    }
  }

  // Segment summaries: thread tid takes segments tid, tid + NT, ... (one
  // load when nseg <= NT). The row's candidate count, the largest
  // per-segment count, and the bracket of the k-th key come out of wave
  // reductions and one barrier: every candidate is at or below hi, and lo
  // (the largest segment floor, or the smallest candidate) is at or below
  // the need_all-th largest candidate key.
  constexpr int SPT = kMaxSeg / NT;
  uint32_t fl = 0u, tp = 0u, bt = 0xffffffffu, cmx = 0u, mine = 0u;
  for (int s = tid; s < nseg; s += NT) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(ginfo + s);
    mine += v.x;
    fl = v.y > fl ? v.y : fl;
    tp = v.z > tp ? v.z : tp;
    bt = v.w < bt ? v.w : bt;
    cmx = v.x > cmx ? v.x : cmx;
  }
  for (int i = tid; i < kFinBins; i += NT) sm.hist[i] = 0u;   // the first histogram level
  if (tid == 0) sm.nbin = 0;
  {
    const uint32_t a = wave_sum_u32(mine), f = wave_max_u32(fl), t = wave_max_u32(tp);
    const uint32_t u = wave_min_u32(bt), m = wave_max_u32(cmx);
    if (lane == 0) {
      sm.red[0][wv] = a;
      sm.red[1][wv] = f;
      sm.red[2][wv] = t;
      sm.red[3][wv] = u;
      sm.red[4][wv] = m;
    }
  }
  // top-delta (final level only): the row's pseudo-max and the key a kept
  // token must reach (0: no filter); its slots are read with the summaries
  uint32_t pm = 0u;
  if constexpr (!MERGE) {
    if (dl.pmax) {                                      // block-uniform
      for (int s = tid; s < dl.nseg0; s += NT) {
        const uint32_t v = dl.pmax[int64_t(row) * dl.nseg0 + s];
        pm = v > pm ? v : pm;
      }
      pm = wave_max_u32(pm);
      if (lane == 0) sm.red[5][wv] = pm;
    }
  }
  __syncthreads();
  int n = 0;
  uint32_t lo = 0u, hi = 0u, lbot = 0xffffffffu, cmax = 0u;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    n += int(sm.red[0][i]);
    lo = sm.red[1][i] > lo ? sm.red[1][i] : lo;
    hi = sm.red[2][i] > hi ? sm.red[2][i] : hi;
    lbot = sm.red[3][i] < lbot ? sm.red[3][i] : lbot;
    cmax = sm.red[4][i] > cmax ? sm.red[4][i] : cmax;
  }
  lo = lbot > lo ? lbot : lo;
  uint32_t thr_key = 0u;
  if constexpr (!MERGE) {
    if (dl.pmax) {
#pragma unroll
      for (int i = 0; i < NW; ++i) pm = sm.red[5][i] > pm ? sm.red[5][i] : pm;
      if (pm != 0u) thr_key = score_key(key_score(pm) - dl.thr_off);   // (-inf: key 0, no filter)
    }
  }
  const bool direct = try_direct && int(cmax) <= dslots;       // block-uniform
  // Offsets of the segments in the row's list: needed only when the list is
  // read by position (not direct).
  if (!direct) {                                       // (thread tid: SPT consecutive segments)
    int c[SPT];
    int mc = 0;
#pragma unroll
    for (int x = 0; x < SPT; ++x) {
      const int s = tid * SPT + x;
      c[x] = s < nseg ? ginfo[s].cnt : 0;
      mc += c[x];
    }
    int tot;
    int run = block_scan<NT>(mc, sm.scan, &tot) - mc;
#pragma unroll
    for (int x = 0; x < SPT; ++x) {
      const int s = tid * SPT + x;
      if (s < nseg) sm.offs[s] = run;
      run += c[x];
    }
    if (tid == 0) sm.offs[nseg] = n;
    __syncthreads();
  }
  // The row's candidate list is its segments one after the other: ascending
  // token order (segments cover ascending token ranges, each in token order).
  auto locate = [&](int i) -> int {      // segment holding list position i < n
    int lo_s = 0, hi_s = nseg - 1;
    while (lo_s < hi_s) {
      const int mid = (lo_s + hi_s + 1) >> 1;
      if (sm.offs[mid] <= i) lo_s = mid; else hi_s = mid - 1;
    }
    return lo_s;
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
    const int cnt = dseg < nseg ? dcnt : 0;
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
  const bool search = n > need_all && need_all > 0;   // block-uniform
  if (search) {
    // Adaptive levels: kFinBins linear bins over the current bracket
    // [lo, hi] of keys; the bin holding the rem-th largest key becomes the
    // next bracket. Every level narrows the bracket by 2^12, so at most three
    // levels reach a single key value.
    uint64_t blo_ = lo, bhi_ = hi;
    int rem = need_all;
    for (int level = 0;; ++level) {
      const uint64_t range = bhi_ - blo_;
      const int sh = range < uint64_t(kFinBins) ? 0 : (64 - __builtin_clzll(range)) - kFinBits;
      if (level > 0) {
        for (int i = tid; i < kFinBins; i += NT) sm.hist[i] = 0u;
        if (tid == 0) sm.nbin = 0;
        __syncthreads();
      }
      for_each_key([&](uint32_t key) {
        if (key >= blo_ && key <= bhi_) atomicAdd(&sm.hist[(key - blo_) >> sh], 1u);
      });
      __syncthreads();
      pick_bin<NT, kFinBins / NT>(sm.hist, rem, true, sm.scan, sm.res);
      const uint64_t D = uint64_t(sm.res[0]);
      rem -= sm.res[1];
      const int cnt = int(sm.hist[D]);
      __syncthreads();
      const uint64_t blo = blo_ + (D << sh);
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
          if (key >= blo_ && key <= bhi_ && ((key - blo_) >> sh) == D) sm.bin[atomicAdd(&sm.nbin, 1)] = key;
        });
        __syncthreads();
        if (wv == 0) {
          const uint32_t mk = lane < cnt ? sm.bin[lane] : 0u;
          int gt = 0, eq = 0;                      // keys of the bin above / equal to this lane's
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
      const uint64_t bhi = blo + (uint64_t(1) << sh) - 1;
      blo_ = blo;
      bhi_ = bhi < bhi_ ? bhi : bhi_;
    }
  }

  if constexpr (LISTS) {
    // (!search: every candidate is taken, so a chunk that dropped any real
    // token leaves it out: the F = 0 test below then fails for it)
    const uint32_t F = search ? tkey : 0u;
    bool bad = false;
    for (int s = tid; s < nseg; s += NT) {
      const int real = min(lists.chunk_len, max(0, Tb - (s0 + s) * lists.chunk_len));
      const u32x4 v = *reinterpret_cast<const u32x4*>(ginfo + s);
      bad = bad || (int(v.x) < real && v.w >= F);
    }
    if (__syncthreads_or(bad)) {                       // block-uniform
      lists_fallback<NT>(lists.scores + int64_t(row) * max_seq, Tb, k, out + int64_t(row) * k, sm.hist, sm.scan,
                         sm.res);
      return;
    }
  }

  // Output in list order, which is ascending token order: two block scans
  // per page of candidates, one ranking the tied candidates and one placing
  // the taken ones.
  int32_t* dst = MERGE ? outs.idx + (int64_t(row) * ng + grp) * outs.cap : out + int64_t(row) * k;
  uint32_t* dkey = MERGE ? outs.key + (int64_t(row) * ng + grp) * outs.cap : nullptr;
  int tie_base = 0, out_base = 0;
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
    int at2 = block_scan<NT>(ns, sm.scan, &st) - ns + out_base;
#pragma unroll
    for (int e = 0; e < EF; ++e)
      if (take >> e & 1u) {
        if constexpr (MERGE) dkey[at2] = ck[e];
        dst[at2] = ci[e];
        ++at2;
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
    // the group's first min(k, n) candidates: all at or above tkey (searched)
    // or lo (all of them taken)
    const uint32_t b = search ? tkey : lo;
    if (tid == 0)
      write_info(outs, int64_t(row) * ng + grp, out_base, out_base >= k ? b : 0u, hi, out_base > 0 ? b : 0xffffffffu);
  } else {
    for (int i = out_base + tid; i < k; i += NT) dst[i] = -1;
    if (dl.counts && tid == 0) dl.counts[row] = out_base;
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
  w.info = reinterpret_cast<SegInfo*>(take(size_t(rows) * nseg * sizeof(SegInfo)));
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
                       cur, cur.nseg, idx, CandSegs{}, dl);
  else
    hipLaunchKernelGGL((final_kernel<1024, 12, false>), dim3(rows), dim3(1024), 0, st, H, max_seq, seq_lens, k,
                       cur, cur.nseg, idx, CandSegs{}, dl);
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
  carve_segs(nullptr, rows, chunks_of(max_seq), seg_cap(k, kChunk), &total);
  total += merge_workspace_bytes(rows, chunks_of(max_seq), k);
  if (use_wide(rows, max_seq, k)) {
    size_t wide = 0;
    carve_segs(nullptr, rows, (max_seq + kWideChunk - 1) / kWideChunk, seg_cap(k, kWideChunk), &wide);
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
    CandSegs segs = carve_segs(wsp, rows, nwide, seg_cap(k, kWideChunk), nullptr);
    hipLaunchKernelGGL(chunk_wide_kernel, dim3(nwide, rows), dim3(kWT), 0, st, H, max_seq, seq_lens, scores, k,
                       segs);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // about nwide * k candidates plus ties: the 12-per-thread final holds them
    hipLaunchKernelGGL((final_kernel<1024, 12, false>), dim3(rows), dim3(1024), 0, st, H, max_seq, seq_lens, k,
                       segs, segs.nseg, idx, CandSegs{}, DeltaArgs{});
    return hipGetLastError();
  }
  size_t main_bytes = 0;
  CandSegs segs = carve_segs(wsp, rows, nchunks, seg_cap(k, kChunk), &main_bytes);
  hipLaunchKernelGGL(chunk_kernel, dim3(nchunks, rows), dim3(kCT), 0, st, H, max_seq, seq_lens, scores, k, segs);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_select_final(rows, H, max_seq, seq_lens, k, segs, idx, static_cast<char*>(wsp) + main_bytes, st);
}

hipError_t launch_topk_lists(int rows, int H, int max_seq, const int32_t* seq_lens, const float* scores, int k,
                             int32_t* idx, CandSegs lists, int chunk_len, hipStream_t st) {
  if (lists.nseg > kMaxSeg) return hipErrorInvalidValue;
  // Rows of up to about 7.7K list candidates (kc = cap / 2 per segment) are
  // held 8 per thread; a segment of up to 1024 / nseg * 8 is then read
  // directly by its threads. Longer lists 12 per thread.
  if (int64_t(lists.nseg) * (lists.cap / 2) <= 7680)
    hipLaunchKernelGGL((final_kernel<1024, 8, false, true>), dim3(rows), dim3(1024), 0, st, H, max_seq, seq_lens, k,
                       lists, lists.nseg, idx, CandSegs{}, DeltaArgs{}, ListArgs{scores, chunk_len});
  else
    hipLaunchKernelGGL((final_kernel<1024, 12, false, true>), dim3(rows), dim3(1024), 0, st, H, max_seq, seq_lens, k,
                       lists, lists.nseg, idx, CandSegs{}, DeltaArgs{}, ListArgs{scores, chunk_len});
  return hipGetLastError();
}

}  // namespace jssa

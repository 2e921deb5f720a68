// Lossless tile screening of the score stream ("DoSA Makes Sparse Attention
// Selection Conditional Without Approximation", cctest.ai, How the method
// works). The scores of a few seed tokens bound the selection threshold from
// below; a candidate whose score cannot reach that bound is never scored
// exactly, and the selected set stays the same.
//
// The score is one r-dim dot product s_t = qp . Kp_t, so a tile of 64
// consecutive tokens has the box bound ub = sum_c max(qp_c lo_c, qp_c hi_c),
// with lo and hi the per-dimension minimum and maximum of its valid
// projected keys: ub >= s_t for every token of the tile. tau, the k-th
// largest score over the distinct valid seed tokens, is at most the k-th
// score of the sequence, so a tile with ub < tau holds no token of the
// top-k; the score stream then does not read it.
//
//  tile_bounds_kernel  lo/hi per (sequence, KV head, tile) from the
//                      projected cache: every tile (set-up), or only the
//                      tiles holding appended tokens (decode)
//  screen_kernel       one block (1024 threads; 512 for r >= 64) per (sequence, KV head):
//                      qp, the distinct seeds (an LDS hash set) and their
//                      scores, tau, then one keep bit per tile
//
// Both sides of the comparison carry fp32 rounding: the stream scores the
// same token in another order than the seed pass, and ub is an fp32 sum.
// A tile is dropped only when ub + eps * U < tau - eps * S, with U a bound
// on every sum_c |qp_c Kp_c| in the tile ((sum_c |qp_c|) max_c max(|lo_c|,
// |hi_c|) for r <= 48, sum_c |qp_c| max(|lo_c|, |hi_c|) above), S the
// largest such sum over the seeds and eps = 2^-16,
// far above the error of a sum of r <= 128 fp32 terms: a tile that exact
// arithmetic would keep is never dropped.
//
// Bounds layout: tiles in groups of 64; for each group, 16-byte vector v of
// every tile of the group in turn (v < r/8: the minima of dims 8v .. 8v+7,
// else the maxima of dims 8(v - r/8) .. 8(v - r/8)+7). A wave that reads
// vector v of 64 consecutive tiles reads 1 KB of consecutive bytes.
#include "internal.hpp"

namespace jssa {
namespace {

constexpr int kTile = 64;
constexpr int kMaxSeed = 4096;
constexpr int kSeedTableBits = 13;                  // 2 * kMaxSeed slots
constexpr int kSeedTable = 1 << kSeedTableBits;
// threads per block: 1024, or 512 for the wide ranks (register room for a
// whole projected row per seed); one histogram bin per thread
constexpr int screen_threads(int R) { return R >= 64 ? 512 : 1024; }
constexpr float kScreenEps = 1.0f / 65536.0f;

// index (in 16-byte vectors) of vector v of a tile; row = b * Hkv + j
__device__ __forceinline__ int64_t bound_vec(int64_t row, int ngroups, int nv2, int tile, int v) {
  return ((row * ngroups + (tile >> 6)) * nv2 + v) * 64 + (tile & 63);
}

// One wave per tile, four tiles per block. pos == nullptr: tile 4x + w of
// block x (set-up, every tile). Otherwise the (4x + w)-th tile holding one
// of the tokens pos[b] .. pos[b] + n_tok - 1 that lie in [0, max_seq) (an
// append); waves past the last such tile only take part in the barrier.
// Lane (row group rg, vector v) loads 16-byte vector v of rows rg, rg + RG,
// ... of the tile, all loads in flight at once (rows past T_b or without a
// valid page read row 0 of the cache and are left out); the row groups'
// minima and maxima then meet in LDS.
template <int R>
__global__ __launch_bounds__(256) void tile_bounds_kernel(GqaDev g, const uint16_t* __restrict__ Kp,
                                                           uint16_t* __restrict__ bounds, int ntiles,
                                                           const int32_t* __restrict__ pos, int n_tok) {
  constexpr int NV = R / 8, RG = 64 / NV, NI = (kTile + RG - 1) / RG;   // row groups, loads per lane
  __shared__ float part[4][2][RG][R];
  const int j = blockIdx.y, b = blockIdx.z, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int Tb = seq_len(g, b);
  int tile = int(blockIdx.x) * 4 + w;
  bool valid = tile < ntiles;
  if (pos) {
    const int64_t t0 = pos[b], t1 = t0 + n_tok - 1;    // first and last appended token
    const int first = int((t0 > 0 ? t0 : 0) / kTile);
    const int last = int((t1 < g.max_seq - 1 ? t1 : g.max_seq - 1) / kTile);
    tile += first;
    valid = t1 >= 0 && t0 < g.max_seq && tile <= last;
  }
  const int v = lane % NV, rg = lane / NV;
  float lo[8], hi[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { lo[e] = __builtin_inff(); hi[e] = -__builtin_inff(); }
  if (valid && rg < RG) {
    u32x4 x[NI];
    bool ok[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = rg + RG * i, t = tile * kTile + r;
      const int64_t off = (r < kTile && t < Tb) ? row_off(g, b, j, t, R) : -1;
      ok[i] = off >= 0;
      x[i] = *reinterpret_cast<const u32x4*>(Kp + (ok[i] ? off : 0) + 8 * v);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (!ok[i]) continue;
      const uint32_t wd[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = (e & 1) ? bf_hi(wd[e >> 1]) : bf_lo(wd[e >> 1]);
        lo[e] = f < lo[e] ? f : lo[e];
        hi[e] = f > hi[e] ? f : hi[e];
      }
    }
  }
  if (rg < RG) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      part[w][0][rg][8 * v + e] = lo[e];
      part[w][1][rg][8 * v + e] = hi[e];
    }
  }
  __syncthreads();
  if (!valid) return;
  const int ngroups = (ntiles + 63) / 64, row = b * g.Hkv + j;
  for (int c = lane; c < R; c += 64) {
    float l = __builtin_inff(), h = -__builtin_inff();
#pragma unroll
    for (int q = 0; q < RG; ++q) {
      l = fminf(l, part[w][0][q][c]);
      h = fmaxf(h, part[w][1][q][c]);
    }
    // min and max of bf16 values are bf16 values: the conversion is exact
    // (and +-inf for a tile without a valid token)
    bounds[bound_vec(row, ngroups, 2 * NV, tile, c / 8) * 8 + c % 8] = uint16_t(__float_as_uint(l) >> 16);
    bounds[bound_vec(row, ngroups, 2 * NV, tile, NV + c / 8) * 8 + c % 8] = uint16_t(__float_as_uint(h) >> 16);
  }
}

template <int R>
__global__ __launch_bounds__(screen_threads(R)) void screen_kernel(GqaDev g, const uint16_t* __restrict__ q,
                                                           const float* __restrict__ P,
                                                           const uint16_t* __restrict__ Kp,
                                                           const uint16_t* __restrict__ bounds, int ntiles,
                                                           const int32_t* __restrict__ seeds, int n_seed, int k,
                                                           uint32_t* __restrict__ keep, int nwords,
                                                           int32_t* __restrict__ kept_tiles) {
  constexpr int NT = screen_threads(R), NW = NT / 64;
  constexpr int kScrBins = NT, kScrBits = NT == 1024 ? 10 : 9;
  constexpr int NS = NT / R, NI = (128 + NS - 1) / NS; // P row slices and rows per slice
  __shared__ float qbar[128];
  __shared__ float qp[128];
  __shared__ uint32_t qsel[64];                         // per dim pair: 0xffff halves where qp_c > 0
  __shared__ float qpart[NS][R];
  __shared__ int32_t table[kSeedTable];                 // distinct seed tokens (open addressing)
  __shared__ uint32_t hist[kScrBins];
  __shared__ ScanSmem<NT> scan;
  __shared__ int res[2];
  __shared__ uint32_t red[3][NW];
  const int row = blockIdx.x, b = row / g.Hkv, j = row % g.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int Tb = seq_len(g, b);

  // qp = P_j^T (sum of the group's query rows), fp32: thread (slice sl,
  // column c) holds rows sl, sl + NS, ... of P's column c; its loads go out
  // with the query rows and the seed indices, in one round trip
  const int pc = tid % R, sl = tid / R;                 // threads with sl >= NS take no part
  float pv[NI];
#pragma unroll
  for (int ii = 0; ii < NI; ++ii) {
    const int i = sl + ii * NS;
    pv[ii] = (sl < NS && i < 128) ? P[(int64_t(j) * 128 + i) * R + pc] : 0.f;
  }
  constexpr int SPT = kMaxSeed / NT;
  int st[SPT];
  bool mine[SPT];
#pragma unroll
  for (int x = 0; x < SPT; ++x) {
    const int i = tid + x * NT;
    st[x] = i < n_seed ? seeds[int64_t(row) * n_seed + i] : -1;
    mine[x] = false;
  }
  // the group's query rows, by the first two waves: up to 8 rows with all
  // loads in flight (heads past G re-read the last one), the rest after
  constexpr int NV = R / 8;
  constexpr int kQh = 8;
  if (__builtin_amdgcn_readfirstlane(wv) < 2) {         // wave-uniform: tid < 128
    const uint16_t* qg = q + (int64_t(b) * g.Hq + int64_t(j) * g.G) * 128 + tid;
    uint16_t qv[kQh];
#pragma unroll
    for (int h = 0; h < kQh; ++h) qv[h] = qg[(h < g.G ? h : g.G - 1) * 128];
    float qs = 0.f;
#pragma unroll
    for (int h = 0; h < kQh; ++h) qs += h < g.G ? bf(qv[h]) : 0.f;
    for (int h = kQh; h < g.G; ++h) qs += bf(qg[h * 128]);
    qbar[tid] = qs;
  }
  for (int i = tid; i < kSeedTable; i += NT) table[i] = -1;
  __syncthreads();
  if (sl < NS) {
    float s = 0.f;
#pragma unroll
    for (int ii = 0; ii < NI; ++ii) {
      const int i = sl + ii * NS;
      s = __builtin_fmaf(pv[ii], qbar[i < 128 ? i : 127], s);
    }
    qpart[sl][pc] = s;
  }
  // seeds: each valid token enters the table once; the thread that inserts
  // it scores it, so repeated entries count once
#pragma unroll
  for (int x = 0; x < SPT; ++x) {
    const int t = st[x];
    if (t < 0 || t >= Tb) continue;
    uint32_t h = (uint32_t(t) * 2654435761u) >> (32 - kSeedTableBits);
    for (;;) {                                          // at most kMaxSeed entries in 2 * kMaxSeed slots
      const int old = atomicCAS(&table[h], -1, t);
      if (old == -1) { mine[x] = true; break; }
      if (old == t) break;
      h = (h + 1) & (kSeedTable - 1);
    }
  }
  __syncthreads();                                      // qpart complete
  if (tid < R) {
    float s = 0.f;
    for (int x = 0; x < NS; ++x) s += qpart[x][tid];
    qp[tid] = s;
    const float s1 = __shfl_down(s, 1, 64);
    if ((tid & 1) == 0) qsel[tid >> 1] = (s > 0.f ? 0xffffu : 0u) | (s1 > 0.f ? 0xffff0000u : 0u);
  }
  __syncthreads();                                      // qp complete
  uint32_t skey[SPT];
  uint32_t kmax = 0u, kmin = 0xffffffffu;
  float amax = 0.f;
  int nvalid = 0;
#pragma unroll
  for (int x = 0; x < SPT; ++x) {
    skey[x] = 0u;
    if (!mine[x]) continue;
    const int64_t off = row_off(g, b, j, st[x], R);
    if (off < 0) continue;                              // no valid page
    const u32x4* rowp = reinterpret_cast<const u32x4*>(Kp + off);
    u32x4 rv[NV];
#pragma unroll
    for (int c8 = 0; c8 < NV; ++c8) rv[c8] = rowp[c8];   // the row's loads all in flight
    float s = 0.f, a = 0.f;
#pragma unroll
    for (int c8 = 0; c8 < R / 8; ++c8) {
      const u32x4 v = rv[c8];
      const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = bf_lo(wd[e]), x1 = bf_hi(wd[e]);
        const float q0 = qp[c8 * 8 + 2 * e], q1 = qp[c8 * 8 + 2 * e + 1];
        s = __builtin_fmaf(q0, x0, s);
        s = __builtin_fmaf(q1, x1, s);
        a = __builtin_fmaf(__builtin_fabsf(q0), __builtin_fabsf(x0), a);
        a = __builtin_fmaf(__builtin_fabsf(q1), __builtin_fabsf(x1), a);
      }
    }
    skey[x] = score_key(s);
    amax = a > amax ? a : amax;
    kmax = skey[x] > kmax ? skey[x] : kmax;
    kmin = skey[x] < kmin ? skey[x] : kmin;
    ++nvalid;
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t x1 = uint32_t(__shfl_xor(int(kmax), o, 64));
    const uint32_t x2 = uint32_t(__shfl_xor(int(kmin), o, 64));
    kmax = x1 > kmax ? x1 : kmax;
    kmin = x2 < kmin ? x2 : kmin;
    amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  }
  int nv_tot;
  block_scan<NT>(nvalid, scan, &nv_tot);
  if (lane == 0) {
    red[0][wv] = kmax;
    red[1][wv] = kmin;
    red[2][wv] = __float_as_uint(amax);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    kmax = red[0][i] > kmax ? red[0][i] : kmax;
    kmin = red[1][i] < kmin ? red[1][i] : kmin;
    amax = fmaxf(amax, __uint_as_float(red[2][i]));
  }

  // tau: the lower edge of the bin holding the k-th largest seed key, over
  // two levels of linear bins (at least k distinct seeds lie at or above it,
  // so it is at or below the k-th largest score)
  const bool screen = nv_tot >= k && k > 0;             // block-uniform
  float tau_lo = -__builtin_inff();
  if (screen && nv_tot == k) {
    // exactly k distinct valid seeds (a previous selection of the same k):
    // the k-th largest is the smallest
    tau_lo = key_score(kmin) - kScreenEps * amax;
  } else if (screen) {
    uint64_t lo = kmin, hi = kmax;
    int rem = k;
    for (int level = 0; level < 2; ++level) {
      const uint64_t range = hi - lo;
      const int sh = range < uint64_t(kScrBins) ? 0 : (64 - __builtin_clzll(range)) - kScrBits;
      for (int i = tid; i < kScrBins; i += NT) hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int x = 0; x < SPT; ++x)
        if (skey[x] != 0u && skey[x] >= lo && skey[x] <= hi) atomicAdd(&hist[(skey[x] - lo) >> sh], 1u);
      __syncthreads();
      pick_bin<NT, kScrBins / NT>(hist, rem, true, scan, res);
      const uint64_t D = uint64_t(res[0]);
      rem -= res[1];
      const uint64_t blo = lo + (D << sh);
      const uint64_t bhi = blo + (uint64_t(1) << sh) - 1;
      lo = blo;
      hi = bhi < hi ? bhi : hi;
      __syncthreads();
      if (sh == 0) break;
    }
    tau_lo = key_score(uint32_t(lo)) - kScreenEps * amax;
  }

  const int nt_row = (Tb + kTile - 1) / kTile, ngroups = (ntiles + 63) / 64;
  // vector v of a tile: the row's base plus v KB (uniform, scalar registers)
  // plus the tile's 32-bit byte offset (one vector register for all v)
  const char* bdr = reinterpret_cast<const char*>(bounds) + int64_t(row) * ngroups * 2 * NV * 64 * 16;
  auto toff = [&](int tile) { return uint32_t(((tile >> 6) * 2 * NV * 64 + (tile & 63)) * 16); };
  auto bvec = [&](uint32_t off, int v) { return *reinterpret_cast<const u32x4*>(bdr + v * 1024 + off); };
  // one keep bit per tile; tiles past the sequence or without a valid token
  // (bounds +inf / -inf in every dim) are dropped.
  //  ranks <= 48: for l <= h, max(q l, q h) is q h when q > 0, else q l: one
  //    bit-select per pair of packed bf16 bounds, then one fma per dim;
  //    max |bound| is tracked on the packed magnitudes (unsigned 16-bit order
  //    is magnitude order for bf16) and the margin is eps (sum |qp|) max|b|.
  //  ranks >= 64 (fewer registers per thread for the loaded bounds): ub as
  //    sum max(q l, q h), the margin eps sum |q| max(|l|, |h|).
  constexpr bool kPacked = R <= 48;
  float qabs = 0.f;
#pragma unroll 8
  for (int c = 0; c < R; ++c) qabs += __builtin_fabsf(qp[c]);
  int kept = 0;
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  // qo: a zero the compiler cannot see through, so that the coefficient
  // reads stay inside the loop over tiles instead of occupying registers
  // for the whole loop
  auto add_bounds = [&](const u32x4& lv, const u32x4& hv, int c8, int qo, float& ub, float& mag) {
    const uint32_t lw[4] = {lv.x, lv.y, lv.z, lv.w}, hw[4] = {hv.x, hv.y, hv.z, hv.w};
    if constexpr (kPacked) {
      uint32_t mw = __float_as_uint(mag);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t qs = qsel[qo + c8 * 4 + e];
        const uint32_t sel = (qs & hw[e]) | (~qs & lw[e]);
        ub = __builtin_fmaf(qp[qo + c8 * 8 + 2 * e], bf_lo(sel), ub);
        ub = __builtin_fmaf(qp[qo + c8 * 8 + 2 * e + 1], bf_hi(sel), ub);
        u16x2 mm = __builtin_bit_cast(u16x2, mw);
        mm = __builtin_elementwise_max(mm, __builtin_bit_cast(u16x2, lw[e] & 0x7fff7fffu));
        mm = __builtin_elementwise_max(mm, __builtin_bit_cast(u16x2, hw[e] & 0x7fff7fffu));
        mw = __builtin_bit_cast(uint32_t, mm);
      }
      mag = __uint_as_float(mw);                        // two packed magnitudes, not a float
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float l = (e & 1) ? bf_hi(lw[e >> 1]) : bf_lo(lw[e >> 1]);
        const float h = (e & 1) ? bf_hi(hw[e >> 1]) : bf_lo(hw[e >> 1]);
        const float qc = qp[c8 * 8 + e];
        ub += fmaxf(qc * l, qc * h);
        mag = __builtin_fmaf(__builtin_fabsf(qc), fmaxf(__builtin_fabsf(l), __builtin_fabsf(h)), mag);
      }
    }
  };
  // the tile test without the empty check
  auto keep_bound = [&](float ub, float mag) {
    float margin;
    if constexpr (kPacked) {
      const uint32_t mw = __float_as_uint(mag);
      margin = qabs * fmaxf(bf_lo(mw), bf_hi(mw));
    } else {
      margin = mag;
    }
    return !screen || ub + kScreenEps * margin >= tau_lo;
  };
  auto emit = [&](int base, bool k_it) {
    const uint64_t bits = __ballot(k_it);
    kept += k_it ? 1 : 0;
    if (lane == 0) {
      const int wbase = (base + wv * 64) / 32;
      if (wbase < nwords) keep[int64_t(row) * nwords + wbase] = uint32_t(bits);
      if (wbase + 1 < nwords) keep[int64_t(row) * nwords + wbase + 1] = uint32_t(bits >> 32);
    }
  };
  for (int base = 0; base < nwords * 32; base += NT) {
    const int tile = base + tid;
    bool k_it = false;
    if (tile < nt_row && tile < ntiles) {
      // in groups of vectors (all of them up to rank 48, 4 per half above),
      // each group's loads all in flight before use
      constexpr int KC = kPacked ? NV : 4, kGroupUnroll = kPacked ? 8 : 1;
      const uint32_t to = toff(tile);
      float ub = 0.f, mag = 0.f;
      bool empty = false;
      int qo = 0;
      if constexpr (kPacked) asm volatile("s_mov_b32 %0, 0" : "=s"(qo));
      // (ranks >= 64: a rolled loop over the groups keeps one group's
      // bounds and coefficients in registers at a time)
#pragma unroll kGroupUnroll
      for (int c0 = 0; c0 < NV; c0 += KC) {
        u32x4 lv[KC], hv[KC];
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          lv[c] = bvec(to, c0 + c);
          hv[c] = bvec(to, NV + c0 + c);
        }
        if (c0 == 0) empty = bf_lo(lv[0].x) > bf_lo(hv[0].x);   // a valid token makes lo <= hi in dim 0
#pragma unroll
        for (int c = 0; c < KC; ++c) add_bounds(lv[c], hv[c], c0 + c, qo, ub, mag);
      }
      k_it = !empty && keep_bound(ub, mag);
    }
    emit(base, k_it);
  }
  if (kept_tiles) {
    int tot;
    block_scan<NT>(kept, scan, &tot);
    if (tid == 0) kept_tiles[row] = tot;
  }
}

}  // namespace

int screen_tiles(int max_seq) { return (max_seq + kTile - 1) / kTile; }
int screen_words(int max_seq) { return 2 * ((screen_tiles(max_seq) + 63) / 64); }
int screen_max_seeds() { return kMaxSeed; }

hipError_t launch_tile_bounds(const GqaDev& g, const uint16_t* Kp, uint16_t* bounds, const int32_t* pos,
                              int n_tok, hipStream_t st) {
  const int nt = screen_tiles(g.max_seq);
  // n_tok tokens from any start touch at most ceil(n_tok / 64) + 1 tiles
  int n = pos ? (n_tok + kTile - 1) / kTile + 1 : nt;
  n = n < nt ? n : nt;
  const dim3 grid((n + 3) / 4, g.Hkv, g.B);
  switch (g.r) {
#define JSSA_TB(RR)                                                                                      \
  case RR:                                                                                               \
    hipLaunchKernelGGL(tile_bounds_kernel<RR>, grid, dim3(256), 0, st, g, Kp, bounds, nt, pos, n_tok); \
    break;
    JSSA_TB(16) JSSA_TB(32) JSSA_TB(48) JSSA_TB(64) JSSA_TB(128)
#undef JSSA_TB
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_screen(const GqaDev& g, const uint16_t* q, const float* P, const uint16_t* Kp,
                         const uint16_t* bounds, const int32_t* seeds, int n_seed, int k, uint32_t* keep,
                         int32_t* kept_tiles, hipStream_t st) {
  switch (g.r) {
#define JSSA_SCR(RR)                                                                                        \
  case RR:                                                                                                  \
    hipLaunchKernelGGL(screen_kernel<RR>, dim3(g.B * g.Hkv), dim3(screen_threads(RR)), 0, st, g, q, P, Kp, bounds, \
                       screen_tiles(g.max_seq), seeds, n_seed, k, keep, screen_words(g.max_seq), kept_tiles); \
    break;
    JSSA_SCR(16) JSSA_SCR(32) JSSA_SCR(48) JSSA_SCR(64) JSSA_SCR(128)
#undef JSSA_SCR
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace jssa

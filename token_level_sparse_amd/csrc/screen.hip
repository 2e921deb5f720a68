// Lossless tile screening of the score stream ("DoSA Makes Sparse Attention
// Selection Conditional Without Approximation", cctest.ai, How the method
// works: a seed set gives a lower bound on the winning threshold, and
// candidates whose upper bound falls below it are dropped before exact
// scoring, leaving the top-k unchanged).
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
//                      projected cache, once and after appends (setup work)
//  screen_kernel       one block per (sequence, KV head): qp, the seeds'
//                      scores, tau, then one keep bit per tile
//
// Both sides of the comparison carry fp32 rounding: the stream scores the
// same token in another order than the seed pass, and ub is an fp32 sum.
// A tile is dropped only when ub + eps * U < tau - eps * S, with U the
// tile's sum_c |qp_c| max(|lo_c|, |hi_c|) (a bound on every sum_c |qp_c
// Kp_c| in the tile), S the largest such sum over the seeds and eps = 2^-16,
// far above the error of a sum of r <= 128 fp32 terms: a tile that exact
// arithmetic would keep is never dropped.
#include "internal.hpp"

namespace jssa {
namespace {

constexpr int kTile = 64;
constexpr int kMaxSeed = 4096;
constexpr int kScreenNT = 256;
constexpr int kScrBins = 256;
constexpr float kScreenEps = 1.0f / 65536.0f;

__global__ __launch_bounds__(64) void tile_bounds_kernel(GqaDev g, const uint16_t* __restrict__ Kp,
                                                          uint16_t* __restrict__ bounds, int ntiles) {
  const int tile = blockIdx.x, j = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int Tb = seq_len(g, b);
  const int R = g.r;
  uint16_t* dst = bounds + ((int64_t(b) * g.Hkv + j) * ntiles + tile) * 2 * R;
  for (int c0 = 0; c0 < R; c0 += 64) {
    const int c = c0 + lane;
    float lo = __builtin_inff(), hi = -__builtin_inff();
    if (c < R) {
      // 16 rows at a time, every load issued before any is used (rows past
      // T_b or without a valid page read row 0 of the tile's sequence head
      // and are left out)
      for (int i0 = 0; i0 < kTile; i0 += 16) {
        float v[16];
        bool ok[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int t = tile * kTile + i0 + i;
          int64_t off = t < Tb ? row_off(g, b, j, t, R) : -1;
          ok[i] = off >= 0;
          off = ok[i] ? off : row_off(g, b, j, 0, R);
          v[i] = off >= 0 ? bf(Kp[off + c]) : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (!ok[i]) continue;
          lo = v[i] < lo ? v[i] : lo;
          hi = v[i] > hi ? v[i] : hi;
        }
      }
      // min and max of bf16 values are bf16 values: the conversion is exact
      // (and +-inf for a tile without a valid token)
      dst[c] = uint16_t(__float_as_uint(lo) >> 16);
      dst[R + c] = uint16_t(__float_as_uint(hi) >> 16);
    }
  }
}

__global__ __launch_bounds__(kScreenNT) void screen_kernel(GqaDev g, const uint16_t* __restrict__ q,
                                                           const float* __restrict__ P,
                                                           const uint16_t* __restrict__ Kp,
                                                           const uint16_t* __restrict__ bounds, int ntiles,
                                                           const int32_t* __restrict__ seeds, int n_seed, int k,
                                                           uint32_t* __restrict__ keep, int nwords,
                                                           int32_t* __restrict__ kept_tiles) {
  constexpr int NT = kScreenNT, NW = NT / 64;
  __shared__ float qbar[128];
  __shared__ float qp[128];
  __shared__ int32_t sidx[kMaxSeed];
  __shared__ uint32_t hist[kScrBins];
  __shared__ ScanSmem<NT> scan;
  __shared__ int res[2];
  __shared__ uint32_t red[3][NW];
  const int row = blockIdx.x, b = row / g.Hkv, j = row % g.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int R = g.r, Tb = seq_len(g, b);

  // qp = P_j^T (sum of the group's query rows), fp32
  if (tid < 128) {
    float s = 0.f;
    for (int h = 0; h < g.G; ++h) s += bf(q[(int64_t(b) * g.Hq + int64_t(j) * g.G + h) * 128 + tid]);
    qbar[tid] = s;
  }
  // the seeds of this row, sorted ascending (bitonic, padded with INT_MAX) so
  // that repeated entries can be counted once
  int npow = 1;
  while (npow < n_seed) npow <<= 1;
  for (int i = tid; i < npow; i += NT) {
    int t = i < n_seed ? seeds[int64_t(row) * n_seed + i] : 0x7fffffff;
    sidx[i] = t;
  }
  __syncthreads();
  if (tid < R) {
    float s = 0.f;
    for (int i = 0; i < 128; ++i) s = __builtin_fmaf(P[(int64_t(j) * 128 + i) * R + tid], qbar[i], s);
    qp[tid] = s;
  }
  for (int size = 2; size <= npow; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < npow / 2; i += NT) {
        const int lo = 2 * i - (i & (stride - 1)), hi = lo + stride;
        const bool up = (lo & size) == 0;
        const int a = sidx[lo], c = sidx[hi];
        if ((a > c) == up) {
          sidx[lo] = c;
          sidx[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  __syncthreads();

  // score each distinct valid seed (key 0: none); S = the largest sum |qp_c Kp_c|
  constexpr int SPT = kMaxSeed / NT;
  uint32_t skey[SPT];
  uint32_t kmax = 0u, kmin = 0xffffffffu;
  float amax = 0.f;
  int nvalid = 0;
#pragma unroll
  for (int x = 0; x < SPT; ++x) {
    const int i = tid + x * NT;
    skey[x] = 0u;
    if (i < n_seed) {
      const int t = sidx[i];
      const bool first = i == 0 || sidx[i - 1] != t;
      if (first && t >= 0 && t < Tb) {
        const int64_t off = row_off(g, b, j, t, R);
        if (off >= 0) {
          float s = 0.f, a = 0.f;
          for (int c = 0; c < R; ++c) {
            const float v = bf(Kp[off + c]);
            s = __builtin_fmaf(qp[c], v, s);
            a = __builtin_fmaf(__builtin_fabsf(qp[c]), __builtin_fabsf(v), a);
          }
          skey[x] = score_key(s);
          amax = a > amax ? a : amax;
          kmax = skey[x] > kmax ? skey[x] : kmax;
          kmin = skey[x] < kmin ? skey[x] : kmin;
          ++nvalid;
        }
      }
    }
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
  // two levels of 256 linear bins (at least k distinct seeds lie at or above
  // it, so it is at or below the k-th largest score)
  bool screen = nv_tot >= k && k > 0;                   // block-uniform
  float tau_lo = -__builtin_inff();
  if (screen) {
    uint64_t lo = kmin, hi = kmax;
    int rem = k;
    for (int level = 0; level < 2; ++level) {
      const uint64_t range = hi - lo;
      const int sh = range < uint64_t(kScrBins) ? 0 : (64 - __builtin_clzll(range)) - 8;
      hist[tid] = 0u;
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
    const float tau = key_score(uint32_t(lo));
    tau_lo = tau - kScreenEps * amax;
  }

  // one keep bit per tile; tiles past the sequence or without a valid token
  // are dropped
  const int nt_row = (Tb + kTile - 1) / kTile;
  int kept = 0;
  for (int base = 0; base < nwords * 32; base += NT) {
    const int tile = base + tid;
    bool k_it = false;
    if (tile < nt_row && tile < ntiles) {
      const uint16_t* bd = bounds + ((int64_t(b) * g.Hkv + j) * ntiles + tile) * 2 * R;
      float ub = 0.f, U = 0.f;
      bool empty = false;
      for (int c = 0; c < R; ++c) {
        const float l = bf(bd[c]), h = bf(bd[R + c]);
        empty = empty || l > h;
        ub += fmaxf(qp[c] * l, qp[c] * h);
        U = __builtin_fmaf(__builtin_fabsf(qp[c]), fmaxf(__builtin_fabsf(l), __builtin_fabsf(h)), U);
      }
      k_it = !empty && (!screen || ub + kScreenEps * U >= tau_lo);
    }
    const uint64_t bits = __ballot(k_it);
    kept += k_it ? 1 : 0;
    if (lane == 0) {
      const int wbase = (base + wv * 64) / 32;
      if (wbase < nwords) keep[int64_t(row) * nwords + wbase] = uint32_t(bits);
      if (wbase + 1 < nwords) keep[int64_t(row) * nwords + wbase + 1] = uint32_t(bits >> 32);
    }
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

hipError_t launch_tile_bounds(const GqaDev& g, const uint16_t* Kp, uint16_t* bounds, hipStream_t st) {
  const int nt = screen_tiles(g.max_seq);
  hipLaunchKernelGGL(tile_bounds_kernel, dim3(nt, g.Hkv, g.B), dim3(64), 0, st, g, Kp, bounds, nt);
  return hipGetLastError();
}

hipError_t launch_screen(const GqaDev& g, const uint16_t* q, const float* P, const uint16_t* Kp,
                         const uint16_t* bounds, const int32_t* seeds, int n_seed, int k, uint32_t* keep,
                         int32_t* kept_tiles, hipStream_t st) {
  hipLaunchKernelGGL(screen_kernel, dim3(g.B * g.Hkv), dim3(kScreenNT), 0, st, g, q, P, Kp, bounds,
                     screen_tiles(g.max_seq), seeds, n_seed, k, keep, screen_words(g.max_seq), kept_tiles);
  return hipGetLastError();
}

}  // namespace jssa

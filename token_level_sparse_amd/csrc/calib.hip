// Second moments for subspace calibration (JSSA abstract on weekinpapers,
// Abstract: the shared query-key subspace is the closed-form spectral
// solution of a marginal bound on the token-score preservation error). The
// bound depends on the second moment S_q of the group-summed decode queries
// and S_k of the keys only; these kernels compute both, per KV head, on the
// GPU. The spectral step (a 128 x 128 symmetric eigenproblem per head) runs
// on the host (calib_host.cpp).
//
// Key moments: S_k[j] = (1/N_j) sum over the valid tokens of KV head j, in
// every sequence, of k k^T (d = 128). It is the Gram matrix X^T X of the
// head's cache rows: one pass over the K cache, 32K flops per 256-byte row
// (128 flop/byte, below the bf16 MFMA ridge of ~312), so HBM bounds it and
// v_mfma_f32_16x16x32_bf16 (exact bf16 products, fp32 sums) keeps up easily.
//
// Wave layout. A step is 32 consecutive rows. Lane L (g = L/16, m = L%16)
// loads rows 8g..8g+7 of the step at dims 8m..8m+7 (eight 16-byte loads;
// each load instruction of the wave reads four whole 256-byte rows) and
// transposes that 8 x 8 bf16 block in registers: w[i] then holds dim 8m+i of
// the lane's eight rows. Read as an MFMA operand, w[i] is both
//   A[m][k] = X[k][8m+i]   (A: 16 x 32, lane m = L%16, k = 8g..8g+7)  and
//   B[k][n] = X[k][8n+i]   (B: 32 x 16, lane n = L%16, k = 8g..8g+7),
// so mfma(w[i], w[jj]) accumulates G[8m+i][8n+jj] for all m, n < 16. The 36
// pairs i <= jj cover the symmetric matrix with no LDS traffic; each lane
// ends with D[4g+v][L%16] (v < 4) of each of the 36 tiles.
//
// Work split: units are (sequence, 8192-token chunk) of one KV head; block p
// of head j takes units p, p + npb, ...; its 4 waves take interleaved steps.
// Each wave writes its 36 tiles and its valid-row count to a partial slot of
// the workspace; a second kernel sums the partials in a fixed order (the
// result does not depend on scheduling), mirrors the off-diagonal tiles and
// divides by N_j.
#include "internal.hpp"

namespace jssa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kCD = 128;              // head dim
constexpr int kCalChunk = 8192;       // tokens per unit
constexpr int kCalWaves = 4;
constexpr int kPairs = 36;            // (i, jj) with i <= jj < 8
constexpr int kTileFloats = kPairs * 256;

__host__ __device__ constexpr int pair_index(int i, int jj) { return i * 8 - i * (i - 1) / 2 + (jj - i); }

__device__ __forceinline__ uint32_t pack_half(uint32_t lo_word, uint32_t hi_word, bool upper) {
  // low 16 bits from lo_word, high 16 bits from hi_word; `upper` picks which
  // bf16 of each word (bits 16..31 instead of 0..15)
  return __builtin_amdgcn_perm(hi_word, lo_word, upper ? 0x07060302u : 0x05040100u);
}

__global__ __launch_bounds__(kCalWaves * 64) void gram_kernel(GqaDev g, const uint16_t* __restrict__ K,
                                                             float* __restrict__ partial,
                                                             int* __restrict__ counts, int npb) {
  __shared__ int pid[kCalChunk / kPage];
  const int j = blockIdx.y, p = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gq = lane >> 4, m = lane & 15;
  const bool paged = g.page_size != 0;
  const int nch = (g.max_seq + kCalChunk - 1) / kCalChunk;
  const int units = g.B * nch;

  f32x4v acc[kPairs];
#pragma unroll
  for (int x = 0; x < kPairs; ++x) acc[x] = f32x4v{0.f, 0.f, 0.f, 0.f};
  int cnt = 0;

  for (int u = p; u < units; u += npb) {                // block-uniform
    const int b = u / nch, t0 = (u % nch) * kCalChunk;
    const int Tb = seq_len(g, b);
    if (t0 >= Tb) continue;
    const int t1 = Tb - t0 < kCalChunk ? Tb : t0 + kCalChunk;
    if (paged) {
      __syncthreads();                                  // previous unit's reads of pid are done
      for (int i = tid; i < kCalChunk / kPage; i += kCalWaves * 64) {
        int t = t0 + i * kPage;
        t = t < t1 ? t : t1 - 1;
        const int pg = g.page_table[int64_t(b) * g.max_pages + (t >> 4)];
        pid[i] = pg >= 0 && pg < g.num_pages ? pg : -1;
      }
      __syncthreads();
    }
    const int64_t ubase = (int64_t(b) * g.Hkv + j) * int64_t(g.max_seq);
    // rows of step s of this wave: t0 + (s*4 + w)*32 + 8*gq + 0..7
    const int nsteps = (t1 - t0 - w * 32 + 127) / 128;  // wave-uniform, may be <= 0
    auto load_step = [&](int s, u32x4 (&v)[8], uint32_t& ok) {
      const int r0 = t0 + (s * kCalWaves + w) * 32 + 8 * gq;   // 8-aligned: one page for all 8 rows
      int64_t rowbase;
      bool pg_ok = true;
      if (!paged) {
        rowbase = ubase;
      } else {
        const int rc = r0 < t1 ? r0 : t1 - 1;
        const int pg = pid[(rc - t0) >> 4];
        pg_ok = pg >= 0;
        rowbase = (int64_t(pg_ok ? pg : 0) * g.Hkv + j) * kPage - (rc & ~(kPage - 1));
      }
      ok = 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = r0 + e;
        const bool valid = t < t1 && pg_ok;
        ok |= valid ? (1u << e) : 0u;
        const int tc = t < t1 ? t : t1 - 1;
        v[e] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(K + (rowbase + tc) * kCD + 8 * m));
      }
    };
    auto compute_step = [&](const u32x4 (&v)[8], uint32_t ok) {
      u32x4 x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool valid = (ok >> e) & 1u;
        x[e] = valid ? v[e] : u32x4{0u, 0u, 0u, 0u};
      }
      u32x4 wv[8];                                      // wv[i].word[p] = rows 2p (low), 2p+1 (high) of dim i
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) wv[i][q] = pack_half(x[2 * q][i >> 1], x[2 * q + 1][i >> 1], i & 1);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, wv[i]);
#pragma unroll
        for (int jj = i; jj < 8; ++jj)
          acc[pair_index(i, jj)] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, wv[jj]), acc[pair_index(i, jj)], 0, 0, 0);
      }
      if (m == 0) cnt += __builtin_popcount(ok);
    };
    // two register buffers rotate: the loads of the next step are in flight
    // while the current one is multiplied (steps past the end read a valid
    // row and are masked out)
    u32x4 va[8], vb[8];
    uint32_t oka, okb;
    if (nsteps > 0) load_step(0, va, oka);
    for (int s = 0; s < nsteps; s += 2) {
      load_step(s + 1, vb, okb);
      compute_step(va, oka);
      if (s + 2 < nsteps) load_step(s + 2, va, oka);
      if (s + 1 < nsteps) compute_step(vb, okb);
    }
  }

  // partial slot of this wave
  const int64_t slot = (int64_t(j) * npb + p) * kCalWaves + w;
  float* dst = partial + slot * kTileFloats;
#pragma unroll
  for (int x = 0; x < kPairs; ++x) {
    f32x4 o = {acc[x][0], acc[x][1], acc[x][2], acc[x][3]};
    *reinterpret_cast<f32x4*>(dst + x * 256 + lane * 4) = o;
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) cnt += __shfl_xor(cnt, o, 64);
  if (lane == 0) counts[slot] = cnt;
}

// out[j] = (sum of the head's partials) / N_j as a full symmetric 128 x 128
// matrix. Block (j, pair): lane L sums its 4 values of tile `pair` over the
// partials in slot order, then writes D[4g+v][L%16] to G[8(4g+v)+i][8n+jj]
// and, off the diagonal tiles, to the mirrored entry.
__global__ __launch_bounds__(64) void gram_reduce_kernel(const float* __restrict__ partial,
                                                         const int* __restrict__ counts, int nslots,
                                                         float* __restrict__ out) {
  const int j = blockIdx.x, x = blockIdx.y, lane = threadIdx.x;
  int i = 0;
  while (pair_index(i, 7) < x) ++i;                     // tile x = (i, jj)
  const int jj = i + (x - pair_index(i, i));
  const float* src = partial + int64_t(j) * nslots * kTileFloats + x * 256 + lane * 4;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  int64_t n = 0;
#pragma unroll 8
  for (int q = 0; q < nslots; ++q) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(src + int64_t(q) * kTileFloats);
    s = s + v;
    n += counts[int64_t(j) * nslots + q];
  }
  const float inv = n > 0 ? float(1.0 / double(n)) : 0.f;
  float* G = out + int64_t(j) * kCD * kCD;
  const int gq = lane >> 4, nn = lane & 15;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int mm = 4 * gq + v;
    const int row = 8 * mm + i, col = 8 * nn + jj;
    const float val = s[v] * inv;
    G[row * kCD + col] = val;
    if (i != jj) G[col * kCD + row] = val;
  }
}

// Query moments: out[j] = (1/N) sum_n qbar_n qbar_n^T, qbar_n the fp32 sum of
// the bf16 query rows of KV head j's group in sample n. Block (j, p) takes
// the samples of slice p (kQSplit slices) 64 at a time through LDS; thread
// tid accumulates the 8 x 8 patch of rows 8(tid/16).., columns 8(tid%16)..
// of its slice's sum, written as a partial; qmoment_reduce_kernel sums the
// slices in order and divides by N.
constexpr int kQSplit = 32;

__global__ __launch_bounds__(256) void qmoment_kernel(int N, int Hq, int Hkv, const uint16_t* __restrict__ q,
                                                      float* __restrict__ partial) {
  __shared__ float qs[64][kCD + 4];
  const int j = blockIdx.x, p = blockIdx.y, tid = threadIdx.x;
  const int G = Hq / Hkv;
  const int per = (N + kQSplit - 1) / kQSplit;
  const int n_lo = p * per, n_hi = N < n_lo + per ? N : n_lo + per;
  const int r0 = 8 * (tid >> 4), c0 = 8 * (tid & 15);
  float acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[a][c] = 0.f;
  for (int n0 = n_lo; n0 < n_hi; n0 += 64) {
    __syncthreads();
    for (int e = tid; e < 64 * kCD; e += 256) {
      const int n = e / kCD, dim = e % kCD;
      float s = 0.f;
      if (n0 + n < n_hi) {
        const uint16_t* row = q + (int64_t(n0 + n) * Hq + int64_t(j) * G) * kCD + dim;
        for (int h = 0; h < G; ++h) s += bf(row[h * kCD]);
      }
      qs[n][dim] = s;
    }
    __syncthreads();
    const int nb = n_hi - n0 < 64 ? n_hi - n0 : 64;
    for (int n = 0; n < nb; ++n) {
      float ra[8], cb[8];
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        ra[a] = qs[n][r0 + a];
        cb[a] = qs[n][c0 + a];
      }
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[a][c] = __builtin_fmaf(ra[a], cb[c], acc[a][c]);
    }
  }
  float* dst = partial + (int64_t(j) * kQSplit + p) * kCD * kCD;
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    f32x4 lo = {acc[a][0], acc[a][1], acc[a][2], acc[a][3]};
    f32x4 hi = {acc[a][4], acc[a][5], acc[a][6], acc[a][7]};
    *reinterpret_cast<f32x4*>(dst + (r0 + a) * kCD + c0) = lo;
    *reinterpret_cast<f32x4*>(dst + (r0 + a) * kCD + c0 + 4) = hi;
  }
}

__global__ __launch_bounds__(256) void qmoment_reduce_kernel(int N, const float* __restrict__ partial,
                                                             float* __restrict__ out) {
  const int j = blockIdx.x;
  const int e = blockIdx.y * 256 + threadIdx.x;        // element of the 128 x 128 matrix
  float s = 0.f;
#pragma unroll 8
  for (int p = 0; p < kQSplit; ++p) s += partial[(int64_t(j) * kQSplit + p) * kCD * kCD + e];
  out[int64_t(j) * kCD * kCD + e] = N > 0 ? s * float(1.0 / double(N)) : 0.f;
}

}  // namespace

int calib_blocks_per_head(int Hkv) { return Hkv >= 512 ? 1 : 512 / Hkv; }

size_t calib_workspace_bytes(int Hkv) {
  const size_t slots = size_t(Hkv) * calib_blocks_per_head(Hkv) * kCalWaves;
  return align256(slots * kTileFloats * sizeof(float)) + align256(slots * sizeof(int));
}

hipError_t launch_calib_key_moments(const GqaDev& g, const uint16_t* K, float* out, void* ws, hipStream_t st) {
  const int npb = calib_blocks_per_head(g.Hkv);
  const size_t slots = size_t(g.Hkv) * npb * kCalWaves;
  float* partial = static_cast<float*>(ws);
  int* counts = reinterpret_cast<int*>(static_cast<char*>(ws) + align256(slots * kTileFloats * sizeof(float)));
  hipLaunchKernelGGL(gram_kernel, dim3(npb, g.Hkv), dim3(kCalWaves * 64), 0, st, g, K, partial, counts, npb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gram_reduce_kernel, dim3(g.Hkv, kPairs), dim3(64), 0, st, partial, counts, npb * kCalWaves, out);
  return hipGetLastError();
}

size_t calib_query_workspace_bytes(int Hkv) { return size_t(Hkv) * kQSplit * kCD * kCD * sizeof(float); }

hipError_t launch_calib_query_moments(int N, int Hq, int Hkv, const uint16_t* q, float* out, void* ws,
                                      hipStream_t st) {
  float* partial = static_cast<float*>(ws);
  hipLaunchKernelGGL(qmoment_kernel, dim3(Hkv, kQSplit), dim3(256), 0, st, N, Hq, Hkv, q, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(qmoment_reduce_kernel, dim3(Hkv, kCD * kCD / 256), dim3(256), 0, st, N, partial, out);
  return hipGetLastError();
}

}  // namespace jssa

// MLA shared-latent path: selection over the shared latent cache and
// attention over the selected latent rows.
//
// On MLA models the selection runs on the one latent cache that every head
// reads (ai4snews digest, Perspective). Per head h the key of token t is
// [W_uk[h] c_t[:512]; c_t[512:]] and its value c_t[:512]; absorbing W_uk into
// the query (q_abs = [W_uk[h]^T q_nope; q_rope]) turns the logits into one
// 576-dim dot per (head, token) and the output into W_uv[h] (sum_t p_t c_t).
// All heads share the latent rows, so with 128 heads the per-token work is a
// genuine dense contraction: QK^T and PV run on bf16 MFMA (gfx950
// v_mfma_f32_16x16x32_bf16). The query enters QK^T, and the softmax weights
// enter PV, as hi + lo pairs of bf16 (two MFMAs each), so logits and weighted
// sums keep ~fp32 accuracy.
#include "internal.hpp"

namespace jssa {
namespace {

constexpr int kDc = 576;        // latent + rope
constexpr int kDl = 512;        // latent (value) width
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int mla_len(const MlaDev& m, int b) {
  if (!m.seq_lens) return m.max_seq;
  int t = m.seq_lens[b];
  return t < 0 ? 0 : (t > m.max_seq ? m.max_seq : t);
}

// ---------------------------------------------------------------------------
// Kp_lat = bf16_rne(c . P), fp64 accumulation (same rounding argument as the
// GQA key projection), on fp64 MFMA: v_mfma_f64_16x16x4f64 takes A[m][k]
// from lane 16k + m, B[k][n] from lane 16k + n, and leaves D[k' + 4i][n] in
// register i of lane 16k' + n. Block: 64 tokens (16 per wave) x R columns.
// The 576 dims go in 9 chunks of 64; in chunk c, step s, lane group kq
// covers dim 64c + 16kq + s (the same order for A and B), so a lane's A
// values are 16 consecutive dims of its token (32 bytes), and the chunk's
// P rows sit in LDS. The next chunk's A loads are in flight during the
// current chunk's products.
// ---------------------------------------------------------------------------
typedef double f64x4 __attribute__((ext_vector_type(4)));

template <int R>
__global__ __launch_bounds__(256) void mla_project_kernel(MlaDev m, const uint16_t* __restrict__ lat,
                                                          const float* __restrict__ P,
                                                          uint16_t* __restrict__ Kp) {
  static_assert(R % 16 == 0, "columns in tiles of 16");
  constexpr int TOK = 64, CH = 64, NCH = kDc / CH;
  static_assert(kDc % CH == 0, "whole chunks");
  __shared__ __attribute__((aligned(16))) float Pc[CH * R];
  const int b = blockIdx.y, t0 = blockIdx.x * TOK;
  const int Tb = mla_len(m, b);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int mm = lane & 15, kq = lane >> 4;
  const int tok = t0 + 16 * w + mm;                      // this lane's A row
  const bool aval = tok < Tb;
  const uint16_t* arow = lat + (int64_t(b) * m.max_seq + (aval ? tok : 0)) * kDc + 16 * kq;
  auto load_a = [&](int c, u32x4 (&v)[2]) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
      v[q] = aval ? reinterpret_cast<const u32x4*>(arow + c * CH)[q] : u32x4{0u, 0u, 0u, 0u};
  };
  f64x4 acc[R / 16];
#pragma unroll
  for (int ct = 0; ct < R / 16; ++ct) acc[ct] = f64x4{0.0, 0.0, 0.0, 0.0};
  u32x4 av[2], an[2];
  load_a(0, av);
#pragma unroll 1
  for (int c = 0; c < NCH; ++c) {
    load_a(c + 1 < NCH ? c + 1 : c, an);                // (the last chunk reloads itself, unused)
    __syncthreads();                                    // the previous chunk's P rows are read
    for (int e = tid * 4; e < CH * R; e += 256 * 4)
      *reinterpret_cast<f32x4*>(Pc + e) = *reinterpret_cast<const f32x4*>(P + int64_t(c) * CH * R + e);
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < R / 16; ++ct) {
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const uint32_t wd = av[s >> 3][(s >> 1) & 3];
        const double x = double(__uint_as_float((s & 1) ? (wd & 0xffff0000u) : (wd << 16)));
        const double y = double(Pc[(16 * kq + s) * R + 16 * ct + mm]);
        acc[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(x, y, acc[ct], 0, 0, 0);
      }
    }
    av[0] = an[0];
    av[1] = an[1];
  }
#pragma unroll
  for (int ct = 0; ct < R / 16; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 16 * w + kq + 4 * i;
      if (t < Tb) Kp[(int64_t(b) * m.max_seq + t) * R + 16 * ct + mm] = f64_to_bf16_rne(acc[ct][i]);
    }
}

// ---------------------------------------------------------------------------
// Folded selection weights (set-up): U[h][n][c] = sum_d W_uk[h][n][d] P[d][c]
// over the 512 latent dims, in fp64 (bf16 x fp32 products are exact in
// fp64), rounded once to fp32. Since the selection query is linear in the
// absorbed query, P_lat^T sum_h W_uk[h]^T q_nope[b,h] = sum_h U[h]^T
// q_nope[b,h], so the per-step selection query needs U and q_nope only, not
// the absorbed query. Block (h, n), one thread per column c.
// ---------------------------------------------------------------------------
template <int R>
__global__ __launch_bounds__(R) void mla_fold_kernel(const uint16_t* __restrict__ Wuk, const float* __restrict__ P,
                                                     float* __restrict__ U) {
  const int h = blockIdx.x, n = blockIdx.y, c = threadIdx.x;
  const uint16_t* w = Wuk + (int64_t(h) * 128 + n) * kDl;
  double s = 0.0;
  for (int d = 0; d < kDl; ++d) s = __builtin_fma(double(bf(w[d])), double(P[int64_t(d) * R + c]), s);
  U[(int64_t(h) * 128 + n) * R + c] = float(s);
}

// ---------------------------------------------------------------------------
// One launch forms both per-step queries; its two kinds of blocks are
// independent, so the selection query does not wait for the absorbed one.
//
// Selection query, in kMlaSelParts parts (blocks 0 .. kMlaSelParts-1):
// part g covers the heads of class g (h = g, g + 64, ...), q_sel[b,g,:] =
// sum over those heads of (U[h]^T q_nope[b,h] + P_rope^T q_rope[b,h]); the
// score passes add the parts in order, which gives P^T sum_h q_abs[b,h].
// A class's heads go in chunks of 2: 320 reduction rows per chunk (256 rows
// U[h][n] against q_nope[b,h,n], 64 rows P[512 + e] against the chunk's
// rope values summed over its heads in head order). Thread (rq, sl) owns
// columns 4rq .. 4rq+3 and rows sl, sl + NS, ... (all its row loads in
// flight at once, after the query loads); the NS slices meet in LDS in
// order. Fixed summation orders throughout: every call gives the same
// query.
//
// Absorbed query (the other blocks, one per (h, column quarter)):
// q_abs[b,h,c] = sum_i q_nope[b,h,i] W_uk[h,i,c] for c < 512 (fp32), then
// the rope part copied. 128 columns as 64 bf16 pairs; wave w sums rows
// i = 32w .. 32w+31, whose 32 pair loads per lane are issued before any is
// used; the four partial sums meet in LDS. Each W_uk element is read once
// and serves every sequence.
// ---------------------------------------------------------------------------
constexpr int kSelBT = 4;                 // sequences per pass of a selection block
constexpr int kSelHC = 2;                 // heads per chunk
constexpr int kSelRows = kSelHC * 128 + 64;   // reduction rows per chunk
constexpr int kAbsBT = 8;                 // sequences per pass of an absorb block
static_assert(kMlaSelParts == 64, "selection query parts: one per head class h % 64");

template <int R>
__device__ __forceinline__ void mla_sel_part(const MlaDev& m, int g, const uint16_t* __restrict__ qn,
                                             const uint16_t* __restrict__ qr, const float* __restrict__ U,
                                             const float* __restrict__ P, float* __restrict__ qsel) {
  constexpr int NQ = R / 4, NS = 256 / NQ, NU = kSelRows / NS;
  static_assert(kSelRows % NS == 0, "whole rows per slice");
  __shared__ float qs[kSelBT][kSelRows];  // the chunk's query values per row
  __shared__ __attribute__((aligned(16))) float pp[NS][kSelBT][R];   // slice partial sums
  const int tid = threadIdx.x, rq = tid % NQ, sl = tid / NQ;
  const int nh = g < m.H ? (m.H - g + kMlaSelParts - 1) / kMlaSelParts : 0;   // heads of class g
  for (int b0 = 0; b0 < m.B; b0 += kSelBT) {
    const int nb = min(kSelBT, m.B - b0);
    f32x4v acc[kSelBT];
#pragma unroll
    for (int bb = 0; bb < kSelBT; ++bb) acc[bb] = f32x4v{0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < nh; i0 += kSelHC) {
      const int hc = min(kSelHC, nh - i0);              // heads in this chunk
      auto head = [&](int hi) { return g + kMlaSelParts * (i0 + (hi < hc ? hi : 0)); };   // clamped: valid
      // query values (loads clamped to valid rows; values past the chunk or
      // the batch zeroed): q_nope pairs, then rope pairs, one per head
      constexpr int kNP = kSelBT * kSelHC * 64 / 256;   // q_nope pairs per thread
      uint32_t qv[kNP];
#pragma unroll
      for (int u = 0; u < kNP; ++u) {
        const int e = tid + 256 * u, bb = e / (kSelHC * 64), x = 2 * (e % (kSelHC * 64)), hi = x / 128;
        qv[u] = *reinterpret_cast<const uint32_t*>(qn + (int64_t(b0 + (bb < nb ? bb : 0)) * m.H + head(hi)) * 128 +
                                                   x % 128);
      }
      constexpr int kRP = kSelBT * 32 * kSelHC / 256;   // rope pairs per thread
      uint32_t rv[kRP];
#pragma unroll
      for (int u = 0; u < kRP; ++u) {
        const int e = tid + 256 * u, hi = e % kSelHC, pr = (e / kSelHC) % 32, bb = e / (32 * kSelHC);
        rv[u] = *reinterpret_cast<const uint32_t*>(qr + (int64_t(b0 + (bb < nb ? bb : 0)) * m.H + head(hi)) * 64 + 2 * pr);
      }
      f32x4v uv[NU];
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int x = sl + NS * u;
        const float* row = x < kSelHC * 128 ? U + (int64_t(head(x / 128)) * 128 + x % 128) * R
                                             : P + int64_t(512 + x - kSelHC * 128) * R;
        uv[u] = reinterpret_cast<const f32x4v*>(row)[rq];
      }
#pragma unroll
      for (int u = 0; u < kNP; ++u) {
        const int e = tid + 256 * u, bb = e / (kSelHC * 64), x = 2 * (e % (kSelHC * 64)), hi = x / 128;
        const bool ok = bb < nb && hi < hc;
        qs[bb][x] = ok ? bf_lo(qv[u]) : 0.f;
        qs[bb][x + 1] = ok ? bf_hi(qv[u]) : 0.f;
      }
      // rope: the chunk's heads of one (sequence, pair) sit in kSelHC
      // consecutive lanes and are added in head order
      static_assert(kSelHC == 2, "rope sum over lane pairs");
#pragma unroll
      for (int u = 0; u < kRP; ++u) {
        const int e = tid + 256 * u, hi = e % kSelHC, pr = (e / kSelHC) % 32, bb = e / (32 * kSelHC);
        const bool ok = bb < nb && hi < hc;
        const float lo = ok ? bf_lo(rv[u]) : 0.f, hv = ok ? bf_hi(rv[u]) : 0.f;
        const float lo1 = __shfl_down(lo, 1, 2), hv1 = __shfl_down(hv, 1, 2);
        if (hi == 0) {
          qs[bb][kSelHC * 128 + 2 * pr] = lo + lo1;
          qs[bb][kSelHC * 128 + 2 * pr + 1] = hv + hv1;
        }
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int x = sl + NS * u;
#pragma unroll
        for (int bb = 0; bb < kSelBT; ++bb) acc[bb] += qs[bb][x] * uv[u];
      }
      __syncthreads();                                  // qs is rewritten by the next chunk
    }
#pragma unroll
    for (int bb = 0; bb < kSelBT; ++bb) *reinterpret_cast<f32x4v*>(&pp[sl][bb][4 * rq]) = acc[bb];
    __syncthreads();
    for (int e = tid; e < nb * R; e += 256) {
      const int bb = e / R, c = e % R;
      float t = 0.f;
      for (int x = 0; x < NS; ++x) t += pp[x][bb][c];
      qsel[(int64_t(b0 + bb) * kMlaSelParts + g) * R + c] = t;
    }
    __syncthreads();                                    // pp is rewritten by the next pass
  }
}

__device__ __forceinline__ void mla_absorb_block(const MlaDev& m, int h, int cq, const uint16_t* __restrict__ qn,
                                                 const uint16_t* __restrict__ qr, const uint16_t* __restrict__ Wuk,
                                                 float* __restrict__ qa) {
  __shared__ float qs[kAbsBT][128];
  __shared__ float part[4][kAbsBT][128];
  const int tid = threadIdx.x;
  const int cp = tid & 63, w = tid >> 6;
  const uint16_t* W = Wuk + (int64_t(h) * 128 + w * 32) * kDl + cq * 128 + 2 * cp;
  uint32_t wr[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) wr[i] = *reinterpret_cast<const uint32_t*>(W + int64_t(i) * kDl);
  for (int b0 = 0; b0 < m.B; b0 += kAbsBT) {
    const int nb = min(kAbsBT, m.B - b0);
    __syncthreads();
    for (int e = tid; e < kAbsBT * 128; e += 256) {
      const int bb = e / 128, i = e % 128;
      qs[bb][i] = bb < nb ? bf(qn[(int64_t(b0 + bb) * m.H + h) * 128 + i]) : 0.f;
    }
    __syncthreads();
    float acc[kAbsBT][2];
#pragma unroll
    for (int bb = 0; bb < kAbsBT; ++bb) acc[bb][0] = acc[bb][1] = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float w0 = bf_lo(wr[i]), w1 = bf_hi(wr[i]);
#pragma unroll
      for (int bb = 0; bb < kAbsBT; ++bb) {
        const float q = qs[bb][w * 32 + i];
        acc[bb][0] = __builtin_fmaf(q, w0, acc[bb][0]);
        acc[bb][1] = __builtin_fmaf(q, w1, acc[bb][1]);
      }
    }
#pragma unroll
    for (int bb = 0; bb < kAbsBT; ++bb) {
      part[w][bb][2 * cp] = acc[bb][0];
      part[w][bb][2 * cp + 1] = acc[bb][1];
    }
    __syncthreads();
    for (int e = tid; e < nb * 128; e += 256) {
      const int bb = e / 128, c = e % 128;
      const float v = ((part[0][bb][c] + part[1][bb][c]) + part[2][bb][c]) + part[3][bb][c];
      qa[(int64_t(b0 + bb) * m.H + h) * kDc + cq * 128 + c] = v;
    }
    if (cq == 0)
      for (int e = tid; e < nb * 64; e += 256) {
        const int bb = e / 64, j = e % 64;
        qa[(int64_t(b0 + bb) * m.H + h) * kDc + kDl + j] = bf(qr[(int64_t(b0 + bb) * m.H + h) * 64 + j]);
      }
  }
}

template <int R>
__global__ __launch_bounds__(256) void mla_queries_kernel(MlaDev m, const uint16_t* __restrict__ qn,
                                                          const uint16_t* __restrict__ qr,
                                                          const uint16_t* __restrict__ Wuk,
                                                          const float* __restrict__ U, const float* __restrict__ P,
                                                          float* __restrict__ qa, float* __restrict__ qsel) {
  const int x = blockIdx.x;                             // (block-uniform role)
  if (x < kMlaSelParts)
    mla_sel_part<R>(m, x, qn, qr, U, P, qsel);
  else
    mla_absorb_block(m, (x - kMlaSelParts) >> 2, (x - kMlaSelParts) & 3, qn, qr, Wuk, qa);
}

// ---------------------------------------------------------------------------
// Indexed MLA attention on MFMA. Block = 2 waves = 16 heads x one split of
// the selected slots; wave w takes the w-th half of the split's slots, in
// steps of 16 tokens, and the two halves meet in LDS at the end.
//  QK^T: S^T[16 tok x 16 heads] += C[16 tok x 32 dims] . Qt[32 dims x 16 heads]
//        over 18 dim blocks (v_mfma_f32_16x16x32_bf16), twice (q hi and q
//        lo). Lane (n, g) (n = lane % 16, g = lane / 16) supplies dims
//        32 kb + 8g .. +7 of token n of the step, and receives the logits of
//        tokens 4g .. 4g+3 for head n: the A operand of PV below as it is.
//  PV:   O[16 heads x 16 dims] += P[16 heads x 16 tok] . V[16 tok x 16 dims],
//        32 dim tiles (v_mfma_f32_16x16x16_bf16), the weights as hi + lo
//        bf16 pairs. The step's value rows go to the wave's LDS as loaded
//        (row-major, one 16-byte store per piece); the B operand of dim tile
//        t, tokens 4g .. 4g+3 of dim 16 t + n in lane (n, g), comes back with
//        one transposing LDS read (ds_read_b64_tr_b16: within a group of 16
//        lanes, lane 4a + c receives element c of the 8 bytes that lanes 4j + a
//        address, j = 0..3; so lane s of group g addresses token 4g + s / 4,
//        dims 16 t + 4 (s % 4) .. +3).
// Two waves per block and 69 KB of LDS per block keep two blocks, one wave
// per SIMD, on every CU; the query's hi and lo parts sit in LDS once per
// block (both waves serve the same heads), the registers holding the
// accumulators and two steps of row loads.
// ---------------------------------------------------------------------------
constexpr int kVRS = kDl + 8;   // u16 per staged value row (16-byte aligned rows, banks staggered)
constexpr float kLazy = 8.f;    // log2 headroom of the running softmax base

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// x combined with its partner in lane ^ 16 (permlane16_swap: odd 16-lane
// rows of the first register trade places with even rows of the second) or
// lane ^ 32 (permlane32_swap: upper half of the first with lower half of the
// second). Both registers start as x, so afterwards each lane holds {x,
// partner} in some order and max of the pair is the same in both lanes.
// (The pair's elements are copied out by value: bit-casting a vector-element
// lvalue reads element 0.)
__device__ __forceinline__ float max_x16(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  return fmaxf(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}
__device__ __forceinline__ float max_x32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  return fmaxf(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}

__device__ __forceinline__ s16x4 pack_bf16x4(__bf16 a, __bf16 b, __bf16 c, __bf16 d) {
  s16x4 r;
  r[0] = __builtin_bit_cast(short, a);
  r[1] = __builtin_bit_cast(short, b);
  r[2] = __builtin_bit_cast(short, c);
  r[3] = __builtin_bit_cast(short, d);
  return r;
}

__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(1, 1))) void mla_indexed_kernel(
    MlaDev m, const float* __restrict__ qa, const uint16_t* __restrict__ lat, const int32_t* __restrict__ idx, int k,
    int S, float scale, float* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][16 * kVRS];
  __shared__ bf16x8 qhi_s[18][64], qlo_s[18][64];
  __shared__ float xm[2][16], xl[2][16];
  const int s = blockIdx.x, ht = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Tb = mla_len(m, b);
  const int cs = (k + S - 1) / S;
  const int r0 = min(s * cs, k), r1 = min(r0 + cs, k);
  const int hl = ((r1 - r0 + 1) / 2 + 15) / 16 * 16;   // slots per wave, whole steps
  const int w0 = min(r0 + wv * hl, r1), w1 = min(w0 + hl, r1);
  const int h = ht * 16 + n;                            // this lane's head in the QK B operand
  uint16_t* vs = Vs[wv];

  // Row loads are pipelined by steps: while one step's 18 pieces per lane
  // are multiplied, the next step's are in flight, and the slot indices are
  // read a step further ahead, so no wait for an index stands between two
  // steps. No load sits under a data-dependent branch: slots past the wave's
  // range or with an invalid index read token 0 of the sequence (finite
  // data) and are masked out of the softmax.
  const int32_t* irow = idx + int64_t(b) * k;
  const uint16_t* lrow = lat + int64_t(b) * m.max_seq * kDc;
  const int smax = w1 > w0 ? w1 - 1 : 0;               // (a wave without slots reads slot 0, unused)
  auto tok_of = [&](int base) -> int {                 // token of row n of the step at slot base
    const int sl = base + n;
    return irow[sl < w1 ? sl : smax];
  };
  auto rows = [&](int base, int t, bool& ok, u32x4 (&A)[18]) {
    ok = base + n < w1 && t >= 0 && t < Tb;
    const uint16_t* crow = lrow + int64_t(ok ? t : 0) * kDc + 8 * g;
#pragma unroll
    for (int kb = 0; kb < 18; ++kb) A[kb] = *reinterpret_cast<const u32x4*>(crow + kb * 32);
  };
  u32x4 A0[18], A1[18];
  bool ok0 = false, ok1 = false;
  int tb = 0;                                           // token of the step after the current one
  // Prologue loads, all issued unconditionally (clamped and masked: a load
  // under a branch would make the waits after the join count conservatively):
  // the slot indices, the first step's rows, then the query. (An L2 prefetch
  // of the next steps' rows here was measured: the steps did not get faster,
  // they wait on LDS and MFMA latency, not on the rows.)
  const int ta = tok_of(w0);
  tb = tok_of(w0 + 16);
  __builtin_amdgcn_sched_barrier(0);
  rows(w0, ta, ok0, A0);
  const float* qrow = qa + (int64_t(b) * m.H + h) * kDc;
  f32x4v qv[9][2];
#pragma unroll
  for (int j = 0; j < 9; ++j) {
    const f32x4v* p = reinterpret_cast<const f32x4v*>(qrow + (9 * wv + j) * 32 + 8 * g);
    qv[j][0] = p[0];
    qv[j][1] = p[1];
  }
  __builtin_amdgcn_sched_barrier(0);

  // B operand of QK^T (Q^T): lane holds Q[head n][dims kb*32 + 8g .. +8] as
  // hi and lo bf16, kept in LDS (registers go to the accumulators and the
  // loads in flight); wave w converts dim blocks 9w .. 9w+8.
  {
    const float qs = scale * kLog2e;
#pragma unroll
    for (int j = 0; j < 9; ++j) {
      const int kb = 9 * wv + j;
      const f32x4v a = qv[j][0], c = qv[j][1];
      float x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
      bf16x8 hv, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = x[e] * qs;
        const __bf16 hi = __bf16(v);
        hv[e] = hi;
        lo[e] = __bf16(v - float(hi));
      }
      qhi_s[kb][lane] = hv;
      qlo_s[kb][lane] = lo;
    }
  }
  __syncthreads();

  f32x4v O[32];
#pragma unroll
  for (int t = 0; t < 32; ++t) O[t] = f32x4v{0.f, 0.f, 0.f, 0.f};
  float mrun = -__builtin_inff();    // running max for head n (log2 domain), uniform over g
  float lrun = 0.f;                  // partial sum over this lane group's tokens

  // one step: QK^T (stashing the value part transposed), the online softmax
  // update and PV. Four independent accumulator chains (hi/lo x even/odd dim
  // blocks) keep the MFMA pipe busy.
  auto step = [&](const u32x4 (&A)[18], bool ok) {
    f32x4v acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = f32x4v{0.f, 0.f, 0.f, 0.f};
    wave_lds_sync();                                    // the previous step's PV has read vs
#pragma unroll
    for (int kb = 0; kb < 18; ++kb) {
      if (kb < 16) *reinterpret_cast<u32x4*>(&vs[n * kVRS + kb * 32 + 8 * g]) = A[kb];   // value dims
      const bf16x8 a = __builtin_bit_cast(bf16x8, A[kb]);
      acc[kb & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qhi_s[kb][lane], acc[kb & 1], 0, 0, 0);
      acc[2 + (kb & 1)] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qlo_s[kb][lane], acc[2 + (kb & 1)], 0, 0, 0);
    }
    const f32x4v St = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    // St[i] = logit (log2 domain) of head n, token 4g + i; row r's validity
    // is bit r of one ballot (lanes 0..15 hold rows 0..15)
    const uint64_t vm = __ballot(ok);
    float lg[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) lg[i] = ((vm >> (4 * g + i)) & 1ull) ? St[i] : -__builtin_inff();
    float bm = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
    bm = max_x16(bm);                                   // (permlane swaps: no LDS round trip)
    bm = max_x32(bm);
    // Lazy rescaling: the exponent base mrun moves only when a logit exceeds
    // it by more than kLazy (so every weight stays below 2^kLazy, exact in
    // the hi + lo pair and harmless to the fp32 sums), and the 128
    // accumulators are rescaled only on such a move of a head that already
    // holds weight. The base cancels in O / l and enters the lse exactly.
    const bool grow = bm > mrun + kLazy;                // (mrun = -inf: any finite bm)
    const float mnew = grow ? bm : mrun;
    float alpha = 1.f;
    float p[4];
    if (mnew == -__builtin_inff()) {
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = 0.f;
    } else {
      alpha = grow ? __builtin_amdgcn_exp2f(mrun - mnew) : 1.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(lg[i] - mnew);
    }
    const bool held = mrun != -__builtin_inff();         // O of this head is not all zero
    mrun = mnew;
    lrun = lrun * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    if (__ballot(grow && held) != 0) {                  // wave-uniform
      // rescale O: accumulator rows are heads 4g+i; their alpha sits in lane n = 4g+i
      float ar[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
      for (int t = 0; t < 32; ++t) {
        O[t][0] *= ar[0]; O[t][1] *= ar[1]; O[t][2] *= ar[2]; O[t][3] *= ar[3];
      }
    }
    // The weights enter PV as a hi + lo pair of bf16 (two MFMAs), like the
    // query in QK^T: p = hi + lo to about 2^-16 relative, so the weighted sum
    // matches the fp32 denominator lrun instead of carrying bf16 rounding
    // (2^-9 relative per weight).
    __bf16 ph[4], pl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ph[i] = __bf16(p[i]);
      pl[i] = __bf16(p[i] - float(ph[i]));
    }
    const s16x4 pa = pack_bf16x4(ph[0], ph[1], ph[2], ph[3]);
    const s16x4 pb = pack_bf16x4(pl[0], pl[1], pl[2], pl[3]);
    wave_lds_sync();                                    // this step's vs is written
    const uint16_t* vrd = vs + (4 * g + (n >> 2)) * kVRS + 4 * (n & 3);
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vrd + 16 * t));
      O[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, O[t], 0, 0, 0);
      O[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pb, vb, O[t], 0, 0, 0);
    }
  };

  for (int base = w0; base < w1; base += 32) {
    const int tc = tok_of(base + 32);                   // (past the range: clamped, masked)
    rows(base + 16, tb, ok1, A1);
    step(A0, ok0);
    const int td = tok_of(base + 48);
    rows(base + 32, tc, ok0, A0);
    step(A1, ok1);
    tb = td;
  }
  // total softmax denominator of head n over this wave's tokens
  lrun = xor_sum(xor_sum(lrun, 16), 32);

  // The halves meet: wave 0 keeps dims 0..255 (tiles 0..15), wave 1 dims
  // 256..511 (tiles 16..31); each hands the other tiles to the other wave
  // through its own (now free) transposed-value buffer.
  __syncthreads();                                      // both waves are done with their vs
  float* xo = reinterpret_cast<float*>(vs);             // 16 tiles x 64 lanes x 4 = 16 KB
  // (constant indexes into O in both branches: a wave-dependent index would
  // put the accumulators in scratch memory)
  if (wv == 0) {
#pragma unroll
    for (int t = 0; t < 16; ++t) *reinterpret_cast<f32x4v*>(xo + (t * 64 + lane) * 4) = O[16 + t];
  } else {
#pragma unroll
    for (int t = 0; t < 16; ++t) *reinterpret_cast<f32x4v*>(xo + (t * 64 + lane) * 4) = O[t];
  }
  if (g == 0) {
    xm[wv][n] = mrun;
    xl[wv][n] = lrun;
  }
  __syncthreads();
  const float* yo = reinterpret_cast<const float*>(Vs[1 - wv]);
  // O[t][i] is head 4g+i, dim t*16+n
  float fa[4], fb[4], inv[4], lse[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = 4 * g + i;
    const float ma = xm[wv][hh], mb = xm[1 - wv][hh];
    const float la = xl[wv][hh], lb = xl[1 - wv][hh];
    const float M = fmaxf(ma, mb);
    fa[i] = M == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(ma - M);
    fb[i] = M == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mb - M);
    const float L = la * fa[i] + lb * fb[i];
    inv[i] = L > 0.f ? 1.f / L : 0.f;
    lse[i] = L > 0.f ? (M + __builtin_log2f(L)) * kLn2 : -__builtin_inff();
  }
  auto finish = [&](const f32x4v* mine, int keep) {    // mine: this wave's tiles keep .. keep+15
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = ht * 16 + 4 * g + i;
      const int64_t ob = (int64_t(b) * m.H + hh) * S + s;
      float* dst = part_o + ob * kDl;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const float other = yo[(t * 64 + lane) * 4 + i];
        dst[(keep + t) * 16 + n] = (mine[t][i] * fa[i] + other * fb[i]) * inv[i];
      }
      if (wv == 0 && n == 0) part_lse[ob] = lse[i];
    }
  };
  if (wv == 0)
    finish(O, 0);
  else
    finish(O + 16, 16);
}

// ---------------------------------------------------------------------------
// out[b,h,v] = sum_c W_uv[h,v,c] o_lat[b,h,c]. Block (h, quarter of v): each
// wave takes 8 rows of W_uv[h] (lane l holds dims 8l..8l+7 of each, all 8
// rows loaded before any is used) and applies them to every sequence, four
// at a time, reducing each dot over the 64 lanes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mla_up_v_kernel(MlaDev m, const float* __restrict__ olat,
                                                       const uint16_t* __restrict__ Wuv,
                                                       float* __restrict__ out) {
  const int h = blockIdx.x, vq = blockIdx.y, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int v0 = vq * 32 + w * 8;
  const uint16_t* W = Wuv + (int64_t(h) * 128 + v0) * kDl;
  u32x4 wr[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) wr[j] = reinterpret_cast<const u32x4*>(W + int64_t(j) * kDl)[lane];
  for (int b0 = 0; b0 < m.B; b0 += 4) {
    f32x4v o[4][2];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const int b = b0 + bb < m.B ? b0 + bb : m.B - 1;
      const f32x4v* op = reinterpret_cast<const f32x4v*>(olat + (int64_t(b) * m.H + h) * kDl + lane * 8);
      o[bb][0] = op[0];
      o[bb][1] = op[1];
    }
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const u32x4 r = wr[j];
        float a = 0.f;
        a = __builtin_fmaf(o[bb][0].x, bf_lo(r.x), a);
        a = __builtin_fmaf(o[bb][0].y, bf_hi(r.x), a);
        a = __builtin_fmaf(o[bb][0].z, bf_lo(r.y), a);
        a = __builtin_fmaf(o[bb][0].w, bf_hi(r.y), a);
        a = __builtin_fmaf(o[bb][1].x, bf_lo(r.z), a);
        a = __builtin_fmaf(o[bb][1].y, bf_hi(r.z), a);
        a = __builtin_fmaf(o[bb][1].z, bf_lo(r.w), a);
        a = __builtin_fmaf(o[bb][1].w, bf_hi(r.w), a);
        a = row16_sum(a);
        a = xor_sum(xor_sum(a, 16), 32);
        if (lane == 0 && b0 + bb < m.B) out[(int64_t(b0 + bb) * m.H + h) * 128 + v0 + j] = a;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Split merge and value up-projection in one pass (A6 + the W_uv step): one
// block per head h. The S partials of rows (b, h) are merged, with weights
// exp(lse_s - M) over their sum L as jssa_combine does, into the latent
// outputs (kCB sequences at a time); then out[b,h,:] = W_uv[h] o_lat[b] runs
// on MFMA: D[b][v] += A[b][32 dims] . B[32 dims][v] over 16 dim blocks
// (v_mfma_f32_16x16x32_bf16), B = W_uv[h] rows as stored (bf16), A = o_lat
// split exactly into three bf16 terms (8 significant bits each; three
// MFMAs into three accumulators), so the products are exact, the sums fp32,
// and no dot needs a cross-lane reduction.
//  Wave w owns outputs v = 16w .. 16w+15: lane (n, g) holds
//  W_uv[h][16w + n][32kb + 8g .. +7] for every kb, loaded at the start with
//  the split weights' and the partials' loads.
//  Merge: thread (q, c4) = (tid / 128, tid % 128) takes sequence b0 + q,
//  columns 4c4 .. +3, 16 splits per batch of 16-byte loads; each wave
//  computes its sequence's split weights itself (lane s: split s), so no
//  barrier stands before the merge. The thread splits its merged values into
//  the three bf16 terms once and stores them to LDS, where every wave reads
//  its A operands (A rows past the group's sequences read a valid row; the
//  D rows they produce are not stored).
// ---------------------------------------------------------------------------
constexpr int kCB = 4;          // sequences merged per pass (one per pair of waves)

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(512) void mla_combine_up_kernel(MlaDev m, int S, const float* __restrict__ part_o,
                                                             const float* __restrict__ part_lse,
                                                             const uint16_t* __restrict__ Wuv,
                                                             float* __restrict__ out, float* __restrict__ lse_out) {
  __shared__ __attribute__((aligned(16))) __bf16 ol3[3][kCB][kDl];   // o_lat = hi + mid + lo
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int q = tid >> 7, c4 = tid & 127;
  constexpr int kSP = 16;
  for (int b0 = 0; b0 < m.B; b0 += kCB) {
    const int nb = m.B - b0 < kCB ? m.B - b0 : kCB;
    const int64_t row = int64_t(b0 + (q < nb ? q : nb - 1)) * m.H + h;   // past B: row B-1, unused
    // split weights of this wave's sequence: lane s holds split s
    const float x = part_lse[row * S + (lane < S ? lane : 0)];
    f32x4v pv[kSP];
    auto load = [&](int s0) {
      const f32x4v* po = reinterpret_cast<const f32x4v*>(part_o + (row * S + s0) * kDl) + c4;
#pragma unroll
      for (int i = 0; i < kSP; ++i) pv[i] = po[int64_t(s0 + i < S ? i : S - 1 - s0) * (kDl / 4)];
    };
    load(0);
    u32x4 wb[16];                                       // (re-read per group: cache hits after the first)
    {
      const uint16_t* W = Wuv + (int64_t(h) * 128 + 16 * w + n) * kDl + 8 * g;
#pragma unroll
      for (int kb = 0; kb < 16; ++kb) wb[kb] = *reinterpret_cast<const u32x4*>(W + kb * 32);
    }
    float M = lane < S ? x : -__builtin_inff();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    const float wgt = lane < S && M != -__builtin_inff() ? __expf(x - M) : 0.f;
    float L = wgt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) L += __shfl_xor(L, o, 64);
    const float wt = L > 0.f ? wgt / L : 0.f;
    if (lse_out && (w & 1) == 0 && lane == 0 && q < nb) lse_out[row] = L > 0.f ? M + __logf(L) : -__builtin_inff();
    f32x4v acc = f32x4v{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += kSP) {
      if (s0 > 0) load(s0);
#pragma unroll
      for (int i = 0; i < kSP; ++i) {
        // lanes >= S hold weight 0, so splits past S (clamped loads) add nothing
        const float ws = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wt), s0 + i < 64 ? s0 + i : 63));
        acc += ws * pv[i];
      }
    }
    bf16x4 t0, t1, t2;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const __bf16 hb = __bf16(acc[e]);
      const float r1 = acc[e] - float(hb);              // exact
      const __bf16 mb = __bf16(r1);
      t0[e] = hb;
      t1[e] = mb;
      t2[e] = __bf16(r1 - float(mb));                   // exact: acc = hi + mid + lo
    }
    __syncthreads();                                    // the previous group's ol3 is read
    *reinterpret_cast<bf16x4*>(&ol3[0][q][4 * c4]) = t0;
    *reinterpret_cast<bf16x4*>(&ol3[1][q][4 * c4]) = t1;
    *reinterpret_cast<bf16x4*>(&ol3[2][q][4 * c4]) = t2;
    __syncthreads();
    f32x4v D[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) D[j] = f32x4v{0.f, 0.f, 0.f, 0.f};
    const int r = n & (kCB - 1);                        // A row n: sequence b0 + n for n < nb
#pragma unroll
    for (int kb = 0; kb < 16; ++kb) {
      const bf16x8 bw = __builtin_bit_cast(bf16x8, wb[kb]);
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&ol3[j][r][32 * kb + 8 * g]);
        D[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bw, D[j], 0, 0, 0);
      }
    }
    // D of lane (n, g), register i: sequence b0 + 4g + i, output v = 16w + n
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * g + i < nb) out[(int64_t(b0 + 4 * g + i) * m.H + h) * 128 + 16 * w + n] = (D[0][i] + D[1][i]) + D[2][i];
  }
}

}  // namespace

hipError_t launch_mla_project(const MlaDev& m, const uint16_t* latent, const float* P, uint16_t* Kp,
                              hipStream_t st) {
  dim3 grid((m.max_seq + 63) / 64, m.B);
  switch (m.r) {
    case 16: hipLaunchKernelGGL(mla_project_kernel<16>, grid, dim3(256), 0, st, m, latent, P, Kp); break;
    case 32: hipLaunchKernelGGL(mla_project_kernel<32>, grid, dim3(256), 0, st, m, latent, P, Kp); break;
    case 64: hipLaunchKernelGGL(mla_project_kernel<64>, grid, dim3(256), 0, st, m, latent, P, Kp); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_mla_fold(const MlaDev& m, const uint16_t* W_uk, const float* P, float* U, hipStream_t st) {
  const dim3 grid(m.H, 128);
  switch (m.r) {
    case 16: hipLaunchKernelGGL(mla_fold_kernel<16>, grid, dim3(16), 0, st, W_uk, P, U); break;
    case 32: hipLaunchKernelGGL(mla_fold_kernel<32>, grid, dim3(32), 0, st, W_uk, P, U); break;
    case 64: hipLaunchKernelGGL(mla_fold_kernel<64>, grid, dim3(64), 0, st, W_uk, P, U); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_mla_absorb(const MlaDev& m, const uint16_t* q_nope, const uint16_t* q_rope,
                             const uint16_t* W_uk, const float* P, const float* U, float* q_abs, float* q_sel,
                             hipStream_t st) {
  // the selection parts first in launch order: the score pass waits on them
  const dim3 grid(kMlaSelParts + m.H * (kDl / 128));
  switch (m.r) {
    case 16: hipLaunchKernelGGL(mla_queries_kernel<16>, grid, dim3(256), 0, st, m, q_nope, q_rope, W_uk, U, P, q_abs, q_sel); break;
    case 32: hipLaunchKernelGGL(mla_queries_kernel<32>, grid, dim3(256), 0, st, m, q_nope, q_rope, W_uk, U, P, q_abs, q_sel); break;
    case 64: hipLaunchKernelGGL(mla_queries_kernel<64>, grid, dim3(256), 0, st, m, q_nope, q_rope, W_uk, U, P, q_abs, q_sel); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_mla_indexed(const MlaDev& m, const float* q_abs, const uint16_t* latent,
                              const int32_t* idx, int k, int S, float scale, float* part_o,
                              float* part_lse, hipStream_t st) {
  dim3 grid(S, m.H / 16, m.B);
  hipLaunchKernelGGL(mla_indexed_kernel, grid, dim3(128), 0, st, m, q_abs, latent, idx, k, S, scale,
                     part_o, part_lse);
  return hipGetLastError();
}

hipError_t launch_mla_combine_up(const MlaDev& m, int S, const float* part_o, const float* part_lse,
                                 const uint16_t* W_uv, float* out, float* lse, hipStream_t st) {
  hipLaunchKernelGGL(mla_combine_up_kernel, dim3(m.H), dim3(512), 0, st, m, S, part_o, part_lse, W_uv, out, lse);
  return hipGetLastError();
}

hipError_t launch_mla_up_v(const MlaDev& m, const float* o_lat, const uint16_t* W_uv, float* out,
                           hipStream_t st) {
  hipLaunchKernelGGL(mla_up_v_kernel, dim3(m.H, 128 / 32), dim3(256), 0, st, m, o_lat, W_uv, out);
  return hipGetLastError();
}

}  // namespace jssa

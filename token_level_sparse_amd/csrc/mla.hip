// MLA shared-latent path: selection over the shared latent cache and
// attention over the selected latent rows.
//
// For MLA models JSSA's selection operates over the shared latent cache
// (ai4snews digest, Perspective). Per head h the key of token t is
// [W_uk[h] c_t[:512]; c_t[512:]] and its value c_t[:512]; absorbing W_uk into
// the query (q_abs = [W_uk[h]^T q_nope; q_rope]) turns the logits into one
// 576-dim dot per (head, token) and the output into W_uv[h] (sum_t p_t c_t).
// All heads share the latent rows, so with 128 heads the per-token work is a
// genuine dense contraction: QK^T and PV run on bf16 MFMA (gfx950
// v_mfma_f32_16x16x32_bf16). The query enters QK^T as a hi + lo pair of bf16
// (two MFMAs) so the logits keep ~fp32 accuracy.
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
// Absorbed query: q_abs[b,h,c] = sum_i q_nope[b,h,i] W_uk[h,i,c] for c < 512
// (fp32), then the rope part copied. Block (h, column quarter): 128 columns
// as 64 bf16 pairs; wave w sums rows i = 32w .. 32w+31, whose 32 pair loads
// per lane are all issued before any is used; the four partial sums meet in
// LDS. Each W_uk element is read once and serves every sequence.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mla_absorb_kernel(MlaDev m, const uint16_t* __restrict__ qn,
                                                         const uint16_t* __restrict__ qr,
                                                         const uint16_t* __restrict__ Wuk,
                                                         float* __restrict__ qa) {
  constexpr int BT = 8;                  // sequences per pass
  __shared__ float qs[BT][128];
  __shared__ float part[4][BT][128];
  const int h = blockIdx.x, cq = blockIdx.y, tid = threadIdx.x;
  const int cp = tid & 63, w = tid >> 6;
  const uint16_t* W = Wuk + (int64_t(h) * 128 + w * 32) * kDl + cq * 128 + 2 * cp;
  uint32_t wr[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) wr[i] = *reinterpret_cast<const uint32_t*>(W + int64_t(i) * kDl);
  for (int b0 = 0; b0 < m.B; b0 += BT) {
    const int nb = min(BT, m.B - b0);
    __syncthreads();
    for (int e = tid; e < BT * 128; e += 256) {
      const int bb = e / 128, i = e % 128;
      qs[bb][i] = bb < nb ? bf(qn[(int64_t(b0 + bb) * m.H + h) * 128 + i]) : 0.f;
    }
    __syncthreads();
    float acc[BT][2];
#pragma unroll
    for (int bb = 0; bb < BT; ++bb) acc[bb][0] = acc[bb][1] = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float w0 = bf_lo(wr[i]), w1 = bf_hi(wr[i]);
#pragma unroll
      for (int bb = 0; bb < BT; ++bb) {
        const float q = qs[bb][w * 32 + i];
        acc[bb][0] = __builtin_fmaf(q, w0, acc[bb][0]);
        acc[bb][1] = __builtin_fmaf(q, w1, acc[bb][1]);
      }
    }
#pragma unroll
    for (int bb = 0; bb < BT; ++bb) {
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

// ---------------------------------------------------------------------------
// Selection query of a sequence: q_sel[b,:] = P^T (sum_h q_abs[b,h,:]), the
// subspace query the latent score stream dots with every projected row
// (fixed summation order: deterministic). Block per sequence, 1024 threads:
// the head sum is split over 4 head quarters (unrolled loads) and merged in
// LDS, then R columns x 1024/R row slices of P.
// ---------------------------------------------------------------------------
template <int R>
__global__ __launch_bounds__(1024) void mla_selq_kernel(MlaDev m, const float* __restrict__ qa,
                                                        const float* __restrict__ P,
                                                        float* __restrict__ qsel) {
  __shared__ float part[4][kDc];
  __shared__ float qbar[kDc];
  __shared__ float ppart[1024];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int hq = tid >> 8, ct = tid & 255;              // head quarter, column thread
  const int hpq = (m.H + 3) / 4;
  const int h0 = hq * hpq, h1 = min(m.H, h0 + hpq);
  // up to 32 heads per quarter: all loads of a column issued at once
  // (clamped to a valid head, zero weight past the quarter)
  for (int c = ct; c < kDc; c += 256) {
    const float* qc = qa + int64_t(b) * m.H * kDc + c;
    float s = 0.f;
    for (int hb = h0; hb < h1; hb += 32) {
      float a[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int h = hb + u < h1 ? hb + u : h1 - 1;
        a[u] = qc[int64_t(h) * kDc];
      }
#pragma unroll
      for (int u = 0; u < 32; ++u) s += hb + u < h1 ? a[u] : 0.f;
    }
    part[hq][c] = s;
  }
  __syncthreads();
  for (int c = tid; c < kDc; c += 1024) qbar[c] = ((part[0][c] + part[1][c]) + part[2][c]) + part[3][c];
  __syncthreads();
  constexpr int NS = 1024 / R;                          // row slices
  constexpr int NI = (kDc + NS - 1) / NS;
  const int c = tid % R, sl = tid / R;
  float s = 0.f;
  float pv[NI];
#pragma unroll
  for (int ii = 0; ii < NI; ++ii) {                   // every P load in flight at once
    const int i = sl + ii * NS;
    pv[ii] = P[(i < kDc ? i : kDc - 1) * R + c];
  }
#pragma unroll
  for (int ii = 0; ii < NI; ++ii) {
    const int i = sl + ii * NS;
    s = __builtin_fmaf(pv[ii], i < kDc ? qbar[i < kDc ? i : kDc - 1] : 0.f, s);
  }
  ppart[sl * R + c] = s;
  __syncthreads();
  if (tid < R) {
    float t = 0.f;
    for (int x = 0; x < NS; ++x) t += ppart[x * R + tid];
    qsel[int64_t(b) * R + tid] = t;
  }
}

// ---------------------------------------------------------------------------
// Indexed MLA attention on MFMA. Block = 1 wave = 16 heads x one split of the
// selected slots, processed 32 tokens at a time.
//  QK^T: S^T[16 tok x 16 heads] += C[16 tok x 32 dims] . Qt[32 dims x 16 heads]
//        over 18 dim blocks, twice (q hi and q lo), for two 16-token halves.
//        Row m of half hf is token 8*(m/4) + 4*hf + m%4 of the 32-token block,
//        so that lane group g (= lane/16) ends up with the logits of tokens
//        8g..8g+7 for head lane%16: exactly the A operand of the PV MFMA.
//  PV:   O[16 heads x 16 dims] += P[16 heads x 32 tok] . V[32 tok x 16 dims],
//        32 dim tiles; V is staged transposed in LDS ([dim][token]) from the
//        same loads that fed QK^T, so each lane reads its 8 tokens with one
//        ds_read_b128.
// ---------------------------------------------------------------------------
constexpr int kVtStride = 40;   // u16 per transposed row (32 tokens + pad)

__global__ __launch_bounds__(64) void mla_indexed_kernel(MlaDev m, const float* __restrict__ qa,
                                                         const uint16_t* __restrict__ lat,
                                                         const int32_t* __restrict__ idx, int k,
                                                         int S, float scale,
                                                         float* __restrict__ part_o,
                                                         float* __restrict__ part_lse) {
  __shared__ __attribute__((aligned(16))) uint16_t Vt[kDl * kVtStride];
  const int s = blockIdx.x, ht = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x, g = lane >> 4, n = lane & 15;
  const int Tb = mla_len(m, b);
  const int cs = (k + S - 1) / S;
  const int r0 = min(s * cs, k), r1 = min(r0 + cs, k);
  const int h = ht * 16 + n;                       // this lane's head in the QK B operand

  // B operand of QK^T (Q^T): lane holds Q[head n][dims kb*32 + 8g .. +8], as hi and lo bf16;
  // the lo parts wait in LDS (registers go to the accumulators and loads in flight).
  __shared__ bf16x8 qlo_s[18][64];
  bf16x8 qhi[18];
  {
    const float* qrow = qa + (int64_t(b) * m.H + h) * kDc;
    const float qs = scale * kLog2e;
#pragma unroll
    for (int kb = 0; kb < 18; ++kb) {
      const f32x4v* p = reinterpret_cast<const f32x4v*>(qrow + kb * 32 + 8 * g);
      const f32x4v a = p[0], c = p[1];
      float x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
      bf16x8 lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = x[e] * qs;
        const __bf16 hi = __bf16(v);
        qhi[kb][e] = hi;
        lo[e] = __bf16(v - float(hi));
      }
      qlo_s[kb][lane] = lo;
    }
  }

  f32x4v O[32];
#pragma unroll
  for (int t = 0; t < 32; ++t) O[t] = f32x4v{0.f, 0.f, 0.f, 0.f};
  float mrun = -__builtin_inff();    // running max for head n (log2 domain), uniform over g
  float lrun = 0.f;                  // partial sum over this lane group's tokens

  // Loads are pipelined by half tiles: while one half's 18 pieces per lane
  // are multiplied, the other half's (or the next tile's first half's) are
  // in flight. No load sits under a data-dependent branch: rows past the
  // split or with an invalid index read token 0 of the sequence (finite
  // data) and are masked out of the softmax.
  const int32_t* irow = idx + int64_t(b) * k;
  const uint16_t* lrow = lat + int64_t(b) * m.max_seq * kDc;
  auto tile_index = [&](int base) -> int {           // lane l < 32: index of slot base + l
    const int sl = base + (lane & 31);
    return irow[sl < r1 ? sl : r1 - 1];
  };
  auto row_of = [&](int base, int tv, int hf, bool& ok) -> const uint16_t* {
    const int tl = 8 * (n >> 2) + 4 * hf + (n & 3);  // token of MFMA row n in half hf
    const int t = __shfl(tv, tl, 64);
    ok = base + tl < r1 && t >= 0 && t < Tb;
    return lrow + int64_t(ok ? t : 0) * kDc + 8 * g;
  };
  auto load_half = [&](const uint16_t* crow, u32x4 (&A)[18]) {
#pragma unroll
    for (int kb = 0; kb < 18; ++kb) A[kb] = *reinterpret_cast<const u32x4*>(crow + kb * 32);
  };
  // QK^T of one half tile; stashes the value part transposed in LDS. Four
  // independent accumulator chains (hi/lo x even/odd dim blocks) keep the
  // MFMA pipe busy instead of waiting on one chain's previous result.
  auto qk_half = [&](const u32x4 (&A)[18], int hf) -> f32x4v {
    const int tl = 8 * (n >> 2) + 4 * hf + (n & 3);
    f32x4v acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 18; ++kb) {
      if (kb < 16) {
        const u32x4 raw = A[kb];
        const uint16_t* e16 = reinterpret_cast<const uint16_t*>(&raw);
#pragma unroll
        for (int e = 0; e < 8; ++e) Vt[(kb * 32 + 8 * g + e) * kVtStride + tl] = e16[e];
      }
      const bf16x8 a = __builtin_bit_cast(bf16x8, A[kb]);
      acc[kb & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qhi[kb], acc[kb & 1], 0, 0, 0);
      acc[2 + (kb & 1)] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qlo_s[kb][lane], acc[2 + (kb & 1)], 0, 0, 0);
    }
    return (acc[0] + acc[1]) + (acc[2] + acc[3]);
  };

  u32x4 A0[18], A1[18];
  int tv = r0 < r1 ? tile_index(r0) : 0;
  bool ok0 = false, ok1 = false;
  if (r0 < r1) load_half(row_of(r0, tv, 0, ok0), A0);
  for (int base = r0; base < r1; base += 32) {
    load_half(row_of(base, tv, 1, ok1), A1);
    const int nb = base + 32 < r1 ? base + 32 : base;    // next tile (or this one again: unused)
    const int tvn = tile_index(nb);
    f32x4v St[2];
    bool okrow[2];
    St[0] = qk_half(A0, 0);
    okrow[0] = ok0;
    load_half(row_of(nb, tvn, 0, ok0), A0);            // next tile's first half
    St[1] = qk_half(A1, 1);
    okrow[1] = ok1;
    tv = tvn;
    // St[hf][i] = logit (log2 domain) of head n, token 8g + 4hf + i.
    // validity of those tokens: rows 4g+i of each half belong to lanes n' = 4g+i
    float lg[8];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int src = (lane & 48) | (4 * g + i);    // any lane whose n == 4g+i; same group
        const int okv = __shfl(okrow[hf] ? 1 : 0, src, 64);
        lg[hf * 4 + i] = okv ? St[hf][i] : -__builtin_inff();
      }
    float bm = lg[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) bm = fmaxf(bm, lg[i]);
    bm = xor_max(bm, 16);
    bm = xor_max(bm, 32);
    const float mnew = fmaxf(mrun, bm);
    float alpha = 1.f;
    float p[8];
    if (mnew == -__builtin_inff()) {
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = 0.f;
    } else {
      alpha = __builtin_amdgcn_exp2f(mrun - mnew);
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(lg[i] - mnew);
    }
    mrun = mnew;
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ps += p[i];
    lrun = lrun * alpha + ps;
    // rescale O: accumulator rows are heads 4g+i; their alpha sits in lane n = 4g+i
    float ar[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      O[t][0] *= ar[0]; O[t][1] *= ar[1]; O[t][2] *= ar[2]; O[t][3] *= ar[3];
    }
    bf16x8 pa;
#pragma unroll
    for (int i = 0; i < 8; ++i) pa[i] = __bf16(p[i]);
    wave_lds_sync();
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const u32x4 vraw = *reinterpret_cast<const u32x4*>(&Vt[(t * 16 + n) * kVtStride + 8 * g]);
      O[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf16x8, vraw), O[t], 0, 0, 0);
    }
    wave_lds_sync();
  }
  // total softmax denominator of head n: sum over the 4 lane groups
  lrun = xor_sum(xor_sum(lrun, 16), 32);
  // O[t][i] is head 4g+i, dim t*16+n
  float lh[4], mh[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lh[i] = __shfl(lrun, 4 * g + i, 64);
    mh[i] = __shfl(mrun, 4 * g + i, 64);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = ht * 16 + 4 * g + i;
    const int64_t ob = (int64_t(b) * m.H + hh) * S + s;
    const float inv = lh[i] > 0.f ? 1.f / lh[i] : 0.f;
    float* dst = part_o + ob * kDl;
#pragma unroll
    for (int t = 0; t < 32; ++t) dst[t * 16 + n] = O[t][i] * inv;
    if (n == 0) part_lse[ob] = lh[i] > 0.f ? (mh[i] + __builtin_log2f(lh[i])) * kLn2 : -__builtin_inff();
  }
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

hipError_t launch_mla_absorb(const MlaDev& m, const uint16_t* q_nope, const uint16_t* q_rope,
                             const uint16_t* W_uk, const float* P, float* q_abs, float* q_sel, hipStream_t st) {
  hipLaunchKernelGGL(mla_absorb_kernel, dim3(m.H, kDl / 128), dim3(256), 0, st, m, q_nope, q_rope, W_uk, q_abs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (m.r) {
    case 16: hipLaunchKernelGGL(mla_selq_kernel<16>, dim3(m.B), dim3(1024), 0, st, m, q_abs, P, q_sel); break;
    case 32: hipLaunchKernelGGL(mla_selq_kernel<32>, dim3(m.B), dim3(1024), 0, st, m, q_abs, P, q_sel); break;
    case 64: hipLaunchKernelGGL(mla_selq_kernel<64>, dim3(m.B), dim3(1024), 0, st, m, q_abs, P, q_sel); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_mla_indexed(const MlaDev& m, const float* q_abs, const uint16_t* latent,
                              const int32_t* idx, int k, int S, float scale, float* part_o,
                              float* part_lse, hipStream_t st) {
  dim3 grid(S, m.H / 16, m.B);
  hipLaunchKernelGGL(mla_indexed_kernel, grid, dim3(64), 0, st, m, q_abs, latent, idx, k, S, scale,
                     part_o, part_lse);
  return hipGetLastError();
}

hipError_t launch_mla_up_v(const MlaDev& m, const float* o_lat, const uint16_t* W_uv, float* out,
                           hipStream_t st) {
  hipLaunchKernelGGL(mla_up_v_kernel, dim3(m.H, 128 / 32), dim3(256), 0, st, m, o_lat, W_uv, out);
  return hipGetLastError();
}

}  // namespace jssa

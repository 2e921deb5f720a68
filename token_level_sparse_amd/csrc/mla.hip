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
// GQA key projection). Block: 64 tokens x R columns; P read through L2.
// ---------------------------------------------------------------------------
template <int R>
__global__ __launch_bounds__(256) void mla_project_kernel(MlaDev m, const uint16_t* __restrict__ lat,
                                                          const float* __restrict__ P,
                                                          uint16_t* __restrict__ Kp) {
  constexpr int TOK = 64;
  constexpr int TG = 256 / R;            // token groups
  constexpr int TPT = TOK / TG;          // tokens per thread
  __shared__ uint16_t Cs[TOK * kDc];
  const int b = blockIdx.y, t0 = blockIdx.x * TOK;
  const int Tb = mla_len(m, b);
  const int tid = threadIdx.x;
  const uint16_t* src = lat + (int64_t(b) * m.max_seq + t0) * kDc;
  const int nrows = min(TOK, max(0, Tb - t0));
  for (int e = tid; e < TOK * kDc / 8; e += 256) {
    const int row = e / (kDc / 8);
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (row < nrows) v = reinterpret_cast<const u32x4*>(src)[e];
    reinterpret_cast<u32x4*>(Cs)[e] = v;
  }
  __syncthreads();
  const int c = tid % R, tg = tid / R;
  double acc[TPT];
#pragma unroll
  for (int i = 0; i < TPT; ++i) acc[i] = 0.0;
  for (int i = 0; i < kDc; ++i) {
    const double p = double(P[i * R + c]);
#pragma unroll
    for (int x = 0; x < TPT; ++x) acc[x] = __builtin_fma(double(bf(Cs[(tg + x * TG) * kDc + i])), p, acc[x]);
  }
#pragma unroll
  for (int x = 0; x < TPT; ++x) {
    const int t = t0 + tg + x * TG;
    if (t < Tb) Kp[(int64_t(b) * m.max_seq + t) * R + c] = f64_to_bf16_rne(acc[x]);
  }
}

// ---------------------------------------------------------------------------
// Absorbed query. Block per head h: q_abs[b,h,c] = sum_i q_nope[b,h,i] W_uk[h,i,c]
// for c < 512 (fp32), then the rope part copied.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mla_absorb_kernel(MlaDev m, const uint16_t* __restrict__ qn,
                                                         const uint16_t* __restrict__ qr,
                                                         const uint16_t* __restrict__ Wuk,
                                                         float* __restrict__ qa) {
  constexpr int BT = 8;                  // sequences per pass
  __shared__ float qs[BT][128];
  const int h = blockIdx.x, tid = threadIdx.x;
  const uint16_t* W = Wuk + int64_t(h) * 128 * kDl;
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
    for (int i = 0; i < 128; ++i) {
      const uint32_t w2 = reinterpret_cast<const uint32_t*>(W + int64_t(i) * kDl)[tid];
      const float w0 = bf_lo(w2), w1 = bf_hi(w2);
#pragma unroll
      for (int bb = 0; bb < BT; ++bb) {
        acc[bb][0] = __builtin_fmaf(qs[bb][i], w0, acc[bb][0]);
        acc[bb][1] = __builtin_fmaf(qs[bb][i], w1, acc[bb][1]);
      }
    }
    for (int bb = 0; bb < nb; ++bb) {
      float* dst = qa + (int64_t(b0 + bb) * m.H + h) * kDc;
      dst[2 * tid] = acc[bb][0];
      dst[2 * tid + 1] = acc[bb][1];
      if (tid < 64) dst[kDl + tid] = bf(qr[(int64_t(b0 + bb) * m.H + h) * 64 + tid]);
    }
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

  // B operand of QK^T (Q^T): lane holds Q[head n][dims kb*32 + 8g .. +8], as hi and lo bf16.
  bf16x8 qhi[18], qlo[18];
  {
    const float* qrow = qa + (int64_t(b) * m.H + h) * kDc;
    const float qs = scale * kLog2e;
#pragma unroll
    for (int kb = 0; kb < 18; ++kb) {
      const f32x4v* p = reinterpret_cast<const f32x4v*>(qrow + kb * 32 + 8 * g);
      const f32x4v a = p[0], c = p[1];
      float x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = x[e] * qs;
        const __bf16 hi = __bf16(v);
        qhi[kb][e] = hi;
        qlo[kb][e] = __bf16(v - float(hi));
      }
    }
  }

  f32x4v O[32];
#pragma unroll
  for (int t = 0; t < 32; ++t) O[t] = f32x4v{0.f, 0.f, 0.f, 0.f};
  float mrun = -__builtin_inff();    // running max for head n (log2 domain), uniform over g
  float lrun = 0.f;                  // partial sum over this lane group's tokens

  const int32_t* irow = idx + int64_t(b) * k;
  for (int base = r0; base < r1; base += 32) {
    f32x4v St[2];
    bool okrow[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      // token handled by MFMA row n of half hf
      const int tok_local = 8 * (n >> 2) + 4 * hf + (n & 3);
      const int slot = base + tok_local;
      int t = -1;
      if (slot < r1) t = irow[slot];
      const bool ok = t >= 0 && t < Tb;
      okrow[hf] = ok;
      const uint16_t* crow = lat + (int64_t(b) * m.max_seq + (ok ? t : 0)) * kDc;
      f32x4v acc = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 18; ++kb) {
        u32x4 raw = u32x4{0u, 0u, 0u, 0u};
        if (ok) raw = *reinterpret_cast<const u32x4*>(crow + kb * 32 + 8 * g);
        if (kb < 16) {
          // transposed stash of the value part: Vt[dim][token]
          const uint16_t* e16 = reinterpret_cast<const uint16_t*>(&raw);
#pragma unroll
          for (int e = 0; e < 8; ++e) Vt[(kb * 32 + 8 * g + e) * kVtStride + tok_local] = e16[e];
        }
        const bf16x8 a = __builtin_bit_cast(bf16x8, raw);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qhi[kb], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qlo[kb], acc, 0, 0, 0);
      }
      St[hf] = acc;
    }
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
// out[b,h,v] = sum_c W_uv[h,v,c] o_lat[b,h,c]. Block per head, wave per 32 v.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mla_up_v_kernel(MlaDev m, const float* __restrict__ olat,
                                                       const uint16_t* __restrict__ Wuv,
                                                       float* __restrict__ out) {
  const int h = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint16_t* W = Wuv + int64_t(h) * 128 * kDl;
  for (int b = 0; b < m.B; ++b) {
    const f32x4v* op = reinterpret_cast<const f32x4v*>(olat + (int64_t(b) * m.H + h) * kDl + lane * 8);
    const f32x4v o0 = op[0], o1 = op[1];
    for (int v = w * 32; v < w * 32 + 32; ++v) {
      const u32x4 wr = reinterpret_cast<const u32x4*>(W + int64_t(v) * kDl)[lane];
      float a = 0.f;
      a = __builtin_fmaf(o0.x, bf_lo(wr.x), a);
      a = __builtin_fmaf(o0.y, bf_hi(wr.x), a);
      a = __builtin_fmaf(o0.z, bf_lo(wr.y), a);
      a = __builtin_fmaf(o0.w, bf_hi(wr.y), a);
      a = __builtin_fmaf(o1.x, bf_lo(wr.z), a);
      a = __builtin_fmaf(o1.y, bf_hi(wr.z), a);
      a = __builtin_fmaf(o1.z, bf_lo(wr.w), a);
      a = __builtin_fmaf(o1.w, bf_hi(wr.w), a);
      a = row16_sum(a);
      a = xor_sum(xor_sum(a, 16), 32);
      if (lane == 0) out[(int64_t(b) * m.H + h) * 128 + v] = a;
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
                             const uint16_t* W_uk, float* q_abs, hipStream_t st) {
  hipLaunchKernelGGL(mla_absorb_kernel, dim3(m.H), dim3(256), 0, st, m, q_nope, q_rope, W_uk, q_abs);
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
  hipLaunchKernelGGL(mla_up_v_kernel, dim3(m.H), dim3(256), 0, st, m, o_lat, W_uv, out);
  return hipGetLastError();
}

}  // namespace jssa

// Per-(sequence, head) top-k with lowest-index ties.
//
// JSSA keeps a distinct selected token set for each KV head (JSSA abstract;
// ai4snews digest, Synopsis). The result is the first min(k, T_b) tokens of
// the total order (score descending, index ascending), listed ascending.
//
// Two-level deterministic selection, no global sorting:
//  round 0: each block takes one chunk of C scores of one row, keeps them in
//           registers (256 or 1024 threads x 4..16 each) as order-preserving uint32 keys and radix-selects the
//           chunk's own top-k (three digit levels, 11+11+10 bits, with LDS
//           histograms; the last digit level is skipped once the threshold
//           bin holds exactly the tokens still needed). Ties at the threshold
//           key are resolved by position, so the chunk's list is the chunk's
//           prefix of the total order. Survivors are written in position
//           order (ballot ranks + a prefix over (element, wave) blocks).
//  merge:   a 1024-thread block concatenates the chunk lists of a row (still
//           ascending by token) and runs the same selection; a token dropped
//           inside a chunk has k better tokens in that chunk, so the union of
//           chunk lists contains the row's top-k. Long rows with small k take
//           extra merge rounds.
// Every decision depends only on keys and positions, so results do not
// depend on scheduling.
#include "internal.hpp"

namespace jssa {
namespace {

constexpr int kBins = 2048;

template <int NT>
struct SelectSmem {
  int hist[kBins];
  int blk[(NT / 64) * 64 + 1];
  int scan_tot[NT / 64];
  int sel_bin, sel_gt, total;
  int offs[1025];
};

// Inclusive scan over threads (tid order); returns inclusive value, writes
// the block total to *total (visible after the call).
template <int NT>
__device__ int block_incl_scan(int v, SelectSmem<NT>& sm) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) sm.scan_tot[w] = v;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int x = sm.scan_tot[i];
    pre += (i < w) ? x : 0;
    tot += x;
  }
  __syncthreads();
  if (threadIdx.x == 0) sm.total = tot;
  return v + pre;
}

// Position-order rank of set flags; element e of thread tid has position
// e*NT + tid. Returns ranks in rank[], count of set flags via return.
template <int NT, int E>
__device__ int ordered_rank(const bool (&flag)[E], int (&rank)[E], SelectSmem<NT>& sm) {
  constexpr int NW = NT / 64;
  constexpr int NB = E * NW;                 // (element, wave) blocks in position order
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t ball = __ballot(flag[e]);
    rank[e] = __popcll(ball & lt);
    if (lane == 0) sm.blk[e * NW + w] = __popcll(ball);
  }
  __syncthreads();
  if (w == 0) {
    constexpr int PER = (NB + 63) / 64;
    int loc[PER];
    int s = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int ix = lane * PER + i;
      loc[i] = ix < NB ? sm.blk[ix] : 0;
      s += loc[i];
    }
    int incl = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    int run = incl - s;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int ix = lane * PER + i;
      if (ix < NB) sm.blk[ix] = run;
      run += loc[i];
    }
    if (lane == 63) sm.blk[NB] = incl;
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) rank[e] += sm.blk[e * NW + w];
  const int tot = sm.blk[NB];
  __syncthreads();
  return tot;
}

// Selects `need` = min(k, n) elements; on return take[e] marks them.
template <int NT, int E>
__device__ void select_top(const uint32_t (&key)[E], const bool (&valid)[E], int n, int k,
                           bool (&take)[E], SelectSmem<NT>& sm) {
  const int tid = threadIdx.x;
  if (n <= k) {
#pragma unroll
    for (int e = 0; e < E; ++e) take[e] = valid[e];
    return;
  }
  int rem = k;
  uint32_t pre = 0;
  int res_shift = 0;
  constexpr int BPT = kBins / NT;
  for (int L = 0; L < 3; ++L) {
    const int shift = L == 0 ? 21 : (L == 1 ? 10 : 0);
    const int bits = L == 2 ? 10 : 11;
    const uint32_t mask = (1u << bits) - 1u;
    for (int i = tid; i < kBins; i += NT) sm.hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool in = valid[e] && (L == 0 || (key[e] >> (shift + bits)) == pre);
      if (in) atomicAdd(&sm.hist[(key[e] >> shift) & mask], 1);
    }
    __syncthreads();
    int loc[BPT];
    int mine = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      loc[i] = sm.hist[tid * BPT + i];
      mine += loc[i];
    }
    const int incl = block_incl_scan<NT>(mine, sm);
    __syncthreads();
    int running = sm.total - incl;          // elements in higher bins (higher threads)
#pragma unroll
    for (int i = BPT - 1; i >= 0; --i) {
      if (running < rem && running + loc[i] >= rem) {
        sm.sel_bin = tid * BPT + i;
        sm.sel_gt = running;
      }
      running += loc[i];
    }
    __syncthreads();
    const int D = sm.sel_bin;
    rem -= sm.sel_gt;
    const int cntD = sm.hist[D];
    pre = (pre << bits) | uint32_t(D);
    res_shift = shift;
    __syncthreads();
    if (cntD == rem) break;
  }
  bool gt[E], eq[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t top = key[e] >> res_shift;
    gt[e] = valid[e] && top > pre;
    eq[e] = valid[e] && top == pre;
  }
  int rk[E];
  ordered_rank<NT, E>(eq, rk, sm);
#pragma unroll
  for (int e = 0; e < E; ++e) take[e] = gt[e] || (eq[e] && rk[e] < rem);
}

struct SegIn {
  const int32_t* cnt;    // [rows][nseg]
  const uint32_t* key;   // [rows][nseg][k]
  const int32_t* idx;
  int nseg, spc;
};
struct SegOut {
  int32_t* cnt;          // [rows][gridDim.x]
  uint32_t* key;         // [rows][gridDim.x][k]
  int32_t* idx;
};

template <int NT, int E, bool FROM_SCORES, bool FINAL>
__global__ __launch_bounds__(NT) void select_kernel(int H, int max_seq, const int32_t* seq_lens,
                                                    const float* __restrict__ scores, SegIn in,
                                                    int k, SegOut out, int32_t* __restrict__ idx_out) {
  __shared__ SelectSmem<NT> sm;
  const int tid = threadIdx.x;
  const int row = blockIdx.y, chunk = blockIdx.x;
  uint32_t key[E];
  int32_t idx[E];
  bool valid[E];
  int n;
  if constexpr (FROM_SCORES) {
    const int b = row / H;
    int Tb = seq_lens ? seq_lens[b] : max_seq;
    Tb = Tb < 0 ? 0 : (Tb > max_seq ? max_seq : Tb);
    const int start = chunk * (NT * E);
    n = Tb - start;
    n = n < 0 ? 0 : (n > NT * E ? NT * E : n);
    const float* src = scores + int64_t(row) * max_seq + start;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int p = e * NT + tid;
      valid[e] = p < n;
      key[e] = valid[e] ? score_key(src[p]) : 0u;
      idx[e] = start + p;
    }
  } else {
    const int s0 = chunk * in.spc;
    const int ns = min(in.spc, in.nseg - s0);
    int c = 0;
    if (tid < ns) c = in.cnt[int64_t(row) * in.nseg + s0 + tid];
    const int incl = block_incl_scan<NT>(c, sm);
    if (tid < ns) sm.offs[tid + 1] = incl;
    if (tid == 0) sm.offs[0] = 0;
    __syncthreads();
    n = sm.offs[ns];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int p = e * NT + tid;
      valid[e] = p < n;
      key[e] = 0u;
      idx[e] = -1;
      if (valid[e]) {
        int lo = 0, hi = ns - 1;         // largest s with offs[s] <= p
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (sm.offs[mid] <= p) lo = mid; else hi = mid - 1;
        }
        const int64_t at = (int64_t(row) * in.nseg + s0 + lo) * k + (p - sm.offs[lo]);
        key[e] = in.key[at];
        idx[e] = in.idx[at];
      }
    }
    __syncthreads();
  }

  bool take[E];
  select_top<NT, E>(key, valid, n, k, take, sm);
  int rk[E];
  const int cnt = ordered_rank<NT, E>(take, rk, sm);
  if constexpr (FINAL) {
    int32_t* dst = idx_out + int64_t(row) * k;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (take[e]) dst[rk[e]] = idx[e];
    for (int i = cnt + tid; i < k; i += NT) dst[i] = -1;
  } else {
    const int64_t seg = int64_t(row) * gridDim.x + chunk;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (take[e]) {
        out.key[seg * k + rk[e]] = key[e];
        out.idx[seg * k + rk[e]] = idx[e];
      }
    if (tid == 0) out.cnt[seg] = cnt;
  }
}

constexpr int kMergeCap = 16384;   // candidates one merge block holds (1024 x 16)

int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

struct TopkPlan {
  int C0, n0;                       // round-0 chunk length and chunk count
  int rounds;                       // merge rounds after round 0 (last one final)
  int nseg[8], spc[8];              // per merge round: input segments, segments per block
  size_t seg_bytes[2];              // ping-pong segment buffers
};

TopkPlan plan(int rows, int max_seq, int k) {
  TopkPlan p{};
  int C0 = next_pow2(16 * k);
  C0 = C0 < 1024 ? 1024 : (C0 > 16384 ? 16384 : C0);
  if (max_seq <= C0) {
    C0 = next_pow2(max_seq);
    if (C0 < 1024) C0 = 1024;
  }
  p.C0 = C0;
  p.n0 = (max_seq + C0 - 1) / C0;
  auto bytes = [&](int nseg) { return size_t(rows) * nseg * (size_t(k) * 8 + 4) + 256; };
  p.seg_bytes[0] = p.n0 > 1 ? bytes(p.n0) : 0;
  p.seg_bytes[1] = 0;
  int nseg = p.n0;
  p.rounds = 0;
  while (nseg > 1) {
    int spc;
    if (int64_t(nseg) * k <= kMergeCap && nseg <= 1024) {
      spc = nseg;
    } else {
      spc = kMergeCap / k;
      if (spc > 1024) spc = 1024;
    }
    p.nseg[p.rounds] = nseg;
    p.spc[p.rounds] = spc;
    const int next = (nseg + spc - 1) / spc;
    if (next > 1) {
      const size_t nb = bytes(next);
      size_t& slot = p.seg_bytes[(p.rounds + 1) & 1];
      if (nb > slot) slot = nb;
    }
    ++p.rounds;
    nseg = next;
  }
  return p;
}

template <int NT, int E>
void launch_round0(dim3 grid, bool final_, int H, int max_seq, const int32_t* seq_lens,
                   const float* scores, int k, SegOut out, int32_t* idx, hipStream_t st) {
  SegIn none{nullptr, nullptr, nullptr, 0, 0};
  if (final_)
    hipLaunchKernelGGL((select_kernel<NT, E, true, true>), grid, dim3(NT), 0, st, H, max_seq,
                       seq_lens, scores, none, k, out, idx);
  else
    hipLaunchKernelGGL((select_kernel<NT, E, true, false>), grid, dim3(NT), 0, st, H, max_seq,
                       seq_lens, scores, none, k, out, idx);
}

template <int E>
void launch_merge(dim3 grid, bool final_, int H, SegIn in, int k, SegOut out, int32_t* idx,
                  hipStream_t st) {
  if (final_)
    hipLaunchKernelGGL((select_kernel<1024, E, false, true>), grid, dim3(1024), 0, st, H, 0,
                       nullptr, nullptr, in, k, out, idx);
  else
    hipLaunchKernelGGL((select_kernel<1024, E, false, false>), grid, dim3(1024), 0, st, H, 0,
                       nullptr, nullptr, in, k, out, idx);
}

SegOut seg_view(void* base, int rows, int nseg, int k) {
  char* p = static_cast<char*>(base);
  SegOut s;
  s.key = reinterpret_cast<uint32_t*>(p);
  s.idx = reinterpret_cast<int32_t*>(p + size_t(rows) * nseg * k * 4);
  s.cnt = reinterpret_cast<int32_t*>(p + size_t(rows) * nseg * k * 8);
  return s;
}

}  // namespace

size_t topk_workspace_bytes(int rows, int max_seq, int k) {
  TopkPlan p = plan(rows, max_seq, k);
  return p.seg_bytes[0] + p.seg_bytes[1];
}

hipError_t launch_topk(int B, int H, int max_seq, const int32_t* seq_lens, const float* scores,
                       int k, int32_t* idx, void* ws, hipStream_t st) {
  const int rows = B * H;
  TopkPlan p = plan(rows, max_seq, k);
  void* buf[2] = {ws, static_cast<char*>(ws) + p.seg_bytes[0]};
  const bool single = p.n0 == 1;
  SegOut out0 = single ? SegOut{nullptr, nullptr, nullptr} : seg_view(buf[0], rows, p.n0, k);
  dim3 g0(p.n0, rows);
  switch (p.C0) {
    case 1024: launch_round0<256, 4>(g0, single, H, max_seq, seq_lens, scores, k, out0, idx, st); break;
    case 2048: launch_round0<256, 8>(g0, single, H, max_seq, seq_lens, scores, k, out0, idx, st); break;
    case 4096: launch_round0<256, 16>(g0, single, H, max_seq, seq_lens, scores, k, out0, idx, st); break;
    case 8192: launch_round0<1024, 8>(g0, single, H, max_seq, seq_lens, scores, k, out0, idx, st); break;
    case 16384: launch_round0<1024, 16>(g0, single, H, max_seq, seq_lens, scores, k, out0, idx, st); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  SegOut cur = out0;
  for (int r = 0; r < p.rounds; ++r) {
    const int nseg = p.nseg[r], spc = p.spc[r];
    const int next = (nseg + spc - 1) / spc;
    const bool fin = next == 1;
    SegIn in{cur.cnt, cur.key, cur.idx, nseg, spc};
    SegOut o = fin ? SegOut{nullptr, nullptr, nullptr} : seg_view(buf[(r + 1) & 1], rows, next, k);
    const int64_t cap = int64_t(spc) * k;
    if (cap <= 8192)
      launch_merge<8>(dim3(next, rows), fin, H, in, k, o, idx, st);
    else
      launch_merge<16>(dim3(next, rows), fin, H, in, k, o, idx, st);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    cur = o;
  }
  return hipSuccess;
}

}  // namespace jssa

// Subspace score stream: scores[b,j,t] = qp(b,j) . Kp[b,j,t,:], and the
// same stream fused with the chunk stage of the top-k selection.
//
// JSSA ranks candidate tokens in a low-dimensional space that holds queries
// and keys together (ai4snews digest, Synopsis and Interpretation). A KV
// head's score sums its G query heads' scores; by linearity that is one dot of
// qp = P_j^T (sum_h q_h) with the stored projected key, so the stream reads
// 2r bytes per token and does r FMAs. For the MLA latent cache the same
// stream runs with the selection query qp = P^T (sum over all heads of the
// absorbed query), which the absorb step writes as kMlaSelParts partial
// sums (one per class of heads); every block adds them in the same fixed
// order in its prologue.
//
// HBM-bound streaming kernel. Each wave reads a tile of 64 tokens' projected
// keys as 64*r/8 contiguous 16-byte pieces, one coalesced dwordx4 load per
// piece column (1 KB per wave instruction, whole cache lines). Lane l of load
// m holds piece 64m+l; the r/8 lanes holding one token's pieces are adjacent,
// so their 8-element partial dots are summed with DPP moves, and one
// ds_bpermute per load column hands token i's score to lane i: every lane
// then owns one token of the tile. Scores are staged in LDS and leave after
// the stream as 16-byte stores. The next tile's loads are in flight while the
// current tile is reduced, and the first tile's loads are issued before the
// qp prologue. r = 48 (6 lanes per token, not aligned to DPP rows) sums its
// partials through LDS instead.
//
// Fused variant (score -> top-k chunk stage): after the stream the block runs the
// chunk selection of the top-k (chunk_select) on its 8192 tokens and writes
// the surviving candidates, so the row's final selection never has to read
// the whole score row back. Writing the scores themselves is optional.
#include "internal.hpp"
#include "select.hpp"

namespace jssa {
namespace {

constexpr int kD = 128;
constexpr int kDc = 576;
constexpr int kWaves = 4;
constexpr int kFusedTiles = 32;            // tiles of 64 tokens per wave: 8192-token chunks
constexpr int kPlainTiles = 16;            // 4096-token chunks for the score-only stream
constexpr int kMlaTiles = 4;               // 1024-token chunks: the latent cache has only B rows
// Tiles per wave whose loads are in flight together. The plain score stream
// takes four for r <= 32 (measured: 199 -> 192 us at 128K x B = 16); the
// fused stream keeps two (four measured no faster: its time beyond the pure
// stream is the select and the XCD tail, not the loads in flight), as do
// larger ranks, whose buffers would not fit beside the select's registers.
constexpr int depth_of(int r, bool fused) { return r <= 32 && !fused ? 4 : 2; }
constexpr int kPackMaxB = 64;              // sequences up to which blocks take packed work items

// sum over aligned groups of PP lanes (PP = 1, 2, 4, 8 or 16), left in every
// lane of the group (a butterfly; the lanes' sums are bit-identical)
template <int PP>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (PP >= 2) x += dpp_mov<0xb1>(x);     // quad_perm [1,0,3,2]
  if constexpr (PP >= 4) x += dpp_mov<0x4e>(x);     // quad_perm [2,3,0,1]
  if constexpr (PP >= 8) x += dpp_mov<0x141>(x);    // row_half_mirror
  if constexpr (PP >= 16) x += dpp_mov<0x140>(x);   // row_mirror
  return x;
}

__device__ __forceinline__ float dot8(const float (&q)[8], u32x4 v) {
  float a = 0.f;
  a = __builtin_fmaf(q[0], bf_lo(v.x), a);
  a = __builtin_fmaf(q[1], bf_hi(v.x), a);
  a = __builtin_fmaf(q[2], bf_lo(v.y), a);
  a = __builtin_fmaf(q[3], bf_hi(v.y), a);
  a = __builtin_fmaf(q[4], bf_lo(v.z), a);
  a = __builtin_fmaf(q[5], bf_hi(v.z), a);
  a = __builtin_fmaf(q[6], bf_lo(v.w), a);
  a = __builtin_fmaf(q[7], bf_hi(v.w), a);
  return a;
}

enum Mode { kGqa = 0, kMla = 1 };

constexpr int tiles_per_wave(int mode, bool fused) {
  return fused ? kFusedTiles : (mode == kMla ? kMlaTiles : kPlainTiles);
}

struct FusedOut {
  CandSegs segs;
  int k;
  int write_scores;
  uint32_t* pmax;           // top-delta: per segment, the largest key of the row's sink/local tokens in it
  int n_sink, n_local;      // sink tokens: t < n_sink; local tokens: t >= T_b - n_local
  const uint32_t* keep;     // screening: one bit per 64-token tile ([rows, keep_words]); nullptr: all kept
  int keep_words;
  // fused stream keeping chunk lists (the chunk's own top k, which need not
  // hold the row's top k; segment floor 0, no selection slack), with the
  // scores written for the final pass's per-row fallback; scores2: a second
  // destination for the scores (the caller's buffer), or nullptr
  int lists;
  float* scores2;
};
// A token of a dropped tile is staged with this value: a NaN whose score_key
// is 0, the key of no token (finite scores map to keys above 0).
constexpr uint32_t kDroppedBits = 0xffffffffu;

template <int R>
struct ScoreSmem {
  union {
    struct {
      float qbar[kD];
      float qpart[kWaves * 64];
    } pro;                                                   // prologue only
    float part[(R / 8) & (R / 8 - 1) ? kWaves * 4 * R : 1];  // stream: LDS reduction (r = 48 only)
  } u;
  float qp[R];
};

template <int R, int MODE, bool FUSED, bool SCREEN>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(FUSED && R <= 64 ? 4 : 1))) void score_kernel(GqaDev g, const uint16_t* __restrict__ q,
                                                    const float* __restrict__ qsel,
                                                    const float* __restrict__ P,
                                                    const uint16_t* __restrict__ Kp,
                                                    float* __restrict__ scores, FusedOut fo) {
  constexpr int PP = R / 8;                   // lanes (16-byte pieces) per token
  constexpr bool kDpp = (PP & (PP - 1)) == 0; // power of two -> DPP groups
  // qp slices held per lane: load m of a tile gives lane l piece
  // (64 m + l) % PP, which repeats with period PP / gcd(64, PP) in m
  constexpr int kLow = PP & -PP;              // gcd(64, PP) for PP <= 64
  constexpr int NSL = kDpp ? 1 : PP / kLow;
  constexpr int TPW = tiles_per_wave(MODE, FUSED);
  __shared__ ScoreSmem<R> sm;
  // Fused: token o of the chunk is staged at (o % TPW) * SS + o / TPW with
  // SS = NT + 64/TPW, so thread i later reads its TPW consecutive tokens
  // o = i*TPW + e at e*SS + i; the pad makes both the tile writes (64
  // consecutive o) and those reads hit 64 distinct LDS banks. Score-only:
  // staged at o.
  constexpr int NT = kWaves * 64;
  static_assert(!FUSED || (64 % TPW == 0 || TPW % 64 == 0), "fused staging pad");
  constexpr int SS = NT + (TPW <= 64 ? 64 / TPW : 1);
  constexpr int kStageBytes = FUSED ? TPW * SS * 4 : NT * TPW * 4;
  constexpr int kBufBytes = kStageBytes > int(sizeof(ChunkSmem<NT, TPW>)) ? kStageBytes : int(sizeof(ChunkSmem<NT, TPW>));
  __shared__ __attribute__((aligned(16))) char sbuf[kBufBytes];   // staged scores, then selection scratch

  // Work item of this block. Blocks go to the XCDs round-robin by launch
  // position. When some chunks lie past their sequence's end (per-sequence
  // lengths, up to kPackMaxB sequences), the first launch positions take the
  // sequences' real chunks in order, the KV head varying fastest (the heads
  // of one token range, which share the cache pages, are read together:
  // 1-2% on a paged cache), and the rest the empty ones, which
  // only record an empty segment: the real work is dealt evenly over the
  // XCDs and CUs instead of leaving the slots of empty chunks idle. Otherwise
  // launch position x holds chunk (x + row) mod nx, so chunk c of every row
  // does not land on one XCD.
  const int nx = int(gridDim.x);
  int b, j, cx;
  const int chunk_len = kWaves * 64 * TPW;
  auto nch = [&](int bb) { return (seq_len(g, bb) + chunk_len - 1) / chunk_len; };   // <= nx
  int real = g.B * g.Hkv * nx;                          // chunks before the sequences' ends
  if (g.seq_lens && g.B <= kPackMaxB) {
    real = 0;
#pragma unroll 8
    for (int bb = 0; bb < g.B; ++bb) real += g.Hkv * nch(bb);
  }
  if (real < g.B * g.Hkv * nx) {                        // some chunk lies past its sequence's end
    const int lin = int(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
    b = 0;
    j = 0;
    cx = 0;
    int acc = lin < real ? 0 : real;
    for (int bb = 0; bb < g.B; ++bb) {
      const int n = lin < real ? nch(bb) : nx - nch(bb), c = g.Hkv * n;   // chunks of each row of bb in this part
      if (lin < acc + c) {
        const int r = lin - acc;
        b = bb;
        j = r % g.Hkv;
        cx = (lin < real ? 0 : nx - n) + r / g.Hkv;
        break;
      }
      acc += c;
    }
  } else {
    b = int(blockIdx.z);
    j = int(blockIdx.y);
    cx = int((blockIdx.x + unsigned(b * g.Hkv + j) % 8u) % unsigned(nx));
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);     // wave index, kept scalar
  const int Tb = seq_len(g, b);
  const int chunk = kWaves * 64 * TPW;
  const int t_begin = cx * chunk;
  float* srow = scores ? scores + (int64_t(b) * g.Hkv + j) * g.max_seq : nullptr;
  const bool paged = g.page_size != 0;
  const int64_t ubase = (int64_t(b) * g.Hkv + j) * int64_t(g.max_seq) * R;   // contiguous unit base

  const bool lists = !FUSED && fo.segs.info != nullptr;   // score-only stream writing chunk lists (kernel-uniform)
  const int64_t seg = FUSED || lists ? int64_t(b * g.Hkv + j) * fo.segs.nseg + cx : 0;
  float* srow2 = FUSED && fo.scores2 ? fo.scores2 + (int64_t(b) * g.Hkv + j) * g.max_seq : nullptr;
  if (t_begin >= Tb) {                       // whole chunk past the sequence's end
    if (!FUSED || (fo.write_scores && !fo.lists)) {   // (list mode: its own copy is read below T_b only)
      const int lim = g.max_seq - t_begin < chunk ? g.max_seq - t_begin : chunk;
      for (int i = tid; i < lim; i += NT) __builtin_nontemporal_store(-__builtin_inff(), srow + t_begin + i);
        }
    if (srow2) {
      const int lim = g.max_seq - t_begin < chunk ? g.max_seq - t_begin : chunk;
      for (int i = tid; i < lim; i += NT) __builtin_nontemporal_store(-__builtin_inff(), srow2 + t_begin + i);
    }
    if (FUSED && tid == 0) {
      write_info(fo.segs, seg, 0, 0u, 0u, 0xffffffffu);
      if (fo.pmax) fo.pmax[seg] = 0u;
    }
    if (lists && tid == 0) write_info(fo.segs, seg, 0, 0u, 0u, 0xffffffffu);
    return;
  }
  // Tokens of this block are [t_begin, tend); loads of later positions are
  // clamped to token tend - 1 (a cache hit) and masked out of the result, so
  // every tile's loads are issued without a branch.
  const int tend = Tb - t_begin < chunk ? Tb : t_begin + chunk;
  __shared__ int pid[FUSED ? kWaves * 64 * kFusedTiles / kPage : kWaves * 64 * kPlainTiles / kPage];
  if (paged) {                               // page ids of the chunk (-1: no valid page)
    for (int i = tid; i < chunk / kPage; i += NT) {
      int t = t_begin + i * kPage;
      t = t < tend ? t : tend - 1;
      const int pg = g.page_table[int64_t(b) * g.max_pages + (t >> 4)];
      pid[i] = pg >= 0 && pg < g.num_pages ? pg : -1;
    }
    __syncthreads();
  }
  // Screening (SCREEN, a separate instantiation: the plain stream carries
  // none of this): the chunk's 128 tiles of 64 tokens have one keep bit
  // each. A wave streams only its kept tiles; its dropped tiles are staged
  // as dropped and cost no HBM bytes.
  uint32_t kw[4] = {~0u, ~0u, ~0u, ~0u};
  if (SCREEN) {
    const uint32_t* kp = fo.keep + int64_t(b * g.Hkv + j) * fo.keep_words;
    const int w0 = t_begin / (64 * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) kw[i] = w0 + i < fo.keep_words ? kp[w0 + i] : 0u;
  }
  if (SCREEN && (kw[0] | kw[1] | kw[2] | kw[3]) == 0u) {   // every tile dropped (block-uniform)
    if (tid == 0) {
      write_info(fo.segs, seg, 0, 0u, 0u, 0xffffffffu);
      if (fo.pmax) fo.pmax[seg] = 0u;
    }
    return;
  }
  auto load_tile = [&](int tile, u32x4 (&buf)[PP]) {
    const int t0 = t_begin + (tile * kWaves + w) * 64;
#pragma unroll
    for (int m = 0; m < PP; ++m) {
      const int p = m * 64 + lane;
      int t = t0 + p / PP;
      t = t < tend ? t : tend - 1;
      int64_t off;
      if (!paged) {
        off = ubase + int64_t(t) * R;
      } else {
        int pg = pid[(t - t_begin) >> 4];
        pg = pg < 0 ? 0 : pg;
        off = ((int64_t(pg) * g.Hkv + j) * kPage + (t & (kPage - 1))) * R;
      }
      buf[m] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Kp + off) + p % PP);
    }
  };
  auto token_ok = [&](int t) -> bool {
    if (t >= tend) return false;
    return !paged || pid[(t - t_begin) >> 4] >= 0;
  };

  // Screening: the wave streams only its kept tiles, in order. Lane r holds
  // the r-th kept tile of the wave (pushed there by the lane of that tile),
  // read back with a uniform readlane; past the last one the last is
  // repeated (loads hit the cache, the stage write repeats the same scores).
  int nkept = TPW, klist = 0;
  uint32_t kmask = 0u;
  if constexpr (SCREEN) {
    // lane l < TPW: is tile l of this wave (chunk tile l * kWaves + w) kept?
    const int ct = lane * kWaves + w;
    const uint32_t word = ct < 32 ? kw[0] : (ct < 64 ? kw[1] : (ct < 96 ? kw[2] : kw[3]));
    const bool kb = lane < TPW && ((word >> (ct & 31)) & 1u) != 0u;
    kmask = uint32_t(__ballot(kb));
    nkept = __builtin_popcount(kmask);
    const int rank = __builtin_popcount(kmask & ((1u << (lane & 31)) - 1u));
    klist = __builtin_amdgcn_ds_permute((kb ? rank : 63) * 4, lane);
  }
  auto kept_tile = [&](int i) -> int {
    if constexpr (!SCREEN) return i;
    return __builtin_amdgcn_readlane(klist, i < nkept ? i : nkept - 1);
  };

  constexpr int kDepth = depth_of(R, FUSED);
  u32x4 bufs[kDepth][PP];
  // the first tiles' loads: in flight during the prologue, issued after the
  // prologue's own loads (a wave's loads complete in issue order, so the
  // prologue then waits for its query and P values only, not for a tile)
  auto first_tiles = [&]() {
    if (nkept > 0) {
#pragma unroll
      for (int u = 0; u < kDepth - 1; ++u) load_tile(kept_tile(u), bufs[u]);
    }
    // keep the scheduler from moving the prologue's arithmetic (which waits
    // for the query values) above these loads
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- prologue: qp = P_j^T qbar (fp32). The slice of P this thread needs
  // and the group's query rows are loaded together (one round trip, not two),
  // with every loop unrolled so that its loads are all in flight at once.
  if constexpr (MODE == kGqa) {
    constexpr int NS = NT / R;                 // row slices of P
    constexpr int NI = (kD + NS - 1) / NS;     // rows per slice
    constexpr bool kPreP = NI <= 32;           // hold the slice in registers
    constexpr int kMaxG = 16;                  // query heads per KV head (validated on the host)
    const int c = tid % R, sl = tid / R;
    const float* Pj = P + int64_t(j) * kD * R;
    float pv[kPreP ? NI : 1];
    if constexpr (kPreP) {
#pragma unroll
      for (int ii = 0; ii < NI; ++ii) {
        const int i = sl + ii * NS;
        pv[ii] = Pj[(i < kD ? i : kD - 1) * R + c];   // unconditional load, zero weight past d
      }
    }
    // column tid of the group's query rows, loaded by every thread (column 0
    // past d, unused): loads under a branch would make the compiler wait for
    // them before issuing the tiles' loads
    uint16_t qh[kMaxG];
    {
      const uint16_t* qg = q + (int64_t(b) * g.Hq + int64_t(j) * g.G) * kD + (tid < kD ? tid : 0);
#pragma unroll
      for (int h = 0; h < kMaxG; ++h) qh[h] = qg[(h < g.G ? h : g.G - 1) * kD];   // clamped: a valid row
    }
    first_tiles();
    if (tid < kD) {
      float s = 0.f;
#pragma unroll
      for (int h = 0; h < kMaxG; ++h) s += h < g.G ? bf(qh[h]) : 0.f;
      sm.u.pro.qbar[tid] = s;
    }
    __syncthreads();
    if (sl < NS) {
      float s = 0.f;
#pragma unroll 16
      for (int ii = 0; ii < NI; ++ii) {
        const int i = sl + ii * NS;
        const int ic = i < kD ? i : kD - 1;
        const float p = kPreP ? pv[kPreP ? ii : 0] : Pj[ic * R + c];
        s = __builtin_fmaf(p, i < kD ? sm.u.pro.qbar[ic] : 0.f, s);
      }
      sm.u.pro.qpart[sl * R + c] = s;
    }
    __syncthreads();
    if (tid < R) {
      float s = 0.f;
      for (int x = 0; x < NS; ++x) s += sm.u.pro.qpart[x * R + tid];
      sm.qp[tid] = s;
    }
    __syncthreads();
  } else {
    // MLA: the selection query qp = sum of its kMlaSelParts rows qsel[b,x,:]
    // (written by the absorb step). Thread (c, part) adds rows part, part +
    // NP, ... of column c, in order; the NP partial sums then meet in LDS,
    // in order (a fixed summation order: every block of the sequence gets
    // the same qp). The rows are loaded before the first tiles go out.
    constexpr int NP = NT / R;
    constexpr int kRows = (kMlaSelParts + NP - 1) / NP;   // rows per thread
    const int c = tid % R, part = tid / R;
    const float* qb = qsel + int64_t(b) * kMlaSelParts * R + c;
    float hv[kRows];
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      const int x = part + u * NP;
      hv[u] = qb[int64_t(x < kMlaSelParts ? x : 0) * R];   // clamped: a valid row, not added
    }
    first_tiles();
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < kRows; ++u) acc += part + u * NP < kMlaSelParts ? hv[u] : 0.f;
    sm.u.pro.qpart[part * R + c] = acc;
    __syncthreads();
    if (tid < R) {
      float t = 0.f;
      for (int x = 0; x < NP; ++x) t += sm.u.pro.qpart[x * R + tid];
      sm.qp[tid] = t;
    }
    __syncthreads();
  }
  float qr[NSL][8];
#pragma unroll
  for (int m = 0; m < NSL; ++m) {
    const int sl = (m * 64 + lane) % PP;
#pragma unroll
    for (int e = 0; e < 8; ++e) qr[m][e] = sm.qp[sl * 8 + e];
  }

  // score of token t0 + lane of the current tile
  auto tile_scores = [&](const u32x4 (&v)[PP]) -> float {
    if constexpr (kDpp) {
      constexpr int TPI = 64 / PP;            // tokens per load column
      // Every lane of a group holds the group sum; lane g*PP + i keeps the
      // sum of load i (token i*TPI + g), so one permute hands each lane its
      // token: token t is in load t / TPI, group t % TPI.
      float r = 0.f;
#pragma unroll
      for (int m = 0; m < PP; ++m) {
        const float s = group_sum<PP>(dot8(qr[0], v[m]));
        r = (lane % PP) == m ? s : r;
      }
      return __shfl(r, (lane % TPI) * PP + lane / TPI, 64);
    } else {
      // Token t of the tile sits in lanes PP*t .. PP*t+PP-1 of the loads taken
      // as one 64*PP-lane row; the first PP/2 loads hold tokens 0..31 and the
      // rest tokens 32..63, so the partials go through LDS half at a time.
      static_assert(PP % 2 == 0, "a tile's loads split into two halves of 32 tokens");
      constexpr int HALF = PP / 2;
      float* pw = sm.u.part + w * 32 * PP;
      float s = 0.f;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int m = 0; m < HALF; ++m) pw[m * 64 + lane] = dot8(qr[(hh * HALF + m) % NSL], v[hh * HALF + m]);
        wave_lds_sync();
        if ((lane >> 5) == hh) {
#pragma unroll
          for (int pc = 0; pc < PP; ++pc) s += pw[(lane & 31) * PP + pc];
        }
        wave_lds_sync();
      }
      return s;
    }
  };

  // Stream the chunk's tiles; the scores are staged in LDS and leave only
  // after the stream, as non-temporal stores (they are not read again in
  // this kernel; kept out of the caches, they do not crowd the stream's
  // loads: the score-only stream at 128K x B = 16 went from 192.7 to 183.9
  // us). (A store inside the loop would sit in the in-order
  // vmcnt queue between tile loads, so every wait for a tile would also wait
  // for the previous store's write acknowledgement; holding them in
  // registers would cost occupancy.)
  float* stage = reinterpret_cast<float*>(sbuf);
  auto sidx = [](int o) { return FUSED ? (o % TPW) * SS + o / TPW : o; };
  auto stage_tile = [&](int tile, const u32x4 (&buf)[PP]) {
    const int off = (tile * kWaves + w) * 64;
    const float x = tile_scores(buf);
    const float v = token_ok(t_begin + off + lane) ? x : -__builtin_inff();
    stage[sidx(off + lane)] = v;
  };
  // kDepth register buffers rotate with no copies between them (a copy of a
  // buffer whose loads are in flight would wait for them): while one tile's
  // scores are computed, the loads of the next kDepth - 1 tiles are in flight.
  static_assert(TPW % kDepth == 0, "tiles are streamed in groups of kDepth");
  if constexpr (SCREEN) {
    for (int tile = 0; tile < TPW; ++tile)             // dropped tiles: staged as such, nothing read
      if (!((kmask >> tile) & 1u)) stage[sidx((tile * kWaves + w) * 64 + lane)] = __uint_as_float(kDroppedBits);
  }
  for (int i = 0; i < nkept; i += kDepth) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      // past the chunk (or the last kept tile) on the last group: clamped, unused
      load_tile(kept_tile(i + u + kDepth - 1), bufs[(u + kDepth - 1) % kDepth]);
      stage_tile(kept_tile(i + u), bufs[u]);
    }
  }
  __syncthreads();
  if (!FUSED || fo.write_scores) {
    float* dst = srow + t_begin;
    float* dst2 = srow2 ? srow2 + t_begin : nullptr;
    const int lim = g.max_seq - t_begin;                 // > 0
    // list mode: the workspace copy is only read below T_b (the caller's copy,
    // dst2, is the whole row)
    const int lim1 = FUSED && fo.lists ? (Tb - t_begin + 3) & ~3 : lim;
    if ((g.max_seq & 3) == 0) {                          // 16-byte aligned row chunk
      for (int i = tid * 4; i < chunk && i < lim; i += 4 * NT) {
        const f32x4 v = f32x4{stage[sidx(i)], stage[sidx(i + 1)], stage[sidx(i + 2)], stage[sidx(i + 3)]};
        if (i < lim1) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst + i));
        if (dst2) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst2 + i));
      }
    } else {
      for (int i = tid; i < chunk && i < lim; i += NT) {
        if (i < lim1) dst[i] = stage[sidx(i)];
        if (dst2) dst2[i] = stage[sidx(i)];
      }
    }
  }
  if constexpr (!FUSED) {
    if (lists) {
      // The chunk's own top fo.k (every real token at or above its fo.k-th
      // key, chunk_select), written as the chunk's candidate segment in
      // token order; thread tid takes tokens tid*TPW .. tid*TPW+TPW-1 (the
      // stage is in token order, and positions past the end hold -inf: key 0).
      uint32_t key[TPW];
#pragma unroll
      for (int e = 0; e < TPW; ++e) key[e] = score_key(stage[tid * TPW + e]);
      int n = Tb - t_begin;
      n = n > chunk ? chunk : n;
      __syncthreads();                                   // the stage is reused below
      ChunkSmem<NT, TPW>& csm = *reinterpret_cast<ChunkSmem<NT, TPW>*>(sbuf);
      // (no slack: the union of these lists is what the final pass selects from)
      chunk_select<NT, TPW>(key, t_begin, Tb, n, fo.k, csm, fo.segs, seg, 0);
      // a list of one chunk bounds nothing about the row's k-th key: no floor
      if (tid == 0) fo.segs.info[seg].floor = 0u;
    }
  }
  if constexpr (FUSED) {
    if (fo.pmax) {                                       // top-delta pseudo-max contribution of this chunk
      const int e1 = fo.n_sink < tend ? fo.n_sink : tend;
      const int s2 = Tb - fo.n_local > t_begin ? Tb - fo.n_local : t_begin;
      uint32_t pm = 0u;
      if (e1 > t_begin || tend > s2) {                   // block-uniform
        __shared__ uint32_t pred[kWaves];
        uint32_t v = 0u;
        for (int t = t_begin + tid; t < e1; t += NT) {
          const uint32_t x = score_key(stage[sidx(t - t_begin)]);
          v = x > v ? x : v;
        }
        for (int t = s2 + tid; t < tend; t += NT) {
          const uint32_t x = score_key(stage[sidx(t - t_begin)]);
          v = x > v ? x : v;
        }
        v = wave_max_u32(v);
        if (lane == 0) pred[w] = v;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kWaves; ++i) pm = pred[i] > pm ? pred[i] : pm;
      }
      if (tid == 0) fo.pmax[seg] = pm;
    }
    __shared__ Top2Smem<NT> tsm;
    uint32_t key[TPW];
#pragma unroll
    for (int e = 0; e < TPW; ++e) key[e] = score_key(stage[e * SS + tid]);   // token tid*TPW + e
    int n = Tb - t_begin;
    n = n < 0 ? 0 : (n > chunk ? chunk : n);
    // the top-two bound first (block-uniform; it leaves the stage intact),
    // the histogram select when it does not apply or keeps too many
    const bool done = n == chunk && fo.k <= NT && !fo.lists &&
                      chunk_select_top2<NT, TPW>(key, t_begin, fo.k, tsm, stage, SS, fo.segs, seg);
    if (!done) {
      __syncthreads();                                   // stage is reused below
      ChunkSmem<NT, TPW>& csm = *reinterpret_cast<ChunkSmem<NT, TPW>*>(sbuf);
      chunk_select<NT, TPW>(key, t_begin, Tb, n, fo.k, csm, fo.segs, seg, fo.lists ? 0 : kSelSlack);
      // a list of one chunk bounds nothing about the row's k-th key: no floor
      if (fo.lists && tid == 0) fo.segs.info[seg].floor = 0u;
    }
  }
}

template <int MODE, bool FUSED, bool SCREEN = false>
hipError_t launch_score_t(const GqaDev& g, const uint16_t* q, const float* qsel, const float* P,
                          const uint16_t* Kp, float* scores, hipStream_t st, FusedOut fo) {
  const int64_t chunk = kWaves * 64 * tiles_per_wave(MODE, FUSED);
  dim3 grid(unsigned((g.max_seq + chunk - 1) / chunk), g.Hkv, g.B);
  switch (g.r) {
#define JSSA_CASE(R)                                                                                  \
  case R:                                                                                             \
    hipLaunchKernelGGL((score_kernel<R, MODE, FUSED, SCREEN>), grid, dim3(kWaves * 64), 0, st, g, q, qsel, P, Kp, \
                       scores, fo);                                                                   \
    break;
    JSSA_CASE(16) JSSA_CASE(32) JSSA_CASE(48) JSSA_CASE(64) JSSA_CASE(128)
#undef JSSA_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score(const GqaDev& g, const uint16_t* q, const float* P, const uint16_t* Kp,
                        float* scores, hipStream_t st) {
  return launch_score_t<kGqa, false>(g, q, nullptr, P, Kp, scores, st, FusedOut{});
}

hipError_t launch_mla_score(const MlaDev& m, const float* q_sel, const uint16_t* Kp, float* scores,
                            hipStream_t st) {
  GqaDev g{};
  g.B = m.B;
  g.Hq = 1;
  g.Hkv = 1;
  g.G = 1;
  g.d = kDc;
  g.r = m.r;
  g.max_seq = m.max_seq;
  g.seq_lens = m.seq_lens;
  return launch_score_t<kMla, false>(g, nullptr, q_sel, nullptr, Kp, scores, st, FusedOut{});
}

hipError_t launch_mla_score_lists(const MlaDev& m, const float* q_sel, const uint16_t* Kp, float* scores,
                                  CandSegs lists, int list_k, hipStream_t st) {
  GqaDev g{};
  g.B = m.B;
  g.Hq = 1;
  g.Hkv = 1;
  g.G = 1;
  g.d = kDc;
  g.r = m.r;
  g.max_seq = m.max_seq;
  g.seq_lens = m.seq_lens;
  FusedOut fo{};
  fo.segs = lists;
  fo.k = list_k;
  return launch_score_t<kMla, false>(g, nullptr, q_sel, nullptr, Kp, scores, st, fo);
}

int mla_score_chunks(int max_seq) {
  const int chunk = kWaves * 64 * kMlaTiles;
  return (max_seq + chunk - 1) / chunk;
}

int score_topk_segments(int max_seq) {
  const int chunk = kWaves * 64 * kFusedTiles;
  return (max_seq + chunk - 1) / chunk;
}

int score_topk_segment_cap(int k) { return seg_cap(k, kWaves * 64 * kFusedTiles); }

int score_topk_chunk_len() { return kWaves * 64 * kFusedTiles; }

hipError_t launch_score_chunks(const GqaDev& g, const uint16_t* q, const float* P, const uint16_t* Kp, int k,
                               float* scores, CandSegs segs, hipStream_t st, uint32_t* pmax, int n_sink,
                               int n_local, const uint32_t* keep, int keep_words) {
  FusedOut fo{segs, k, scores ? 1 : 0, pmax, n_sink, n_local, keep, keep_words};
  if (keep) return launch_score_t<kGqa, true, true>(g, q, nullptr, P, Kp, scores, st, fo);
  return launch_score_t<kGqa, true>(g, q, nullptr, P, Kp, scores, st, fo);
}

hipError_t launch_score_chunks_lists(const GqaDev& g, const uint16_t* q, const float* P, const uint16_t* Kp, int kc,
                                     float* scores_ws, float* scores_user, CandSegs lists, hipStream_t st,
                                     const uint32_t* keep, int keep_words) {
  FusedOut fo{lists, kc, 1, nullptr, 0, 0, keep, keep_words, 1, scores_user};
  if (keep) return launch_score_t<kGqa, true, true>(g, q, nullptr, P, Kp, scores_ws, st, fo);
  return launch_score_t<kGqa, true>(g, q, nullptr, P, Kp, scores_ws, st, fo);
}

hipError_t launch_score_topk(const GqaDev& g, const uint16_t* q, const float* P, const uint16_t* Kp, int k,
                             float* scores, int32_t* idx, CandSegs segs, void* merge_ws, hipStream_t st) {
  hipError_t e = launch_score_chunks(g, q, P, Kp, k, scores, segs, st);
  if (e != hipSuccess) return e;
  return launch_select_final(g.B * g.Hkv, g.Hkv, g.max_seq, g.seq_lens, k, segs, idx, merge_ws, st);
}

}  // namespace jssa

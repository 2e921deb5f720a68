// C ABI of the JSSA library: host-side validation, then the call's launches.
// Declarations and the contract of every entry point are in include/jssa.h.
#include "../../include/jssa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <vector>

#include "internal.hpp"

namespace {

thread_local char g_err[512] = "";

jssa_status fail(jssa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

jssa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) {
    g_err[0] = 0;
    return JSSA_OK;
  }
  return fail(JSSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE_PTR(p)                                                          \
  do {                                                                          \
    if (!(p)) return fail(JSSA_ERR_NULL, "%s: %s is NULL", __func__, #p);       \
    if (!aligned(p)) return fail(JSSA_ERR_ALIGN, "%s: %s is not 16-byte aligned", __func__, #p); \
  } while (0)
#define REQUIRE_ALIGNED_OPT(p)                                                  \
  do {                                                                          \
    if ((p) && !aligned(p))                                                     \
      return fail(JSSA_ERR_ALIGN, "%s: %s is not 16-byte aligned", __func__, #p); \
  } while (0)

constexpr int32_t kMaxSeq = 1 << 24;

jssa_status check_desc(const char* fn, const jssa_gqa_desc* d, bool need_rank) {
  if (!d) return fail(JSSA_ERR_NULL, "%s: desc is NULL", fn);
  if (d->B < 1 || d->Hq < 1 || d->Hkv < 1)
    return fail(JSSA_ERR_SHAPE, "%s: B, Hq, Hkv must be >= 1 (got %d, %d, %d)", fn, d->B, d->Hq, d->Hkv);
  if (d->Hq % d->Hkv != 0)
    return fail(JSSA_ERR_SHAPE, "%s: Hq (%d) is not a multiple of Hkv (%d)", fn, d->Hq, d->Hkv);
  if (d->Hq / d->Hkv > 16)
    return fail(JSSA_ERR_UNSUPPORTED, "%s: group size %d > 16", fn, d->Hq / d->Hkv);
  if (d->d != 128) return fail(JSSA_ERR_UNSUPPORTED, "%s: head width %d (only 128)", fn, d->d);
  if (need_rank && d->r != 16 && d->r != 32 && d->r != 48 && d->r != 64 && d->r != 128)
    return fail(JSSA_ERR_UNSUPPORTED, "%s: rank %d (16, 32, 48, 64 or 128)", fn, d->r);
  if (d->max_seq < 1 || d->max_seq > kMaxSeq)
    return fail(JSSA_ERR_SHAPE, "%s: max_seq %d outside [1, 2^24]", fn, d->max_seq);
  if (int64_t(d->B) * d->Hq > (1 << 24))
    return fail(JSSA_ERR_SHAPE, "%s: B*Hq too large", fn);
  if (d->page_size != 0 && d->page_size != 16)
    return fail(JSSA_ERR_UNSUPPORTED, "%s: page_size %d (0 or 16)", fn, d->page_size);
  if (d->page_size == 16) {
    if (!d->page_table) return fail(JSSA_ERR_NULL, "%s: page_table is NULL for a paged cache", fn);
    if (d->num_pages < 1) return fail(JSSA_ERR_SHAPE, "%s: num_pages %d", fn, d->num_pages);
    if (d->max_pages_per_seq < (d->max_seq + 15) / 16)
      return fail(JSSA_ERR_SHAPE, "%s: max_pages_per_seq %d < ceil(max_seq/16)", fn, d->max_pages_per_seq);
  }
  return JSSA_OK;
}

jssa::GqaDev to_dev(const jssa_gqa_desc* d) {
  jssa::GqaDev g;
  g.B = d->B;
  g.Hq = d->Hq;
  g.Hkv = d->Hkv;
  g.G = d->Hq / d->Hkv;
  g.d = d->d;
  g.r = d->r;
  g.max_seq = d->max_seq;
  g.page_size = d->page_size;
  g.num_pages = d->page_size ? d->num_pages : 0;
  g.max_pages = d->page_size ? d->max_pages_per_seq : 0;
  g.page_table = d->page_size ? d->page_table : nullptr;
  g.seq_lens = d->seq_lens;
  return g;
}

hipStream_t S(void* s) { return static_cast<hipStream_t>(s); }

jssa_status check_mla(const char* fn, const jssa_mla_desc* m) {
  if (!m) return fail(JSSA_ERR_NULL, "%s: desc is NULL", fn);
  if (m->B < 1 || m->H < 1) return fail(JSSA_ERR_SHAPE, "%s: B and H must be >= 1", fn);
  if (m->H % 16 != 0 || m->H > 1024)
    return fail(JSSA_ERR_UNSUPPORTED, "%s: H %d (a multiple of 16, <= 1024)", fn, m->H);
  if (m->d_latent != 512 || m->d_rope != 64 || m->d_nope != 128 || m->d_v != 128)
    return fail(JSSA_ERR_UNSUPPORTED, "%s: widths latent/rope/nope/v must be 512/64/128/128", fn);
  if (m->r != 16 && m->r != 32 && m->r != 64)
    return fail(JSSA_ERR_UNSUPPORTED, "%s: rank %d (16, 32 or 64)", fn, m->r);
  if (m->max_seq < 1 || m->max_seq > kMaxSeq)
    return fail(JSSA_ERR_SHAPE, "%s: max_seq %d outside [1, 2^24]", fn, m->max_seq);
  return JSSA_OK;
}

jssa::MlaDev to_mla(const jssa_mla_desc* m) {
  return jssa::MlaDev{m->B, m->H, m->d_latent, m->d_rope, m->d_nope, m->d_v, m->r, m->max_seq,
                      m->seq_lens};
}

}  // namespace

namespace {
// Workspace of the fused score -> top-k selection (jssa_score_topk and the
// split _chunks / _final calls). Classic: each 8192-token chunk keeps every
// token that can be among its row's top k (candidate segments of
// score_topk_segment_cap(k)), merged level by level when a row's lists are
// too long for one final pass. Lists (budgets whose candidates would need a
// merge level): each chunk keeps only its own top kc, kc = 3x the chunk's
// share of k; one final pass selects from their union and checks that the
// union held the row's top k, selecting the row again from its scores when
// it did not (so the stream also writes the scores, into the workspace).
struct TopkWs {
  jssa::CandSegs segs;
  void* merge_ws;   // classic: merge levels
  float* scores;    // lists: the rows' scores [rows, max_seq]; classic: nullptr
  int kc;           // lists: per-chunk list length; classic: 0
  size_t bytes;
};

int gqa_list_k(int max_seq, int k) {
  const int nseg = jssa::score_topk_segments(max_seq);
  if (nseg <= 1 || int64_t(nseg) * k <= 8192) return 0;          // one final pass already
  int kc = 3 * ((k + nseg - 1) / nseg);
  kc = kc < 64 ? 64 : kc;
  kc = (kc + 3) & ~3;
  return 2 * kc <= k ? kc : 0;
}

TopkWs topk_ws(const jssa_gqa_desc* d, int k, void* ws, bool allow_lists) {
  TopkWs w{};
  const int rows = d->B * d->Hkv, nseg = jssa::score_topk_segments(d->max_seq);
  w.kc = allow_lists ? gqa_list_k(d->max_seq, k) : 0;
  size_t main_bytes = 0;
  if (w.kc) {
    w.segs = jssa::carve_segs(ws, rows, nseg, jssa::seg_cap(w.kc, jssa::score_topk_chunk_len()), &main_bytes);
    w.scores = ws ? reinterpret_cast<float*>(static_cast<char*>(ws) + main_bytes) : nullptr;
    w.merge_ws = nullptr;
    w.bytes = main_bytes + jssa::align256(size_t(rows) * d->max_seq * sizeof(float));
  } else {
    w.segs = jssa::carve_segs(ws, rows, nseg, jssa::score_topk_segment_cap(k), &main_bytes);
    w.merge_ws = ws ? static_cast<char*>(ws) + main_bytes : nullptr;
    w.scores = nullptr;
    w.bytes = main_bytes + jssa::merge_workspace_bytes(rows, nseg, k);
  }
  return w;
}

// the final pass of either layout
hipError_t topk_ws_final(const jssa_gqa_desc* d, int k, const TopkWs& w, int32_t* idx, hipStream_t st) {
  if (w.kc)
    return jssa::launch_topk_lists(d->B * d->Hkv, d->Hkv, d->max_seq, d->seq_lens, w.scores, k, idx, w.segs,
                                   jssa::score_topk_chunk_len(), st);
  return jssa::launch_select_final(d->B * d->Hkv, d->Hkv, d->max_seq, d->seq_lens, k, w.segs, idx, w.merge_ws, st);
}

// the fused stream of either layout (scores: the caller's optional buffer)
hipError_t topk_ws_chunks(const jssa_gqa_desc* d, const void* q, const float* P, const void* Kp, int k,
                          float* scores, const TopkWs& w, hipStream_t st) {
  const auto* q16 = static_cast<const uint16_t*>(q);
  const auto* Kp16 = static_cast<const uint16_t*>(Kp);
  if (w.kc) return jssa::launch_score_chunks_lists(to_dev(d), q16, P, Kp16, w.kc, w.scores, scores, w.segs, st);
  return jssa::launch_score_chunks(to_dev(d), q16, P, Kp16, k, scores, w.segs, st);
}

hipError_t score_topk_impl(const jssa_gqa_desc* d, const void* q, const float* P, const void* Kp, int k,
                           float* scores, int32_t* idx, void* ws, bool allow_lists, hipStream_t st) {
  const TopkWs w = topk_ws(d, k, ws, allow_lists);
  hipError_t e = topk_ws_chunks(d, q, P, Kp, k, scores, w, st);
  if (e == hipSuccess) e = topk_ws_final(d, k, w, idx, st);
  return e;
}
}  // namespace

extern "C" {

int32_t jssa_version(void) { return 100; }

const char* jssa_last_error(void) { return g_err; }

const char* jssa_status_string(jssa_status s) {
  switch (s) {
    case JSSA_OK: return "ok";
    case JSSA_ERR_NULL: return "null pointer";
    case JSSA_ERR_SHAPE: return "bad shape";
    case JSSA_ERR_UNSUPPORTED: return "unsupported size";
    case JSSA_ERR_ALIGN: return "misaligned pointer";
    case JSSA_ERR_WORKSPACE: return "workspace too small";
    case JSSA_ERR_HIP: return "HIP runtime error";
    case JSSA_ERR_NUMERIC: return "numerical routine did not converge";
    default: return "unknown status";
  }
}

jssa_status jssa_append_kv(const jssa_gqa_desc* desc, void* K, void* V, void* Kp, const void* k_new,
                           const void* v_new, const float* P, const int32_t* pos, int32_t n_new,
                           void* stream) {
  if (jssa_status s = check_desc(__func__, desc, true)) return s;
  REQUIRE_PTR(K); REQUIRE_PTR(V); REQUIRE_PTR(Kp); REQUIRE_PTR(k_new); REQUIRE_PTR(v_new);
  REQUIRE_PTR(P); REQUIRE_PTR(pos);
  if (n_new < 1 || n_new > desc->max_seq)
    return fail(JSSA_ERR_SHAPE, "%s: n_new %d outside [1, max_seq]", __func__, n_new);
  return hip_status(jssa::launch_project(to_dev(desc), static_cast<const uint16_t*>(k_new), 0, pos,
                                         n_new, true, static_cast<uint16_t*>(K),
                                         static_cast<uint16_t*>(V),
                                         static_cast<const uint16_t*>(v_new), P,
                                         static_cast<uint16_t*>(Kp), S(stream)),
                    __func__);
}

jssa_status jssa_project_keys(const jssa_gqa_desc* desc, const void* K, const float* P, void* Kp,
                              void* stream) {
  if (jssa_status s = check_desc(__func__, desc, true)) return s;
  REQUIRE_PTR(K); REQUIRE_PTR(P); REQUIRE_PTR(Kp);
  return hip_status(jssa::launch_project(to_dev(desc), static_cast<const uint16_t*>(K), 0, nullptr,
                                         desc->max_seq, false, nullptr, nullptr, nullptr, P,
                                         static_cast<uint16_t*>(Kp), S(stream)),
                    __func__);
}

jssa_status jssa_score(const jssa_gqa_desc* desc, const void* q, const float* P, const void* Kp,
                       float* scores, void* stream) {
  if (jssa_status s = check_desc(__func__, desc, true)) return s;
  REQUIRE_PTR(q); REQUIRE_PTR(P); REQUIRE_PTR(Kp); REQUIRE_PTR(scores);
  return hip_status(jssa::launch_score(to_dev(desc), static_cast<const uint16_t*>(q), P,
                                       static_cast<const uint16_t*>(Kp), scores, S(stream)),
                    __func__);
}

jssa_status jssa_topk_workspace_size(int32_t B, int32_t H, int32_t max_seq, int32_t k, size_t* bytes) {
  if (!bytes) return fail(JSSA_ERR_NULL, "%s: bytes is NULL", __func__);
  if (B < 1 || H < 1 || int64_t(B) * H > (1 << 24))
    return fail(JSSA_ERR_SHAPE, "%s: B %d, H %d", __func__, B, H);
  if (max_seq < 1 || max_seq > kMaxSeq)
    return fail(JSSA_ERR_SHAPE, "%s: max_seq %d outside [1, 2^24]", __func__, max_seq);
  if (k < 1 || k > 4096 || k > max_seq)
    return fail(JSSA_ERR_SHAPE, "%s: k %d outside [1, min(4096, max_seq)]", __func__, k);
  *bytes = jssa::topk_workspace_bytes(B * H, max_seq, k);
  return JSSA_OK;
}

jssa_status jssa_topk(int32_t B, int32_t H, int32_t max_seq, const int32_t* seq_lens,
                      const float* scores, int32_t k, int32_t* idx, void* ws, size_t ws_bytes,
                      void* stream) {
  size_t need = 0;
  if (jssa_status s = jssa_topk_workspace_size(B, H, max_seq, k, &need)) return s;
  REQUIRE_PTR(scores); REQUIRE_PTR(idx); REQUIRE_ALIGNED_OPT(seq_lens);
  if (need > 0) REQUIRE_PTR(ws);
  if (ws_bytes < need)
    return fail(JSSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__, ws_bytes, need);
  return hip_status(jssa::launch_topk(B, H, max_seq, seq_lens, scores, k, idx, ws, S(stream)),
                    __func__);
}

jssa_status jssa_score_topk_workspace_size(const jssa_gqa_desc* desc, int32_t k, size_t* bytes) {
  if (jssa_status s = check_desc(__func__, desc, true)) return s;
  if (!bytes) return fail(JSSA_ERR_NULL, "%s: bytes is NULL", __func__);
  if (k < 1 || k > 4096 || k > desc->max_seq)
    return fail(JSSA_ERR_SHAPE, "%s: k %d outside [1, min(4096, max_seq)]", __func__, k);
  *bytes = topk_ws(desc, k, nullptr, true).bytes;
  return JSSA_OK;
}

jssa_status jssa_score_topk(const jssa_gqa_desc* desc, const void* q, const float* P, const void* Kp, int32_t k,
                            float* scores, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  if (jssa_status s = jssa_score_topk_workspace_size(desc, k, &need)) return s;
  REQUIRE_PTR(q); REQUIRE_PTR(P); REQUIRE_PTR(Kp); REQUIRE_PTR(idx); REQUIRE_PTR(ws);
  REQUIRE_ALIGNED_OPT(scores);
  if (ws_bytes < need)
    return fail(JSSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__, ws_bytes, need);
  return hip_status(score_topk_impl(desc, q, P, Kp, k, scores, idx, ws, true, S(stream)), __func__);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// jssa_score_topk without a caller workspace: the candidate lists live in a
// file-scope device array of this library (each GPU the library runs on
// holds its own copy until the process ends). Host code never passes the
// array's name to a kernel: its device address is taken once per device
// with hipGetSymbolAddress, with that device current, and kept.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the scratch array on the current device.
jssa_status scratch_address(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  if (dev < 0 || dev >= kMaxDevices) return fail(JSSA_ERR_UNSUPPORTED, "%s: device ordinal %d", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, fn);
    if (!p) return fail(JSSA_ERR_HIP, "%s: no device address for the scratch array", fn);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return JSSA_OK;
}

}  // namespace

extern "C" {

jssa_status jssa_score_topk_noalloc(const jssa_gqa_desc* desc, const void* q, const float* P, const void* Kp,
                                   int32_t k, float* scores, int32_t* idx, void* stream) {
  size_t need = 0;
  if (jssa_status s = jssa_score_topk_workspace_size(desc, k, &need)) return s;   // (validation)
  REQUIRE_PTR(q); REQUIRE_PTR(P); REQUIRE_PTR(Kp); REQUIRE_PTR(idx);
  REQUIRE_ALIGNED_OPT(scores);
  need = topk_ws(desc, k, nullptr, false).bytes;        // the candidate-list layout: no score rows
  if (need > kScratchBytes)
    return fail(JSSA_ERR_WORKSPACE,
                "%s: this shape needs %zu bytes of candidate lists, more than the %zu-byte static scratch; "
                "use jssa_score_topk with a workspace",
                __func__, need, kScratchBytes);
  void* ws = nullptr;
  if (jssa_status s = scratch_address(__func__, &ws)) return s;
  return hip_status(score_topk_impl(desc, q, P, Kp, k, scores, idx, ws, false, S(stream)), __func__);
}

jssa_status jssa_score_topk_chunks(const jssa_gqa_desc* desc, const void* q, const float* P, const void* Kp,
                                   int32_t k, float* scores, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  if (jssa_status s = jssa_score_topk_workspace_size(desc, k, &need)) return s;
  REQUIRE_PTR(q); REQUIRE_PTR(P); REQUIRE_PTR(Kp); REQUIRE_PTR(ws);
  REQUIRE_ALIGNED_OPT(scores);
  if (ws_bytes < need)
    return fail(JSSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__, ws_bytes, need);
  return hip_status(topk_ws_chunks(desc, q, P, Kp, k, scores, topk_ws(desc, k, ws, true), S(stream)), __func__);
}

jssa_status jssa_score_topk_final(const jssa_gqa_desc* desc, int32_t k, const void* ws, size_t ws_bytes,
                                  int32_t* idx, void* stream) {
  size_t need = 0;
  if (jssa_status s = jssa_score_topk_workspace_size(desc, k, &need)) return s;
  REQUIRE_PTR(idx); REQUIRE_PTR(ws);
  if (ws_bytes < need)
    return fail(JSSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__, ws_bytes, need);
  return hip_status(topk_ws_final(desc, k, topk_ws(desc, k, const_cast<void*>(ws), true), idx, S(stream)),
                    __func__);
}

jssa_status jssa_score_topk_final_attend(const jssa_gqa_desc* desc, int32_t k, const void* ws, size_t ws_bytes,
                                         const void* q, const void* K, const void* V, float scale, int32_t* idx,
                                         float* out, float* lse, void* stream) {
  size_t need = 0;
  if (jssa_status s = jssa_score_topk_workspace_size(desc, k, &need)) return s;
  REQUIRE_PTR(ws); REQUIRE_PTR(q); REQUIRE_PTR(K); REQUIRE_PTR(V); REQUIRE_PTR(idx); REQUIRE_PTR(out);
  REQUIRE_PTR(lse);
  if (ws_bytes < need)
    return fail(JSSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__, ws_bytes, need);
  const TopkWs w = topk_ws(desc, k, const_cast<void*>(ws), true);
  const jssa::GqaDev g = to_dev(desc);
  const auto* q16 = static_cast<const uint16_t*>(q);
  const auto* K16 = static_cast<const uint16_t*>(K);
  const auto* V16 = static_cast<const uint16_t*>(V);
  if (!w.kc && jssa::select_attend_fused(w.segs, k, g.G))
    return hip_status(jssa::launch_select_attend(g, k, w.segs, q16, K16, V16, scale, idx, out, lse, S(stream)),
                      __func__);
  hipError_t e = topk_ws_final(desc, k, w, idx, S(stream));
  if (e == hipSuccess) e = jssa::launch_indexed(g, q16, K16, V16, idx, k, 1, scale, out, lse, S(stream));
  return hip_status(e, __func__);
}

jssa_status jssa_indexed_decode(const jssa_gqa_desc* desc, const void* q, const void* K, const void* V,
                                const int32_t* idx, int32_t k, int32_t S_, float scale, float* part_o,
                                float* part_lse, void* stream) {
  if (jssa_status s = check_desc(__func__, desc, false)) return s;
  REQUIRE_PTR(q); REQUIRE_PTR(K); REQUIRE_PTR(V); REQUIRE_PTR(idx); REQUIRE_PTR(part_o);
  REQUIRE_PTR(part_lse);
  if (k < 1 || k > 4096 || k > desc->max_seq)
    return fail(JSSA_ERR_SHAPE, "%s: k %d outside [1, min(4096, max_seq)]", __func__, k);
  if (S_ < 1 || S_ > 64) return fail(JSSA_ERR_SHAPE, "%s: S %d outside [1, 64]", __func__, S_);
  return hip_status(jssa::launch_indexed(to_dev(desc), static_cast<const uint16_t*>(q),
                                         static_cast<const uint16_t*>(K),
                                         static_cast<const uint16_t*>(V), idx, k, S_, scale, part_o,
                                         part_lse, S(stream)),
                    __func__);
}

jssa_status jssa_combine(int32_t B, int32_t H, int32_t S_, int32_t dv, const float* part_o,
                         const float* part_lse, void* out, int32_t out_bf16, float* lse,
                         void* stream) {
  if (B < 1 || H < 1 || int64_t(B) * H > (1 << 24))
    return fail(JSSA_ERR_SHAPE, "%s: B %d, H %d", __func__, B, H);
  if (S_ < 1 || S_ > 256) return fail(JSSA_ERR_SHAPE, "%s: S %d outside [1, 256]", __func__, S_);
  if (dv < 4 || dv > 1024 || dv % 4)
    return fail(JSSA_ERR_UNSUPPORTED, "%s: dv %d (a multiple of 4, <= 1024)", __func__, dv);
  REQUIRE_PTR(part_o); REQUIRE_PTR(part_lse); REQUIRE_PTR(out);
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(JSSA_ERR_ALIGN, "%s: lse is not 4-byte aligned", __func__);
  return hip_status(jssa::launch_combine(B, H, S_, dv, part_o, part_lse, out, out_bf16 != 0, lse,
                                         S(stream)),
                    __func__);
}

jssa_status jssa_dense_decode(const jssa_gqa_desc* desc, const void* q, const void* K, const void* V,
                              int32_t S_, float scale, float* part_o, float* part_lse, void* stream) {
  if (jssa_status s = check_desc(__func__, desc, false)) return s;
  REQUIRE_PTR(q); REQUIRE_PTR(K); REQUIRE_PTR(V); REQUIRE_PTR(part_o); REQUIRE_PTR(part_lse);
  if (S_ < 1 || S_ > 256) return fail(JSSA_ERR_SHAPE, "%s: S %d outside [1, 256]", __func__, S_);
  return hip_status(jssa::launch_dense(to_dev(desc), static_cast<const uint16_t*>(q),
                                       static_cast<const uint16_t*>(K),
                                       static_cast<const uint16_t*>(V), S_, scale, part_o, part_lse,
                                       S(stream)),
                    __func__);
}

jssa_status jssa_gather_kv(const jssa_gqa_desc* desc, const void* K, const void* V,
                           const int32_t* idx, int32_t k, void* Kg, void* Vg, int32_t* lens_out,
                           void* stream) {
  if (jssa_status s = check_desc(__func__, desc, false)) return s;
  REQUIRE_PTR(K); REQUIRE_PTR(V); REQUIRE_PTR(idx); REQUIRE_PTR(Kg); REQUIRE_PTR(Vg);
  REQUIRE_ALIGNED_OPT(lens_out);
  if (k < 1 || k > 4096 || k > desc->max_seq)
    return fail(JSSA_ERR_SHAPE, "%s: k %d outside [1, min(4096, max_seq)]", __func__, k);
  return hip_status(jssa::launch_gather(to_dev(desc), static_cast<const uint16_t*>(K),
                                        static_cast<const uint16_t*>(V), idx, k,
                                        static_cast<uint16_t*>(Kg), static_cast<uint16_t*>(Vg),
                                        lens_out, S(stream)),
                    __func__);
}

jssa_status jssa_mla_project_latent(const jssa_mla_desc* desc, const void* latent, const float* P,
                                    void* Kp_lat, void* stream) {
  if (jssa_status s = check_mla(__func__, desc)) return s;
  REQUIRE_PTR(latent); REQUIRE_PTR(P); REQUIRE_PTR(Kp_lat); REQUIRE_ALIGNED_OPT(desc->seq_lens);
  return hip_status(jssa::launch_mla_project(to_mla(desc), static_cast<const uint16_t*>(latent), P,
                                             static_cast<uint16_t*>(Kp_lat), S(stream)),
                    __func__);
}

jssa_status jssa_mla_fold_selection(const jssa_mla_desc* desc, const void* W_uk, const float* P, float* U,
                                    void* stream) {
  if (jssa_status s = check_mla(__func__, desc)) return s;
  REQUIRE_PTR(W_uk); REQUIRE_PTR(P); REQUIRE_PTR(U);
  return hip_status(jssa::launch_mla_fold(to_mla(desc), static_cast<const uint16_t*>(W_uk), P, U, S(stream)),
                    __func__);
}

jssa_status jssa_mla_absorb_q(const jssa_mla_desc* desc, const void* q_nope, const void* q_rope,
                              const void* W_uk, const float* P, const float* U, float* q_abs, float* q_sel,
                              void* stream) {
  if (jssa_status s = check_mla(__func__, desc)) return s;
  REQUIRE_PTR(q_nope); REQUIRE_PTR(q_rope); REQUIRE_PTR(W_uk); REQUIRE_PTR(P); REQUIRE_PTR(U);
  REQUIRE_PTR(q_abs); REQUIRE_PTR(q_sel);
  return hip_status(jssa::launch_mla_absorb(to_mla(desc), static_cast<const uint16_t*>(q_nope),
                                            static_cast<const uint16_t*>(q_rope),
                                            static_cast<const uint16_t*>(W_uk), P, U, q_abs, q_sel, S(stream)),
                    __func__);
}

jssa_status jssa_mla_score(const jssa_mla_desc* desc, const float* q_sel, const void* Kp_lat, float* scores,
                           void* stream) {
  if (jssa_status s = check_mla(__func__, desc)) return s;
  REQUIRE_PTR(q_sel); REQUIRE_PTR(Kp_lat); REQUIRE_PTR(scores);
  REQUIRE_ALIGNED_OPT(desc->seq_lens);
  return hip_status(jssa::launch_mla_score(to_mla(desc), q_sel, static_cast<const uint16_t*>(Kp_lat), scores,
                                           S(stream)),
                    __func__);
}

namespace {
// Per-chunk list length for the latent top-k: the score stream keeps each
// 1024-token chunk's own top kc, and the final pass selects from the union
// of those lists; the union holds the row's top k unless some chunk holds
// more than about kc of them (checked on the device; such a row is selected
// from its scores instead, so the result is exact either way). kc is 3x the
// average per-chunk share of k, at least 48; 0 (no lists: score, then the
// plain top-k) when that exceeds 256 or a row has more chunks than one final
// block takes.
int mla_list_k(int max_seq, int k) {
  const int nb = jssa::mla_score_chunks(max_seq);
  if (nb > 4096) return 0;
  int kc = 3 * ((k + nb - 1) / nb);
  kc = kc < 48 ? 48 : kc;
  kc = (kc + 3) & ~3;
  return kc <= 256 ? kc : 0;
}
constexpr int kMlaChunk = 1024;
}  // namespace

jssa_status jssa_mla_score_topk_workspace_size(const jssa_mla_desc* desc, int32_t k, size_t* bytes) {
  if (jssa_status s = check_mla(__func__, desc)) return s;
  size_t plain = 0;
  if (jssa_status s = jssa_topk_workspace_size(desc->B, 1, desc->max_seq, k, &plain)) return s;
  const int kc = mla_list_k(desc->max_seq, k);
  if (kc == 0) {
    *bytes = plain;
    return JSSA_OK;
  }
  size_t lists = 0;
  jssa::carve_segs(nullptr, desc->B, jssa::mla_score_chunks(desc->max_seq), jssa::seg_cap(kc, kMlaChunk), &lists);
  *bytes = lists;
  return JSSA_OK;
}

jssa_status jssa_mla_score_topk(const jssa_mla_desc* desc, const float* q_sel, const void* Kp_lat, int32_t k,
                                float* scores, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  if (jssa_status s = jssa_mla_score_topk_workspace_size(desc, k, &need)) return s;
  REQUIRE_PTR(q_sel); REQUIRE_PTR(Kp_lat); REQUIRE_PTR(scores); REQUIRE_PTR(idx);
  REQUIRE_ALIGNED_OPT(desc->seq_lens);
  if (need > 0) REQUIRE_PTR(ws);
  if (ws_bytes < need)
    return fail(JSSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__, ws_bytes, need);
  const jssa::MlaDev m = to_mla(desc);
  const auto* Kp = static_cast<const uint16_t*>(Kp_lat);
  const hipStream_t st = S(stream);
  const int kc = mla_list_k(desc->max_seq, k);
  hipError_t e;
  if (kc == 0) {
    e = jssa::launch_mla_score(m, q_sel, Kp, scores, st);
    if (e == hipSuccess) e = jssa::launch_topk(desc->B, 1, desc->max_seq, desc->seq_lens, scores, k, idx, ws, st);
  } else {
    const jssa::CandSegs lists = jssa::carve_segs(ws, desc->B, jssa::mla_score_chunks(desc->max_seq),
                                                  jssa::seg_cap(kc, kMlaChunk), nullptr);
    e = jssa::launch_mla_score_lists(m, q_sel, Kp, scores, lists, kc, st);
    if (e == hipSuccess)
      e = jssa::launch_topk_lists(desc->B, 1, desc->max_seq, desc->seq_lens, scores, k, idx, lists, kMlaChunk, st);
  }
  return hip_status(e, __func__);
}

jssa_status jssa_mla_indexed_decode(const jssa_mla_desc* desc, const float* q_abs,
                                    const void* latent, const int32_t* idx, int32_t k, int32_t S_,
                                    float scale, float* part_o, float* part_lse, void* stream) {
  if (jssa_status s = check_mla(__func__, desc)) return s;
  REQUIRE_PTR(q_abs); REQUIRE_PTR(latent); REQUIRE_PTR(idx); REQUIRE_PTR(part_o);
  REQUIRE_PTR(part_lse); REQUIRE_ALIGNED_OPT(desc->seq_lens);
  if (k < 1 || k > 4096 || k > desc->max_seq)
    return fail(JSSA_ERR_SHAPE, "%s: k %d outside [1, min(4096, max_seq)]", __func__, k);
  if (S_ < 1 || S_ > 64) return fail(JSSA_ERR_SHAPE, "%s: S %d outside [1, 64]", __func__, S_);
  return hip_status(jssa::launch_mla_indexed(to_mla(desc), q_abs,
                                             static_cast<const uint16_t*>(latent), idx, k, S_,
                                             scale, part_o, part_lse, S(stream)),
                    __func__);
}

jssa_status jssa_mla_up_v(const jssa_mla_desc* desc, const float* o_lat, const void* W_uv,
                          float* out, void* stream) {
  if (jssa_status s = check_mla(__func__, desc)) return s;
  REQUIRE_PTR(o_lat); REQUIRE_PTR(W_uv); REQUIRE_PTR(out);
  return hip_status(jssa::launch_mla_up_v(to_mla(desc), o_lat, static_cast<const uint16_t*>(W_uv),
                                          out, S(stream)),
                    __func__);
}

jssa_status jssa_mla_combine_up_v(const jssa_mla_desc* desc, int32_t n_split, const float* part_o, const float* part_lse,
                                  const void* W_uv, float* out, float* lse, void* stream) {
  if (jssa_status s = check_mla(__func__, desc)) return s;
  if (n_split < 1 || n_split > 64) return fail(JSSA_ERR_SHAPE, "%s: S %d outside [1, 64]", __func__, n_split);
  REQUIRE_PTR(part_o); REQUIRE_PTR(part_lse); REQUIRE_PTR(W_uv); REQUIRE_PTR(out);
  return hip_status(jssa::launch_mla_combine_up(to_mla(desc), n_split, part_o, part_lse,
                                                static_cast<const uint16_t*>(W_uv), out, lse, S(stream)),
                    __func__);
}

jssa_status jssa_score_topdelta_workspace_size(const jssa_gqa_desc* desc, int32_t k_max, size_t* bytes) {
  size_t base = 0;
  if (jssa_status s = jssa_score_topk_workspace_size(desc, k_max, &base)) return s;   // (validation)
  base = topk_ws(desc, k_max, nullptr, false).bytes;   // the candidate-list layout
  const size_t rows = size_t(desc->B) * desc->Hkv, nseg = size_t(jssa::score_topk_segments(desc->max_seq));
  *bytes = jssa::align256(base) + jssa::align256(rows * nseg * sizeof(uint32_t));
  return JSSA_OK;
}

}  // extern "C"

namespace {

// Shared checks and set-up of the two top-delta entry points: the candidate
// segments, the merge workspace, the pseudo-max slots and the filter.
struct TopDelta {
  jssa::CandSegs segs;
  void* merge_ws;
  uint32_t* pmax;
  jssa::DeltaArgs dl;
};

jssa_status topdelta_setup(const char* fn, const jssa_gqa_desc* desc, int32_t k_max, const jssa_topdelta_rule* rule,
                           float scale, int32_t* counts, void* ws, size_t ws_bytes, TopDelta* td) {
  size_t need = 0;
  if (jssa_status s = jssa_score_topdelta_workspace_size(desc, k_max, &need)) return s;
  if (!rule) return fail(JSSA_ERR_NULL, "%s: rule is NULL", fn);
  if (!(rule->delta >= 0.0f)) return fail(JSSA_ERR_SHAPE, "%s: delta %g (must be >= 0)", fn, double(rule->delta));
  if (rule->n_sink < 0 || rule->n_local < 0)
    return fail(JSSA_ERR_SHAPE, "%s: n_sink %d, n_local %d (must be >= 0)", fn, rule->n_sink, rule->n_local);
  if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(JSSA_ERR_SHAPE, "%s: scale %g", fn, double(scale));
  if (!ws) return fail(JSSA_ERR_NULL, "%s: ws is NULL", fn);
  if (!aligned(ws)) return fail(JSSA_ERR_ALIGN, "%s: ws is not 16-byte aligned", fn);
  if (counts && !aligned(counts)) return fail(JSSA_ERR_ALIGN, "%s: counts is not 16-byte aligned", fn);
  if (ws_bytes < need) return fail(JSSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  size_t base = 0;
  base = topk_ws(desc, k_max, nullptr, false).bytes;
  size_t main_bytes = 0;
  const int rows = desc->B * desc->Hkv, nseg = jssa::score_topk_segments(desc->max_seq);
  td->segs = jssa::carve_segs(ws, rows, nseg, jssa::score_topk_segment_cap(k_max), &main_bytes);
  td->merge_ws = static_cast<char*>(ws) + main_bytes;
  td->pmax = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + jssa::align256(base));
  td->dl = jssa::DeltaArgs{td->pmax, nseg, rule->delta * float(desc->Hq / desc->Hkv) / scale, counts};
  return JSSA_OK;
}

}  // namespace

extern "C" {

jssa_status jssa_score_topdelta(const jssa_gqa_desc* desc, const void* q, const float* P, const void* Kp,
                                int32_t k_max, const jssa_topdelta_rule* rule, float scale, int32_t* idx,
                                int32_t* counts, void* ws, size_t ws_bytes, void* stream) {
  TopDelta td;
  if (jssa_status s = topdelta_setup(__func__, desc, k_max, rule, scale, counts, ws, ws_bytes, &td)) return s;
  REQUIRE_PTR(q); REQUIRE_PTR(P); REQUIRE_PTR(Kp); REQUIRE_PTR(idx);
  const jssa::GqaDev g = to_dev(desc);
  hipError_t e = jssa::launch_score_chunks(g, static_cast<const uint16_t*>(q), P, static_cast<const uint16_t*>(Kp),
                                           k_max, nullptr, td.segs, S(stream), td.pmax, rule->n_sink, rule->n_local);
  if (e == hipSuccess)
    e = jssa::launch_select_final(g.B * g.Hkv, g.Hkv, g.max_seq, g.seq_lens, k_max, td.segs, idx, td.merge_ws,
                                  S(stream), td.dl);
  return hip_status(e, __func__);
}

jssa_status jssa_score_topdelta_attend(const jssa_gqa_desc* desc, const void* q, const float* P, const void* Kp,
                                       const void* K, const void* V, int32_t k_max, const jssa_topdelta_rule* rule,
                                       float scale, int32_t* idx, int32_t* counts, float* out, float* lse, void* ws,
                                       size_t ws_bytes, void* stream) {
  TopDelta td;
  if (jssa_status s = topdelta_setup(__func__, desc, k_max, rule, scale, counts, ws, ws_bytes, &td)) return s;
  REQUIRE_PTR(q); REQUIRE_PTR(P); REQUIRE_PTR(Kp); REQUIRE_PTR(K); REQUIRE_PTR(V); REQUIRE_PTR(idx);
  REQUIRE_PTR(out); REQUIRE_PTR(lse);
  const jssa::GqaDev g = to_dev(desc);
  const auto* q16 = static_cast<const uint16_t*>(q);
  const auto* K16 = static_cast<const uint16_t*>(K);
  const auto* V16 = static_cast<const uint16_t*>(V);
  hipError_t e = jssa::launch_score_chunks(g, q16, P, static_cast<const uint16_t*>(Kp), k_max, nullptr, td.segs,
                                           S(stream), td.pmax, rule->n_sink, rule->n_local);
  if (e != hipSuccess) return hip_status(e, __func__);
  if (jssa::select_attend_fused(td.segs, k_max, g.G))
    return hip_status(jssa::launch_select_attend(g, k_max, td.segs, q16, K16, V16, scale, idx, out, lse,
                                                 S(stream), td.dl),
                      __func__);
  e = jssa::launch_select_final(g.B * g.Hkv, g.Hkv, g.max_seq, g.seq_lens, k_max, td.segs, idx, td.merge_ws,
                                S(stream), td.dl);
  if (e == hipSuccess) e = jssa::launch_indexed(g, q16, K16, V16, idx, k_max, 1, scale, out, lse, S(stream));
  return hip_status(e, __func__);
}

jssa_status jssa_tile_bounds_size(const jssa_gqa_desc* desc, size_t* bytes) {
  if (jssa_status s = check_desc(__func__, desc, true)) return s;
  if (!bytes) return fail(JSSA_ERR_NULL, "%s: bytes is NULL", __func__);
  *bytes = size_t(desc->B) * desc->Hkv * ((jssa::screen_tiles(desc->max_seq) + 63) / 64 * 64) * 2 * desc->r *
           sizeof(uint16_t);
  return JSSA_OK;
}

jssa_status jssa_build_tile_bounds(const jssa_gqa_desc* desc, const void* Kp, void* bounds, void* stream) {
  if (jssa_status s = check_desc(__func__, desc, true)) return s;
  REQUIRE_PTR(Kp); REQUIRE_PTR(bounds); REQUIRE_ALIGNED_OPT(desc->seq_lens);
  return hip_status(jssa::launch_tile_bounds(to_dev(desc), static_cast<const uint16_t*>(Kp),
                                             static_cast<uint16_t*>(bounds), nullptr, 0, S(stream)),
                    __func__);
}

jssa_status jssa_update_tile_bounds(const jssa_gqa_desc* desc, const void* Kp, const int32_t* pos, int32_t n_new,
                                    void* bounds, void* stream) {
  if (jssa_status s = check_desc(__func__, desc, true)) return s;
  REQUIRE_PTR(Kp); REQUIRE_PTR(pos); REQUIRE_PTR(bounds); REQUIRE_ALIGNED_OPT(desc->seq_lens);
  if (n_new < 1 || n_new > desc->max_seq)
    return fail(JSSA_ERR_SHAPE, "%s: n_new %d outside [1, max_seq]", __func__, n_new);
  return hip_status(jssa::launch_tile_bounds(to_dev(desc), static_cast<const uint16_t*>(Kp),
                                             static_cast<uint16_t*>(bounds), pos, n_new, S(stream)),
                    __func__);
}

jssa_status jssa_score_topk_screened_workspace_size(const jssa_gqa_desc* desc, int32_t k, size_t* bytes) {
  size_t base = 0;
  if (jssa_status s = jssa_score_topk_workspace_size(desc, k, &base)) return s;   // (the jssa_score_topk layout)
  const size_t rows = size_t(desc->B) * desc->Hkv;
  *bytes = jssa::align256(base) + jssa::align256(rows * jssa::screen_words(desc->max_seq) * sizeof(uint32_t));
  return JSSA_OK;
}

jssa_status jssa_score_topk_screened_chunks(const jssa_gqa_desc* desc, const void* q, const float* P, const void* Kp,
                                           const void* bounds, const int32_t* seeds, int32_t n_seed, int32_t k,
                                           int32_t* kept_tiles, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  if (jssa_status s = jssa_score_topk_screened_workspace_size(desc, k, &need)) return s;
  REQUIRE_PTR(q); REQUIRE_PTR(P); REQUIRE_PTR(Kp); REQUIRE_PTR(bounds); REQUIRE_PTR(ws);
  REQUIRE_ALIGNED_OPT(kept_tiles); REQUIRE_ALIGNED_OPT(desc->seq_lens);
  if (n_seed < 0 || n_seed > jssa::screen_max_seeds())
    return fail(JSSA_ERR_SHAPE, "%s: n_seed %d outside [0, %d]", __func__, n_seed, jssa::screen_max_seeds());
  if (n_seed > 0) REQUIRE_PTR(seeds);
  if (ws_bytes < need)
    return fail(JSSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__, ws_bytes, need);
  size_t base = 0;
  jssa_score_topk_workspace_size(desc, k, &base);
  const TopkWs w = topk_ws(desc, k, ws, true);      // the jssa_score_topk layout: its final pass follows
  auto* keep = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + jssa::align256(base));
  const jssa::GqaDev g = to_dev(desc);
  const auto* q16 = static_cast<const uint16_t*>(q);
  const auto* Kp16 = static_cast<const uint16_t*>(Kp);
  hipError_t e = jssa::launch_screen(g, q16, P, Kp16, static_cast<const uint16_t*>(bounds), seeds, n_seed, k, keep,
                                     kept_tiles, S(stream));
  if (e == hipSuccess) {
    if (w.kc)
      e = jssa::launch_score_chunks_lists(g, q16, P, Kp16, w.kc, w.scores, nullptr, w.segs, S(stream), keep,
                                          jssa::screen_words(desc->max_seq));
    else
      e = jssa::launch_score_chunks(g, q16, P, Kp16, k, nullptr, w.segs, S(stream), nullptr, 0, 0, keep,
                                    jssa::screen_words(desc->max_seq));
  }
  return hip_status(e, __func__);
}

jssa_status jssa_calib_workspace_size(const jssa_gqa_desc* desc, size_t* bytes) {
  if (jssa_status s = check_desc(__func__, desc, false)) return s;
  if (!bytes) return fail(JSSA_ERR_NULL, "%s: bytes is NULL", __func__);
  *bytes = jssa::calib_workspace_bytes(desc->Hkv);
  return JSSA_OK;
}

jssa_status jssa_calib_key_moments(const jssa_gqa_desc* desc, const void* K, float* moments, void* ws,
                                   size_t ws_bytes, void* stream) {
  size_t need = 0;
  if (jssa_status s = jssa_calib_workspace_size(desc, &need)) return s;
  REQUIRE_PTR(K); REQUIRE_PTR(moments); REQUIRE_PTR(ws); REQUIRE_ALIGNED_OPT(desc->seq_lens);
  if (ws_bytes < need)
    return fail(JSSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__, ws_bytes, need);
  return hip_status(jssa::launch_calib_key_moments(to_dev(desc), static_cast<const uint16_t*>(K), moments, ws,
                                                   S(stream)),
                    __func__);
}

jssa_status jssa_calib_query_workspace_size(int32_t Hkv, size_t* bytes) {
  if (!bytes) return fail(JSSA_ERR_NULL, "%s: bytes is NULL", __func__);
  if (Hkv < 1 || Hkv > 4096) return fail(JSSA_ERR_SHAPE, "%s: Hkv %d", __func__, Hkv);
  *bytes = jssa::calib_query_workspace_bytes(Hkv);
  return JSSA_OK;
}

jssa_status jssa_calib_query_moments(int32_t N, int32_t Hq, int32_t Hkv, const void* q, float* moments, void* ws,
                                     size_t ws_bytes, void* stream) {
  if (N < 1 || N > (1 << 24)) return fail(JSSA_ERR_SHAPE, "%s: N %d outside [1, 2^24]", __func__, N);
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Hq / Hkv > 16 || int64_t(N) * Hq > (int64_t(1) << 31))
    return fail(JSSA_ERR_SHAPE, "%s: Hq %d, Hkv %d", __func__, Hq, Hkv);
  REQUIRE_PTR(q); REQUIRE_PTR(moments); REQUIRE_PTR(ws);
  const size_t need = jssa::calib_query_workspace_bytes(Hkv);
  if (ws_bytes < need)
    return fail(JSSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__, ws_bytes, need);
  return hip_status(jssa::launch_calib_query_moments(N, Hq, Hkv, static_cast<const uint16_t*>(q), moments, ws,
                                                     S(stream)),
                    __func__);
}

jssa_status jssa_calib_projection(int32_t d, int32_t r, const float* S_q, const float* S_k, float* P,
                                  double* eigvals) {
  if (d < 1 || d > 1024 || r < 1 || r > d)
    return fail(JSSA_ERR_SHAPE, "%s: d %d, r %d (need 1 <= r <= d <= 1024)", __func__, d, r);
  if (!S_q || !S_k || !P) return fail(JSSA_ERR_NULL, "%s: S_q, S_k and P must be non-NULL", __func__);
  double tq = 0.0, tk = 0.0;
  for (int i = 0; i < d; ++i) {
    tq += S_q[size_t(i) * d + i];
    tk += S_k[size_t(i) * d + i];
  }
  if (!(tq > 0.0) && !(tk > 0.0))
    return fail(JSSA_ERR_SHAPE, "%s: both moments have zero (or invalid) trace", __func__);
  std::vector<double> M(size_t(d) * d, 0.0), V(size_t(d) * r), w(r);
  for (size_t e = 0; e < M.size(); ++e)
    M[e] = (tq > 0.0 ? double(S_q[e]) / tq : 0.0) + (tk > 0.0 ? double(S_k[e]) / tk : 0.0);
  if (!jssa::symmetric_top_eigen(d, r, M.data(), V.data(), w.data()))
    return fail(JSSA_ERR_NUMERIC, "%s: eigen-solver did not converge", __func__);
  for (size_t e = 0; e < V.size(); ++e) P[e] = float(V[e]);
  if (eigvals)
    for (int c = 0; c < r; ++c) eigvals[c] = w[c];
  g_err[0] = 0;
  return JSSA_OK;
}

}  // extern "C"

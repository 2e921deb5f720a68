// Launchers shared between the kernel sources and the C-ABI layer. Every
// launcher assumes its arguments were validated by abi.cpp and returns the
// status of the launch (hipGetLastError after the launch).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.hpp"
#include "select.hpp"

namespace jssa {

hipError_t launch_project(const GqaDev& g, const uint16_t* src, int64_t src_row_stride_tok,
                          const int32_t* pos, int n_tok, bool append, uint16_t* K, uint16_t* V,
                          const uint16_t* v_src, const float* P, uint16_t* Kp, hipStream_t st);

hipError_t launch_score(const GqaDev& g, const uint16_t* q, const float* P, const uint16_t* Kp,
                        float* scores, hipStream_t st);

size_t topk_workspace_bytes(int rows, int max_seq, int k);
CandSegs carve_segs(void* base, int rows, int nseg, int cap, size_t* total);
int score_topk_segments(int max_seq);
int score_topk_segment_cap(int k);
hipError_t launch_score_topk(const GqaDev& g, const uint16_t* q, const float* P, const uint16_t* Kp, int k,
                             float* scores, int32_t* idx, CandSegs segs, void* merge_ws, hipStream_t st);
hipError_t launch_score_chunks(const GqaDev& g, const uint16_t* q, const float* P, const uint16_t* Kp, int k,
                               float* scores, CandSegs segs, hipStream_t st, uint32_t* pmax = nullptr,
                               int n_sink = 0, int n_local = 0, const uint32_t* keep = nullptr,
                               int keep_words = 0);

// The fused stream keeping per-chunk lists of kc (not necessarily the row's
// top k; segment floor 0), writing the scores to scores_ws (and to
// scores_user too when non-null) for the final pass's per-row fallback;
// keep: screening bits as in launch_score_chunks (dropped tiles are written
// as no token).
hipError_t launch_score_chunks_lists(const GqaDev& g, const uint16_t* q, const float* P, const uint16_t* Kp, int kc,
                                     float* scores_ws, float* scores_user, CandSegs lists, hipStream_t st,
                                     const uint32_t* keep = nullptr, int keep_words = 0);

// Lossless tile screening (screen.hip): 64-token tile bounds of the projected
// cache, and one keep bit per tile from a seed-set threshold.
int screen_tiles(int max_seq);
int screen_words(int max_seq);
int screen_max_seeds();
hipError_t launch_tile_bounds(const GqaDev& g, const uint16_t* Kp, uint16_t* bounds, const int32_t* pos,
                              int n_tok, hipStream_t st);
hipError_t launch_screen(const GqaDev& g, const uint16_t* q, const float* P, const uint16_t* Kp,
                         const uint16_t* bounds, const int32_t* seeds, int n_seed, int k, uint32_t* keep,
                         int32_t* kept_tiles, hipStream_t st);
hipError_t launch_topk(int B, int H, int max_seq, const int32_t* seq_lens, const float* scores,
                       int k, int32_t* idx, void* ws, hipStream_t st);

hipError_t launch_indexed(const GqaDev& g, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                          const int32_t* idx, int k, int S, float scale, float* part_o,
                          float* part_lse, hipStream_t st);
hipError_t launch_dense(const GqaDev& g, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                        int S, float scale, float* part_o, float* part_lse, hipStream_t st);
hipError_t launch_combine(int B, int H, int S, int dv, const float* part_o, const float* part_lse,
                          void* out, bool out_bf16, float* lse, hipStream_t st);
hipError_t launch_gather(const GqaDev& g, const uint16_t* K, const uint16_t* V, const int32_t* idx,
                         int k, uint16_t* Kg, uint16_t* Vg, int32_t* lens_out, hipStream_t st);

size_t align256(size_t x);

// Subspace calibration (calib.hip, calib_host.cpp).
int calib_blocks_per_head(int Hkv);
size_t calib_workspace_bytes(int Hkv);
hipError_t launch_calib_key_moments(const GqaDev& g, const uint16_t* K, float* out, void* ws, hipStream_t st);
size_t calib_query_workspace_bytes(int Hkv);
hipError_t launch_calib_query_moments(int N, int Hq, int Hkv, const uint16_t* q, float* out, void* ws,
                                      hipStream_t st);
// Top-r eigenvectors of the symmetric d x d matrix M (row-major, fp64), by
// cyclic Jacobi rotations; columns by descending eigenvalue, each signed so
// its entry of largest magnitude (first on a tie) is positive. V: [d, r]
// row-major; w: the r eigenvalues. Returns false if it did not converge.
bool symmetric_top_eigen(int d, int r, const double* M, double* V, double* w);

struct MlaDev {
  int B, H, d_latent, d_rope, d_nope, d_v, r, max_seq;
  const int32_t* seq_lens;
};
hipError_t launch_mla_project(const MlaDev& m, const uint16_t* latent, const float* P,
                              uint16_t* Kp, hipStream_t st);
// The MLA selection query P^T sum_h q_abs[b,h] is passed as kMlaSelParts
// partial sums [B, kMlaSelParts, r]: part g over the heads h = g, g + 64,
// ... The score stream adds the parts in order.
constexpr int kMlaSelParts = 64;
// U[h] = W_uk[h] . P[0 .. 512) (set-up; fp32 [H, 128, r], fp64 sums).
hipError_t launch_mla_fold(const MlaDev& m, const uint16_t* W_uk, const float* P, float* U, hipStream_t st);
// The absorbed query and the selection query parts, in one launch.
hipError_t launch_mla_absorb(const MlaDev& m, const uint16_t* q_nope, const uint16_t* q_rope,
                             const uint16_t* W_uk, const float* P, const float* U, float* q_abs, float* q_sel,
                             hipStream_t st);
hipError_t launch_mla_score(const MlaDev& m, const float* q_sel, const uint16_t* Kp, float* scores,
                            hipStream_t st);
int mla_score_chunks(int max_seq);
// The MLA score stream writing, per 1024-token chunk, the chunk's own top
// list_k (chunk_select; segment floor 0) to segment (b, chunk) of `lists`.
hipError_t launch_mla_score_lists(const MlaDev& m, const float* q_sel, const uint16_t* Kp, float* scores,
                                  CandSegs lists, int list_k, hipStream_t st);
// Exact top-k of B score rows from their chunk lists (final select with the
// list check; rows whose lists fall short are selected from their scores).
hipError_t launch_topk_lists(int rows, int H, int max_seq, const int32_t* seq_lens, const float* scores, int k,
                             int32_t* idx, CandSegs lists, int chunk_len, hipStream_t st);
// chunk length of the fused GQA stream (its segments)
int score_topk_chunk_len();
hipError_t launch_mla_indexed(const MlaDev& m, const float* q_abs, const uint16_t* latent,
                              const int32_t* idx, int k, int S, float scale, float* part_o,
                              float* part_lse, hipStream_t st);
hipError_t launch_mla_up_v(const MlaDev& m, const float* o_lat, const uint16_t* W_uv, float* out,
                           hipStream_t st);
hipError_t launch_mla_combine_up(const MlaDev& m, int S, const float* part_o, const float* part_lse,
                                 const uint16_t* W_uv, float* out, float* lse, hipStream_t st);

}  // namespace jssa

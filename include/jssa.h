/*
 * jssa.h -- C ABI of the MI355X (gfx950) JSSA sparse decode library.
 *
 * Joint Subspace Sparse Attention decodes one token per sequence by
 *   (1) scoring every cached token in a low-dimensional subspace shared by
 *       queries and keys,
 *   (2) keeping a distinct top-k token set for each KV head, and
 *   (3) running attention over those tokens read in place from the
 *       standard GQA cache through their indices, with no staging copy.
 * Sources: the JSSA abstract ("Joint Subspace Sparse Attention for Efficient
 * Long-Context Decoding", weekinpapers page of arXiv 2610.19026v1, section
 * Abstract) and the ai4snews digest of the same paper (sections Synopsis,
 * Interpretation, Perspective).
 *
 * Conventions for every entry point
 *  - Pointers named "device" point to GPU memory owned by the caller; the
 *    library never allocates, frees or retains them. Descriptors are read on
 *    the host during the call only.
 *  - bf16 tensors are arrays of uint16 bit patterns; P and scores are fp32;
 *    indices int32. All device pointers must be 16-byte aligned.
 *  - Every call validates its arguments on the host before any HIP call. On
 *    failure it returns a nonzero status, launches nothing and leaves the
 *    outputs untouched; jssa_last_error() then describes the problem
 *    (thread-local). Launch failures return JSSA_ERR_HIP.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *    null stream). Faults inside kernels surface at the caller's next
 *    synchronisation.
 *  - Device-side values (seq_lens, page tables, indices) are not read on the
 *    host. Kernels clamp seq_lens to [0, max_seq] and treat a page-table
 *    entry outside [0, num_pages) or an index outside [0, T_b) as an absent
 *    token: it is never read, scores -inf, is never selected and never
 *    attended. In a score row, -inf marks such a position.
 *  - Inputs must be finite; results for NaN or Inf inputs are unspecified.
 *  - No entry point keeps state between calls; calls on different streams
 *    may run concurrently as long as they do not write the same memory.
 */
#ifndef JSSA_H
#define JSSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define JSSA_API __attribute__((visibility("default")))

typedef int32_t jssa_status;
enum {
  JSSA_OK = 0,
  JSSA_ERR_NULL = 1,        /* a required pointer is NULL */
  JSSA_ERR_SHAPE = 2,       /* inconsistent or out-of-range sizes */
  JSSA_ERR_UNSUPPORTED = 3, /* a size outside the supported set below */
  JSSA_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned */
  JSSA_ERR_WORKSPACE = 5,   /* workspace smaller than jssa_topk_workspace_size */
  JSSA_ERR_HIP = 6,         /* the HIP runtime reported an error */
  JSSA_ERR_NUMERIC = 7      /* a host numerical routine did not converge */
};

/*
 * One layer's GQA cache (JSSA abstract: the indexed-attention kernel works
 * under the standard grouped-query-attention KV-cache layout).
 *
 *  B          sequences in the batch (>= 1)
 *  Hq, Hkv    query and KV heads; Hq % Hkv == 0; G = Hq / Hkv <= 16.
 *             Query head h reads KV head h / G.
 *  d          head width; must be 128
 *  r          rank of the scoring subspace; one of 16, 32, 48, 64, 128
 *  max_seq    cache capacity per sequence (tokens), 1 .. 2^24
 *  page_size  0: contiguous caches K,V [B,Hkv,max_seq,d], Kp [B,Hkv,max_seq,r]
 *             16: paged pools K,V [num_pages,Hkv,16,d], Kp [num_pages,Hkv,16,r];
 *                 token t of sequence b lives in page
 *                 page_table[b*max_pages_per_seq + t/16], slot t%16
 *  num_pages, max_pages_per_seq, page_table (device int32) -- paged only;
 *             max_pages_per_seq >= ceil(max_seq/16)
 *  seq_lens   device int32 [B]: tokens held by each sequence (T_b), or NULL
 *             meaning T_b = max_seq for every b
 */
typedef struct jssa_gqa_desc {
  int32_t B, Hq, Hkv, d, r, max_seq;
  int32_t page_size, num_pages, max_pages_per_seq;
  const int32_t* page_table;
  const int32_t* seq_lens;
} jssa_gqa_desc;

/*
 * Append n_new tokens per sequence to the cache (decode-step write).
 * Source: digest Synopsis (scoring in the shared subspace) -- the projected
 * key row is written next to the key so that scoring reads r values/token.
 *
 *  k_new, v_new  device bf16 [B,Hkv,n_new,d]
 *  P             device fp32 [Hkv,d,r]: per-KV-head basis (calibrated
 *                offline, outside the decode path)
 *  pos           device int32 [B]: first slot written for sequence b
 *  K, V, Kp      device caches (layout per desc) -- written at slots
 *                pos[b] .. pos[b]+n_new-1 that lie in [0, max_seq) and,
 *                when paged, map to a valid page; other slots are skipped.
 *  Kp[b,j,t,c] = bf16_rne(sum_i k[i] * P[j,i,c]), the sum accumulated in
 *  fp64 so that the stored value is the correctly rounded exact product.
 *  1 <= n_new <= max_seq.
 */
JSSA_API jssa_status jssa_append_kv(const jssa_gqa_desc* desc, void* K, void* V, void* Kp,
                           const void* k_new, const void* v_new, const float* P,
                           const int32_t* pos, int32_t n_new, void* stream);

/*
 * Build the projected key cache for tokens [0, T_b) of an existing cache
 * (set-up, or after a basis change). Source: digest Synopsis (tokens are
 * scored in the shared low-dimensional subspace), as for jssa_append_kv, of
 * which this is the bulk form with the same arithmetic.
 *  K   device bf16 cache (read); P device fp32 [Hkv,d,r]; Kp device bf16 (written)
 */
JSSA_API jssa_status jssa_project_keys(const jssa_gqa_desc* desc, const void* K, const float* P,
                              void* Kp, void* stream);

/*
 * Subspace scores (digest Synopsis and Interpretation: candidates are ranked
 * in a low-dimensional space that holds queries and keys together).
 *  q       device bf16 [B,Hq,d]
 *  P       device fp32 [Hkv,d,r]
 *  Kp      device bf16 projected key cache (layout per desc)
 *  scores  device fp32 [B,Hkv,max_seq] (written):
 *          scores[b,j,t] = qp . Kp[b,j,t,:] for t < T_b, -inf for t >= T_b,
 *          where qp = P_j^T (sum of q[b,h] over the G query heads of KV
 *          head j), accumulated in fp32.
 */
JSSA_API jssa_status jssa_score(const jssa_gqa_desc* desc, const void* q, const float* P, const void* Kp,
                       float* scores, void* stream);

/*
 * Workspace bytes needed by jssa_topk for `rows` = B*H score rows of length
 * max_seq and budget k (host-only; no HIP call). The selection it serves is
 * the per-KV-head top-k of the JSSA abstract (Abstract); the workspace holds
 * the per-chunk candidate lists of this library's two-level selection.
 */
JSSA_API jssa_status jssa_topk_workspace_size(int32_t B, int32_t H, int32_t max_seq, int32_t k, size_t* bytes);

/*
 * Distinct top-k token set per (sequence, head) (JSSA abstract: distinct
 * per-KV-head selections; digest Synopsis).
 *  scores   device fp32 [B,H,max_seq]
 *  seq_lens device int32 [B] or NULL (= max_seq)
 *  idx      device int32 [B,H,k] (written): the first min(k,n) tokens of
 *           the order (score descending, index ascending; -0.0 == +0.0),
 *           listed ascending by token index, then -1 padding; n counts the
 *           positions t < T_b whose score is not -inf (a -inf score marks a
 *           position without a token, which is never selected).
 *  ws       device workspace of at least jssa_topk_workspace_size bytes
 *  1 <= k <= 4096, k <= max_seq. Deterministic: identical inputs give
 *  identical outputs whatever the scheduling.
 */
JSSA_API jssa_status jssa_topk(int32_t B, int32_t H, int32_t max_seq, const int32_t* seq_lens,
                      const float* scores, int32_t k, int32_t* idx, void* ws, size_t ws_bytes,
                      void* stream);

/*
 * Fused score -> top-k: the subspace score stream of jssa_score and the
 * selection of jssa_topk in one pass over the projected key cache. Each
 * 8192-token chunk keeps its scores on chip (LDS) and emits only the tokens
 * that can still be among its row's k best, so the fp32 score row is never
 * written and read back (unless `scores` is given). Two launches: the chunk
 * pass (jssa_score_topk_chunks) and the per-row final pass
 * (jssa_score_topk_final); jssa_score_topk issues both.
 * For budgets whose per-chunk candidates would need more than one final
 * pass (chunks x k > 8192), each chunk instead keeps only its own best
 * (3x its share of k) and writes its scores below T_b to the
 * workspace; the final pass checks, once the row's k-th key is known, that
 * every chunk that dropped tokens dropped only keys below it, and selects a
 * row that fails that check again from its scores. The indices are the same
 * either way.
 *  q, P, Kp  as jssa_score; k as jssa_topk (1 <= k <= min(4096, max_seq))
 *  scores    device fp32 [B,Hkv,max_seq] or NULL: if given, written exactly
 *            as by jssa_score
 *  idx       device int32 [B,Hkv,k]: exactly what jssa_topk returns for the
 *            scores jssa_score computes
 *  ws        device workspace of at least jssa_score_topk_workspace_size bytes
 *            (candidate lists, plus the score rows [B*Hkv, max_seq] fp32 in
 *            the list mode above); its contents are scratch
 */
JSSA_API jssa_status jssa_score_topk_workspace_size(const jssa_gqa_desc* desc, int32_t k, size_t* bytes);
JSSA_API jssa_status jssa_score_topk(const jssa_gqa_desc* desc, const void* q, const float* P, const void* Kp,
                                     int32_t k, float* scores, int32_t* idx, void* ws, size_t ws_bytes,
                                     void* stream);

/*
 * jssa_score_topk for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and results, with the candidate lists in a static
 * scratch array of the library instead of a caller workspace.
 *  Arguments as jssa_score_topk without ws / ws_bytes.
 *  Always the candidate-list layout (no list mode, no score rows in the
 *  scratch). Limit: shapes whose candidate lists exceed 16 MiB (16 << 20
 *  bytes) are rejected with JSSA_ERR_WORKSPACE, launching nothing; 128K
 *  tokens x B = 16 x Hkv = 8 at k = 256 needs about 8 MiB.
 *  The call allocates nothing; the scratch array (16 MiB per GPU) exists from
 *  library load to process exit, and its device address is looked up once
 *  per GPU, on the first call made with that GPU current.
 *  Every call on one GPU uses that GPU's one array: calls that overlap in
 *  time on one GPU (different streams, or threads) race and give undefined
 *  results. The array needs no clearing: each call writes every part of it
 *  that it reads.
 */
JSSA_API jssa_status jssa_score_topk_noalloc(const jssa_gqa_desc* desc, const void* q, const float* P, const void* Kp,
                                             int32_t k, float* scores, int32_t* idx, void* stream);

/*
 * The two halves of jssa_score_topk, for callers that schedule or time them
 * separately. jssa_score_topk_chunks streams Kp once and leaves, per 8192-
 * token chunk of each (sequence, KV head) row, that chunk's candidates in
 * `ws`; jssa_score_topk_final reads them back and writes idx. Between the two
 * calls `ws` must not be modified, and both calls must get the same desc
 * (shapes and seq_lens contents) and k; the pair then writes exactly what
 * jssa_score_topk writes. Arguments, errors and workspace size as
 * jssa_score_topk.
 */
JSSA_API jssa_status jssa_score_topk_chunks(const jssa_gqa_desc* desc, const void* q, const float* P,
                                            const void* Kp, int32_t k, float* scores, void* ws,
                                            size_t ws_bytes, void* stream);
JSSA_API jssa_status jssa_score_topk_final(const jssa_gqa_desc* desc, int32_t k, const void* ws, size_t ws_bytes,
                                           int32_t* idx, void* stream);

/*
 * The final half of jssa_score_topk fused with jssa_indexed_decode at one
 * split: each (sequence, KV head) row's block selects its k tokens from the
 * candidates jssa_score_topk_chunks left in `ws` and at once runs the
 * gather-free attention of the row's query heads over them (digest
 * Interpretation: selected rows read in place through the indices).
 *  desc, k, ws, ws_bytes  as jssa_score_topk_final (same desc and k as the
 *                         jssa_score_topk_chunks call that filled ws)
 *  q, K, V, scale         as jssa_indexed_decode
 *  idx  device int32 [B,Hkv,k] (written, as jssa_topk)
 *  out  device fp32 [B,Hq,d] (written): softmax-weighted values
 *  lse  device fp32 [B,Hq] (written): log-sum-exp (-inf for an empty set)
 * out/lse equal jssa_indexed_decode's partials for S = 1 on the same idx.
 * Fused in one kernel when k <= 512, the row's candidates need no merge
 * level and G <= 16; otherwise the same results come from the separate
 * launches (final select, then indexed attention).
 */
JSSA_API jssa_status jssa_score_topk_final_attend(const jssa_gqa_desc* desc, int32_t k, const void* ws,
                                                  size_t ws_bytes, const void* q, const void* K, const void* V,
                                                  float scale, int32_t* idx, float* out, float* lse, void* stream);

/*
 * Gather-free indexed attention, split-K partials (digest Interpretation:
 * selected tokens are read where they lie through scattered indices rather
 * than copied into a contiguous buffer; JSSA abstract).
 *  q        device bf16 [B,Hq,d]
 *  K, V     device bf16 caches (layout per desc), read in place
 *  idx      device int32 [B,Hkv,k] (as written by jssa_topk; -1 = none)
 *  S        splits, 1 <= S <= 64: split s covers idx slots
 *           [s*ceil(k/S), (s+1)*ceil(k/S))
 *  scale    logit scale (1/sqrt(d) for standard attention)
 *  part_o   device fp32 [B,Hq,S,d]  (written) softmax-weighted V of split s
 *  part_lse device fp32 [B,Hq,S]    (written) log-sum-exp of split s's
 *           logits; -inf (and part_o = 0) for a split with no valid token
 */
JSSA_API jssa_status jssa_indexed_decode(const jssa_gqa_desc* desc, const void* q, const void* K,
                                const void* V, const int32_t* idx, int32_t k, int32_t S,
                                float scale, float* part_o, float* part_lse, void* stream);

/*
 * Log-sum-exp merge of split partials. Source: the split-K indexed decode
 * of the JSSA abstract (Abstract: attention runs on the selected tokens)
 * evaluated in S parts; the merge weights part s by exp(lse_s), which makes
 * the result equal to attention over the union of the parts.
 *  part_o [B,H,S,dv] fp32, part_lse [B,H,S] fp32 (device)
 *  out    device [B,H,dv] fp32 (out_bf16 = 0) or bf16 bits (out_bf16 = 1)
 *  lse    device fp32 [B,H] or NULL
 *  1 <= S <= 64; dv a multiple of 4, <= 1024. Rows whose splits are all
 *  empty give out = 0, lse = -inf.
 */
JSSA_API jssa_status jssa_combine(int32_t B, int32_t H, int32_t S, int32_t dv, const float* part_o,
                         const float* part_lse, void* out, int32_t out_bf16, float* lse,
                         void* stream);

/*
 * Dense full-KV decode (the baseline the method is compared with; JSSA
 * abstract reports decode throughput relative to full-KV attention).
 * Attention of every query head over all tokens t < T_b; split s covers
 * tokens [s*ceil(T_b/S), (s+1)*ceil(T_b/S)). Outputs as jssa_indexed_decode.
 *  1 <= S <= 256.
 */
JSSA_API jssa_status jssa_dense_decode(const jssa_gqa_desc* desc, const void* q, const void* K,
                              const void* V, int32_t S, float scale, float* part_o,
                              float* part_lse, void* stream);

/*
 * Gather ablation (digest Interpretation: the common implementation copies
 * the selected entries into a contiguous buffer before a dense kernel).
 *  Kg, Vg    device bf16 [B,Hkv,k,d] (written): row i = cache row idx[b,j,i];
 *            rows for -1 entries are zero
 *  lens_out  device int32 [B] (written): min(k, T_b), the valid rows per
 *            sequence, for use as seq_lens of a contiguous desc with
 *            max_seq = k
 */
JSSA_API jssa_status jssa_gather_kv(const jssa_gqa_desc* desc, const void* K, const void* V,
                           const int32_t* idx, int32_t k, void* Kg, void* Vg, int32_t* lens_out,
                           void* stream);

/*
 * MLA shared latent cache (digest Perspective: on MLA models the selection
 * runs on the one latent cache all heads read).
 *  B, H (query heads), d_latent (512), d_rope (64), d_nope (128), d_v (128),
 *  r (scoring rank, 64), max_seq, seq_lens (device int32 [B] or NULL).
 *  The latent cache is [B,max_seq,d_latent+d_rope] bf16, its projected copy
 *  Kp_lat [B,max_seq,r] bf16.
 */
typedef struct jssa_mla_desc {
  int32_t B, H, d_latent, d_rope, d_nope, d_v, r, max_seq;
  const int32_t* seq_lens;
} jssa_mla_desc;

/* Kp_lat = bf16_rne(latent . P) for tokens [0, T_b); P device fp32 [d_c, r]. */
JSSA_API jssa_status jssa_mla_project_latent(const jssa_mla_desc* desc, const void* latent, const float* P,
                                    void* Kp_lat, void* stream);

/*
 * Folded selection weights, computed once per layer (set-up, like the latent
 * projection): U[h] = W_uk[h] . P[0 .. d_latent) (fp32 [H,d_nope,r]; fp64
 * sums rounded once to fp32). The selection query is linear in the absorbed
 * query (digest Perspective: selection over the shared latent cache), so
 * P_lat^T sum_h W_uk[h]^T q_nope[b,h] = sum_h U[h]^T q_nope[b,h]: with U the
 * per-step selection query needs q_nope, not the absorbed query.
 *  W_uk device bf16 [H,d_nope,d_latent], P device fp32 [d_c,r], U device
 *  fp32 [H,d_nope,r] (written).
 */
JSSA_API jssa_status jssa_mla_fold_selection(const jssa_mla_desc* desc, const void* W_uk, const float* P,
                                             float* U, void* stream);

/*
 * Absorbed query and selection query, in one launch (digest Perspective:
 * selection over the shared latent cache).
 *  q_abs[b,h] = [W_uk[h]^T q_nope[b,h] ; q_rope[b,h]] (fp32): the attention
 *               query of head h against latent rows;
 *  q_sel[b,g] = sum over the heads h = g, g + 64, ... (< H) of
 *               U[h]^T q_nope[b,h] + P[d_latent .. d_c)^T q_rope[b,h],
 *               g < 64 (fp32, fixed summation order): the one subspace
 *               query of sequence b, P^T sum_h q_abs[b,h], in 64 parts by
 *               class of heads; the MLA score passes add the parts
 *               themselves, in order. Parts of classes with no head are 0.
 *  q_nope device bf16 [B,H,d_nope], q_rope device bf16 [B,H,d_rope],
 *  W_uk device bf16 [H,d_nope,d_latent], P device fp32 [d_c,r], U from
 *  jssa_mla_fold_selection (same W_uk and P), q_abs device fp32 [B,H,d_c]
 *  (written), q_sel device fp32 [B,64,r] (written).
 */
JSSA_API jssa_status jssa_mla_absorb_q(const jssa_mla_desc* desc, const void* q_nope, const void* q_rope,
                              const void* W_uk, const float* P, const float* U, float* q_abs, float* q_sel,
                              void* stream);

/*
 * MLA selection scores: scores[b,t] = (sum_j q_sel[b,j]) . Kp_lat[b,t] for
 * t < T_b, -inf beyond; the 64 parts are added in order (the same query in
 * every pass and every block). q_sel device fp32 [B,64,r] (from
 * jssa_mla_absorb_q, or any split of the query into 64 rows), scores device
 * fp32 [B,max_seq].
 */
JSSA_API jssa_status jssa_mla_score(const jssa_mla_desc* desc, const float* q_sel, const void* Kp_lat,
                           float* scores, void* stream);

/*
 * jssa_mla_score followed by the latent top-k (jssa_topk with H = 1): the same
 * scores and the same idx [B,k], in fewer and cheaper passes (per sequence
 * one selection over the shared latent cache, digest Perspective; ties and
 * absent tokens as jssa_topk). The score stream also keeps each 1024-token
 * chunk's own best tokens (3x its share of k, at least 48), and one
 * final pass per sequence selects from the union of those lists. The union
 * holds the sequence's top k unless a chunk held more of them than its list
 * (checked on the device once the k-th key is known); such a sequence is
 * selected again from its scores. The selection is exact either way.
 *  k in [1, min(4096, max_seq)]; scores device fp32 [B,max_seq] (written),
 *  idx device int32 [B,k] (written); ws device, at least
 *  jssa_mla_score_topk_workspace_size bytes, its contents scratch.
 */
JSSA_API jssa_status jssa_mla_score_topk_workspace_size(const jssa_mla_desc* desc, int32_t k, size_t* bytes);
JSSA_API jssa_status jssa_mla_score_topk(const jssa_mla_desc* desc, const float* q_sel, const void* Kp_lat,
                                int32_t k, float* scores, int32_t* idx, void* ws, size_t ws_bytes,
                                void* stream);

/*
 * MLA attention over the selected latent rows, read in place (bf16 MFMA):
 * logits = scale * q_abs[b,h] . latent[b,t] (all d_c dims), values are
 * latent[b,t,:d_latent]. idx device int32 [B,k] (jssa_topk with H = 1).
 *  part_o   device fp32 [B,H,S,d_latent], part_lse device fp32 [B,H,S]
 *  H must be a multiple of 16; 1 <= S <= 64.
 */
JSSA_API jssa_status jssa_mla_indexed_decode(const jssa_mla_desc* desc, const float* q_abs,
                                    const void* latent, const int32_t* idx, int32_t k, int32_t S,
                                    float scale, float* part_o, float* part_lse, void* stream);

/*
 * Value up-projection: out[b,h] = W_uv[h] . o_lat[b,h].
 *  o_lat device fp32 [B,H,d_latent], W_uv device bf16 [H,d_v,d_latent],
 *  out device fp32 [B,H,d_v] (written)
 */
JSSA_API jssa_status jssa_mla_up_v(const jssa_mla_desc* desc, const float* o_lat, const void* W_uv,
                          float* out, void* stream);

/*
 * jssa_combine of the S partials of jssa_mla_indexed_decode followed by
 * jssa_mla_up_v, in one pass (the log-sum-exp merge of split partials, then
 * the value up-projection of the absorbed attention, digest Perspective):
 *  o_lat[b,h] = sum_s exp(lse_s - M) part_o[b,h,s] / sum_s exp(lse_s - M),
 *  out[b,h]   = W_uv[h] . o_lat[b,h];   lse[b,h] = M + log(sum_s exp(lse_s - M)).
 *  part_o device fp32 [B,H,S,d_latent], part_lse device fp32 [B,H,S],
 *  W_uv device bf16 [H,d_v,d_latent], out device fp32 [B,H,d_v] (written),
 *  lse device fp32 [B,H] (written; NULL: not written). 1 <= S <= 64.
 *  o_lat stays on chip. Same results as the two calls up to fp32 summation
 *  order.
 */
JSSA_API jssa_status jssa_mla_combine_up_v(const jssa_mla_desc* desc, int32_t S, const float* part_o,
                                  const float* part_lse, const void* W_uv, float* out, float* lse,
                                  void* stream);

/*
 * Top-delta selection (Faster Than Flash review on evolve.pub, Summary, Key
 * claims and FAQ: a token stays when its log-weight is at most delta below a
 * stand-in for the maximum taken over the first and most recent tokens;
 * since the stand-in cannot exceed the true maximum, a poor stand-in can
 * only keep more tokens). Applied here per token
 * and per KV head to the subspace score s_t: the approximate logit is the
 * group-mean scale * s_t / G; the pseudo-max m is the largest s_t over the
 * first n_sink and the last n_local positions of the sequence; token t is
 * kept iff s_t >= m - delta * G / scale, at most k_max of them, chosen by
 * (score desc, index asc). Tokens without a valid page are never kept; with
 * no special token (n_sink = n_local = 0) nothing is filtered. The result is
 * the same as the top-k_max selection with its members below the threshold
 * removed. Scores, m and the threshold are fp32.
 */
typedef struct {
  float delta;       /* >= 0, in natural-log units of the group-mean logit; +inf: plain top-k */
  int32_t n_sink;    /* >= 0: positions 0 .. n_sink-1 inform the pseudo-max */
  int32_t n_local;   /* >= 0: positions T_b-n_local .. T_b-1 inform the pseudo-max */
} jssa_topdelta_rule;

/* Workspace of the top-delta calls (the score + top-k workspace plus one
 * pseudo-max slot per 8192-token chunk). */
JSSA_API jssa_status jssa_score_topdelta_workspace_size(const jssa_gqa_desc* desc, int32_t k_max, size_t* bytes);

/*
 * Score stream + top-delta selection (two launches or more: the fused chunk
 * pass, then the final selection).
 *  q, P, Kp  as jssa_score_topk; scale > 0 converts delta to score units
 *  idx       device int32 [B,Hkv,k_max]: kept tokens ascending, -1 padded
 *  counts    device int32 [B,Hkv] or NULL: number kept per (b, j)
 * ws holds the candidate lists and pseudo-max slots; no initialisation.
 */
JSSA_API jssa_status jssa_score_topdelta(const jssa_gqa_desc* desc, const void* q, const float* P, const void* Kp,
                                         int32_t k_max, const jssa_topdelta_rule* rule, float scale, int32_t* idx,
                                         int32_t* counts, void* ws, size_t ws_bytes, void* stream);

/*
 * jssa_score_topdelta followed by the attention of every query head over
 * its KV head's kept tokens, read in place (one split: out is the
 * normalised output, lse the log-sum-exp; an empty set gives 0 and -inf).
 * The final selection and the attention share a kernel when the selection
 * needs no merge level, k_max <= 512 and G <= 16; otherwise
 * jssa_indexed_decode (S = 1) follows it.
 *  K, V  device bf16 (layout of desc); out device fp32 [B,Hq,128]; lse [B,Hq]
 */
JSSA_API jssa_status jssa_score_topdelta_attend(const jssa_gqa_desc* desc, const void* q, const float* P,
                                                const void* Kp, const void* K, const void* V, int32_t k_max,
                                                const jssa_topdelta_rule* rule, float scale, int32_t* idx,
                                                int32_t* counts, float* out, float* lse, void* ws, size_t ws_bytes,
                                                void* stream);

/*
 * Lossless tile screening ("DoSA Makes Sparse Attention Selection
 * Conditional Without Approximation", cctest.ai, How the method works: a
 * seed set bounds the winning threshold from below; candidates whose upper
 * bound is lower are dropped before exact scoring; the top-k is unchanged).
 * Tiles are 64 consecutive tokens of one (sequence, KV head). A tile's box
 * bound ub = sum_c max(qp_c lo_c, qp_c hi_c), lo/hi the per-dimension min/max
 * of its valid projected keys, is >= each of its scores. tau is the k-th
 * largest score over the distinct valid seed tokens (caller-given, e.g. the
 * previous decode step's selection), so tau <= the k-th score; a tile with
 * ub < tau is not read by the score stream. The comparison carries a margin
 * of 2^-16 * sum|qp_c Kp_c| on both sides so that fp32 rounding never drops
 * a tile that exact arithmetic keeps. The selection is exactly that of
 * jssa_score_topk; only the bytes read change. With fewer than k distinct
 * valid seeds nothing is dropped.
 */

/* Size of the tile bounds: device bf16 [B,Hkv,ntg,2r/8,64,8] with
 * ntg = ceil(ceil(max_seq/64)/64): tiles in groups of 64; per group, 8-dim
 * vector v of each of its 64 tiles in turn, v < r/8 holding the minima of
 * dims 8v..8v+7 and v >= r/8 the maxima of dims 8(v-r/8)..8(v-r/8)+7 (+inf /
 * -inf for a tile with no valid token). Tiles past ceil(max_seq/64) are
 * never written or read. */
JSSA_API jssa_status jssa_tile_bounds_size(const jssa_gqa_desc* desc, size_t* bytes);

/* Builds every tile's bounds from the projected cache Kp (layout of desc).
 * Exact (the min and max of bf16 values). After appends, build again (the
 * tiles holding new tokens change). */
JSSA_API jssa_status jssa_build_tile_bounds(const jssa_gqa_desc* desc, const void* Kp, void* bounds, void* stream);

/* Rebuilds only the tiles that hold appended tokens pos[b] .. pos[b]+n_new-1
 * (those in [0, max_seq)), with the arguments of jssa_append_kv: the bounds
 * of a tile depend on its valid tokens alone. After jssa_append_kv, with
 * desc->seq_lens grown by at most the appended run (pos[b] <= the previous
 * T_b, new T_b <= max(previous T_b, pos[b] + n_new)), the result equals
 * jssa_build_tile_bounds, at the cost of at most ceil(n_new/64) + 1 tiles
 * per (sequence, KV head). Tokens made valid in any other way need a full
 * build.
 *  pos    device int32 [B]
 *  1 <= n_new <= max_seq */
JSSA_API jssa_status jssa_update_tile_bounds(const jssa_gqa_desc* desc, const void* Kp, const int32_t* pos,
                                             int32_t n_new, void* bounds, void* stream);

/* Workspace of jssa_score_topk_screened_chunks: the jssa_score_topk workspace
 * (same layout, at the start) plus one keep bit per tile. */
JSSA_API jssa_status jssa_score_topk_screened_workspace_size(const jssa_gqa_desc* desc, int32_t k, size_t* bytes);

/*
 * Screening, then the fused score stream + chunk selection over the kept
 * tiles only. Finish with jssa_score_topk_final or
 * jssa_score_topk_final_attend on the same workspace; the indices are those
 * of jssa_score_topk.
 *  bounds      from jssa_build_tile_bounds
 *  seeds       device int32 [B,Hkv,n_seed] token indices (entries outside
 *              [0, T_b), repeats and tokens without a page are ignored);
 *              NULL allowed when n_seed = 0; 0 <= n_seed <= 4096
 *  kept_tiles  device int32 [B,Hkv] or NULL: tiles read per (b, j)
 */
JSSA_API jssa_status jssa_score_topk_screened_chunks(const jssa_gqa_desc* desc, const void* q, const float* P,
                                                     const void* Kp, const void* bounds, const int32_t* seeds,
                                                     int32_t n_seed, int32_t k, int32_t* kept_tiles, void* ws,
                                                     size_t ws_bytes, void* stream);

/*
 * Subspace calibration (JSSA abstract on weekinpapers, Abstract: the shared
 * query-key subspace minimises a token-score preservation error through a
 * marginal upper bound that has a closed-form spectral solution; the
 * formulas are not on the pages). Reading used here: the error of a (query,
 * key) pair is e = qbar^T (I - P P^T) k for the group-summed query qbar;
 * Cauchy-Schwarz and AM-GM bound its mean by
 * tr((I - P P^T)(lam S_q + S_k / lam)) / 2, with S_q = E[qbar qbar^T],
 * S_k = E[k k^T], lam = sqrt(tr S_k / tr S_q). The bound is smallest for P =
 * the top-r eigenvectors of M = S_q / tr S_q + S_k / tr S_k. These calls
 * compute S_k and S_q per KV head on the GPU and P on the host; P [Hkv,d,r]
 * from jssa_calib_projection (one head per call) is the projection that
 * jssa_project_keys / jssa_score take. Offline: not part of a decode step.
 */

/* Workspace of jssa_calib_key_moments, in bytes (depends on desc->Hkv only). */
JSSA_API jssa_status jssa_calib_workspace_size(const jssa_gqa_desc* desc, size_t* bytes);

/*
 * Key second moments over the cache:
 *   moments[j] = (1/N_j) sum_{b, t < T_b, page valid} K[b,j,t] K[b,j,t]^T
 * with N_j the number of those tokens (a zero matrix when N_j = 0).
 *  K        device bf16, layout of desc (contiguous or paged, d = 128)
 *  moments  device fp32 [Hkv,128,128], written (symmetric)
 *  ws       device workspace of jssa_calib_workspace_size bytes (partials;
 *           its contents need no initialisation and are overwritten)
 * bf16 products are exact; sums are fp32 (MFMA accumulation, then a fixed-
 * order sum of per-wave partials), so repeated calls give identical bits.
 * desc->r is not used.
 */
JSSA_API jssa_status jssa_calib_key_moments(const jssa_gqa_desc* desc, const void* K, float* moments, void* ws,
                                            size_t ws_bytes, void* stream);

/* Workspace of jssa_calib_query_moments (per-slice partial sums). */
JSSA_API jssa_status jssa_calib_query_workspace_size(int32_t Hkv, size_t* bytes);

/*
 * Query second moments over N decode-query samples:
 *   moments[j] = (1/N) sum_n qbar_n qbar_n^T, qbar_n = sum_{h in group j} q[n,h]
 *  q        device bf16 [N,Hq,128]; Hq a multiple of Hkv, Hq/Hkv <= 16
 *  moments  device fp32 [Hkv,128,128], written
 *  ws       device workspace of jssa_calib_query_workspace_size bytes
 * qbar is summed in fp32; the outer products accumulate in fp32 over 32
 * slices of the samples, summed in a fixed order (repeatable bits).
 */
JSSA_API jssa_status jssa_calib_query_moments(int32_t N, int32_t Hq, int32_t Hkv, const void* q, float* moments,
                                              void* ws, size_t ws_bytes, void* stream);

/*
 * Spectral step, HOST pointers (no GPU work): P = the top-r eigenvectors of
 * M = S_q / tr S_q + S_k / tr S_k (a term with zero trace is left out),
 * computed in fp64 by cyclic Jacobi rotations.
 *  S_q, S_k  host fp32 [d,d] (symmetric)
 *  P         host fp32 [d,r] row-major, written: orthonormal columns by
 *            descending eigenvalue, each signed so that its entry of largest
 *            magnitude (the first on a tie) is positive
 *  eigvals   host fp64 [r] or NULL: the r eigenvalues of M
 * JSSA_ERR_SHAPE if both traces are zero, JSSA_ERR_NUMERIC if the rotations
 * do not converge.
 */
JSSA_API jssa_status jssa_calib_projection(int32_t d, int32_t r, const float* S_q, const float* S_k, float* P,
                                           double* eigvals);

/* Diagnostics (host only). */
JSSA_API const char* jssa_status_string(jssa_status s);
JSSA_API const char* jssa_last_error(void);
JSSA_API int32_t jssa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* JSSA_H */

/*
 * gqla.h -- C ABI of libgqla: GQLA (Group-Query Latent Attention) decode
 * attention for AMD Instinct MI355X (gfx950).
 *
 * Method: "GQLA: Group-Query Latent Attention for Hardware-Adaptive Large
 * Language Model Decoding" (arXiv 2605.15250).  One set of group-indexed
 * latent weights (W_UK[G], W_UV[G], G < g) exposes two algebraically
 * equivalent decode paths (paperlayer.ai summary, section 3 "Methods", bullet
 * "Two equivalent decoding paths"; gist.science technical summary, section 2
 * "Architektur"):
 *   - the MQA-absorb path: W_UK[G] folded into each query head, attention of
 *     all h_q heads over the shared latent cache (c^KV_t ++ k^R_t), output
 *     up-projected by W_UV[G];
 *   - the GQA path: the latent cache expanded once into g K/V groups plus the
 *     shared rope key; conventional grouped-query attention with s_q query
 *     tokens per sequence (multi-token prediction) and no per-step expansion.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller; the library
 *   never allocates, frees or retains them and never synchronises.  Every
 *   call only enqueues kernels on `stream` (a hipStream_t passed as void*;
 *   NULL = the null stream) and returns.
 * - bf16 tensors are passed as void* to 16-bit bfloat16 storage; fp32 as
 *   float*; indices as int32_t*.  Every tensor pointer must be 16-byte
 *   aligned and densely packed in the row-major shape given.
 * - Head h belongs to group G = h / (h_q / g).  W_UK[G] is (d_latent x d_nope)
 *   and W_UV[G] is (d_latent x d_v): the key/value of token t in group G are
 *   the row vectors c_t W_UK[G] and c_t W_UV[G].
 * - Logits are (q_nope . k_nope + q_rope . k_rope) * softmax_scale.  q_rope
 *   and k_rope arrive already rotated.
 * - cache_seqlens[b] = L_b counts the s_q new tokens; query row i < s_q of
 *   sequence b sees cache tokens t <= L_b - s_q + i (causal mask between the
 *   MTP rows).  Precondition: s_q <= L_b.
 * - Paged cache: token t of sequence b is slot t % block_size of page
 *   block_table[b * max_blocks + t / block_size].  Only entries t / block_size
 *   < ceil(L_b / block_size) are read.  Precondition: those entries are valid
 *   page indices.
 * - lse outputs are natural-log sum-exp of the scaled logits (fp32).
 * - Split-KV: split_offsets (device, int32 [batch + 1], prefix sums) gives
 *   sequence b the splits split_offsets[b] .. split_offsets[b+1]-1; split j
 *   of b covers tokens [j*split_tokens, min((j+1)*split_tokens, L_b)).
 *   split_tokens must be a positive multiple of block_size and
 *   split_offsets[batch] must equal total_splits (caller's duty: use
 *   ceil(L_b / split_tokens) splits for sequence b).  Partials are the
 *   normalised attention output over the split and its lse; a split in which
 *   a row sees no token holds out = 0, lse = -inf.
 * - Errors: a negative return value means nothing was enqueued.  Argument
 *   checks happen on the host before any HIP call, so they never touch the
 *   device.  GQLA_ERR_HIP reports a launch failure (hipGetLastError).
 *   Calls are reentrant (no mutable global state); calls on different
 *   streams may overlap.
 *
 * Supported shapes (compile-time instantiations; others return
 * GQLA_ERR_UNSUPPORTED_SHAPE): block_size = 64, s_q in {1, 2}, and
 *   (h_q/g, d_latent, d_rope, d_nope, d_v) in
 *     {(16, 512, 64, 128, 128), (32, 512, 64, 128, 128), (4, 512, 64, 128, 128),
 *      (8, 64, 16, 32, 32)}.
 */
#ifndef GQLA_H
#define GQLA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GQLA_OK 0
#define GQLA_ERR_INVALID_ARG (-1)
#define GQLA_ERR_UNSUPPORTED_SHAPE (-2)
#define GQLA_ERR_MISALIGNED (-3)
#define GQLA_ERR_BAD_SPLIT_PLAN (-4)
#define GQLA_ERR_HIP (-5)
#define GQLA_ERR_SCRATCH_LIMIT (-6)

/* Problem dimensions, in the pages' notation (paperlayer.ai section 3
 * "Architecture": h_q heads, g groups of per-head dim d_h, latent c^KV_t,
 * per-head q^R_h and shared k^R; s_q query tokens per step). */
typedef struct gqla_dims {
    int32_t num_heads;     /* h_q */
    int32_t num_groups;    /* g: number of distinct W_UK[G] / W_UV[G] */
    int32_t d_latent;      /* r_kv: latent width of c^KV_t */
    int32_t d_rope;        /* d^R_h: shared decoupled-RoPE key width */
    int32_t d_nope;        /* per-head K-NoPE width */
    int32_t d_v;           /* per-head V width */
    int32_t s_q;           /* query tokens per sequence per step (1 + MTP heads) */
    int32_t block_size;    /* tokens per cache page */
    float softmax_scale;   /* 0 => 1/sqrt(d_nope + d_rope) */
} gqla_dims;

/* Elements per page of each cache format.
 * Latent page:   [block_size][d_latent + d_rope]   (c_t ++ k_rope_t per slot;
 *                576 elements = 1152 B per token for the DeepSeek-V3 shape,
 *                paperlayer.ai section 5 "Conversion setup").
 * Expanded page: for G in 0..g-1: K block [block_size][d_nope] then V block
 *                [block_size][d_v] (both token-major); then rope
 *                [block_size][d_rope].
 *                2*g*d_h + d_rope elements per token (same passage; 4224 B per
 *                token at g = 8, section 4 "GQA path"). */
int64_t gqla_latent_page_elems(const gqla_dims* d);
int64_t gqla_expanded_page_elems(const gqla_dims* d);

/* One-shot cache expansion (latent -> per-group K/V), the deployment-time
 * switch to the GQA path (paperlayer.ai section 3, "Two equivalent decoding
 * paths": a one-shot cache compression or expansion; pwwt.cn section 3).
 *   latent_pages   bf16 [num_pages][block_size][d_latent + d_rope]
 *   w_uk           bf16 [g][d_latent][d_nope]
 *   w_uv           bf16 [g][d_latent][d_v]
 *   page_ids       int32 [num_pages_to_expand] or NULL (= pages 0..num_pages-1)
 *   expanded_pages bf16 [num_pages][gqla_expanded_page_elems]; page p of the
 *                  output corresponds to latent page p, so one block table
 *                  indexes both caches.
 * Every slot of each listed page is expanded: K = RNE_bf16(c W_UK[G]),
 * V = RNE_bf16(c W_UV[G]) with fp32 accumulation; the rope key is copied
 * bit-exactly. */
int gqla_expand_cache(const gqla_dims* d, const void* latent_pages, const void* w_uk,
                      const void* w_uv, int64_t num_pages, const int32_t* page_ids,
                      int64_t num_pages_to_expand, void* expanded_pages, void* stream);

/* Incremental append (the step beside decode that live serving needs): after
 * the one-shot conversion the latent pages stay the stored state and the GQA
 * path decodes with no per-step latent expansion (paperlayer.ai section 4
 * "GQA path"), but each step's new tokens still need their latent rows and,
 * for the GQA path, their per-group K/V.
 *   new_rows  bf16 [batch][n_new][d_latent + d_rope]: the new tokens' c ++ k_rope,
 *             written to positions cache_seqlens[b] - n_new .. cache_seqlens[b] - 1
 *             of sequence b (cache_seqlens counts the new tokens, as the decode
 *             calls take it; 1 <= n_new <= block_size <= cache_seqlens[b]);
 *   latent_pages, num_pages, block_table, max_blocks: as for the decode calls;
 *   expanded_pages  NULL, or the expanded cache: then the new tokens' K, V and
 *             rope slots are written too (w_uk and w_uv required), computed
 *             exactly as gqla_expand_cache computes them, so the expanded cache
 *             stays bit-identical to a full expansion of the latent cache; no
 *             other slot is written.
 * The latent rows are written before the expansion reads them (one stream).
 * Two new tokens must not share a slot.  A new token whose position is below 0
 * (cache_seqlens[b] < n_new) or whose page index is >= max_blocks breaks the
 * precondition; nothing is written for it, in either mode. */
int gqla_append_tokens(const gqla_dims* d, int32_t batch, int32_t n_new, const void* new_rows,
                       void* latent_pages, int64_t num_pages, const int32_t* block_table,
                       int32_t max_blocks, const int32_t* cache_seqlens, const void* w_uk,
                       const void* w_uv, void* expanded_pages, void* stream);

/* MQA-absorb decode over the latent cache (paperlayer.ai section 4,
 * "MQA-absorb path"; gist.science section 2 "MQA-Absorb-Pfad"):
 *   q_abs = W_UK[G] q_nope,  s_t = (q_abs . c_t + q_rope . k_rope_t) * scale,
 *   o_lat = softmax(s) C,     out = o_lat W_UV[G].
 *   q_nope  bf16 [batch][s_q][h_q][d_nope]     q_rope bf16 [batch][s_q][h_q][d_rope]
 *   latent_pages as for gqla_expand_cache; block_table int32 [batch][max_blocks];
 *   cache_seqlens int32 [batch]; w_uk, w_uv as for gqla_expand_cache.
 *   split_offsets   NULL => one split per sequence, else the split plan
 *                   described above.
 *   out      bf16 [batch][s_q][h_q][d_v], required in both modes.
 *   lse      fp32 [batch][s_q][h_q] or NULL.
 *   workspace  device scratch of at least
 *            gqla_mqa_absorb_workspace_bytes(d, batch, split_offsets ? total_splits : 0)
 *            bytes, 16-byte aligned, owned by the caller; it must not be shared
 *            by calls that may run concurrently.  Too small or NULL returns
 *            GQLA_ERR_INVALID_ARG.  Its four regions (byte offsets from
 *            gqla_mqa_absorb_workspace_offsets) hold, after the call:
 *              [0] the absorbed query rows q_abs ++ q_rope, bf16
 *                  [batch][s_q][h_q][d_latent + d_rope];
 *              [1] W_UV transposed, bf16, g x d_v x d_latent elements (internal
 *                  order: the merge's MFMA operand chunks);
 *              [2] the per-split normalised latent outputs o_lat, bf16
 *                  [units][s_q][h_q][d_latent] (units = total_splits under a
 *                  split plan, else batch with unit b = sequence b);
 *              [3] their lse, fp32 [units][s_q][h_q] (-inf and o_lat = 0 for a
 *                  row that sees no token of the split).
 * The splits are merged in the latent space (log-sum-exp weights, fp32) and
 * the merged o_lat is up-projected once per row; by linearity this equals
 * merging per-split up-projected outputs.  No part_out / part_lse buffers. */
int gqla_decode_mqa_absorb(const gqla_dims* d, int32_t batch, const void* q_nope,
                           const void* q_rope, const void* latent_pages,
                           const int32_t* block_table, int32_t max_blocks,
                           const int32_t* cache_seqlens, const void* w_uk, const void* w_uv,
                           const int32_t* split_offsets, int32_t split_tokens,
                           int32_t total_splits, void* out, float* lse, void* workspace,
                           uint64_t workspace_bytes, void* stream);

/* Bytes of device workspace gqla_decode_mqa_absorb needs for `batch` sequences
 * and `total_splits` splits (0 = no split plan); 0 for batch <= 0,
 * total_splits < 0 or d == NULL. */
uint64_t gqla_mqa_absorb_workspace_bytes(const gqla_dims* d, int32_t batch, int32_t total_splits);

/* Byte offsets of the four workspace regions listed above (offsets[0..3]);
 * GQLA_ERR_INVALID_ARG for the arguments gqla_mqa_absorb_workspace_bytes
 * answers 0 for, or offsets == NULL. */
int gqla_mqa_absorb_workspace_offsets(const gqla_dims* d, int32_t batch, int32_t total_splits,
                                      uint64_t* offsets);

/* gqla_decode_mqa_absorb without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, checks and results as
 * gqla_decode_mqa_absorb; the workspace is a device array of
 * GQLA_NOALLOC_SCRATCH_BYTES bytes compiled into the library, one per GPU,
 * resolved on the first call on that GPU (the current device, which must be
 * the stream's device) and held until the process ends.  The call allocates
 * nothing.  A call whose workspace would exceed the array
 * (gqla_mqa_absorb_workspace_bytes(d, batch, split_offsets ? total_splits : 0)
 * > GQLA_NOALLOC_SCRATCH_BYTES) returns GQLA_ERR_SCRATCH_LIMIT before any HIP
 * call.  Every call on one GPU uses the same array: calls that may overlap on
 * one GPU (concurrent streams or threads) race and must be serialised by the
 * caller.  The kernels write every scratch byte they later read, so nothing
 * is cleared between calls. */
#define GQLA_NOALLOC_SCRATCH_BYTES (32u << 20)
int gqla_decode_mqa_absorb_noalloc(const gqla_dims* d, int32_t batch, const void* q_nope,
                                   const void* q_rope, const void* latent_pages,
                                   const int32_t* block_table, int32_t max_blocks,
                                   const int32_t* cache_seqlens, const void* w_uk, const void* w_uv,
                                   const int32_t* split_offsets, int32_t split_tokens,
                                   int32_t total_splits, void* out, float* lse, void* stream);

/* Merge of MQA-absorb split partials in the latent space, then the
 * up-projection (paperlayer.ai section 4, "MQA-absorb path": attention runs
 * over the latent and W_UV[G] maps its output back; the up-projection is
 * linear, so the splits may be merged before it).  For each query row
 * (b, i, h) of group G = h / (h_q / g), over the units s of sequence b:
 *   m = max_s lse_s,  w_s = exp(lse_s - m),  o = sum_s w_s part_lat_s / sum_s w_s,
 *   lse = m + ln sum_s w_s,  out = o W_UV[G]   (fp32 throughout, bf16 out).
 *   part_lat   bf16 [units][s_q][h_q][d_latent]: each split's normalised
 *              latent output;
 *   part_lse   fp32 [units][s_q][h_q]; -inf marks a split that saw no token
 *              of the row (its part_lat row then carries weight 0);
 *   split_offsets  int32 [batch + 1] or NULL: sequence b owns units
 *              split_offsets[b] .. split_offsets[b + 1] - 1; NULL means unit b
 *              is sequence b (units = batch);
 *   total_splits   units when split_offsets is given (>= batch, else
 *              GQLA_ERR_BAD_SPLIT_PLAN); ignored otherwise;
 *   w_uv       bf16 [g][d_latent][d_v];
 *   out        bf16 [batch][s_q][h_q][d_v];  lse fp32 [batch][s_q][h_q] or NULL;
 *   workspace  at least gqla_mqa_absorb_merge_workspace_bytes(d) bytes of
 *              device scratch, 16-byte aligned, owned by the caller (W_UV
 *              transposed); too small or NULL returns GQLA_ERR_INVALID_ARG.
 * part_lat and part_lse have the layouts of regions [2] and [3] of the
 * gqla_decode_mqa_absorb workspace, so this call also re-merges the partials a
 * decode call left there.  A row whose units all have lse = -inf gets out = 0
 * and lse = -inf.  The same checks as the decode calls run on the host before
 * anything is enqueued; batch = 0 is a no-op. */
int gqla_mqa_absorb_merge(const gqla_dims* d, int32_t batch, const void* part_lat, const float* part_lse,
                          const int32_t* split_offsets, int32_t total_splits, const void* w_uv, void* out,
                          float* lse, void* workspace, uint64_t workspace_bytes, void* stream);

/* Bytes of workspace gqla_mqa_absorb_merge needs; 0 for d == NULL or
 * non-positive g, d_v or d_latent. */
uint64_t gqla_mqa_absorb_merge_workspace_bytes(const gqla_dims* d);

/* GQA decode over the per-group expanded cache (paperlayer.ai section 4,
 * "GQA path"; gist.science section 2 "GQA-Pfad": conventional grouped-query
 * attention with no per-step latent expansion).  Arguments as for
 * gqla_decode_mqa_absorb, with expanded_pages (bf16 [num_pages]
 * [gqla_expanded_page_elems]) in place of the latent cache, no weights and no
 * workspace, and:
 *   out      bf16 [batch][s_q][h_q][d_v]: required without a split plan; with
 *            one and out != NULL, gqla_splitkv_combine is enqueued after the
 *            decode.
 *   part_out fp32 [total_splits][s_q][h_q][d_v], part_lse fp32
 *            [total_splits][s_q][h_q]: the per-split partials, required iff
 *            split_offsets != NULL. */
int gqla_decode_gqa(const gqla_dims* d, int32_t batch, const void* q_nope, const void* q_rope,
                    const void* expanded_pages, const int32_t* block_table, int32_t max_blocks,
                    const int32_t* cache_seqlens, const int32_t* split_offsets,
                    int32_t split_tokens, int32_t total_splits, void* out, float* lse,
                    float* part_out, float* part_lse, void* stream);

/* Sparse GQA decode over per-group token selections (sparse GQLA:
 * gist.science section 2, subsection "Sparse GQLA"; pwwt.cn section 5 on the
 * sparse extension; ai-feeds.com "Methods", the optional sparse extension).
 * Each KV group attends to its own listed subset of the cached tokens, shared
 * by all h_q/g heads and all s_q query rows of the group, so the group's rows
 * stay one dense matrix tile.  How the subset is chosen (an indexer) is left
 * to the caller.  Arguments as for gqla_decode_gqa without a split plan, and:
 *   num_pages  pages in expanded_pages (>= 1, at most 2^28 / block_size);
 *   indices    int32 [batch][g][topk]: token positions of sequence b chosen
 *              for group G.  Entries outside [0, cache_seqlens[b]), or whose
 *              block-table page is outside [0, num_pages), are ignored (-1
 *              pads a short list); an entry listed twice counts twice; query
 *              row i still sees only positions <= L_b - s_q + i.  A row that
 *              sees no entry gets out = 0 and lse = -inf.
 *   topk       entries per list (>= 1).
 *   split_entries  0: one workgroup per (sequence, group) over its whole
 *              list; else a multiple of 32: each list (rounded up to 32
 *              entries) is cut into ranges of this many entries, one
 *              workgroup per (sequence, range, group), whose fp32 partials
 *              are merged by log-sum-exp as gqla_splitkv_combine merges them
 *              (a third kernel).  Splitting fills the GPU at small batch.
 *   out, lse   as for gqla_decode_gqa (out required).
 *   workspace  device scratch of at least gqla_sparse_workspace_bytes(d,
 *              batch, topk, split_entries) bytes, 16-byte aligned, owned by
 *              the caller and not shared by calls that may run concurrently.
 *              Regions (byte offsets from gqla_sparse_workspace_offsets):
 *                [0] each entry's resolved cache row, uint32 [batch][g][topk
 *                    rounded up to 32]: bits 0..27 page * block_size + slot,
 *                    bits 28..30 the first query row that sees the entry (7:
 *                    none);
 *                [1] with a split: the split plan, int32 [batch + 1]
 *                    (b * ranges per list);
 *                [2], [3] with a split: the partial outputs fp32 [batch *
 *                    ranges][s_q][h_q][d_v] and their lse fp32 [batch *
 *                    ranges][s_q][h_q];
 *                [4] the end.
 * Kernels are enqueued on `stream`: the row resolution, the decode, and with a
 * split the merge. */
int gqla_decode_gqa_sparse(const gqla_dims* d, int32_t batch, const void* q_nope,
                           const void* q_rope, const void* expanded_pages, int64_t num_pages,
                           const int32_t* block_table, int32_t max_blocks,
                           const int32_t* cache_seqlens, const int32_t* indices, int32_t topk,
                           int32_t split_entries, void* out, float* lse, void* workspace,
                           uint64_t workspace_bytes, void* stream);

/* Bytes of workspace gqla_decode_gqa_sparse needs; 0 for the arguments
 * gqla_sparse_workspace_offsets rejects. */
uint64_t gqla_sparse_workspace_bytes(const gqla_dims* d, int32_t batch, int32_t topk,
                                     int32_t split_entries);

/* Byte offsets of the sparse workspace regions listed above (offsets[0..4]);
 * GQLA_ERR_INVALID_ARG for d == NULL, offsets == NULL, batch <= 0, topk <= 0
 * or split_entries < 0. */
int gqla_sparse_workspace_offsets(const gqla_dims* d, int32_t batch, int32_t topk,
                                  int32_t split_entries, uint64_t* offsets);

/* Log-sum-exp merge of split partials (the pages are silent on split-KV; this
 * is the exact decomposition of a softmax over disjoint token ranges):
 *   m = max_s lse_s, w_s = exp(lse_s - m), out = sum_s w_s o_s / sum_s w_s
 *   (rounded to bf16), lse = m + log(sum_s w_s).  Splits with lse = -inf carry
 *   weight 0; a row whose splits are all empty gets out = 0, lse = -inf.
 *   part_out fp32 [total_splits][s_q][h_q][d_v], part_lse fp32 [total_splits][s_q][h_q],
 *   out bf16 [batch][s_q][h_q][d_v], lse fp32 [batch][s_q][h_q] or NULL. */
int gqla_splitkv_combine(const gqla_dims* d, int32_t batch, const int32_t* split_offsets,
                         int32_t total_splits, const float* part_out, const float* part_lse,
                         void* out, float* lse, void* stream);

/* ---- Path selector (roofline advisor) ----------------------------------
 * The pages pick the path per hardware by comparing each path's arithmetic
 * intensity with the ridge point (paperlayer.ai section 4 "Roofline
 * analysis" and "Hardware operating points"; gist.science section 2
 * "Pfadauswahl"); they state no policy beyond that.  This estimates one
 * decode call of each path over a batch with the pages' roofline model,
 * time = max(bytes / bandwidth, FLOPs / peak), divided by the fraction of that
 * bound the path reaches on the given hardware, and recommends the path with
 * the higher query tokens per second (ties go to the absorb path, which needs
 * no expanded cache).  Host-only: no device memory, no stream. */
typedef struct {
  double hbm_gbps;        /* memory bandwidth, GB/s (> 0) */
  double mfma_tflops;     /* dense bf16 matrix peak, TFLOP/s (> 0) */
  double frac_absorb;     /* fraction of its roofline the absorb path reaches, (0, 1] */
  double frac_gqa;        /* same for the GQA path */
  int32_t cache_only;     /* 1: count only cache bytes and attention FLOPs (the pages'
                             step-time convention); 0: also the query, output and, on
                             the absorb path, the weights and the two projections */
} gqla_hw;

typedef struct {
  double bytes;           /* algorithmic bytes of the call (each operand moved once) */
  double flops;           /* algorithmic FLOPs, 2 per multiply-accumulate */
  double t_hbm_us;        /* bytes / bandwidth */
  double t_mfma_us;       /* FLOPs / peak */
  double t_roofline_us;   /* max of the two */
  double t_expected_us;   /* t_roofline_us / frac */
  double tokens_per_s;    /* batch * s_q / t_expected_us */
  int32_t bound;          /* 0 = memory-bound, 1 = compute-bound */
} gqla_path_estimate;

#define GQLA_PATH_ABSORB 0
#define GQLA_PATH_GQA 1

/* Estimates of one gqla_decode_mqa_absorb call with s_q_absorb query tokens
 * per sequence and one gqla_decode_gqa call with s_q_gqa (e.g. 1 and 2 with
 * one MTP head), over `batch` sequences of lengths cache_seqlens_host (HOST
 * int32 [batch], each >= the larger s_q).  d->s_q and d->block_size are not
 * used.  Writes *absorb and *gqa (either may be NULL) and returns
 * GQLA_PATH_ABSORB or GQLA_PATH_GQA; GQLA_ERR_INVALID_ARG for NULL d, hw or
 * lengths, batch < 1, s_q outside [1, 2], a length below s_q, a
 * non-positive rate or a fraction outside (0, 1]. */
int gqla_select_path(const gqla_dims* d, int32_t batch, const int32_t* cache_seqlens_host,
                     int32_t s_q_absorb, int32_t s_q_gqa, const gqla_hw* hw,
                     gqla_path_estimate* absorb, gqla_path_estimate* gqa);

/* Human-readable text for a status code (static storage; never NULL). */
const char* gqla_status_string(int status);

/* ABI version (major * 100 + minor). */
int gqla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GQLA_H */

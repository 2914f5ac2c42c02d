/*
 * vt.h -- C ABI of the draft-sampling / verification hot path for AMD Instinct MI355X (gfx950).
 *
 * Three operations make one speculative-decoding block:
 *   vt_lmhead_trimmed  drafter logits through a vocabulary-trimmed LM head
 *   vt_softmax_temp    temperature softmax (log-normaliser, optional probabilities) with an
 *                      optional inverse-CDF draw per row
 *   vt_spec_verify     batched modified rejection sampling: accept scan, residual or bonus draw,
 *                      trimmed-id -> full-id remap
 * and vt_spec_block runs all of them for one block in a single call, with fused kernels.
 * vt_keepset.h builds the kept vocabulary and the trimmed head; vt_generate.h chains blocks into
 * a generation loop for table models.
 *
 * Pages cited (title, section):
 *   [VT] "VocabTrim: Vocabulary Pruning for Efficient Speculative Decoding in LLMs" (arXiv 2506.22694v2)
 *   [GL] "Speculative decoding" (glossary page)
 *   [RR] "A rejection rule keeps speculative decoding's output exact"
 *
 * Conventions for every entry point
 *   - Every array pointer is a DEVICE pointer owned by the caller.  The library never allocates,
 *     frees or synchronises; it only enqueues kernels on `stream` (0 = the null stream) and
 *     returns.  Outputs are valid once the caller has synchronised the stream; inputs must stay
 *     unchanged until then.  There is no global state (apart from the fixed device scratch of
 *     vt_spec_block_noalloc): calls on distinct streams (with distinct workspaces) may overlap.
 *   - Arguments are validated on the host before any HIP call.  A failed check returns an error
 *     code and enqueues nothing.  Nothing is thrown across the ABI and nothing aborts.
 *   - Random numbers the method draws are inputs: uniforms u in (0, 1].  Using u = (k+1) * 2^-24
 *     for a 24-bit integer k keeps them exact in fp32.
 *   - Documented but unchecked preconditions (violations give unspecified results, never an
 *     out-of-bounds access unless stated): logits are finite or -inf with at least one finite
 *     entry per row; keep_ids entries are distinct and in [0, V_rows); full_to_trim is the
 *     inverse of keep_ids (-1 elsewhere); an lse passed in was produced by vt_softmax_temp from
 *     the same logits and temperature.
 *   - Workspaces: a caller-owned device buffer of at least the size the matching
 *     *_workspace_bytes function returns, holding per-chunk partial results between the
 *     launches of one call.  Its contents need no initialisation and carry nothing between
 *     calls; two calls in flight at once must not share a workspace.
 */
#ifndef VT_H_
#define VT_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VT_OK = 0,
  VT_ERR_INVALID_ARG = 1, /* a NULL required pointer, a size out of range, a bad temperature */
  VT_ERR_UNSUPPORTED = 2, /* valid arguments this build does not handle (alignment, H % 8, gamma > 64) */
  VT_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than the *_workspace_bytes size */
  VT_ERR_HIP = 4          /* hipLaunchKernel reported an error for one of the launches */
} vt_status_t;

typedef enum { VT_F32 = 0, VT_BF16 = 1 } vt_dtype_t;

/*
 * vt_lmhead_trimmed -- drafter logits over the trimmed vocabulary.
 *   [VT] §3, Eq. 1: the trimmed head keeps the rows of the full LM head W that belong to the kept
 *   vocabulary (Top-K of a token-frequency count), in that order; [VT] Appendix C.1, Algorithm 2:
 *   the trimmed drafter scores only those rows.
 *
 *   logits[m][j] = sum_{k < H} hidden[m][k] * weight[row(j)][k],   row(j) = keep_ids ? keep_ids[j] : j
 *
 *   hidden   bf16 bit patterns, row-major [M][H]
 *   weight   bf16 bit patterns, row-major [V_rows][H] (the full head; rows are gathered through
 *            keep_ids, so no trimmed copy is needed; pass a pre-gathered W^Trim with keep_ids=NULL)
 *   keep_ids int32 [Vt] or NULL (then row(j) = j and Vt <= V_rows)
 *   logits   fp32 row-major [M][Vt], written in full
 *   Products of bf16 values are exact in fp32; sums are accumulated in fp32 in an order that does
 *   not depend on the row, so trimmed logits equal untrimmed logits gathered at keep_ids bit for bit.
 *   The order does depend on M, which picks the kernel: a GEMV when M <= 8 and
 *   M * ceil(H / 512) <= 48 (lanes hold partial sums over 16-byte pieces of a row, reduced across
 *   lanes); otherwise an MFMA kernel: when H % 32 == 0 one block of all M rows (padded to a
 *   multiple of 32) per 256 head rows up to M = 192 (when the head has fewer than 256 blocks of
 *   256 rows: per 128 head rows up to M = 256, and in two row blocks up to M = 384), 256 x 256
 *   tiles beyond; for other H 128 x 128
 *   tiles up to M = 128, register-staged 256 x 256 tiles beyond.  Every MFMA kernel sums a
 *   logit's products in MFMA steps of 16 in ascending K, so they all give the same bits; between
 *   the GEMV and the MFMA kernels a hidden row's logits may differ in the last bits (each within
 *   the recursive-summation bound H 2^-24 sum_k |h_k w_k|), and so may a decision taken on them,
 *   but only where it lies within rounding of its uniform.
 *   Errors: INVALID_ARG for NULL hidden/weight/logits, M, H, Vt or V_rows <= 0, Vt > V_rows when
 *   keep_ids is NULL; UNSUPPORTED for H % 8 != 0 or a hidden/weight base not 16-byte aligned.
 */
vt_status_t vt_lmhead_trimmed(const uint16_t *hidden, const uint16_t *weight, const int32_t *keep_ids,
                              int64_t M, int64_t H, int64_t Vt, int64_t V_rows, float *logits,
                              hipStream_t stream);

/*
 * vt_softmax_temp -- temperature softmax over each row of a [rows][n] matrix (row stride ld
 * elements), with an optional inverse-CDF draw.
 *   [GL] "Distributional exactness has conditions": temperature must be applied to the very
 *   distributions the correction uses; [RR] "A target and a draft small enough to print in full":
 *   the categorical sampler walks the tokens in index order accumulating mass.
 *
 *   lse[r]      = log sum_j exp(x[r][j] / T)                      (fp64 output, fp32 reduction)
 *   probs[r][j] = exp(x[r][j] / T - lse[r])                       (optional, fp32, row stride n)
 *   sampled[r]  = min { j : u[r] * Z <= C[j] }                    (optional, int32)
 *     where C is the running sum of the row's weights exp((x[r][j] - max_j x[r][j]) / T) in index
 *     order and Z is the last entry of that same running sum, so for u in (0, 1] an index exists
 *     and a zero-weight entry is never returned.  The running sum is formed in fp32 over fixed
 *     4096-element chunks (chunk sums, a prefix over chunks, then a prefix inside the selected
 *     chunk), independent of rows and of the row count.  Rows of more than one chunk take two
 *     launches (chunk partials, then one workgroup per row), plus one for probs.  Where the two levels disagree by a
 *     rounding step at a chunk's end, the last positive-weight entry of that chunk is returned.
 *
 *   logits  fp32 or bf16 (dtype), [rows][ld] with ld >= n
 *   lse     required, fp64 [rows]
 *   probs   optional (NULL), fp32 [rows][n]
 *   u       optional (NULL), fp32 [rows] in (0, 1]; sampled must be non-NULL exactly when u is
 *   workspace / workspace_bytes: see vt_softmax_temp_workspace_bytes
 *   T = 0 is the greedy limit ([VT] §4 decodes the target greedily): sampled[r] (if non-NULL) is
 *   the index of the row maximum, the lowest such index on ties; lse[r] holds the row maximum
 *   (the limit of T * logsumexp(x / T)); probs is one-hot at sampled[r]; u is not read.
 *   Errors: INVALID_ARG for NULL logits/lse, rows or n <= 0, ld < n, T not finite or < 0,
 *   exactly one of u/sampled NULL (T > 0), an unknown dtype; WORKSPACE if the workspace is too small.
 */
vt_status_t vt_softmax_temp(const void *logits, vt_dtype_t dtype, int64_t rows, int64_t n, int64_t ld,
                            float temperature, double *lse, float *probs, const float *u, int32_t *sampled,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace vt_softmax_temp needs for this shape (0 when no row spans two chunks). */
size_t vt_softmax_temp_workspace_bytes(int64_t rows, int64_t n);

/*
 * vt_spec_verify -- modified rejection sampling for B independent sequences of gamma drafts.
 *   [GL] "Propose a block, keep a prefix" and "Why a rejection needs a special draw";
 *   [RR] "What the accept/reject rule has to balance" and "Extending the rule from one token to a
 *   drafted run"; [VT] Appendix C.1, Algorithm 2 (the token index mapper back to the full vocabulary).
 *
 *   For each sequence b, with p_i = softmax(target row i / target_T) over the V full ids and
 *   q_i = softmax(draft row i / draft_T) over the Vt kept ids (q_i = 0 off the kept set):
 *     1. left to right for i < gamma: x = draft_ids[b][i] (trimmed id), y = keep_ids[x] (full id);
 *        accept iff u_accept[b][i] <= min(1, p_i(y) / q_i(x)); n = index of the first rejection,
 *        or gamma if none;
 *     2. if n < gamma: final ~ max(0, p_n - q_n) over full ids 0..V-1 (if that sums to 0 in fp32:
 *        p_n); else final ~ p_gamma (the bonus token); drawn with u_final[b] by the running-sum
 *        rule of vt_softmax_temp over full ids, in fixed 4096-id chunks;
 *     3. out_tokens[b] = { y_0 .. y_{n-1}, final, -1 ... } (gamma+1 entries), out_num_accepted[b] = n.
 *   The accept ratio is evaluated in fp64 from the fp32/bf16 logits and the fp64 lse.
 *   target_T = 0 selects greedy verification ([VT] §4, App. C.1 Algorithm 2 under greedy
 *   decoding): accept iff y_i == a_i, the lowest id of target row i's maximum; final = a_n (a_gamma
 *   after full acceptance); target_lse, draft_logits, draft_lse, draft_T, u_accept and u_final
 *   are not read (may be NULL).
 *   A draft id outside [0, Vt) (or mapping outside [0, V)) among the first gamma makes that
 *   sequence's out_num_accepted -1 and all its tokens -1; this is checked on the device.
 *
 *   target_logits fp32 or bf16 (target_dtype), [B][gamma+1][V]
 *   target_lse    fp64 [B][gamma+1]     (from vt_softmax_temp with target_T)
 *   draft_logits  fp32 [B][R][Vt], R >= gamma (rows gamma..R-1 are not read)
 *   draft_lse     fp64 [B][R]           (from vt_softmax_temp with draft_T)
 *   draft_ids     int32 [B][R] trimmed ids (from vt_softmax_temp's draw)
 *   keep_ids      int32 [Vt], full_to_trim int32 [V]: both NULL (untrimmed head, Vt == V) or both set
 *   u_accept      fp32 [B][gamma];  u_final fp32 [B]
 *   out_tokens    int32 [B][gamma+1];  out_num_accepted int32 [B]
 *   Errors: INVALID_ARG for NULL required pointers, B, gamma, V, Vt <= 0, Vt > V, R < gamma,
 *   a temperature not finite or <= 0 (target_T > 0), keep_ids/full_to_trim NULL with Vt < V or
 *   only one of them NULL; UNSUPPORTED for gamma > 64; WORKSPACE if the workspace is too small.
 */
vt_status_t vt_spec_verify(int64_t B, int64_t gamma, int64_t V, int64_t Vt, const void *target_logits,
                           vt_dtype_t target_dtype, const double *target_lse, float target_T,
                           const float *draft_logits, int64_t R, const double *draft_lse, float draft_T,
                           const int32_t *draft_ids, const int32_t *keep_ids, const int32_t *full_to_trim,
                           const float *u_accept, const float *u_final, int32_t *out_tokens,
                           int32_t *out_num_accepted, void *workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Bytes of workspace vt_spec_verify needs for B sequences of gamma drafts over a V-id vocabulary. */
size_t vt_spec_verify_workspace_bytes(int64_t B, int64_t gamma, int64_t V);

/*
 * vt_spec_block -- one whole speculative block in one call: the trimmed LM head, the draft
 * softmax with draws, the target softmax and the verification, i.e. the four calls above, with
 * the kernels fused where the dependencies allow.  Decode-sized batches (B*R <= 8, both sides
 * sampled) take 3 launches instead of 7: the LM head launch also emits the draft softmax's
 * first pass and, in extra workgroups, the target rows' first pass; one chunk pass over the
 * full vocabulary forms the log-normalisers, draft draws, accept tests and residual chunk sums;
 * one final pass draws the last token.  Past the GEMV sizes, for up to 32 hidden rows in at most 4
 * sequences of up to 8 draft rows or 2 of up to 16, the same two passes follow the target partials
 * and the MFMA head (4 launches).
 * Larger batches take 5 (target partials, LM head with the draft partials, one combine launch
 * for both row sets, two verify passes).  Past the GEMV
 * sizes with H % 32 == 0 the target partials launch also copies the hidden rows K-tiled into the
 * workspace (the head then reads each K step of a block of hidden rows as one contiguous run; same
 * products, same logits); without target partials (V <= 4096 or greedy verification) the copy is
 * a launch of its own.  That head takes one block of all hidden rows up to B*R = 192 (on heads
 * of fewer than 256 blocks of 256 rows: one block up to 256 rows, two up to 384), and beyond
 * 384 x 256 tiles (384 hidden rows) when they give each CU no more hidden rows than 256 x 256
 * tiles, counting one tile per CU at a time (B*R = 2304 or 288 against 256 head blocks), else
 * 256 x 256 tiles (B*R = 512 against 128 head blocks); all sum the same products in the same
 * order as the separate call's kernel.
 *   The call issues kernel launches (and the optional events) only: no allocation, memset or copy,
 *   so it can be captured into a HIP graph with its workspace and replayed.
 *   Pages: as for the four calls above.
 *
 *   hidden bf16 [B*R][H] (row b*R + i is sequence b's i-th draft position); weight bf16 [V][H]
 *   (the full head); weight_tiled: NULL, or W^Trim in the K-tiled layout vt_trim_head_tiled makes
 *   from this weight and keep_ids (vt_keepset.h), which the MFMA head then reads in place of
 *   gathering rows of weight (only past the GEMV sizes and when H % 32 == 0; ignored otherwise;
 *   same products in the same order, so the same logits bits; the library cannot check
 *   that it matches weight and keep_ids); keep_ids int32 [Vt] and full_to_trim int32 [V] (both
 *   NULL iff the head is untrimmed, Vt == V); target_logits [B][gamma+1][V] (fp32 or bf16);
 *   u_draft fp32 [B*R], u_accept fp32 [B][gamma], u_final fp32 [B].
 *   Outputs: draft_logits fp32 [B*R][Vt], draft_lse fp64 [B*R], draft_ids int32 [B*R] (trimmed
 *   ids), target_lse fp64 [B*(gamma+1)], out_tokens int32 [B][gamma+1], out_num_accepted int32 [B].
 *   lmhead_begin / lmhead_end: optional (NULL) events, recorded on `stream` immediately before and
 *   after the LM-head kernel, for timing it inside the call.
 *   Results are those of the four calls (the logits and target_lse bit for bit), except that on
 *   the fused paths the draft running sums are chunked by the LM head's own blocks of head rows
 *   instead of 4096-element chunks: ceil(Vt / 256) rounded up to a multiple of 4 rows on the GEMV,
 *   256 rows on the MFMA heads with partials (H % 32 == 0, or B*R > 128).  Draws can then differ
 *   from the separate calls only where a CDF boundary lies within rounding of the uniform.
 *   Sequences are independent: a sequence's outputs are those it gets alone, up to the LM head's
 *   batch-size-dependent summation order and draft chunking (GEMV or MFMA head, see
 *   vt_lmhead_trimmed), i.e. they can differ only at a decision within rounding of its
 *   uniform; every target-side quantity (target_lse, p, the residual) is computed per row in an
 *   order that depends on neither B nor the row.
 *   target_T = 0 selects greedy verification as in vt_spec_verify ([VT] §4): no target softmax
 *   runs, target_lse is not written, u_accept and u_final are not read (all three may be NULL).
 *   draft_T = 0 (allowed only with target_T = 0) makes each draft the lowest id of its row's
 *   maximum, draft_lse the row maximum, and u_draft is not read (may be NULL); the LM head then
 *   emits argmax partials instead of softmax partials: at decode sizes (B*R <= 8) per block of
 *   head rows for the draft rows and, in extra workgroups, per 4096-chunk for the target rows,
 *   and one more launch finishes the block (2 launches); on the MFMA heads per column block of
 *   head rows (the same kernels, K-tiled copies and weight_tiled as with sampled drafts), after a
 *   launch that takes the target rows' per-4096-chunk argmaxes, and one more launch finishes the
 *   block (3 launches; with more than 16 draft rows per sequence the combine and the verify passes
 *   finish it); otherwise (the GEMV without the decode path, or H % 32 != 0 with B*R <= 128) the
 *   head runs without partials and a separate pass finds the draft rows' argmaxes.
 *   Errors: INVALID_ARG for NULL required pointers, B, gamma, H, V or Vt <= 0, R < gamma, Vt > V,
 *   a temperature not finite or < 0, draft_T = 0 with target_T > 0, keep_ids/full_to_trim
 *   inconsistent with Vt; UNSUPPORTED for
 *   gamma > 64, H % 8 != 0, a hidden/weight/weight_tiled base not 16-byte aligned, weight_tiled
 *   with H % 32 != 0; WORKSPACE if the workspace
 *   is smaller than vt_spec_block_workspace_bytes.
 */
vt_status_t vt_spec_block(const uint16_t *hidden, const uint16_t *weight, const uint16_t *weight_tiled,
                          const int32_t *keep_ids,
                          const int32_t *full_to_trim, int64_t B, int64_t gamma, int64_t R, int64_t H, int64_t Vt,
                          int64_t V, const void *target_logits, vt_dtype_t target_dtype, float target_T,
                          float draft_T, const float *u_draft, const float *u_accept, const float *u_final,
                          float *draft_logits, double *draft_lse, int32_t *draft_ids, double *target_lse,
                          int32_t *out_tokens, int32_t *out_num_accepted, hipEvent_t lmhead_begin,
                          hipEvent_t lmhead_end, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace vt_spec_block needs for this shape. */
size_t vt_spec_block_workspace_bytes(int64_t B, int64_t gamma, int64_t R, int64_t H, int64_t Vt, int64_t V);

/*
 * vt_spec_block_noalloc -- vt_spec_block for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * results and errors as vt_spec_block, without workspace / workspace_bytes: the workspace is a
 * fixed 64 MiB array of device memory inside the library, one per device, held until the process
 * ends (its address is looked up once per device, on the first call with that device current).
 * Nothing is allocated or freed by this call.
 *   Limit: shapes whose vt_spec_block_workspace_bytes exceeds 64 MiB return VT_ERR_WORKSPACE
 *   before anything is enqueued (for example B = 256, gamma = 8, H = 4096, Vt = 65536,
 *   V = 128256 needs 24.5 MiB, most of it the K-tiled copy of the hidden rows).
 *   Calls that overlap on one device (two streams, or two host threads) share that device's array
 *   and race: serialise them.  The array keeps the last call's partial results; no call depends on
 *   its previous contents.  Errors: as vt_spec_block, plus VT_ERR_HIP if the device or the array's
 *   address cannot be queried, VT_ERR_UNSUPPORTED for a device index of 64 or more.
 */
vt_status_t vt_spec_block_noalloc(const uint16_t *hidden, const uint16_t *weight, const uint16_t *weight_tiled,
                                  const int32_t *keep_ids,
                                  const int32_t *full_to_trim, int64_t B, int64_t gamma, int64_t R, int64_t H,
                                  int64_t Vt, int64_t V, const void *target_logits, vt_dtype_t target_dtype,
                                  float target_T, float draft_T, const float *u_draft, const float *u_accept,
                                  const float *u_final, float *draft_logits, double *draft_lse, int32_t *draft_ids,
                                  double *target_lse, int32_t *out_tokens, int32_t *out_num_accepted,
                                  hipEvent_t lmhead_begin, hipEvent_t lmhead_end, hipStream_t stream);

/* Static description of a status code (never NULL). */
const char *vt_status_string(vt_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* VT_H_ */

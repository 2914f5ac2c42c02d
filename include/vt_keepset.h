/*
 * vt_keepset.h -- building the kept (trimmed) vocabulary on the GPU: the offline step that
 * produces the keep_ids / full_to_trim maps and the trimmed LM head consumed by vt.h.
 *
 *   vt_token_histogram  token-frequency counter over a calibration corpus
 *   vt_keep_select      the kept set from the counter: Top-K, Top-P or minimum frequency
 *   vt_trim_head        the trimmed head W^Trim as a contiguous row gather of W
 *
 * Pages cited (title, section):
 *   [VT] "VocabTrim: Vocabulary Pruning for Efficient Speculative Decoding in LLMs" (arXiv 2506.22694v2)
 *
 * The conventions of vt.h hold here too: device pointers owned by the caller, no allocation or
 * synchronisation inside, host-side validation before any launch, errors as vt_status_t.
 */
#ifndef VT_KEEPSET_H_
#define VT_KEEPSET_H_

#include "vt.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * vt_token_histogram -- [VT] §3, Algorithm 1: a counter over the vocabulary, zero at the start,
 * incremented once for every token of the corpus.
 *
 *   tokens      int32 [n] token ids (4-byte aligned; 16-byte alignment takes the vector path).
 *               Ids outside [0, V) are not tokens of the vocabulary and are skipped.
 *   n           number of tokens, >= 0 (n = 0 writes zeros, or leaves counts as they are when
 *               accumulating)
 *   V           vocabulary size, 1 <= V < 2^31
 *   accumulate  0: counts = histogram of tokens; non-zero: counts += histogram (to count a
 *               corpus in parts).  Counts are uint32 and wrap modulo 2^32.
 *   counts      uint32 [V], written in full
 *   workspace   per-group partial counters; at least vt_token_histogram_workspace_bytes(n, V)
 *               bytes (0 for small n, when NULL is accepted)
 *   Results are exact integers and do not depend on the launch shape.
 *   Errors: INVALID_ARG for NULL tokens (n > 0) or counts, n < 0, V <= 0; UNSUPPORTED for
 *   V >= 2^31 or tokens not 4-byte aligned; WORKSPACE for a short workspace.
 */
size_t vt_token_histogram_workspace_bytes(int64_t n, int64_t V);
vt_status_t vt_token_histogram(const int32_t *tokens, int64_t n, int64_t V, int accumulate, uint32_t *counts,
                               void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Selection rules: [VT] §3 Eq. 1 names Top-K; the same section lists Top-P and a minimum
 * frequency as other criteria for the trimmed vocabulary. */
typedef enum {
  VT_SELECT_TOP_K = 0,    /* the k most frequent ids; ties broken by the lower id */
  VT_SELECT_TOP_P = 1,    /* the shortest prefix of that ranking whose summed count reaches
                             ceil(p * N), N = sum of counts, p * N evaluated in float64;
                             at least one id */
  VT_SELECT_MIN_FREQ = 2  /* every id whose count is >= min_count (possibly none) */
} vt_select_t;

/*
 * vt_keep_select -- the kept vocabulary from a counter, stored in ascending id order.
 *
 *   counts        uint32 [V] (for example from vt_token_histogram)
 *   rule          one of vt_select_t; k is read by TOP_K (1 <= k <= V), p by TOP_P (0 < p <= 1),
 *                 min_count by MIN_FREQ
 *   keep_ids      int32, capacity V: entries [0, K) receive the kept ids, ascending; entries
 *                 past K are left as they were
 *   full_to_trim  int32 [V], written in full: the position of id v in keep_ids, or -1
 *   num_kept      int32 [1]: K
 *   One workgroup does the whole selection (a radix descent over the 32-bit counts, then an
 *   ordered compaction); the sizes involved are a vocabulary, not a corpus.
 *   Errors: INVALID_ARG for NULL counts/keep_ids/full_to_trim/num_kept, V <= 0, an unknown rule,
 *   k outside [1, V] (TOP_K), p outside (0, 1] or NaN (TOP_P); UNSUPPORTED for V >= 2^31.
 */
vt_status_t vt_keep_select(const uint32_t *counts, int64_t V, vt_select_t rule, int64_t k, double p,
                           uint32_t min_count, int32_t *keep_ids, int32_t *full_to_trim, int32_t *num_kept,
                           hipStream_t stream);

/*
 * vt_trim_head -- [VT] §3 Eq. 1, second line: W^Trim = W[keep_ids, :], a contiguous copy of the
 * kept rows in keep_ids order (the layout vt_lmhead_trimmed reads with keep_ids = NULL).
 *
 *   weight    bf16 bit patterns, row-major [V_rows][H], 16-byte aligned
 *   keep_ids  int32 [k]; an id outside [0, V_rows) yields a zero row (nothing is read for it)
 *   trimmed   bf16 bit patterns, row-major [k][H], 16-byte aligned, written in full
 *   Errors: INVALID_ARG for NULL pointers, V_rows, H or k <= 0; UNSUPPORTED for H % 8 != 0, an
 *   unaligned base, or k, V_rows >= 2^31.
 */
vt_status_t vt_trim_head(const uint16_t *weight, int64_t V_rows, int64_t H, const int32_t *keep_ids, int64_t k,
                         uint16_t *trimmed, hipStream_t stream);

/*
 * vt_trim_head_tiled -- the same W^Trim ([VT] §3 Eq. 1, second line: the kept rows in keep_ids
 * order), stored K-tiled for the MFMA LM head of vt_spec_block: row j = 256 b + r,
 * columns 32 s .. 32 s + 31 sit at tiled[b][s][r][0 .. 31], so each 256-row, 32-column slice is
 * one contiguous 16 KB run.  [VT] §3 builds W^Trim once, from calibration counts, before any
 * decoding, so its storage layout is a free choice; this one is what the head's loads read fastest.
 *
 *   weight    bf16 bit patterns, row-major [V_rows][H], 16-byte aligned
 *   keep_ids  int32 [k], or NULL for rows 0 .. k-1 (then k <= V_rows); an id outside [0, V_rows)
 *             yields a zero row (nothing is read for it)
 *   tiled     bf16 bit patterns, [ceil(k / 256)][H / 32][256][32], 16-byte aligned, written in
 *             full (rows k .. 256 ceil(k / 256) - 1 are zeros): vt_trim_head_tiled_bytes(k, H) bytes
 *   Errors: INVALID_ARG for NULL weight/tiled, V_rows, H or k <= 0, k > V_rows without keep_ids;
 *   UNSUPPORTED for H % 32 != 0, an unaligned base, or k, V_rows >= 2^31.
 */
vt_status_t vt_trim_head_tiled(const uint16_t *weight, int64_t V_rows, int64_t H, const int32_t *keep_ids,
                               int64_t k, uint16_t *tiled, hipStream_t stream);

/* Bytes of the K-tiled W^Trim of k rows (0 when k or H <= 0 or H % 32 != 0). */
size_t vt_trim_head_tiled_bytes(int64_t k, int64_t H);

#ifdef __cplusplus
}
#endif

#endif /* VT_KEEPSET_H_ */

// One whole speculative block per call: trimmed LM head, draft softmax + draws, target softmax,
// verification -- the operations of vt_lmhead_trimmed, vt_softmax_temp (twice) and vt_spec_verify
// ("VocabTrim" §3 Eq. 1 and Appendix C.1 Algorithm 2; "Speculative decoding" glossary, "Why a
// rejection needs a special draw"; "A rejection rule keeps speculative decoding's output exact",
// "Extending the rule from one token to a drafted run"), launched as few kernels as the
// dependencies allow:
//   1. target rows' chunk partials (max, sum of exp)                       [if V > 4096]
//   2. LM head; on the GEMV path and on the MFMA paths with whole 32-column K steps its epilogue
//      also emits the draft rows' partials per row block or column tile (no second pass over the
//      logits); otherwise a partials launch follows
//   3. one combine launch for the draft rows (lse + draws) and the target rows (lse)
//   4. verify pass 1 (accept scans, residual chunk sums) and pass 2 (final draws, outputs)
// Launch order never lets an independent kernel sit between the LM head and its consumers.
// Small batches with both sides sampled and at most 8 draft rows per sequence replace 3 and 4
// with two launches: one chunk pass forms every log-normaliser, draft draw, accept scan and
// residual chunk sum from the partials, and the final pass draws the last token; on the GEMV path
// the target partials also ride in extra workgroups of the head launch (3 launches in all).
#include <algorithm>
#include <mutex>

#include "lmhead_impl.hpp"
#include "softmax_impl.hpp"
#include "verify_fused.hpp"
#include "verify_impl.hpp"

namespace vt {
namespace {

// Batches after whose MFMA head the two-pass verification runs: at most kFvMfmaMaxM hidden rows and
// 16 draft rows per sequence, and at most kFvMfmaMaxB sequences, counted twice when each chunk-pass
// wavefront draws two rows.  Each chunk workgroup of a sequence repeats the sequence's draft draws
// and target log-normalisers, which pays at a few sequences and not beyond (batched shape, H =
// 3072, Vt = 32768, 8 draft rows: 2 sequences 55.0 -> 49.6 us per block, 4: 56.3 -> 54.4 us, 8:
// 59.4 -> 66.8 us; large-drafter shape, 9 draft rows: 1 sequence 116.1 -> 112.6 us, 2: 116.0 ->
// 115.1 us, 3: 124.7 us against 120.5 us for 4 without it).
constexpr int64_t kFvMfmaMaxM = 32;
constexpr int64_t kFvMfmaMaxB = 4;

struct BlockPlan {
  bool fused;       // GEMV with draft partials in its epilogue
  bool fused_mfma;  // MFMA head with draft partials (softmax or argmax) in its epilogue
  bool fv;          // small batch, sampling both sides: target partials (in the GEMV launch, or a
                    // launch of their own before an MFMA head), then one chunk pass and one final
                    // pass (verify_fused_chunk / _final)
  bool fg;          // greedy both sides, at most 8 draft rows per sequence after the GEMV or 16
                    // after an MFMA head: argmax partials of the head blocks and of the target
                    // chunks (in extra workgroups of the GEMV launch, or a launch of their own
                    // before the MFMA head), then verify_greedy_small
  int64_t M, rows_t;
  int64_t nchunk_t;  // 4096-chunks of a target row
  int64_t nchunk_d;  // draft partial chunks per row (GEMV row blocks, MFMA column blocks, or 4096-chunks)
  int chunk_d;
  int64_t nchunk_v;
  size_t off_tpart, off_dpart, off_nbuf, off_vpart, off_wbuf, off_hidt, bytes;
  size_t hidt_bytes;  // K-tiled copy of the hidden rows for the MFMA head (0: none)
};

// greedy_t: the target is decoded greedily (no target softmax; verification compares argmaxes).
// greedy_d: the drafts are the draft rows' argmaxes (the LM head runs without softmax partials).
BlockPlan plan_block(int64_t B, int64_t gamma, int64_t R, int64_t H, int64_t Vt, int64_t V, bool trim,
                     bool greedy_t = false, bool greedy_d = false) {
  BlockPlan p{};
  p.M = B * R;
  p.rows_t = B * (gamma + 1);
  // past the GEMV sizes: the direct-to-LDS MFMA heads (and the register-staged one from kBigMinM
  // rows) emit the draft partials in their epilogue (softmax partials, or argmax partials for
  // argmax drafts); the head kernel is the one the separate call takes for the same M and H
  const bool mfma_ok = pick_gemv<kPartsNone>(p.M, H, trim) == nullptr && mfma_head_direct(p.M, H);
  p.fused = !greedy_d && pick_gemv<kPartsSoftmax>(p.M, H, trim) != nullptr;
  const bool fg_gemv = greedy_t && greedy_d && R <= kFvMaxR && pick_gemv<kPartsArgmax>(p.M, H, trim) != nullptr;
  p.fg = fg_gemv || (greedy_t && greedy_d && R <= kFvMaxR2 && mfma_ok);
  p.nchunk_t = greedy_t && !p.fg ? 1 : (V + kChunk - 1) / kChunk;
  p.fused_mfma = !p.fused && !fg_gemv && mfma_ok;
  if (p.fused || fg_gemv) {
    p.nchunk_d = gemv_blocks(Vt);
    p.chunk_d = gemv_rows_per_block(Vt);
  } else if (p.fused_mfma) {
    p.chunk_d = head_tile_cols(p.M, H, Vt);
    p.nchunk_d = (Vt + p.chunk_d - 1) / p.chunk_d;
  } else {
    p.nchunk_d = (Vt + kChunk - 1) / kChunk;
    p.chunk_d = kChunk;
  }
  // the two-pass verification (chunk pass + final pass) after the GEMV head, and after the MFMA
  // head for the small batches above
  const int64_t rows_per_wave = R > kFvMaxR ? 2 : 1;
  p.fv = !greedy_t && R <= kFvMaxR2 && p.nchunk_d <= kFvMaxParts &&
         (p.fused || (p.fused_mfma && p.M <= kFvMfmaMaxM && B * rows_per_wave <= kFvMfmaMaxB));
  p.nchunk_v = (V + (p.fv ? kFvIds : kChunk) - 1) / (p.fv ? kFvIds : kChunk);
  size_t off = 0;
  p.off_tpart = off;
  if (p.nchunk_t > 1 || p.fv || p.fg)
    off += align_up(static_cast<size_t>(p.rows_t * p.nchunk_t) * sizeof(float2), 256);
  p.off_dpart = off;
  if (p.fused || p.fused_mfma || p.fg || p.nchunk_d > 1)
    off += align_up(static_cast<size_t>(p.M * p.nchunk_d) * sizeof(float2), 256);
  p.off_nbuf = off;
  p.off_vpart = off;
  if (p.nchunk_v > 1 || p.fv) {
    off += align_up(static_cast<size_t>(B) * sizeof(int), 256);
    p.off_vpart = off;
    off += align_up(static_cast<size_t>(B * (gamma + 1) * p.nchunk_v) * sizeof(float2), 256);
  }
  p.off_wbuf = off;
  if (p.fv) off += align_up(static_cast<size_t>(2 * B * V) * sizeof(float), 256);  // final-draw weights and p_n
  p.off_hidt = off;
  p.hidt_bytes = p.fused_mfma ? hidden_tiles_bytes(p.M, H, Vt) : 0;
  off += align_up(p.hidt_bytes, 256);
  p.bytes = off;
  return p;
}

template <typename TinT, bool kVecT, bool kVecD>
hipError_t launch_combine(const SmParams &D, bool d_multi, const SmParams &T, bool t_multi, hipStream_t stream) {
  if (d_multi && t_multi)
    return launch(softmax_combine2<float, kVecD, TinT, kVecT>, dim3(static_cast<unsigned>(D.rows + T.rows)),
                  dim3(kBlock), 0, stream, D, T);
  if (d_multi)
    return launch(softmax_combine<float, kVecD>, dim3(static_cast<unsigned>(D.rows)), dim3(kBlock), 0, stream, D);
  if (t_multi)
    return launch(softmax_combine<TinT, kVecT>, dim3(static_cast<unsigned>(T.rows)), dim3(kBlock), 0, stream, T);
  return hipSuccess;
}

// The chunk pass and the final pass of the two-pass verification: every log-normaliser and draft
// draw is formed from the partials the earlier launches left (draft rows per head block, target
// rows per 4096-chunk), then the accept scan, the residual chunk sums and the last token.
template <typename TinT, bool kVecT>
hipError_t launch_fused_verify(const BlockPlan &pl, const SmParams &D, const SmParams &T, const VfParams &Vp,
                               const float *u_draft, float *wbuf, int64_t B, hipStream_t stream) {
  FvParams F{};
  F.v = Vp;
  F.dpart = D.part;
  F.nd = static_cast<int>(pl.nchunk_d);
  F.dper = pl.chunk_d;
  F.udraft = u_draft;
  F.tpart = T.part;
  F.nt = T.nchunk;
  F.dlse_out = D.lse;
  F.dids_out = D.sampled;
  F.tlse_out = T.lse;
  F.wbuf = wbuf;
  F.pbuf = wbuf + B * Vp.V;
  const dim3 grid(static_cast<unsigned>(B * Vp.nchunk));
  const hipError_t e = Vp.R > kFvMaxR ? launch(verify_fused_chunk<TinT, kVecT, 2>, grid, dim3(kFvBlock), 0, stream, F)
                                      : launch(verify_fused_chunk<TinT, kVecT, 1>, grid, dim3(kFvBlock), 0, stream, F);
  if (e != hipSuccess) return e;
  return launch(verify_fused_final<TinT, kVecT>, dim3(static_cast<unsigned>(B)), dim3(kBlock), 0, stream, F);
}

// Small batch, sampling both sides: 3 launches.  The GEMV launch carries the target rows'
// chunk partials in extra workgroups; the chunk pass forms every log-normaliser and draft draw
// itself from the partials; the final pass draws the last token.
template <typename TinT, bool kVecT>
hipError_t run_block_small(const BlockPlan &pl, const SmParams &D, const SmParams &T, const VfParams &Vp,
                           const uint16_t *hidden, const uint16_t *weight, const int32_t *keep, int64_t H,
                           int64_t Vt, float *logits, const float *u_draft, float *wbuf, int64_t B, hipEvent_t ev0,
                           hipEvent_t ev1, hipStream_t stream) {
  hipError_t e = hipSuccess;
  const int vrows = static_cast<int>(Vp.V);  // the head passed in is the full [V][H] one
  GemvParts gp{};
  gp.part = D.part;
  gp.k2 = D.k2;
  gp.tgt = T;
  gp.tsel = sizeof(TinT) == 4 ? (kVecT ? 1 : 2) : (kVecT ? 3 : 4);
  if (ev0 && (e = hipEventRecord(ev0, stream)) != hipSuccess) return e;
  e = launch_gemv(pick_gemv<kPartsSoftmax>(pl.M, H, keep != nullptr), hidden, weight, keep, vrows, H, Vt, logits, gp, stream,
                  T.rows * T.nchunk);
  if (e != hipSuccess) return e;
  if (ev1 && (e = hipEventRecord(ev1, stream)) != hipSuccess) return e;
  return launch_fused_verify<TinT, kVecT>(pl, D, T, Vp, u_draft, wbuf, B, stream);
}

// Small batch past the GEMV sizes, sampling both sides: 4 launches.  The target rows' chunk
// partials (with the K-tiled hidden copy in extra workgroups), the MFMA head with the draft
// partials, then the chunk pass and the final pass as after the GEMV head.
template <typename TinT, bool kVecT>
hipError_t run_block_small_mfma(const BlockPlan &pl, const SmParams &D, const SmParams &T, const VfParams &Vp,
                                const uint16_t *hidden, const uint16_t *weight, const int32_t *keep, int64_t H,
                                int64_t Vt, float *logits, const float *u_draft, float *wbuf, int64_t B,
                                hipEvent_t ev0, hipEvent_t ev1, hipStream_t stream, void *hidt_base,
                                const uint16_t *weight_tiled) {
  hipError_t e = hipSuccess;
  const int vrows = static_cast<int>(Vp.V);  // the head passed in is the full [V][H] one
  uint16_t *hidt = pl.hidt_bytes ? reinterpret_cast<uint16_t *>(hidt_base) : nullptr;
  const TileParams tp = hidden_tiles_params(hidden, pl.M, H, Vt, hidt);
  if (hidt)
    e = launch(softmax_partial_tiles<TinT, kVecT>,
               dim3(static_cast<unsigned>(T.rows * T.nchunk + hidden_tiles_blocks(tp))), dim3(kBlock), 0, stream, T,
               tp);
  else
    e = launch(softmax_partial<TinT, kVecT>, dim3(static_cast<unsigned>(T.rows * T.nchunk)), dim3(kBlock), 0,
               stream, T);
  if (e != hipSuccess) return e;
  if (ev0 && (e = hipEventRecord(ev0, stream)) != hipSuccess) return e;
  e = launch_mfma_head<kPartsSoftmax>(hidden, weight, keep, vrows, pl.M, H, Vt, logits, GemvParts{D.part, D.k2}, stream,
                                      hidt, weight_tiled);
  if (e != hipSuccess) return e;
  if (ev1 && (e = hipEventRecord(ev1, stream)) != hipSuccess) return e;
  return launch_fused_verify<TinT, kVecT>(pl, D, T, Vp, u_draft, wbuf, B, stream);
}

// The greedy compare pass: one workgroup per sequence reduces the argmax partials of the draft
// rows (per head block) and of the target rows (per 4096-chunk), compares and writes the outputs.
inline hipError_t launch_greedy_verify(const BlockPlan &pl, const SmParams &D, const SmParams &T, const VfParams &Vp,
                                       int64_t B, hipStream_t stream) {
  FvParams F{};
  F.v = Vp;
  F.dpart = D.part;
  F.nd = static_cast<int>(pl.nchunk_d);
  F.dper = pl.chunk_d;
  F.tpart = T.part;
  F.nt = T.nchunk;
  F.dlse_out = D.lse;
  F.dids_out = D.sampled;
  return launch(verify_greedy_small, dim3(static_cast<unsigned>(B)), dim3(kFvBlock), 0, stream, F);
}

// Greedy both sides past the GEMV sizes: 3 launches.  The target rows' per-chunk argmaxes (with
// the K-tiled hidden copy in extra workgroups), the MFMA head with the draft rows' argmax
// partials, and the compare pass.
template <typename TinT, bool kVecT>
hipError_t run_block_greedy_small_mfma(const BlockPlan &pl, const SmParams &D, const SmParams &T,
                                       const VfParams &Vp, const uint16_t *hidden, const uint16_t *weight,
                                       const int32_t *keep, int64_t H, int64_t Vt, float *logits, int64_t B,
                                       hipEvent_t ev0, hipEvent_t ev1, hipStream_t stream, void *hidt_base,
                                       const uint16_t *weight_tiled) {
  hipError_t e = hipSuccess;
  const int vrows = static_cast<int>(Vp.V);  // the head passed in is the full [V][H] one
  uint16_t *hidt = pl.hidt_bytes ? reinterpret_cast<uint16_t *>(hidt_base) : nullptr;
  const TileParams tp = hidden_tiles_params(hidden, pl.M, H, Vt, hidt);
  if (hidt)
    e = launch(softmax_partial_tiles<TinT, kVecT>,
               dim3(static_cast<unsigned>(T.rows * T.nchunk + hidden_tiles_blocks(tp))), dim3(kBlock), 0, stream, T,
               tp);
  else
    e = launch(softmax_partial<TinT, kVecT>, dim3(static_cast<unsigned>(T.rows * T.nchunk)), dim3(kBlock), 0,
               stream, T);
  if (e != hipSuccess) return e;
  if (ev0 && (e = hipEventRecord(ev0, stream)) != hipSuccess) return e;
  e = launch_mfma_head<kPartsArgmax>(hidden, weight, keep, vrows, pl.M, H, Vt, logits, GemvParts{D.part, D.k2}, stream,
                                     hidt, weight_tiled);
  if (e != hipSuccess) return e;
  if (ev1 && (e = hipEventRecord(ev1, stream)) != hipSuccess) return e;
  return launch_greedy_verify(pl, D, T, Vp, B, stream);
}

// Small batch, greedy both sides: 2 launches.  The GEMV launch leaves per-block argmax partials
// of the draft rows and, in extra workgroups, per-chunk argmaxes of the target rows; one
// workgroup per sequence reduces, compares and writes the outputs.
template <typename TinT, bool kVecT>
hipError_t run_block_greedy_small(const BlockPlan &pl, const SmParams &D, const SmParams &T, const VfParams &Vp,
                                  const uint16_t *hidden, const uint16_t *weight, const int32_t *keep, int64_t H,
                                  int64_t Vt, float *logits, int64_t B, hipEvent_t ev0, hipEvent_t ev1,
                                  hipStream_t stream) {
  hipError_t e = hipSuccess;
  const int vrows = static_cast<int>(Vp.V);  // the head passed in is the full [V][H] one
  GemvParts gp{};
  gp.part = D.part;
  gp.tgt = T;
  gp.tsel = sizeof(TinT) == 4 ? (kVecT ? 1 : 2) : (kVecT ? 3 : 4);
  if (ev0 && (e = hipEventRecord(ev0, stream)) != hipSuccess) return e;
  e = launch_gemv(pick_gemv<kPartsArgmax>(pl.M, H, keep != nullptr), hidden, weight, keep, vrows, H, Vt, logits, gp, stream,
                  T.rows * T.nchunk);
  if (e != hipSuccess) return e;
  if (ev1 && (e = hipEventRecord(ev1, stream)) != hipSuccess) return e;
  return launch_greedy_verify(pl, D, T, Vp, B, stream);
}

template <typename TinT, bool kVecT, bool kVecD>
hipError_t run_block(const BlockPlan &pl, const SmParams &D, const SmParams &T, const VfParams &Vp,
                     const uint16_t *hidden, const uint16_t *weight, const int32_t *keep, int64_t H, int64_t Vt,
                     float *logits, float *wbuf, int64_t B, hipEvent_t ev0, hipEvent_t ev1, hipStream_t stream,
                     void *hidt_base, const uint16_t *weight_tiled) {
  if (pl.fv && pl.fused)
    return run_block_small<TinT, kVecT>(pl, D, T, Vp, hidden, weight, keep, H, Vt, logits, D.u, wbuf, B, ev0, ev1,
                                        stream);
  if (pl.fv)
    return run_block_small_mfma<TinT, kVecT>(pl, D, T, Vp, hidden, weight, keep, H, Vt, logits, D.u, wbuf, B, ev0,
                                             ev1, stream, hidt_base, weight_tiled);
  if (pl.fg && pl.fused_mfma)
    return run_block_greedy_small_mfma<TinT, kVecT>(pl, D, T, Vp, hidden, weight, keep, H, Vt, logits, B, ev0, ev1,
                                                    stream, hidt_base, weight_tiled);
  if (pl.fg)
    return run_block_greedy_small<TinT, kVecT>(pl, D, T, Vp, hidden, weight, keep, H, Vt, logits, B, ev0, ev1, stream);
  hipError_t e = hipSuccess;
  const int vrows = static_cast<int>(Vp.V);  // the head passed in is the full [V][H] one
  const bool greedy_t = Vp.greedy;
  const bool t_multi = !greedy_t && pl.nchunk_t > 1;
  // the MFMA head reads the hidden rows K-tiled (one contiguous run per K step of a block of
  // hidden rows); the copy rides in extra workgroups of the target partials launch when there is one
  uint16_t *hidt = pl.hidt_bytes ? reinterpret_cast<uint16_t *>(hidt_base) : nullptr;
  const TileParams tp = hidden_tiles_params(hidden, pl.M, H, Vt, hidt);
  // 1. target partials (or a whole single-chunk target softmax); greedy verification needs none
  if (t_multi && hidt)
    e = launch(softmax_partial_tiles<TinT, kVecT>,
               dim3(static_cast<unsigned>(T.rows * T.nchunk + hidden_tiles_blocks(tp))), dim3(kBlock), 0, stream, T,
               tp);
  else if (t_multi)
    e = launch(softmax_partial<TinT, kVecT>, dim3(static_cast<unsigned>(T.rows * T.nchunk)), dim3(kBlock), 0,
               stream, T);
  else if (!greedy_t)
    e = launch(softmax_single<TinT, kVecT>, dim3(static_cast<unsigned>(T.rows)), dim3(kBlock), 0, stream, T);
  if (e != hipSuccess) return e;
  if (hidt && !t_multi &&
      (e = launch(hidden_tiles, dim3(static_cast<unsigned>(hidden_tiles_blocks(tp))), dim3(kBlock), 0, stream, tp)) !=
          hipSuccess)
    return e;
  // 2. LM head (+ draft partials), bracketed by the caller's timing events if any
  if (ev0 && (e = hipEventRecord(ev0, stream)) != hipSuccess) return e;
  bool d_multi = true;
  if (pl.fused) {
    const GemvFn fn = pick_gemv<kPartsSoftmax>(pl.M, H, keep != nullptr);
    e = launch_gemv(fn, hidden, weight, keep, vrows, H, Vt, logits, GemvParts{D.part, D.k2}, stream);
    if (e != hipSuccess) return e;
    if (ev1 && (e = hipEventRecord(ev1, stream)) != hipSuccess) return e;
  } else if (pl.fused_mfma) {
    e = D.greedy ? launch_mfma_head<kPartsArgmax>(hidden, weight, keep, vrows, pl.M, H, Vt, logits,
                                                  GemvParts{D.part, D.k2}, stream, hidt, weight_tiled)
                 : launch_mfma_head<kPartsSoftmax>(hidden, weight, keep, vrows, pl.M, H, Vt, logits,
                                                   GemvParts{D.part, D.k2}, stream, hidt, weight_tiled);
    if (e != hipSuccess) return e;
    if (ev1 && (e = hipEventRecord(ev1, stream)) != hipSuccess) return e;
  } else {
    const GemvFn plain = pick_gemv<kPartsNone>(pl.M, H, keep != nullptr);
    e = plain ? launch_gemv(plain, hidden, weight, keep, vrows, H, Vt, logits, GemvParts{}, stream)
              : launch_mfma(hidden, weight, keep, vrows, pl.M, H, Vt, logits, stream);
    if (e != hipSuccess) return e;
    if (ev1 && (e = hipEventRecord(ev1, stream)) != hipSuccess) return e;
    if (pl.nchunk_d > 1) {
      e = launch(softmax_partial<float, kVecD>, dim3(static_cast<unsigned>(D.rows * D.nchunk)), dim3(kBlock), 0,
                 stream, D);
    } else {
      d_multi = false;
      e = launch(softmax_single<float, kVecD>, dim3(static_cast<unsigned>(D.rows)), dim3(kBlock), 0, stream, D);
    }
    if (e != hipSuccess) return e;
  }
  // 3. one combine launch for both row sets
  e = launch_combine<TinT, kVecT, kVecD>(D, d_multi, T, t_multi, stream);
  if (e != hipSuccess) return e;
  // 4. verification
  return vf_launch_all<TinT, kVecT>(Vp, B, stream);
}

}  // namespace
}  // namespace vt

extern "C" size_t vt_spec_block_workspace_bytes(int64_t B, int64_t gamma, int64_t R, int64_t H, int64_t Vt,
                                                int64_t V) {
  if (B <= 0 || gamma <= 0 || R < gamma || H <= 0 || Vt <= 0 || V < Vt) return 0;
  // enough for every temperature mode
  size_t bytes = 0;
  for (int mode = 0; mode < 3; ++mode)
    bytes = std::max(bytes, vt::plan_block(B, gamma, R, H, Vt, V, Vt < V, mode >= 1, mode == 2).bytes);
  return bytes;
}

extern "C" vt_status_t vt_spec_block(const uint16_t *hidden, const uint16_t *weight, const uint16_t *weight_tiled,
                                     const int32_t *keep_ids,
                                     const int32_t *full_to_trim, int64_t B, int64_t gamma, int64_t R, int64_t H,
                                     int64_t Vt, int64_t V, const void *target_logits, vt_dtype_t target_dtype,
                                     float target_T, float draft_T, const float *u_draft, const float *u_accept,
                                     const float *u_final, float *draft_logits, double *draft_lse, int32_t *draft_ids,
                                     double *target_lse, int32_t *out_tokens, int32_t *out_num_accepted,
                                     hipEvent_t lmhead_begin, hipEvent_t lmhead_end, void *workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  using namespace vt;
  const bool greedy_t = target_T == 0.f, greedy_d = draft_T == 0.f;
  if (!hidden || !weight || !target_logits || !draft_logits || !draft_lse || !draft_ids || !out_tokens ||
      !out_num_accepted)
    return VT_ERR_INVALID_ARG;
  if (!greedy_d && !u_draft) return VT_ERR_INVALID_ARG;
  if (!greedy_t && (!u_accept || !u_final || !target_lse)) return VT_ERR_INVALID_ARG;
  if (target_dtype != VT_F32 && target_dtype != VT_BF16) return VT_ERR_INVALID_ARG;
  if (B <= 0 || gamma <= 0 || R < gamma || H <= 0 || Vt <= 0 || V <= 0 || Vt > V) return VT_ERR_INVALID_ARG;
  if (!greedy_t && !finite_positive(target_T)) return VT_ERR_INVALID_ARG;
  if (!greedy_d && !finite_positive(draft_T)) return VT_ERR_INVALID_ARG;
  if (greedy_d && !greedy_t) return VT_ERR_INVALID_ARG;  // sampling verification needs a draft distribution
  if ((keep_ids == nullptr) != (full_to_trim == nullptr)) return VT_ERR_INVALID_ARG;
  if (!keep_ids && Vt != V) return VT_ERR_INVALID_ARG;
  if (gamma > kWave) return VT_ERR_UNSUPPORTED;
  if (H % 8 != 0 || !aligned16(hidden) || !aligned16(weight)) return VT_ERR_UNSUPPORTED;
  if (weight_tiled && (H % kTileK != 0 || !aligned16(weight_tiled))) return VT_ERR_UNSUPPORTED;
  if (V > INT32_MAX || H > INT32_MAX || B * R > INT32_MAX) return VT_ERR_UNSUPPORTED;
  const BlockPlan pl = plan_block(B, gamma, R, H, Vt, V, keep_ids != nullptr, greedy_t, greedy_d);
  if (pl.rows_t * pl.nchunk_t + static_cast<int64_t>(pl.hidt_bytes / (16 * kBlock)) + 1 >
          static_cast<int64_t>(UINT32_MAX) ||
      pl.M * pl.nchunk_d > static_cast<int64_t>(UINT32_MAX) || B * pl.nchunk_v > static_cast<int64_t>(UINT32_MAX))
    return VT_ERR_UNSUPPORTED;
  if (!pl.fused && ((pl.M + kBM - 1) / kBM) * ((Vt + kBN - 1) / kBN) > INT32_MAX) return VT_ERR_UNSUPPORTED;
  if (pl.bytes > 0 && (!workspace || workspace_bytes < pl.bytes)) return VT_ERR_WORKSPACE;
  char *ws = static_cast<char *>(workspace);

  const double log2e = 1.4426950408889634;
  SmParams D{};
  D.logits = draft_logits;
  D.rows = pl.M;
  D.n = Vt;
  D.ld = Vt;
  D.greedy = greedy_d;
  D.T = greedy_d ? 1.0 : draft_T;
  D.invT = 1.0 / D.T;
  D.k2 = greedy_d ? 0.f : static_cast<float>(log2e / static_cast<double>(draft_T));
  D.lse = draft_lse;
  D.u = greedy_d ? nullptr : u_draft;
  D.sampled = draft_ids;
  D.nchunk = static_cast<int>(pl.nchunk_d);
  D.chunk = pl.chunk_d;
  if (pl.fused || pl.fused_mfma || pl.fg || pl.nchunk_d > 1) D.part = reinterpret_cast<float2 *>(ws + pl.off_dpart);

  SmParams T{};
  T.logits = target_logits;
  T.rows = pl.rows_t;
  T.n = V;
  T.ld = V;
  T.T = greedy_t ? 1.0 : target_T;
  T.invT = 1.0 / T.T;
  T.k2 = greedy_t ? 0.f : static_cast<float>(log2e / static_cast<double>(target_T));
  T.lse = target_lse;
  T.nchunk = static_cast<int>(pl.nchunk_t);
  T.chunk = kChunk;
  if ((!greedy_t && (pl.nchunk_t > 1 || pl.fv)) || pl.fg) T.part = reinterpret_cast<float2 *>(ws + pl.off_tpart);
  T.greedy = greedy_t;

  VfParams P{};
  P.target = target_logits;
  P.tlse = target_lse;
  P.draft = draft_logits;
  P.dlse = draft_lse;
  P.ids = draft_ids;
  P.keep = keep_ids;
  P.f2t = full_to_trim;
  P.uacc = u_accept;
  P.ufin = u_final;
  P.out_tokens = out_tokens;
  P.out_n = out_num_accepted;
  P.V = V;
  P.Vt = Vt;
  P.R = R;
  P.greedy = greedy_t;
  P.Tt = greedy_t ? 1.0 : target_T;
  P.Td = greedy_d ? 1.0 : draft_T;
  P.invTt = 1.0 / P.Tt;
  P.invTd = 1.0 / P.Td;
  P.k2t = T.k2;
  P.k2d = D.k2;
  P.gamma = static_cast<int>(gamma);
  P.nchunk = static_cast<int>(pl.nchunk_v);
  if (pl.nchunk_v > 1 || pl.fv) {
    P.nbuf = reinterpret_cast<int *>(ws + pl.off_nbuf);
    P.part = reinterpret_cast<float2 *>(ws + pl.off_vpart);
  }

  const int64_t vec_elems = target_dtype == VT_F32 ? 4 : 8;
  const bool vt_ = aligned16(target_logits) && V % vec_elems == 0;
  const bool vd = aligned16(draft_logits) && Vt % 4 == 0 && pl.chunk_d % 4 == 0;
  auto go = [&](auto run) {
    return run(pl, D, T, P, hidden, weight, keep_ids, H, Vt, draft_logits,
               pl.fv ? reinterpret_cast<float *>(ws + pl.off_wbuf) : nullptr, B, lmhead_begin, lmhead_end, stream,
               pl.hidt_bytes ? static_cast<void *>(ws + pl.off_hidt) : nullptr, weight_tiled);
  };
  hipError_t e;
  if (target_dtype == VT_F32) {
    if (vt_)
      e = vd ? go(run_block<float, true, true>) : go(run_block<float, true, false>);
    else
      e = vd ? go(run_block<float, false, true>) : go(run_block<float, false, false>);
  } else {
    if (vt_)
      e = vd ? go(run_block<uint16_t, true, true>) : go(run_block<uint16_t, true, false>);
    else
      e = vd ? go(run_block<uint16_t, false, true>) : go(run_block<uint16_t, false, false>);
  }
  return hip_status(e);
}

// ------------------------------------------------------------------ variant without a workspace
// For callers that cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc): vt_spec_block with its workspace in a fixed device
// array of this file.  Each device the library runs on holds its own copy until the process ends.
// The array's host-side name is only a stand-in for the symbol: its device address is looked up
// once per device (hipGetSymbolAddress, with that device current) and only that address is
// handed to kernels.  Nothing in the workspace has to start at zero: every launch of a call
// writes the partials it reads later in the same call.
namespace vt {
namespace {
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;  // 64 MiB per device
constexpr int kMaxDevices = 64;
}  // namespace
}  // namespace vt

static __device__ __align__(256) char scratch[vt::kNoAllocScratchBytes];

namespace vt {
namespace {
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first call per device).
vt_status_t scratch_on_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return VT_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return VT_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return VT_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return VT_OK;
}
}  // namespace
}  // namespace vt

extern "C" vt_status_t vt_spec_block_noalloc(const uint16_t *hidden, const uint16_t *weight,
                                             const uint16_t *weight_tiled, const int32_t *keep_ids,
                                             const int32_t *full_to_trim, int64_t B, int64_t gamma, int64_t R,
                                             int64_t H, int64_t Vt, int64_t V, const void *target_logits,
                                             vt_dtype_t target_dtype, float target_T, float draft_T,
                                             const float *u_draft, const float *u_accept, const float *u_final,
                                             float *draft_logits, double *draft_lse, int32_t *draft_ids,
                                             double *target_lse, int32_t *out_tokens, int32_t *out_num_accepted,
                                             hipEvent_t lmhead_begin, hipEvent_t lmhead_end, hipStream_t stream) {
  void *ws = nullptr;
  const vt_status_t st = vt::scratch_on_current_device(&ws);
  if (st != VT_OK) return st;
  // vt_spec_block validates every argument and returns VT_ERR_WORKSPACE when the shape needs more
  // than the fixed scratch holds
  return vt_spec_block(hidden, weight, weight_tiled, keep_ids, full_to_trim, B, gamma, R, H, Vt, V, target_logits,
                       target_dtype, target_T, draft_T, u_draft, u_accept, u_final, draft_logits, draft_lse, draft_ids,
                       target_lse, out_tokens, out_num_accepted, lmhead_begin, lmhead_end, ws,
                       vt::kNoAllocScratchBytes, stream);
}

// Verification of small batches in the single-call block, after the GEMV head or a small MFMA
// head (gfx950).
//
// What is computed is what the separate softmax and verify calls compute ("Speculative
// decoding" glossary, "Propose a block, keep a prefix" and "Why a rejection needs a special
// draw"; "A rejection rule keeps speculative decoding's output exact", "What the accept/reject
// rule has to balance" and "Extending the rule from one token to a drafted run"; "VocabTrim",
// Appendix C.1, Algorithm 2 for the trimmed-to-full map).  Only the work layout differs: at
// batch 1 each of those steps is a short, latency-bound launch, so here they are folded into two.
//
// Chunk pass: one 512-thread workgroup per (sequence b, 1024 ids x of the full vocabulary).
//   0. Issue every load that needs nothing computed first: the workgroup's slice of every target
//      row and (through full_to_trim) of every draft row, and the softmax partials that the head
//      launch left behind (per head row block for the draft rows, per 4096-chunk for the target
//      rows).
//   1. Wave w draws draft row w (log-normaliser from the partials, the block whose running mass
//      reaches u Z, then a scan of that block's logits and keep ids), and row w + 8 as well when a
//      sequence has more than 8 draft rows, forms the log-normaliser of target rows w, w + 8
//      (and w + 16), and runs the accept tests of its drafts (fp64 ratio).  Every
//      workgroup of the sequence repeats this small amount of work, so no workgroup waits for
//      another; the first chunk's workgroup writes the outputs.
//   2. After one barrier every thread reads the verdicts: n = first rejection.
//   3. From the registers loaded in step 0: the chunk sums of w(x) = max(0, p_n(x) - q_n(x))
//      (p_gamma when every draft was kept) and of p_n(x).
// Final pass: one workgroup per sequence locates the 1024-id chunk where the running residual
// mass reaches u_final times its total and rescans it (the shared final-draw code of the verify
// call, at 4 ids per thread).
// Greedy blocks (both temperatures 0) need no chunk pass: verify_greedy_small reduces the argmax
// partials of the head launch and compares.
#pragma once
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "softmax_impl.hpp"
#include "verify_impl.hpp"

namespace vt {
namespace {

constexpr int kFvBlock = 512;
constexpr int kFvWaves = kFvBlock / kWave;      // 8: one draft row per wavefront
constexpr int kFvIds = 1024;                    // full-vocabulary ids per chunk workgroup
constexpr int kFvPer = kFvIds / kFvBlock;       // 2 ids per thread
constexpr int kFvMaxR = 8;                      // draft rows per sequence at one per wavefront
constexpr int kFvMaxT = kFvMaxR + 1;            // target rows per sequence
constexpr int kFvMaxR2 = 2 * kFvMaxR;           // draft rows per sequence at two per wavefront
constexpr int kFvFinalPer = kFvIds / kBlock;    // 4 ids per thread in the final rescan
constexpr int kFvMaxParts = 4 * kWave;          // head row blocks per row (gemv_blocks <= 256)
constexpr int kFvScanBatch = 8;                 // 64-logit groups loaded at once when rescanning a row block

static_assert(kFvWaves == kFvMaxR, "one wavefront per draft row");

struct FvParams {
  VfParams v;            // verification view: target, draft logits, keep set, uniforms, outputs
  const float2 *dpart;   // [B * R][nd] per head row block: (max, sum of exp), or (max, argmax) if greedy
  int nd, dper;          // row blocks per draft row, head rows per block
  const float *udraft;   // [B * R]
  const float2 *tpart;   // [B * (gamma + 1)][nt] per 4096-chunk: (max, sum of exp), or (max, argmax)
  int nt;
  double *dlse_out;      // [B * R]
  int32_t *dids_out;     // [B * R]
  double *tlse_out;      // [B * (gamma + 1)]
  float *wbuf, *pbuf;    // [B][V]: the chunk pass's final-draw weights and p_n, for the final pass
};

// Raw bits of two consecutive elements [e0, e0 + 2) of a row (even e0), loaded unconditionally
// at an index clamped into the row.  Nothing here looks at the loaded values: a select on them
// would make the compiler wait for each load on the spot, so the caller masks entries past the
// row end where it uses them.  kVec: the row start is 16-byte aligned and n a multiple of 4, so
// the pair is one aligned load.
template <typename Tin>
struct RawPair {
  typename std::conditional<sizeof(Tin) == 4, float2, uint32_t>::type v;
};

template <typename Tin, bool kVec>
__device__ __forceinline__ RawPair<Tin> load_pair_raw(const Tin *__restrict__ row, int64_t n, int64_t e0) {
  RawPair<Tin> r;
  if constexpr (sizeof(Tin) == 4) {
    if constexpr (kVec) {
      r.v = *reinterpret_cast<const float2 *>(reinterpret_cast<const float *>(row) + (e0 < n ? e0 : n - 2));
    } else {
      const float *f = reinterpret_cast<const float *>(row);
      r.v.x = f[e0 < n ? e0 : n - 1];
      r.v.y = f[e0 + 1 < n ? e0 + 1 : n - 1];
    }
  } else {
    if constexpr (kVec) {
      r.v = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint16_t *>(row) + (e0 < n ? e0 : n - 2));
    } else {
      const uint16_t *h = reinterpret_cast<const uint16_t *>(row);
      r.v = static_cast<uint32_t>(h[e0 < n ? e0 : n - 1]) | (static_cast<uint32_t>(h[e0 + 1 < n ? e0 + 1 : n - 1]) << 16);
    }
  }
  return r;
}

template <typename Tin>
__device__ __forceinline__ float pair_elem(const RawPair<Tin> &r, int j) {
  if constexpr (sizeof(Tin) == 4)
    return j ? r.v.y : r.v.x;
  else
    return __uint_as_float(j ? (r.v & 0xffff0000u) : (r.v << 16));
}

// Draft row m, one wavefront: lse = M / T + ln Z from the head's per-block partials; the draw
// t = u Z walks the block-level running sum to the first block reaching t, then that block's
// logits.  Lane l holds blocks 4l .. 4l+3 (pv, loaded by the caller) and, in the rescan, logits
// 8l .. 8l+7 of each 512-logit batch: a lane-local running sum plus one wavefront scan per level.
// Returns the drawn trimmed index x (-1 if nothing carries weight), its logit and its full id
// keep[x] (x itself without a keep set).
struct DraftDraw {
  double lse;
  int x;
  int64_t y;
  float xl;
};

__device__ __forceinline__ DraftDraw fv_draft_row(const FvParams &F, int64_t m, const float2 (&pv)[4], float u) {
  const int lane = lane_id();
  const float k2 = F.v.k2d;
  float px[4];  // block maxima, -inf past the last block
#pragma unroll
  for (int j = 0; j < 4; ++j) px[j] = 4 * lane + j < F.nd ? pv[j].x : kNegInf;
  float mx = fmaxf(fmaxf(px[0], px[1]), fmaxf(px[2], px[3]));
  const float M = wave_max(mx);
  float mass[4], lp[4];  // this lane's block masses and their running sum
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    mass[j] = px[j] == kNegInf ? 0.f : pv[j].y * exp2_fast((px[j] - M) * k2);
    acc += mass[j];
    lp[j] = acc;
  }
  const float inc = wave_scan_incl(acc);
  const float excl = wave_prev(inc, 0.f);
  const float Z = lane_value(inc, kWave - 1);
  const float t = u * Z;
  // first block k = 4 lane + j with t <= excl + lp[j]
  int jf = 4;
#pragma unroll
  for (int j = 3; j >= 0; --j)
    if (4 * lane + j < F.nd && t <= excl + lp[j]) jf = j;
  const unsigned long long hit = __ballot(jf < 4);
  int ks;
  float E = 0.f;
  bool fallback = false;
  if (hit) {
    const int l = __ffsll(static_cast<long long>(hit)) - 1;
    float before = excl;
#pragma unroll
    for (int j = 1; j < 4; ++j)
      if (jf == j) before = excl + lp[j - 1];
    ks = 4 * l + lane_value(jf, l);
    E = lane_value(before, l);
  } else {
    // t beyond the running sum (u >= 1 or NaN): the last block with positive mass
    int last = -1;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (4 * lane + j < F.nd && mass[j] > 0.f) last = 4 * lane + j;
    ks = max(wave_max_int(last), 0);
    fallback = true;
  }
  // rescan block ks: first logit whose running weight reaches t, else the last positive one
  const float *row = F.v.draft + m * F.v.Vt;
  const int64_t r0 = static_cast<int64_t>(ks) * F.dper;
  const int64_t r1 = r0 + F.dper < F.v.Vt ? r0 + F.dper : F.v.Vt;
  const float te = fallback ? __builtin_huge_valf() : t;
  float run = fallback ? 0.f : E;
  DraftDraw d{};
  d.lse = static_cast<double>(M) * F.v.invTd + log(static_cast<double>(Z));
  d.x = -1;
  d.xl = kNegInf;
  int lastpos = -1;
  for (int64_t g0 = r0; g0 < r1 && d.x < 0; g0 += kWave * kFvScanBatch) {
    const int64_t e0 = g0 + kFvScanBatch * lane;
    float vals[kFvScanBatch];
    int32_t ids[kFvScanBatch];
#pragma unroll
    for (int q = 0; q < kFvScanBatch; ++q) {
      const int64_t e = e0 + q < r1 ? e0 + q : r1 - 1;  // clamped: unconditional loads
      vals[q] = row[e];
      ids[q] = F.v.keep ? F.v.keep[e] : static_cast<int32_t>(e);
      if (e0 + q >= r1) vals[q] = kNegInf;
    }
    float loc[kFvScanBatch];
    float a = 0.f;
#pragma unroll
    for (int q = 0; q < kFvScanBatch; ++q) {
      const float wgt = M == kNegInf ? 0.f : exp2_fast((vals[q] - M) * k2);
      if (e0 + q < r1 && wgt > 0.f) lastpos = static_cast<int>(e0 + q);
      a += wgt;
      loc[q] = a;
    }
    const float binc = wave_scan_incl(a);
    const float base = run + wave_prev(binc, 0.f);
    int qf = kFvScanBatch;
#pragma unroll
    for (int q = kFvScanBatch - 1; q >= 0; --q)
      if (e0 + q < r1 && te <= base + loc[q]) qf = q;
    const unsigned long long bh = __ballot(qf < kFvScanBatch);
    if (bh) {
      const int l = __ffsll(static_cast<long long>(bh)) - 1;
      float v = vals[0];
      int32_t id = ids[0];
#pragma unroll
      for (int q = 1; q < kFvScanBatch; ++q)
        if (qf == q) {
          v = vals[q];
          id = ids[q];
        }
      const int ql = lane_value(qf, l);
      d.x = static_cast<int>(g0 + kFvScanBatch * l + ql);
      d.xl = lane_value(v, l);
      d.y = lane_value(id, l);
    }
    run = run + lane_value(binc, kWave - 1);
  }
  if (d.x < 0) {
    d.x = wave_max_int(lastpos);
    if (d.x >= 0) {
      d.xl = row[d.x];
      d.y = F.v.keep ? F.v.keep[d.x] : d.x;
    }
  }
  return d;
}

// Log-normaliser of target row r from its 4096-chunk partials, one wavefront, with exactly the
// operations (and so the bits) of the combine pass of the separate softmax call: chunk masses
// scanned 64 at a time, four scans to a 256-chunk pass added in order, passes carried (a group
// past the last chunk adds +0 there, so it is skipped here).  p0: the row's first 64 partials,
// loaded by the caller (lanes past the last chunk hold a repeated entry and are masked here).
__device__ __forceinline__ double fv_target_lse(const FvParams &F, int64_t r, float2 p0) {
  const int lane = lane_id();
  const float2 *pp = F.tpart + r * F.nt;
  if (lane >= F.nt) p0 = make_float2(kNegInf, 0.f);
  float mx = p0.x;
  for (int k0 = kWave; k0 < F.nt; k0 += kWave) {
    const int k = k0 + lane;
    const float2 ps = pp[k < F.nt ? k : F.nt - 1];
    if (k < F.nt) mx = fmaxf(mx, ps.x);
  }
  const float M = wave_max(mx);
  auto mass = [&](float2 ps, int k) -> float {
    return (k < F.nt && ps.x != kNegInf) ? ps.y * exp2_fast((ps.x - M) * F.v.k2t) : 0.f;
  };
  // first 64 chunks from p0 (no load on this path: a load here would wait for every load in flight)
  float total = 0.f;
  total += lane_value(wave_scan_incl(mass(p0, lane)), kWave - 1);
  float carry = 0.f;
  for (int k0 = 0; k0 < F.nt; k0 += kBlock) {
    if (k0 > 0) total = 0.f;
    for (int q = k0 == 0 ? 1 : 0; q < kWavesPerBlock; ++q) {
      if (k0 + kWave * q >= F.nt) break;
      const int k = k0 + kWave * q + lane;
      total += lane_value(wave_scan_incl(mass(pp[k < F.nt ? k : F.nt - 1], k)), kWave - 1);
    }
    carry = carry + total;
  }
  return static_cast<double>(M) * F.v.invTt + log(static_cast<double>(carry));
}

// RPW draft rows per wavefront (wave w: rows w + 8 r, r < RPW; target rows w + 8 s): RPW = 1 up to
// 8 draft rows per sequence, 2 up to kFvMaxR2 (the second draw of a wave runs after its first).
template <typename Tin, bool kVec, int RPW>
__global__ __launch_bounds__(kFvBlock) void verify_fused_chunk(FvParams F) {
  constexpr int kMaxR = kFvWaves * RPW;  // draft rows per sequence
  constexpr int kMaxT = kMaxR + 1;       // target rows per sequence
  constexpr int kTPW = (kMaxT + kFvWaves - 1) / kFvWaves;  // target rows per wavefront
  __shared__ double s_tlse[kMaxT], s_dlse[kMaxR];
  __shared__ int s_acc[kMaxR];  // accept test of draft i: 1 kept, 0 rejected, -1 invalid id
  __shared__ float2 s_red[kFvWaves];
  const VfParams &P = F.v;
  // all chunks of a sequence on one XCD: the gathered draft rows meet in that XCD's L2
  const int64_t bid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t b = bid / P.nchunk;
  const int c = static_cast<int>(bid - b * P.nchunk);
  const int lane = lane_id(), w = static_cast<int>(threadIdx.x) / kWave;
  const int g = P.gamma, R = static_cast<int>(P.R);

  // 0. loads that need nothing computed first, all at clamped in-range indices and none of them
  //    inspected until its use (see load_pair_raw)
  const int64_t x0 = static_cast<int64_t>(c) * kFvIds + kFvPer * static_cast<int64_t>(threadIdx.x);
  int32_t ti[kFvPer];
#pragma unroll
  for (int j = 0; j < kFvPer; ++j) {
    const int64_t x = x0 + j;
    ti[j] = P.f2t ? P.f2t[x < P.V ? x : P.V - 1] : static_cast<int32_t>(x);
  }
  bool my_draft[RPW];  // rows past gamma only feed the outputs
  float2 pv[RPW][4];
  float ud[RPW], ua[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int i = w + kFvWaves * r;
    my_draft[r] = i < R && (i < g || c == 0);
    ud[r] = 0.f;
    if (my_draft[r]) {
      const int64_t m = b * R + i;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = 4 * lane + j;
        pv[r][j] = F.dpart[m * F.nd + (k < F.nd ? k : F.nd - 1)];
      }
      ud[r] = F.udraft[m];
    }
    ua[r] = i < g ? P.uacc[b * g + i] : 0.f;
  }
  float2 tp[kTPW];
#pragma unroll
  for (int s = 0; s < kTPW; ++s) {
    const int i = w + kFvWaves * s;
    tp[s] = make_float2(kNegInf, 0.f);
    if (i <= g) tp[s] = F.tpart[(b * (g + 1) + i) * F.nt + (lane < F.nt ? lane : F.nt - 1)];
  }
  RawPair<Tin> tg[kMaxT];
#pragma unroll
  for (int i = 0; i < kMaxT; ++i) {
    const int ri = i <= g ? i : g;  // rows past gamma repeat row gamma (never selected)
    tg[i] = load_pair_raw<Tin, kVec>(reinterpret_cast<const Tin *>(P.target) + (b * (g + 1) + ri) * P.V, P.V, x0);
  }
  bool on[kFvPer];  // id inside the vocabulary and kept
#pragma unroll
  for (int j = 0; j < kFvPer; ++j) on[j] = x0 + j < P.V && ti[j] >= 0 && ti[j] < P.Vt;
  float dg[kMaxR][kFvPer];
#pragma unroll
  for (int i = 0; i < kMaxR; ++i) {
    const int ri = i < g ? i : g - 1;  // rows past gamma - 1 repeat row gamma - 1 (never selected)
    const float *drow = P.draft + (b * R + ri) * P.Vt;
#pragma unroll
    for (int j = 0; j < kFvPer; ++j) dg[i][j] = drow[on[j] ? ti[j] : 0];
  }

  // 1. wave w: draws of its draft rows; log-normalisers of its target rows; accept tests of its
  //    drafts (fp64 ratio exp(a - d), a and d the two log-probabilities of the drafted token)
  DraftDraw dd[RPW];
  bool valid[RPW];
  float tl[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int i = w + kFvWaves * r;
    dd[r] = DraftDraw{};
    valid[r] = false;
    tl[r] = 0.f;
    if (my_draft[r]) {
      const int64_t m = b * R + i;
      dd[r] = fv_draft_row(F, m, pv[r], ud[r]);
      valid[r] = dd[r].x >= 0 && dd[r].x < P.Vt && dd[r].y >= 0 && dd[r].y < P.V;
      if (i < g && valid[r])  // the target logit of the drafted token, in flight during the target lse
        tl[r] = load_logit(reinterpret_cast<const Tin *>(P.target) + (b * (g + 1) + i) * P.V, dd[r].y);
      if (lane == 0) {
        s_dlse[i] = dd[r].lse;
        if (c == 0) {
          F.dlse_out[m] = dd[r].lse;
          F.dids_out[m] = dd[r].x;
        }
      }
    }
  }
  double tl_w[kTPW];  // log-normalisers of target rows w + 8 s
#pragma unroll
  for (int s = 0; s < kTPW; ++s) {
    const int i = w + kFvWaves * s;
    tl_w[s] = 0.0;
    if (i <= g) {
      tl_w[s] = fv_target_lse(F, b * (g + 1) + i, tp[s]);
      if (lane == 0) {
        s_tlse[i] = tl_w[s];
        if (c == 0) F.tlse_out[b * (g + 1) + i] = tl_w[s];
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int i = w + kFvWaves * r;
    if (i < g && lane == 0) {
      int verdict = -1;
      if (valid[r]) {
        const double a = static_cast<double>(tl[r]) * P.invTt - tl_w[r];
        const double d = static_cast<double>(dd[r].xl) * P.invTd - dd[r].lse;
        verdict = accept_ratio(ua[r], a - d) ? 1 : 0;
      }
      s_acc[i] = verdict;
    }
  }
  __syncthreads();

  // 2. n = first rejected draft, gamma if none, -1 if any draft id is out of range
  int n = g;
  bool bad = false;
  for (int i = 0; i < g; ++i) {
    const int a = s_acc[i];
    bad = bad || a < 0;
    if (a == 0 && n == g) n = i;
  }
  if (bad) n = -1;

  // 3. chunk sums of the final-draw weights of row n and of p_n
  float sw = 0.f, sp = 0.f;
  if (n >= 0) {
    RawPair<Tin> tn = tg[0];
    float d2[kFvPer];
#pragma unroll
    for (int j = 0; j < kFvPer; ++j) d2[j] = dg[0][j];
#pragma unroll
    for (int i = 1; i < kMaxT; ++i)
      if (i == n) {
        tn = tg[i];
#pragma unroll
        for (int j = 0; j < kFvPer; ++j)
          if (i < kMaxR) d2[j] = dg[i][j];
      }
    float t2[kFvPer];
#pragma unroll
    for (int j = 0; j < kFvPer; ++j) {
      t2[j] = x0 + j < P.V ? pair_elem(tn, j) : kNegInf;
      if (!on[j]) d2[j] = kNegInf;
    }
    const RowExp pe = make_row_exp_inv(s_tlse[n], P.Tt, P.invTt, P.k2t);
    float wj[kFvPer], pj[kFvPer];
    if (n < g) {
      const RowExp qe = make_row_exp_inv(s_dlse[n], P.Td, P.invTd, P.k2d);
#pragma unroll
      for (int j = 0; j < kFvPer; ++j) {
        pj[j] = pe(t2[j]);
        wj[j] = fmaxf(pj[j] - qe(d2[j]), 0.f);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kFvPer; ++j) pj[j] = wj[j] = pe(t2[j]);
    }
#pragma unroll
    for (int j = 0; j < kFvPer; ++j) {
      sw += wj[j];
      sp += pj[j];
      if (x0 + j < P.V) {  // kept for the final pass's rescan of one chunk
        F.wbuf[b * P.V + x0 + j] = wj[j];
        F.pbuf[b * P.V + x0 + j] = pj[j];
      }
    }
  }
  sw = wave_sum(sw);
  sp = wave_sum(sp);
  if (lane == 0) s_red[w] = make_float2(sw, sp);
  __syncthreads();
  if (threadIdx.x == 0) {
    float a = 0.f, q = 0.f;
#pragma unroll
    for (int k = 0; k < kFvWaves; ++k) {
      a += s_red[k].x;
      q += s_red[k].y;
    }
    P.part[b * P.nchunk + c] = make_float2(a, q);
    if (c == 0) P.nbuf[b] = n;
  }
}

// Greedy blocks (both temperatures 0; "VocabTrim" §4 and Appendix C.1, Algorithm 2: a draft is
// kept only while it equals the target's most likely token, and the target's own token follows
// the first mismatch).  The head launch leaves per-block (max, lowest index of the max) of every
// draft row, and per-4096-chunk argmaxes of every target row come from extra workgroups of the
// GEMV launch or from a launch of their own before an MFMA head; one 512-thread workgroup per
// sequence reduces them (wave w: draft rows w and w + 8, target rows w, w + 8 and w + 16),
// compares, and writes every output.  No logits are read here.
__device__ __forceinline__ void partial_argmax(const float2 *p, int n, float &bv, int &bi) {
  bv = kNegInf;
  bi = kNoIndex;
  for (int k = lane_id(); k < n; k += kWave) {
    const float2 v = p[k];
    if (argmax_better(v.x, __float_as_int(v.y), bv, bi)) {
      bv = v.x;
      bi = __float_as_int(v.y);
    }
  }
  wave_argmax(bv, bi);
}

__global__ __launch_bounds__(kFvBlock) void verify_greedy_small(FvParams F) {
  __shared__ int s_x[kFvMaxR2];
  __shared__ int s_a[kFvMaxR2 + 1];
  const VfParams &P = F.v;
  const int64_t b = blockIdx.x;
  const int lane = lane_id(), w = static_cast<int>(threadIdx.x) / kWave;
  const int g = P.gamma, R = static_cast<int>(P.R);
  for (int i = w; i < R; i += kFvWaves) {
    const int64_t m = b * R + i;
    float bv;
    int bi;
    partial_argmax(F.dpart + m * F.nd, F.nd, bv, bi);
    if (lane == 0) {
      s_x[i] = bi;
      F.dlse_out[m] = static_cast<double>(bv);  // the greedy limit of the log-normaliser: the row max
      F.dids_out[m] = bi;
    }
  }
  for (int i = w; i <= g; i += kFvWaves) {
    float bv;
    int bi;
    partial_argmax(F.tpart + (b * (g + 1) + i) * F.nt, F.nt, bv, bi);
    if (lane == 0) s_a[i] = bi;
  }
  __syncthreads();
  if (w != 0) return;
  // n = first draft whose full id differs from the target's argmax, gamma if none, -1 if an id
  // is out of range; tokens = the kept drafts, then the target's argmax at n, then -1
  bool valid = true, accept = true;
  int32_t y = -1;
  if (lane < g) {
    const int x = s_x[lane];
    valid = x >= 0 && x < P.Vt;
    if (valid) {
      y = P.keep ? P.keep[x] : x;
      valid = y >= 0 && y < P.V;
    }
    accept = valid && y == s_a[lane];
  }
  const unsigned long long bad = __ballot(lane < g && !valid);
  const unsigned long long rej = __ballot(lane < g && !accept);
  const int n = bad ? -1 : (rej ? __ffsll(static_cast<long long>(rej)) - 1 : g);
  int32_t *tok = P.out_tokens + b * (g + 1);
  for (int i = lane; i <= g; i += kWave) {
    int32_t v = -1;
    if (n >= 0 && i < n) v = y;  // lane i holds draft i's full id
    else if (n >= 0 && i == n) v = s_a[n];
    tok[i] = v;
  }
  if (lane == 0) P.out_n[b] = n;
}

// Final pass: one 256-thread workgroup per sequence draws the final token from the chunk sums
// and writes the outputs (the log-normalisers and draft ids were written by the chunk pass); the
// chunk it rescans comes from the weights the chunk pass kept, so no logit is read here.
template <typename Tin, bool kVec>
__global__ __launch_bounds__(kBlock) void verify_fused_final(FvParams F) {
  const VfParams &P = F.v;
  __shared__ float redf[kWavesPerBlock];
  __shared__ int redi[kWavesPerBlock];
  __shared__ float bcast;
  const int64_t b = blockIdx.x;
  const int n = P.nbuf[b];
  const float2 *part = P.part + b * P.nchunk;
  auto mass = [&](int k, bool use_p) -> float {
    if (k >= P.nchunk) return 0.f;
    const float2 v = part[k];
    return use_p ? v.y : v.x;
  };
  auto weights = [&](int c, bool use_p, float(&wv)[kFvFinalPer]) {
    const float *src = (use_p ? F.pbuf : F.wbuf) + b * P.V;
#pragma unroll
    for (int j = 0; j < kFvFinalPer; ++j) {
      const int64_t x = static_cast<int64_t>(c) * kFvIds + static_cast<int64_t>(threadIdx.x) * kFvFinalPer + j;
      wv[j] = x < P.V ? src[x] : 0.f;
    }
  };
  finish_sequence<Tin, kVec, decltype(mass), kFvFinalPer>(P, b, n, mass, redf, redi, &bcast, weights);
}

}  // namespace
}  // namespace vt

// Verification of small batches in the single-call block, after the GEMV head (gfx950).
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
//      reaches u Z, then a scan of that block's logits) and forms the log-normaliser of target
//      rows w and w + 8.  Every workgroup of the sequence repeats this small amount of work, so
//      no workgroup waits for another; the first chunk's workgroup writes the outputs.
//   2. Wave 0 runs the accept scan (fp64 ratios, a ballot gives n = first rejection).
//   3. From the registers loaded in step 0: the chunk sums of w(x) = max(0, p_n(x) - q_n(x))
//      (p_gamma when every draft was kept) and of p_n(x).
// Final pass: one workgroup per sequence locates the 1024-id chunk where the running residual
// mass reaches u_final times its total and rescans it (the shared final-draw code of the verify
// call, at 4 ids per thread).
#pragma once
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "softmax_impl.hpp"
#include "verify_impl.hpp"

namespace vt {
namespace {

constexpr int kFvBlock = 512;
constexpr int kFvWaves = kFvBlock / kWave;      // 8: one draft row per wavefront
constexpr int kFvIds = 1024;                    // full-vocabulary ids per chunk workgroup
constexpr int kFvPer = kFvIds / kFvBlock;       // 2 ids per thread
constexpr int kFvMaxR = 8;                      // draft rows per sequence (the GEMV head takes M <= 8)
constexpr int kFvMaxT = kFvMaxR + 1;            // target rows per sequence
constexpr int kFvFinalPer = kFvIds / kBlock;    // 4 ids per thread in the final rescan
constexpr int kFvMaxParts = 4 * kWave;          // head row blocks per row (gemv_blocks <= 256)
constexpr int kFvScanBatch = 8;                 // 64-logit groups loaded at once when rescanning a row block

static_assert(kFvWaves == kFvMaxR, "one wavefront per draft row");

struct FvParams {
  VfParams v;            // verification view: target, draft logits, keep set, uniforms, outputs
  const float2 *dpart;   // [B * R][nd]: (max, sum of exp) per head row block
  int nd, dper;          // row blocks per draft row, head rows per block
  const float *udraft;   // [B * R]
  const float2 *tpart;   // [B * (gamma + 1)][nt]: (max, sum of exp) per 4096-chunk
  int nt;
  double *dlse_out;      // [B * R]
  int32_t *dids_out;     // [B * R]
  double *tlse_out;      // [B * (gamma + 1)]
};

// Two consecutive elements [e0, e0 + 2) of a row as fp32; -inf past n.  kVec: the row start is
// 16-byte aligned and n even, so the pair is one aligned load.
template <typename Tin, bool kVec>
__device__ __forceinline__ void load_pair(const Tin *__restrict__ row, int64_t n, int64_t e0, float (&v)[2]) {
  if (kVec && e0 + 2 <= n) {
    if constexpr (sizeof(Tin) == 4) {
      const float2 f = *reinterpret_cast<const float2 *>(reinterpret_cast<const float *>(row) + e0);
      v[0] = f.x;
      v[1] = f.y;
    } else {
      const uint32_t u = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint16_t *>(row) + e0);
      v[0] = __uint_as_float(u << 16);
      v[1] = __uint_as_float(u & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t e = e0 + j;
      v[j] = e < n ? load_logit(row, e) : kNegInf;
    }
  }
}

// Draft row m, one wavefront: lse = M / T + ln Z from the head's per-block partials; the draw
// t = u Z walks the block-level running sum to the first block reaching t, then that block's
// logits.  pv: the row's partials (entry k = 64 j + lane), loaded by the caller.  Returns the
// drawn index (-1 if nothing carries weight) and its logit.
__device__ __forceinline__ void fv_draft_row(const FvParams &F, int64_t m, const float2 (&pv)[4], float u,
                                             double &lse, int &x, float &xl) {
  const int lane = lane_id();
  const float k2 = F.v.k2d;
  float mx = kNegInf;
#pragma unroll
  for (int j = 0; j < 4; ++j) mx = fmaxf(mx, pv[j].x);
  const float M = wave_max(mx);
  float mass[4], inc[4], before[4];
  float carry = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    mass[j] = pv[j].x == kNegInf ? 0.f : pv[j].y * exp2_fast((pv[j].x - M) * k2);
    inc[j] = wave_scan_incl(mass[j]);
    before[j] = carry;
    carry = carry + lane_value(inc[j], kWave - 1);
  }
  const float Z = carry;
  lse = static_cast<double>(M) / F.v.Td + log(static_cast<double>(Z));
  const float t = u * Z;
  int ks = -1;
  float E = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const unsigned long long hit = __ballot(kWave * j + lane < F.nd && t <= before[j] + inc[j]);
    const float prev = wave_prev(inc[j], 0.f);
    if (ks < 0 && hit) {
      const int l = __ffsll(static_cast<long long>(hit)) - 1;
      ks = kWave * j + l;
      E = before[j] + lane_value(prev, l);
    }
  }
  bool fallback = false;
  if (ks < 0) {
    // t beyond the running sum (u >= 1 or NaN): the last block with positive mass
    int last = -1;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (kWave * j + lane < F.nd && mass[j] > 0.f) last = kWave * j + lane;
    ks = max(wave_max_int(last), 0);
    fallback = true;
  }
  // rescan block ks: first logit whose running weight reaches t, else the last positive one
  const float *row = F.v.draft + m * F.v.Vt;
  const int64_t r0 = static_cast<int64_t>(ks) * F.dper;
  const int64_t r1 = r0 + F.dper < F.v.Vt ? r0 + F.dper : F.v.Vt;
  const float te = fallback ? __builtin_huge_valf() : t;
  float run = fallback ? 0.f : E;
  int found = -1, lastpos = -1;
  float fl = kNegInf;
  for (int64_t g0 = r0; g0 < r1 && found < 0; g0 += kWave * kFvScanBatch) {
    float vals[kFvScanBatch];
#pragma unroll
    for (int q = 0; q < kFvScanBatch; ++q) {
      const int64_t e = g0 + kWave * q + lane;
      vals[q] = e < r1 ? row[e] : kNegInf;
    }
#pragma unroll
    for (int q = 0; q < kFvScanBatch; ++q) {
      const int64_t e = g0 + kWave * q + lane;
      const float wgt = M == kNegInf ? 0.f : exp2_fast((vals[q] - M) * k2);
      const float G = run + wave_scan_incl(wgt);
      if (e < r1 && wgt > 0.f) lastpos = static_cast<int>(e);
      const unsigned long long hit = __ballot(e < r1 && te <= G);
      if (found < 0 && hit) {
        const int l = __ffsll(static_cast<long long>(hit)) - 1;
        found = static_cast<int>(g0 + kWave * q + l);
        fl = lane_value(vals[q], l);
      }
      run = lane_value(G, kWave - 1);
    }
  }
  if (found < 0) {
    found = wave_max_int(lastpos);
    if (found >= 0) fl = row[found];
  }
  x = found;
  xl = fl;
}

// Log-normaliser of target row r from its 4096-chunk partials, one wavefront, with exactly the
// operations (and so the bits) of the combine pass of the separate softmax call: chunk masses
// scanned 64 at a time, four scans to a 256-chunk pass added in order, passes carried.  p0: the
// row's first 64 partials, loaded by the caller.
__device__ __forceinline__ double fv_target_lse(const FvParams &F, int64_t r, float2 p0) {
  const int lane = lane_id();
  const float2 *pp = F.tpart + r * F.nt;
  float mx = p0.x;
  for (int k = kWave + lane; k < F.nt; k += kWave) mx = fmaxf(mx, pp[k].x);
  const float M = wave_max(mx);
  float carry = 0.f;
  for (int k0 = 0; k0 < F.nt; k0 += kBlock) {
    float total = 0.f;
#pragma unroll
    for (int q = 0; q < kWavesPerBlock; ++q) {
      const int k = k0 + kWave * q + lane;
      float s = 0.f;
      if (k < F.nt) {
        const float2 ps = k < kWave ? p0 : pp[k];
        s = ps.x == kNegInf ? 0.f : ps.y * exp2_fast((ps.x - M) * F.v.k2t);
      }
      total += lane_value(wave_scan_incl(s), kWave - 1);
    }
    carry = carry + total;
  }
  return static_cast<double>(M) / F.v.Tt + log(static_cast<double>(carry));
}

template <typename Tin, bool kVec>
__global__ __launch_bounds__(kFvBlock) void verify_fused_chunk(FvParams F) {
  __shared__ double s_tlse[kFvMaxT], s_dlse[kFvMaxR];
  __shared__ float s_dlog[kFvMaxR];
  __shared__ int s_x[kFvMaxR];
  __shared__ int s_n;
  __shared__ float2 s_red[kFvWaves];
  const VfParams &P = F.v;
  // all chunks of a sequence on one XCD: the gathered draft rows meet in that XCD's L2
  const int64_t bid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t b = bid / P.nchunk;
  const int c = static_cast<int>(bid - b * P.nchunk);
  const int lane = lane_id(), w = static_cast<int>(threadIdx.x) / kWave;
  const int g = P.gamma, R = static_cast<int>(P.R);

  // 0. loads that need nothing computed first
  const int64_t x0 = static_cast<int64_t>(c) * kFvIds + kFvPer * static_cast<int64_t>(threadIdx.x);
  int32_t ti[kFvPer];
#pragma unroll
  for (int j = 0; j < kFvPer; ++j) {
    const int64_t x = x0 + j;
    ti[j] = x < P.V ? (P.f2t ? P.f2t[x] : static_cast<int32_t>(x)) : -1;
  }
  const bool my_draft = w < R && (w < g || c == 0);  // rows past gamma only feed the outputs
  const int64_t m = b * R + w;
  float2 pv[4];
  float ud = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int k = kWave * j + lane;
    pv[j] = (my_draft && k < F.nd) ? F.dpart[m * F.nd + k] : make_float2(kNegInf, 0.f);
  }
  if (my_draft) ud = F.udraft[m];
  float2 tp[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int i = w + kFvWaves * s;
    tp[s] = (i <= g && lane < F.nt) ? F.tpart[(b * (g + 1) + i) * F.nt + lane] : make_float2(kNegInf, 0.f);
  }
  float tg[kFvMaxT][kFvPer];
#pragma unroll
  for (int i = 0; i < kFvMaxT; ++i) {
    if (i <= g) {
      load_pair<Tin, kVec>(reinterpret_cast<const Tin *>(P.target) + (b * (g + 1) + i) * P.V, P.V, x0, tg[i]);
    } else {
      tg[i][0] = tg[i][1] = kNegInf;
    }
  }
  float dg[kFvMaxR][kFvPer];
#pragma unroll
  for (int i = 0; i < kFvMaxR; ++i) {
    const float *drow = P.draft + (b * R + i) * P.Vt;
#pragma unroll
    for (int j = 0; j < kFvPer; ++j) dg[i][j] = (i < g && ti[j] >= 0 && ti[j] < P.Vt) ? drow[ti[j]] : kNegInf;
  }

  // 1. draft row w: log-normaliser and draw; target rows w, w + 8: log-normalisers
  if (my_draft) {
    double lse;
    int x;
    float xl;
    fv_draft_row(F, m, pv, ud, lse, x, xl);
    if (lane == 0) {
      s_dlse[w] = lse;
      s_x[w] = x;
      s_dlog[w] = xl;
      if (c == 0) {
        F.dlse_out[m] = lse;
        F.dids_out[m] = x;
      }
    }
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int i = w + kFvWaves * s;
    if (i <= g) {
      const double l = fv_target_lse(F, b * (g + 1) + i, tp[s]);
      if (lane == 0) {
        s_tlse[i] = l;
        if (c == 0) F.tlse_out[b * (g + 1) + i] = l;
      }
    }
  }
  __syncthreads();

  // 2. accept scan: lanes 0..gamma-1 of wave 0; n = first rejection, gamma if none, -1 if a
  //    draft id (or its full id) is out of range
  if (w == 0) {
    bool valid = true, accept = true;
    if (lane < g) {
      const int x = s_x[lane];
      valid = x >= 0 && x < P.Vt;
      int64_t y = x;
      if (valid && P.keep) {
        y = P.keep[x];
        valid = y >= 0 && y < P.V;
      }
      if (valid) {
        const Tin *trow = reinterpret_cast<const Tin *>(P.target) + (b * (g + 1) + lane) * P.V;
        const double a = static_cast<double>(load_logit(trow, y)) / P.Tt - s_tlse[lane];
        const double d = static_cast<double>(s_dlog[lane]) / P.Td - s_dlse[lane];
        accept = static_cast<double>(P.uacc[b * g + lane]) <= fmin(1.0, exp(a - d));
      }
    }
    const unsigned long long bad = __ballot(lane < g && !valid);
    const unsigned long long rej = __ballot(lane < g && !accept);
    if (lane == 0) s_n = bad ? -1 : (rej ? __ffsll(static_cast<long long>(rej)) - 1 : g);
  }
  __syncthreads();

  // 3. chunk sums of the final-draw weights of row n and of p_n
  const int n = s_n;
  float sw = 0.f, sp = 0.f;
  if (n >= 0) {
    float t2[kFvPer], d2[kFvPer];
#pragma unroll
    for (int j = 0; j < kFvPer; ++j) {
      t2[j] = tg[0][j];
      d2[j] = dg[0][j];
    }
#pragma unroll
    for (int i = 1; i < kFvMaxT; ++i)
      if (i == n) {
#pragma unroll
        for (int j = 0; j < kFvPer; ++j) {
          t2[j] = tg[i][j];
          if (i < kFvMaxR) d2[j] = dg[i][j];
        }
      }
    const RowExp pe = make_row_exp(s_tlse[n], P.Tt, P.k2t);
    if (n < g) {
      const RowExp qe = make_row_exp(s_dlse[n], P.Td, P.k2d);
#pragma unroll
      for (int j = 0; j < kFvPer; ++j) {
        const float p = pe(t2[j]);
        sw += fmaxf(p - qe(d2[j]), 0.f);
        sp += p;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kFvPer; ++j) {
        const float p = pe(t2[j]);
        sw += p;
        sp += p;
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

// Final pass: one 256-thread workgroup per sequence draws the final token from the chunk sums
// and writes the outputs (the log-normalisers and draft ids were written by the chunk pass).
template <typename Tin, bool kVec>
__global__ __launch_bounds__(kBlock) void verify_fused_final(VfParams P) {
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
  finish_sequence<Tin, kVec, decltype(mass), kFvFinalPer>(P, b, n, mass, redf, redi, &bcast);
}

}  // namespace
}  // namespace vt

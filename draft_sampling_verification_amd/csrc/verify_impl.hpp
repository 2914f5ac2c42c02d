// Batched modified rejection sampling for gfx950 ("Speculative decoding" glossary, sections
// "Propose a block, keep a prefix" and "Why a rejection needs a special draw"; "A rejection rule
// keeps speculative decoding's output exact", sections "What the accept/reject rule has to
// balance" and "Extending the rule from one token to a drafted run"; "VocabTrim", Appendix C.1,
// Algorithm 2 for the map from trimmed ids back to the full vocabulary).
//
// Pass 1: one 256-thread workgroup per (sequence b, 4096-id chunk of the full vocabulary).  Every
// workgroup of a sequence repeats the sequence's accept scan (gamma <= 64 lanes of wave 0, fp64
// ratios, a ballot gives n = first rejection), so all of them know which row feeds the final
// draw.  Each then computes, for its chunk of ids x, the weight w(x) = max(0, p_n(x) - q_n(x))
// (q_n(x) = 0 off the kept set; w = p_gamma when all drafts were accepted) and publishes the chunk
// sums of w and of p.  Pass 2 (next launch, one workgroup per sequence) forms the chunk-level
// running sum, falls back to p_n if the residual mass is 0, draws the final token with u_final by
// rescanning one chunk, and writes the outputs.  Vocabularies of one chunk use a single launch.
#pragma once
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "vt_common.hpp"

namespace vt {
namespace {

constexpr double kLog2e = 1.4426950408889634;

struct VfParams {
  const void *target;
  const double *tlse;
  const float *draft;
  const double *dlse;
  const int32_t *ids;
  const int32_t *keep;
  const int32_t *f2t;
  const float *uacc;
  const float *ufin;
  int32_t *out_tokens;
  int32_t *out_n;
  int *nbuf;     // n per sequence, from pass 1 to pass 2
  float2 *part;  // (sum of final-draw weights, sum of p) per (sequence, chunk)
  int64_t V, Vt, R;
  double Tt, Td;
  double invTt, invTd;  // 1 / T, rounded once on the host
  float k2t, k2d;  // log2(e) / T
  int gamma;
  int nchunk;
  bool greedy;  // target_T = 0: accept iff the draft equals the target's argmax; final = argmax
};

// Per-row constants so that exp(x / T - lse) = 2^((x - c0) * k2 - d2) with c0 = lse * T in logit
// units: the fp32 argument is small for the heavy entries, where accuracy matters.
struct RowExp {
  float c0, d2, k2;
  __device__ __forceinline__ float operator()(float x) const {
    return x == kNegInf ? 0.f : __builtin_amdgcn_exp2f(fmaf(x - c0, k2, -d2));
  }
};

__device__ __forceinline__ RowExp make_row_exp(double lse, double T, float k2) {
  RowExp e;
  e.c0 = static_cast<float>(lse * T);
  e.d2 = static_cast<float>((lse - static_cast<double>(e.c0) / T) * kLog2e);
  e.k2 = k2;
  return e;
}

// The same with a host-rounded 1 / T in place of the division.
__device__ __forceinline__ RowExp make_row_exp_inv(double lse, double T, double invT, float k2) {
  RowExp e;
  e.c0 = static_cast<float>(lse * T);
  e.d2 = static_cast<float>((lse - static_cast<double>(e.c0) * invT) * kLog2e);
  e.k2 = k2;
  return e;
}

// u <= min(1, exp(x)), the accept test with fp64 log-ratio x, decided exactly as in fp64: a
// single-precision 2^(x log2 e) settles it whenever u lies outside a 1e-5 relative band around
// it (its error is below 2^-24 |x| from the exponent's rounding plus one ulp, under 1e-5 for
// every result above 1e-30); otherwise, and for tiny ratios, the fp64 exp decides.
__device__ __forceinline__ bool accept_ratio(float u, double x) {
  if (!(x < 0.0)) return u <= 1.f;  // ratio 1 (a NaN ratio also reads as 1 under fmin)
  const float r = __builtin_amdgcn_exp2f(static_cast<float>(x * kLog2e));
  if (r >= 1e-30f) {
    const float du = u - r;
    if (fabsf(du) > 1e-5f * r) return du < 0.f;
  }
  return static_cast<double>(u) <= exp(x);
}

template <typename Tin>
__device__ __forceinline__ float load_logit(const Tin *row, int64_t i) {
  if constexpr (sizeof(Tin) == 4)
    return reinterpret_cast<const float *>(row)[i];
  else
    return bf16_to_f32(reinterpret_cast<const uint16_t *>(row)[i]);
}

// Weights of the final draw for this thread's 16 ids of chunk c: residual (use_p = false) or
// p itself; also returns p in pv for the fallback sum.  p comes from 16-byte loads of the
// thread's own ids.  q_n is fetched lane-contiguously (consecutive lanes read consecutive
// full_to_trim entries and, for an ascending keep set, consecutive draft entries) into LDS and
// read back in the thread's order: a per-thread loop over its 16 ids would make every load
// instruction touch 64 different cache lines.  All threads of the workgroup must call.
// PER ids per thread: chunks of PER * 256 ids (16: the 4096-id chunks of the separate verify
// call; 4: the 1024-id chunks of the batch-1 block).
template <typename Tin, bool kVec, int PER = kPerThread>
__device__ __forceinline__ void final_weights(const VfParams &P, int64_t b, int n, int c, bool use_p, float (&wv)[PER],
                                              float (&pv)[PER]) {
  constexpr int kIds = PER * kBlock;
  __shared__ __align__(16) float sq[kIds];
  const int row = n < P.gamma ? n : P.gamma;
  const Tin *trow = reinterpret_cast<const Tin *>(P.target) + (b * (P.gamma + 1) + row) * P.V;
  float lt[PER];
  load_run<Tin, kVec, PER>(trow, P.V, static_cast<int64_t>(c) * kIds, lt);
  const RowExp pe = make_row_exp(P.tlse[b * (P.gamma + 1) + row], P.Tt, P.k2t);
#pragma unroll
  for (int j = 0; j < PER; ++j) pv[j] = pe(lt[j]);
  if (n >= P.gamma || use_p) {
#pragma unroll
    for (int j = 0; j < PER; ++j) wv[j] = pv[j];
    return;
  }
  const float *drow = P.draft + (b * P.R + n) * P.Vt;
  const RowExp qe = make_row_exp(P.dlse[b * P.R + n], P.Td, P.k2d);
  const int64_t base = static_cast<int64_t>(c) * kIds;
  __syncthreads();  // a previous call's readers are done with sq
  int32_t tv[PER];
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int64_t x = base + r * kBlock + threadIdx.x;
    tv[r] = x < P.V ? (P.f2t ? P.f2t[x] : static_cast<int32_t>(x)) : -1;
  }
  float dv[PER];
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int32_t t = tv[r];
    dv[r] = (t >= 0 && t < P.Vt) ? drow[t] : kNegInf;
  }
#pragma unroll
  for (int r = 0; r < PER; ++r) sq[r * kBlock + threadIdx.x] = qe(dv[r]);
  __syncthreads();
  const float4 *q4 = reinterpret_cast<const float4 *>(sq + threadIdx.x * PER);
#pragma unroll
  for (int k = 0; k < PER / 4; ++k) {
    const float4 q = q4[k];
    wv[4 * k + 0] = fmaxf(pv[4 * k + 0] - q.x, 0.f);
    wv[4 * k + 1] = fmaxf(pv[4 * k + 1] - q.y, 0.f);
    wv[4 * k + 2] = fmaxf(pv[4 * k + 2] - q.z, 0.f);
    wv[4 * k + 3] = fmaxf(pv[4 * k + 3] - q.w, 0.f);
  }
}

// Accept scan of sequence b by wave 0 (lanes 0..gamma-1): n = first rejected draft, gamma if
// none, -1 if a draft id (or its full id) is out of range.  Broadcast through LDS; all threads
// of the workgroup must call.
template <typename Tin>
__device__ __forceinline__ int accept_scan(const VfParams &P, int64_t b, int *sh_n) {
  const int gamma = P.gamma;
  if (wave_id() == 0) {
    const int i = lane_id();
    bool valid = true, accept = true;
    if (i < gamma) {
      const int64_t x = P.ids[b * P.R + i];
      valid = x >= 0 && x < P.Vt;
      int64_t y = x;
      if (valid && P.keep) {
        y = P.keep[x];
        valid = y >= 0 && y < P.V;
      }
      if (valid) {
        const Tin *trow = reinterpret_cast<const Tin *>(P.target) + (b * (gamma + 1) + i) * P.V;
        const double a = static_cast<double>(load_logit(trow, y)) / P.Tt - P.tlse[b * (gamma + 1) + i];
        const double d = static_cast<double>(P.draft[(b * P.R + i) * P.Vt + x]) / P.Td - P.dlse[b * P.R + i];
        const double ratio = fmin(1.0, exp(a - d));
        accept = static_cast<double>(P.uacc[b * gamma + i]) <= ratio;
      }
    }
    const unsigned long long bad = __ballot(i < gamma && !valid);
    const unsigned long long rej = __ballot(i < gamma && !accept);
    if (i == 0) *sh_n = bad ? -1 : (rej ? __ffsll(static_cast<long long>(rej)) - 1 : gamma);
  }
  __syncthreads();
  return *sh_n;
}

// Final draw and outputs of sequence b, given n and the chunk sums of the residual (or bonus)
// weights and of p (mass(k, use_p)); all threads of the workgroup must call.
// weights (optional): a callable (chunk, use_p, float (&wv)[PER]) giving this thread's weights of
// the chunk when they were kept from pass 1; otherwise they are recomputed from the logits.
template <typename Tin, bool kVec, typename Mass, int PER = kPerThread, typename Weights = std::nullptr_t>
__device__ __forceinline__ void finish_sequence(const VfParams &P, int64_t b, int n, Mass mass, float *redf,
                                                int *redi, float *bcast, Weights weights = nullptr) {
  const int gamma = P.gamma;
  int32_t *tok = P.out_tokens + b * (gamma + 1);
  if (n < 0) {
    for (int i = threadIdx.x; i <= gamma; i += kBlock) tok[i] = -1;
    if (threadIdx.x == 0) P.out_n[b] = -1;
    return;
  }
  // residual mass; if it rounds to zero, draw from p_n instead
  float carry = 0.f;
  for (int k0 = 0; k0 < P.nchunk; k0 += kBlock) {
    float prev, total;
    block_inclusive_scan(mass(k0 + threadIdx.x, false), redf, &prev, &total);
    carry = carry + total;
  }
  const bool use_p = !(carry > 0.f);
  float Z = carry;
  if (use_p) {
    carry = 0.f;
    for (int k0 = 0; k0 < P.nchunk; k0 += kBlock) {
      float prev, total;
      block_inclusive_scan(mass(k0 + threadIdx.x, true), redf, &prev, &total);
      carry = carry + total;
    }
    Z = carry;
  }
  const float t = P.ufin[b] * Z;
  int cstar = 0x7fffffff;
  float Estar = 0.f;
  carry = 0.f;
  for (int k0 = 0; k0 < P.nchunk; k0 += kBlock) {
    float prev, total;
    const float incl = block_inclusive_scan(mass(k0 + threadIdx.x, use_p), redf, &prev, &total);
    const int k = k0 + threadIdx.x;
    const bool hit = k < P.nchunk && t <= carry + incl;
    const int first = block_min_int(hit ? k : 0x7fffffff, redi);
    if (first != 0x7fffffff) {
      if (k == first) *bcast = carry + prev;
      __syncthreads();
      cstar = first;
      Estar = *bcast;
      break;
    }
    carry = carry + total;
  }
  bool fallback = false;
  if (cstar == 0x7fffffff) {
    int lastc = -1;
    for (int k = threadIdx.x; k < P.nchunk; k += kBlock)
      if (mass(k, use_p) > 0.f) lastc = k;
    cstar = max(block_max_int(lastc, redi), 0);  // never below chunk 0, even for a NaN uniform
    fallback = true;
  }
  // rescan chunk c*: running sum inside it, first id reaching t (else last positive id)
  float wv[PER];
  if constexpr (std::is_same<Weights, std::nullptr_t>::value) {
    float pv[PER];
    final_weights<Tin, kVec, PER>(P, b, n, cstar, use_p, wv, pv);
  } else {
    weights(cstar, use_p, wv);
  }
  float loc[PER];
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    acc += wv[j];
    loc[j] = acc;
  }
  float prev, total;
  block_inclusive_scan(acc, redf, &prev, &total);
  const float base = Estar + prev;
  int found = 0x7fffffff;
  if (!fallback) {
#pragma unroll
    for (int j = PER - 1; j >= 0; --j)
      if (t <= base + loc[j]) found = static_cast<int>(threadIdx.x) * PER + j;
  }
  found = block_min_int(found, redi);
  if (found == 0x7fffffff) {
    int last = -1;
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (wv[j] > 0.f) last = static_cast<int>(threadIdx.x) * PER + j;
    found = block_max_int(last, redi);
  }
  const int32_t final_id = static_cast<int32_t>(static_cast<int64_t>(cstar) * (PER * kBlock) + found);
  for (int i = threadIdx.x; i <= gamma; i += kBlock) {
    int32_t v = -1;
    if (i < n) {
      const int32_t x = P.ids[b * P.R + i];
      v = P.keep ? P.keep[x] : x;
    } else if (i == n) {
      v = final_id;
    }
    tok[i] = v;
  }
  if (threadIdx.x == 0) P.out_n[b] = n;
}

// ---- greedy mode (target temperature 0; "VocabTrim" §4: the target is decoded greedily, so a
// draft token is kept only if it equals the target's most likely token; Appendix C.1, Algorithm
// 2: on the first mismatch the target's own token is appended).  a[i] = argmax of target row i
// (lowest id on ties); n = first i with keep[x_i] != a[i]; final = a[n].

// Argmax of this workgroup's chunk c of target row (b, i).
template <typename Tin, bool kVec>
__device__ __forceinline__ void chunk_argmax(const VfParams &P, int64_t b, int i, int c, float &bv, int &bi,
                                             float *redf, int *redi) {
  const Tin *trow = reinterpret_cast<const Tin *>(P.target) + (b * (P.gamma + 1) + i) * P.V;
  float v[16];
  const int64_t e0 = static_cast<int64_t>(c) * kChunk + static_cast<int64_t>(threadIdx.x) * kPerThread;
  load16<Tin, kVec>(trow, P.V, static_cast<int64_t>(c) * kChunk, v);
  bv = kNegInf;
  bi = kNoIndex;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j)
    if (e0 + j < P.V && argmax_better(v[j], static_cast<int>(e0 + j), bv, bi)) {
      bv = v[j];
      bi = static_cast<int>(e0 + j);
    }
  block_argmax(bv, bi, redf, redi);
}

// Greedy decision and outputs of sequence b given the row argmaxes a[0..gamma] (in LDS).
__device__ __forceinline__ void greedy_finish(const VfParams &P, int64_t b, const int *a, int *sh_n) {
  const int gamma = P.gamma;
  if (wave_id() == 0) {
    const int i = lane_id();
    bool valid = true, accept = true;
    if (i < gamma) {
      const int64_t x = P.ids[b * P.R + i];
      valid = x >= 0 && x < P.Vt;
      int64_t y = x;
      if (valid && P.keep) {
        y = P.keep[x];
        valid = y >= 0 && y < P.V;
      }
      accept = valid && y == a[i];
    }
    const unsigned long long bad = __ballot(i < gamma && !valid);
    const unsigned long long rej = __ballot(i < gamma && !accept);
    if (i == 0) *sh_n = bad ? -1 : (rej ? __ffsll(static_cast<long long>(rej)) - 1 : gamma);
  }
  __syncthreads();
  const int n = *sh_n;
  int32_t *tok = P.out_tokens + b * (gamma + 1);
  for (int i = threadIdx.x; i <= gamma; i += kBlock) {
    int32_t v = -1;
    if (n >= 0 && i < n) {
      const int32_t x = P.ids[b * P.R + i];
      v = P.keep ? P.keep[x] : x;
    } else if (n >= 0 && i == n) {
      v = a[n];
    }
    tok[i] = v;
  }
  if (threadIdx.x == 0) P.out_n[b] = n;
}

template <typename Tin, bool kVec>
__device__ __forceinline__ void greedy_single(const VfParams &P, int64_t b, float *redf, int *redi, int *sh_n) {
  __shared__ int a[kWave + 1];
  for (int i = 0; i <= P.gamma; ++i) {
    float bv;
    int bi;
    chunk_argmax<Tin, kVec>(P, b, i, 0, bv, bi, redf, redi);
    if (threadIdx.x == 0) a[i] = bi;
  }
  __syncthreads();
  greedy_finish(P, b, a, sh_n);
}

// Vocabularies of at most 64 ids (the toy): one wavefront per sequence, four per workgroup, lane x
// holding id x; the same decisions as verify_single (fp64 accept ratios, n = first rejection,
// residual max(0, p_n - q_n) or p_gamma, p_n when the residual sums to zero, the first id whose
// running sum reaches u Z, else the last one with positive weight), with wave scans and ballots
// instead of workgroup barriers.
template <typename Tin>
__global__ __launch_bounds__(kBlock) void verify_wave(VfParams P, int64_t B) {
  const int64_t b = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave_id();
  if (b >= B) return;  // the whole wavefront
  const int lane = lane_id(), g = P.gamma;
  const bool in = lane < P.V;
  const int xs = in ? lane : 0;
  auto tlogit = [&](int i, int64_t y) {
    return load_logit(reinterpret_cast<const Tin *>(P.target) + (b * (g + 1) + i) * P.V, y);
  };
  int32_t *tok = P.out_tokens + b * (g + 1);
  // draft i on lane i: its trimmed id, full id, validity
  int32_t x = -1, y = -1;
  bool valid = true;
  if (lane < g) {
    x = P.ids[b * P.R + lane];
    valid = x >= 0 && x < P.Vt;
    if (valid) {
      y = P.keep ? P.keep[x] : x;
      valid = y >= 0 && y < P.V;
    }
  }
  const unsigned long long bad = __ballot(lane < g && !valid);
  int n, fin;
  if (P.greedy) {
    // argmax of every target row (lowest id on ties), one row at a time over the lanes
    // lane i < gamma keeps row i's argmax; row gamma's (the bonus, which has no lane of its own
    // when gamma = 64) is kept wave-uniform
    int am = -1, am_g = -1;
    for (int i = 0; i <= g; ++i) {
      float bv = in ? tlogit(i, xs) : kNegInf;
      int bi = in ? lane : kNoIndex;
      wave_argmax(bv, bi);
      if (lane == i) am = bi;
      if (i == g) am_g = bi;
    }
    const unsigned long long rej = __ballot(lane < g && !(valid && y == am));
    n = bad ? -1 : (rej ? __ffsll(static_cast<long long>(rej)) - 1 : g);
    fin = n < 0 ? -1 : (n == g ? am_g : lane_value(am, n));
  } else {
    bool accept = true;
    if (lane < g && valid) {
      const double a = static_cast<double>(tlogit(lane, y)) / P.Tt - P.tlse[b * (g + 1) + lane];
      const double d = static_cast<double>(P.draft[(b * P.R + lane) * P.Vt + x]) / P.Td - P.dlse[b * P.R + lane];
      accept = static_cast<double>(P.uacc[b * g + lane]) <= fmin(1.0, exp(a - d));
    }
    const unsigned long long rej = __ballot(lane < g && !accept);
    n = bad ? -1 : (rej ? __ffsll(static_cast<long long>(rej)) - 1 : g);
    fin = -1;
    if (n >= 0) {
      const int row = n < g ? n : g;
      const RowExp pe = make_row_exp(P.tlse[b * (g + 1) + row], P.Tt, P.k2t);
      const float p = in ? pe(tlogit(row, xs)) : 0.f;
      float w = p;
      if (n < g) {
        const RowExp qe = make_row_exp(P.dlse[b * P.R + n], P.Td, P.k2d);
        const int32_t t = in ? (P.f2t ? P.f2t[xs] : xs) : -1;
        const bool kept = t >= 0 && t < P.Vt;
        const float q = kept ? qe(P.draft[(b * P.R + n) * P.Vt + (kept ? t : 0)]) : 0.f;
        w = fmaxf(p - q, 0.f);
        if (!(lane_value(wave_scan_incl(w), kWave - 1) > 0.f)) w = p;  // residual rounds to zero
      }
      const float C = wave_scan_incl(w);
      const float tt = P.ufin[b] * lane_value(C, kWave - 1);
      const unsigned long long hit = __ballot(in && tt <= C);
      if (hit) {
        fin = __ffsll(static_cast<long long>(hit)) - 1;
      } else {
        const unsigned long long pos = __ballot(in && w > 0.f);
        fin = pos ? 63 - __clzll(static_cast<long long>(pos)) : -1;
      }
    }
  }
  for (int i = lane; i <= g; i += kWave) {
    int32_t v = -1;
    if (n >= 0 && i < n) v = y;  // lane i holds draft i's full id (g <= 64)
    else if (n >= 0 && i == n) v = fin;
    tok[i] = v;
  }
  if (lane == 0) P.out_n[b] = n;
}

// Vocabularies of one chunk (V <= 4096): one workgroup per sequence does everything.
template <typename Tin, bool kVec>
__global__ __launch_bounds__(kBlock) void verify_single(VfParams P) {
  __shared__ float redf[kWavesPerBlock];
  __shared__ int redi[kWavesPerBlock];
  __shared__ int sh_n;
  __shared__ float bcast;
  const int64_t b = blockIdx.x;
  if (P.greedy) {
    greedy_single<Tin, kVec>(P, b, redf, redi, &sh_n);
    return;
  }
  const int n = accept_scan<Tin>(P, b, &sh_n);
  float sw = 0.f, sp = 0.f;
  if (n >= 0) {
    float wv[16], pv[16];
    final_weights<Tin, kVec>(P, b, n, 0, false, wv, pv);
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      sw += wv[j];
      sp += pv[j];
    }
  }
  sw = block_sum(sw, redf);
  sp = block_sum(sp, redf);
  auto mass = [&](int k, bool use_p) -> float { return k == 0 ? (use_p ? sp : sw) : 0.f; };
  finish_sequence<Tin, kVec>(P, b, n, mass, redf, redi, &bcast);
}

// Larger vocabularies, pass 1: one workgroup per (sequence, chunk) repeats the sequence's accept
// scan, then publishes the chunk sums of the residual (or bonus) weights and of p; chunk 0 also
// records n.  Pass 2 reads them after the kernel boundary.
template <typename Tin, bool kVec>
__global__ __launch_bounds__(kBlock) void verify_partial(VfParams P) {
  __shared__ float redf[kWavesPerBlock];
  __shared__ int sh_n;
  // all chunks of a sequence on one XCD: its draft row (gathered through full_to_trim) stays in
  // that XCD's L2 instead of being fetched from the last-level cache for every random read
  const int64_t bid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t b = bid / P.nchunk;
  const int c = static_cast<int>(bid - b * P.nchunk);
  if (P.greedy) {
    __shared__ int redi[kWavesPerBlock];
    for (int i = 0; i <= P.gamma; ++i) {
      float bv;
      int bi;
      chunk_argmax<Tin, kVec>(P, b, i, c, bv, bi, redf, redi);
      if (threadIdx.x == 0) P.part[(b * (P.gamma + 1) + i) * P.nchunk + c] = make_float2(bv, __int_as_float(bi));
    }
    return;
  }
  const int n = accept_scan<Tin>(P, b, &sh_n);
  float sw = 0.f, sp = 0.f;
  if (n >= 0) {
    float wv[16], pv[16];
    final_weights<Tin, kVec>(P, b, n, c, false, wv, pv);
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      sw += wv[j];
      sp += pv[j];
    }
  }
  sw = block_sum(sw, redf);
  sp = block_sum(sp, redf);
  if (threadIdx.x == 0) {
    P.part[b * P.nchunk + c] = make_float2(sw, sp);
    if (c == 0) P.nbuf[b] = n;
  }
}

// Pass 2: one workgroup per sequence draws the final token and writes the outputs.
template <typename Tin, bool kVec>
__global__ __launch_bounds__(kBlock) void verify_final(VfParams P) {
  __shared__ float redf[kWavesPerBlock];
  __shared__ int redi[kWavesPerBlock];
  __shared__ float bcast;
  const int64_t b = blockIdx.x;
  if (P.greedy) {
    __shared__ int a[kWave + 1];
    __shared__ int sh_n;
    for (int i = 0; i <= P.gamma; ++i) {
      const float2 *pr = P.part + (b * (P.gamma + 1) + i) * P.nchunk;
      float bv = kNegInf;
      int bi = kNoIndex;
      for (int k = threadIdx.x; k < P.nchunk; k += kBlock) {
        const float2 pk = pr[k];
        if (argmax_better(pk.x, __float_as_int(pk.y), bv, bi)) {
          bv = pk.x;
          bi = __float_as_int(pk.y);
        }
      }
      block_argmax(bv, bi, redf, redi);
      if (threadIdx.x == 0) a[i] = bi;
    }
    __syncthreads();
    greedy_finish(P, b, a, &sh_n);
    return;
  }
  const int n = P.nbuf[b];
  const float2 *part = P.part + b * P.nchunk;
  auto mass = [&](int k, bool use_p) -> float {
    if (k >= P.nchunk) return 0.f;
    const float2 v = part[k];
    return use_p ? v.y : v.x;
  };
  finish_sequence<Tin, kVec>(P, b, n, mass, redf, redi, &bcast);
}

struct VFWsLayout {
  size_t nbuf, part, bytes;
};

// pass-1 results: n per sequence, and per (sequence, chunk) sums (sampling) or per (sequence,
// row, chunk) argmaxes (greedy): sized for the larger of the two.
VFWsLayout vf_ws_layout(int64_t B, int64_t gamma, int64_t nchunk) {
  VFWsLayout L{};
  if (nchunk <= 1) return L;
  L.nbuf = 0;
  L.part = align_up(static_cast<size_t>(B) * sizeof(int), 256);
  L.bytes = L.part +
            align_up(static_cast<size_t>(B) * static_cast<size_t>(gamma + 1) * static_cast<size_t>(nchunk) * sizeof(float2),
                     256);
  return L;
}

template <typename Tin, bool kVec>
hipError_t vf_launch_all(const VfParams &P, int64_t B, hipStream_t stream) {
  if (P.nchunk == 1 && P.V <= kWave)
    return launch(verify_wave<Tin>, dim3(static_cast<unsigned>((B + kWavesPerBlock - 1) / kWavesPerBlock)),
                  dim3(kBlock), 0, stream, P, B);
  if (P.nchunk == 1) return launch(verify_single<Tin, kVec>, dim3(static_cast<unsigned>(B)), dim3(kBlock), 0, stream, P);
  const hipError_t e = launch(verify_partial<Tin, kVec>, dim3(static_cast<unsigned>(B * P.nchunk)), dim3(kBlock), 0,
                              stream, P);
  if (e != hipSuccess) return e;
  return launch(verify_final<Tin, kVec>, dim3(static_cast<unsigned>(B)), dim3(kBlock), 0, stream, P);
}

template <typename Tin>
hipError_t launch_verify(const VfParams &P, bool vec, int64_t B, hipStream_t stream) {
  return vec ? vf_launch_all<Tin, true>(P, B, stream) : vf_launch_all<Tin, false>(P, B, stream);
}

}  // namespace
}  // namespace vt


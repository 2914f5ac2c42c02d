// Temperature softmax over rows of logits with an optional inverse-CDF draw (gfx950).
//
// Temperature enters every distribution the correction uses ("Speculative decoding" glossary,
// "Distributional exactness has conditions"); the draw walks the vocabulary in index order and
// returns the first token whose running mass reaches the uniform ("A rejection rule keeps
// speculative decoding's output exact", the categorical sampler of "A target and a draft small
// enough to print in full").
//
// Layout of the work: a row is cut into fixed 4096-element chunks, each thread of a 256-thread
// workgroup owning 16 contiguous elements held in registers.  Rows of one chunk finish in one
// workgroup.  Longer rows take two launches: one workgroup per (row, chunk) computes the chunk's
// (max m_c, sum s_c of exp((x - m_c)/T)); then one workgroup per row combines them into
// M = max m_c, S_c = s_c exp((m_c - M)/T), the chunk-level running sum P_c and Z = P_last, writes
// lse = M/T + ln Z in fp64, and, when asked, draws: t = u Z, c* = first chunk with t <= P_c, then
// a rescan of chunk c* finds the first element whose running sum reaches t.  The two launches
// are ordered by the stream; no device-wide fence is used (on a multi-XCD device such a fence
// writes back and invalidates the L2 of the issuing XCD).  exp(y) is evaluated as 2^(y log2 e) on v_exp_f32 with log2(e)/T folded into one
// fp32 constant, and arguments are formed relative to the row max so the heavy entries carry
// the smallest rounding.
#pragma once
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "vt_common.hpp"

namespace vt {
namespace {

struct SmParams {
  const void *logits;
  int64_t rows, n, ld;
  float k2;   // log2(e) / T
  double T;
  double invT;  // 1 / T, rounded once on the host: log-normalisers take M * invT
  double *lse;
  float *probs;
  const float *u;
  int32_t *sampled;
  float2 *rowstat;  // (M, Z) per row, for the probability pass of multi-chunk rows
  float2 *part;     // (m_c, s_c) per (row, chunk)
  int nchunk;
  int chunk;        // elements per chunk of the partials (<= 4096); 4096 for this file's own partials
  bool greedy;      // T = 0: argmax (lowest index on ties) instead of softmax; lse = row max
};

// Argmax of the thread's 16 elements starting at global index e0 (entries at e >= n never win).
__device__ __forceinline__ void thread_argmax16(const float (&v)[16], int64_t e0, int64_t n, float &bv, int &bi) {
  bv = kNegInf;
  bi = kNoIndex;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int64_t e = e0 + j;
    if (e < n && argmax_better(v[j], static_cast<int>(e), bv, bi)) {
      bv = v[j];
      bi = static_cast<int>(e);
    }
  }
}

// T = 0 (greedy limit) outputs for row r with maximum M at index idx: lse = M, probs one-hot.
__device__ __forceinline__ void greedy_outputs(const SmParams &P, int64_t r, float M, int idx) {
  if (threadIdx.x == 0) {
    P.lse[r] = static_cast<double>(M);
    if (P.sampled) P.sampled[r] = idx;
    if (P.rowstat) P.rowstat[r] = make_float2(M, __int_as_float(idx));
  }
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Weights exp((x - M)/T) of the thread's 16 elements (0 for -inf entries or an all -inf row).
__device__ __forceinline__ void weights16(const float (&v)[16], float M, float k2, float (&w)[16]) {
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) w[j] = (M == kNegInf) ? 0.f : exp2_fast((v[j] - M) * k2);
}

// Draw inside one chunk: G_j = E + prev_t + loc_j is the running sum at element j (loc = the
// thread's own sequential prefix, prev_t = the workgroup scan of thread totals before it).
// Returns the chunk-relative index of the first element with t <= G_j, or of the last element
// with positive weight when rounding leaves none.  All threads must call.
struct ChunkScan {
  float loc[16];
  float base;  // E + prev_t
};

__device__ __forceinline__ void chunk_scan(const float (&w)[16], float E, ChunkScan &cs, float *red) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    acc += w[j];
    cs.loc[j] = acc;
  }
  float prev, total;
  block_inclusive_scan(acc, red, &prev, &total);
  cs.base = E + prev;
}

__device__ __forceinline__ int chunk_find(const float (&w)[16], const ChunkScan &cs, float t, int *redi) {
  int found = 0x7fffffff;
#pragma unroll
  for (int j = kPerThread - 1; j >= 0; --j)
    if (t <= cs.base + cs.loc[j]) found = static_cast<int>(threadIdx.x) * kPerThread + j;
  found = block_min_int(found, redi);
  if (found != 0x7fffffff) return found;
  int last = -1;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j)
    if (w[j] > 0.f) last = static_cast<int>(threadIdx.x) * kPerThread + j;
  return block_max_int(last, redi);
}

// Rows of at most one chunk: the whole row lives in one workgroup.  Z is the running sum at
// the row's last element, so the draw always finds an index.
template <typename Tin, bool kVec>
__global__ __launch_bounds__(kBlock) void softmax_single(SmParams P) {
  __shared__ float redf[kWavesPerBlock];
  __shared__ int redi[kWavesPerBlock];
  __shared__ float bcast;
  const int64_t r = blockIdx.x;
  const Tin *row = reinterpret_cast<const Tin *>(P.logits) + r * P.ld;
  float v[16], w[16];
  load16<Tin, kVec>(row, P.n, 0, v);
  if (P.greedy) {
    float bv;
    int bi;
    thread_argmax16(v, static_cast<int64_t>(threadIdx.x) * kPerThread, P.n, bv, bi);
    block_argmax(bv, bi, redf, redi);
    greedy_outputs(P, r, bv, bi);
    if (P.probs) {
      float *pr = P.probs + r * P.n;
#pragma unroll
      for (int j = 0; j < kPerThread; ++j) {
        const int64_t e = static_cast<int64_t>(threadIdx.x) * kPerThread + j;
        if (e < P.n) pr[e] = e == bi ? 1.f : 0.f;
      }
    }
    return;
  }
  float m = kNegInf;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) m = fmaxf(m, v[j]);
  m = block_max(m, redf);
  weights16(v, m, P.k2, w);
  ChunkScan cs;
  chunk_scan(w, 0.f, cs, redf);
  const int last = static_cast<int>(P.n - 1);
  if (static_cast<int>(threadIdx.x) == last / kPerThread) {
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
      if (j == last % kPerThread) z = cs.base + cs.loc[j];
    bcast = z;
  }
  __syncthreads();
  const float Z = bcast;
  if (threadIdx.x == 0) P.lse[r] = static_cast<double>(m) * P.invT + log(static_cast<double>(Z));
  if (P.probs) {
    const float inv = 1.f / Z;
    float *pr = P.probs + r * P.n;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int64_t e = static_cast<int64_t>(threadIdx.x) * kPerThread + j;
      if (e < P.n) pr[e] = w[j] * inv;
    }
  }
  if (P.u) {
    const float t = P.u[r] * Z;
    const int idx = chunk_find(w, cs, t, redi);
    if (threadIdx.x == 0) P.sampled[r] = idx;
  }
}

// Rows of at most 64 elements (the toy vocabularies): one wavefront per row, four rows per
// workgroup, lane j holding element j; the same definitions as softmax_single (Z is the running
// sum at the row's last element; the draw takes the first element reaching u Z, else the last
// one with positive weight), with the row's sums as wave scans instead of workgroup scans.
template <typename Tin>
__global__ __launch_bounds__(kBlock) void softmax_wave(SmParams P) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave_id();
  if (r >= P.rows) return;  // the whole wavefront
  const int lane = lane_id();
  const bool in = lane < P.n;
  const Tin *row = reinterpret_cast<const Tin *>(P.logits) + r * P.ld;
  float x;
  if constexpr (sizeof(Tin) == 4)
    x = reinterpret_cast<const float *>(row)[in ? lane : 0];
  else
    x = bf16_to_f32(reinterpret_cast<const uint16_t *>(row)[in ? lane : 0]);
  const float v = in ? x : kNegInf;
  if (P.greedy) {
    float bv = v;
    int bi = in ? lane : kNoIndex;
    wave_argmax(bv, bi);
    if (lane == 0) {
      P.lse[r] = static_cast<double>(bv);
      if (P.sampled) P.sampled[r] = bi;
      if (P.rowstat) P.rowstat[r] = make_float2(bv, __int_as_float(bi));
    }
    if (P.probs && in) P.probs[r * P.n + lane] = lane == bi ? 1.f : 0.f;
    return;
  }
  const float M = wave_max(v);
  const float w = M == kNegInf ? 0.f : exp2_fast((v - M) * P.k2);
  const float C = wave_scan_incl(w);
  const float Z = lane_value(C, static_cast<int>(P.n) - 1);
  if (lane == 0) P.lse[r] = static_cast<double>(M) * P.invT + log(static_cast<double>(Z));
  if (P.probs && in) P.probs[r * P.n + lane] = w * (1.f / Z);
  if (P.u) {
    const float t = P.u[r] * Z;
    const unsigned long long hit = __ballot(in && t <= C);
    int idx;
    if (hit) {
      idx = __ffsll(static_cast<long long>(hit)) - 1;
    } else {
      const unsigned long long pos = __ballot(in && w > 0.f);
      idx = pos ? 63 - __clzll(static_cast<long long>(pos)) : -1;
    }
    if (lane == 0) P.sampled[r] = idx;
  }
}

// Rows of several chunks, pass 1: one workgroup per (row, chunk) publishes the chunk's
// (max m_c, sum s_c of exp((x - m_c)/T)).  The next launch reads them (kernel boundaries order
// the two passes; no device-wide fences are needed).
// Workgroup `bid` of the pass: row bid / nchunk, chunk bid % nchunk.  Also run by extra
// workgroups of the batch-1 LM-head launch, so it takes its index as an argument.
template <typename Tin, bool kVec>
__device__ __forceinline__ void partial_chunk(const SmParams &P, int64_t bid) {
  __shared__ float redf[kWavesPerBlock];
  const int64_t r = bid / P.nchunk;
  const int c = static_cast<int>(bid - r * P.nchunk);
  const Tin *row = reinterpret_cast<const Tin *>(P.logits) + r * P.ld;
  float v[16], w[16];
  load16<Tin, kVec>(row, P.n, static_cast<int64_t>(c) * kChunk, v);
  if (P.greedy) {
    __shared__ int redi[kWavesPerBlock];
    float bv;
    int bi;
    thread_argmax16(v, static_cast<int64_t>(c) * kChunk + static_cast<int64_t>(threadIdx.x) * kPerThread, P.n, bv,
                    bi);
    block_argmax(bv, bi, redf, redi);
    if (threadIdx.x == 0) P.part[r * P.nchunk + c] = make_float2(bv, __int_as_float(bi));
    return;
  }
  float m = kNegInf;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) m = fmaxf(m, v[j]);
  m = block_max(m, redf);
  weights16(v, m, P.k2, w);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) s += w[j];
  s = block_sum(s, redf);
  if (threadIdx.x == 0) P.part[r * P.nchunk + c] = make_float2(m, s);
}

template <typename Tin, bool kVec>
__global__ __launch_bounds__(kBlock) void softmax_partial(SmParams P) {
  partial_chunk<Tin, kVec>(P, blockIdx.x);
}

// Pass 2 for one row r: combine the chunks into M = max m_c, S_c = s_c exp((m_c - M)/T), the
// chunk-level running sum P_c and Z = P_last; write lse = M/T + ln Z in fp64; draw by locating the
// chunk (first c with u Z <= P_c) and rescanning it.  Chunks hold P.chunk (<= 4096) elements.
template <typename Tin, bool kVec>
__device__ __forceinline__ void combine_row(const SmParams &P, int64_t r, float *redf, int *redi, float *bcast) {
  const Tin *row = reinterpret_cast<const Tin *>(P.logits) + r * P.ld;
  const float2 *part = P.part + r * P.nchunk;
  if (P.greedy) {
    float bv = kNegInf;
    int bi = kNoIndex;
    for (int k = threadIdx.x; k < P.nchunk; k += kBlock) {
      const float2 pk = part[k];
      if (argmax_better(pk.x, __float_as_int(pk.y), bv, bi)) {
        bv = pk.x;
        bi = __float_as_int(pk.y);
      }
    }
    block_argmax(bv, bi, redf, redi);
    greedy_outputs(P, r, bv, bi);
    return;
  }
  float mm = kNegInf;
  for (int k = threadIdx.x; k < P.nchunk; k += kBlock) mm = fmaxf(mm, part[k].x);
  const float M = block_max(mm, redf);
  auto chunk_mass = [&](int k) -> float {
    if (k >= P.nchunk) return 0.f;
    const float2 ps = part[k];
    return (ps.x == kNegInf) ? 0.f : ps.y * exp2_fast((ps.x - M) * P.k2);
  };
  // chunk-level running sum in passes of 256 chunks with a carry; Z is its last value
  float carry = 0.f;
  for (int k0 = 0; k0 < P.nchunk; k0 += kBlock) {
    float prev, total;
    block_inclusive_scan(chunk_mass(k0 + threadIdx.x), redf, &prev, &total);
    carry = carry + total;
  }
  const float Z = carry;
  if (threadIdx.x == 0) {
    P.lse[r] = static_cast<double>(M) * P.invT + log(static_cast<double>(Z));
    if (P.rowstat) P.rowstat[r] = make_float2(M, Z);
  }
  if (!P.u) return;

  const float t = P.u[r] * Z;
  int cstar = 0x7fffffff;
  float Estar = 0.f;
  carry = 0.f;
  for (int k0 = 0; k0 < P.nchunk; k0 += kBlock) {
    float prev, total;
    const float incl = block_inclusive_scan(chunk_mass(k0 + threadIdx.x), redf, &prev, &total);
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
    // u Z beyond the running sum (only for u > 1 or NaN): last chunk with positive mass
    int lastc = -1;
    for (int k = threadIdx.x; k < P.nchunk; k += kBlock)
      if (chunk_mass(k) > 0.f) lastc = k;
    cstar = max(block_max_int(lastc, redi), 0);  // never below chunk 0
    fallback = true;
  }
  const int64_t c0 = static_cast<int64_t>(cstar) * P.chunk;
  const int64_t c1 = c0 + P.chunk < P.n ? c0 + P.chunk : P.n;
  float v[16], w[16];
  load16<Tin, kVec>(row, c1, c0, v);
  weights16(v, M, P.k2, w);
  ChunkScan cs;
  chunk_scan(w, fallback ? 0.f : Estar, cs, redf);
  const int idx = chunk_find(w, cs, fallback ? __builtin_huge_valf() : t, redi);
  if (threadIdx.x == 0) P.sampled[r] = static_cast<int32_t>(c0 + idx);
}

// Pass 2: one workgroup per row.
template <typename Tin, bool kVec>
__global__ __launch_bounds__(kBlock) void softmax_combine(SmParams P) {
  __shared__ float redf[kWavesPerBlock];
  __shared__ int redi[kWavesPerBlock];
  __shared__ float bcast;
  combine_row<Tin, kVec>(P, blockIdx.x, redf, redi, &bcast);
}

// Pass 2 for two row sets in one launch: workgroups [0, A.rows) take A's rows, the rest B's.
template <typename TinA, bool kVecA, typename TinB, bool kVecB>
__global__ __launch_bounds__(kBlock) void softmax_combine2(SmParams A, SmParams B) {
  __shared__ float redf[kWavesPerBlock];
  __shared__ int redi[kWavesPerBlock];
  __shared__ float bcast;
  const int64_t r = blockIdx.x;
  if (r < A.rows)
    combine_row<TinA, kVecA>(A, r, redf, redi, &bcast);
  else
    combine_row<TinB, kVecB>(B, r - A.rows, redf, redi, &bcast);
}

// Probabilities for rows spanning several chunks: exp((x - M)/T) / Z with the row's (M, Z).
template <typename Tin, bool kVec>
__global__ __launch_bounds__(kBlock) void softmax_probs(SmParams P) {
  const int64_t bid = blockIdx.x;
  const int64_t r = bid / P.nchunk;
  const int c = static_cast<int>(bid - r * P.nchunk);
  const Tin *row = reinterpret_cast<const Tin *>(P.logits) + r * P.ld;
  float v[16], w[16];
  const float2 mz = P.rowstat[r];
  if (P.greedy) {
    const int64_t idx = __float_as_int(mz.y);
    float *pr = P.probs + r * P.n;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int64_t e = static_cast<int64_t>(c) * kChunk + static_cast<int64_t>(threadIdx.x) * kPerThread + j;
      if (e < P.n) pr[e] = e == idx ? 1.f : 0.f;
    }
    return;
  }
  load16<Tin, kVec>(row, P.n, static_cast<int64_t>(c) * kChunk, v);
  weights16(v, mz.x, P.k2, w);
  const float inv = 1.f / mz.y;
  float *pr = P.probs + r * P.n;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int64_t e = static_cast<int64_t>(c) * kChunk + static_cast<int64_t>(threadIdx.x) * kPerThread + j;
    if (e < P.n) pr[e] = w[j] * inv;
  }
}

struct SMWsLayout {
  size_t rowstat, part, bytes;
};

SMWsLayout sm_ws_layout(int64_t rows, int64_t nchunk) {
  SMWsLayout L{};
  if (nchunk <= 1) return L;
  L.rowstat = 0;
  L.part = align_up(static_cast<size_t>(rows) * sizeof(float2), 256);
  L.bytes = L.part + align_up(static_cast<size_t>(rows) * static_cast<size_t>(nchunk) * sizeof(float2), 256);
  return L;
}

template <typename Tin, bool kVec>
hipError_t sm_launch_all(const SmParams &P, hipStream_t stream) {
  const unsigned rows = static_cast<unsigned>(P.rows);
  if (P.nchunk == 1 && P.n <= kWave)
    return launch(softmax_wave<Tin>, dim3(static_cast<unsigned>((P.rows + kWavesPerBlock - 1) / kWavesPerBlock)),
                  dim3(kBlock), 0, stream, P);
  if (P.nchunk == 1) return launch(softmax_single<Tin, kVec>, dim3(rows), dim3(kBlock), 0, stream, P);
  const unsigned grid = static_cast<unsigned>(P.rows * P.nchunk);
  hipError_t e = launch(softmax_partial<Tin, kVec>, dim3(grid), dim3(kBlock), 0, stream, P);
  if (e != hipSuccess) return e;
  e = launch(softmax_combine<Tin, kVec>, dim3(rows), dim3(kBlock), 0, stream, P);
  if (e != hipSuccess || !P.probs) return e;
  return launch(softmax_probs<Tin, kVec>, dim3(grid), dim3(kBlock), 0, stream, P);
}

template <typename Tin>
hipError_t sm_launch_dtype(const SmParams &P, bool vec, hipStream_t stream) {
  return vec ? sm_launch_all<Tin, true>(P, stream) : sm_launch_all<Tin, false>(P, stream);
}

}  // namespace
}  // namespace vt


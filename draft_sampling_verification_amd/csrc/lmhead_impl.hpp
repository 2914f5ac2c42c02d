// Trimmed LM head for gfx950: logits[m][j] = sum_k hidden[m][k] * weight[row(j)][k],
// row(j) = keep_ids ? keep_ids[j] : j  ("VocabTrim", §3 Eq. 1; Appendix C.1, Algorithm 2).
//
// Two kernels, picked by the number of hidden rows M:
//  * lmhead_gemv  (M small): the batch-1 decode case.  The head is read once from HBM and every
//    weight row is used M times, so the kernel is bandwidth-bound.  Each wavefront owns whole
//    weight rows; lane l reads 16-byte pieces l, l+64, ... of a row (coalesced 1 KiB per load
//    instruction, non-temporal since the head is streamed once), multiplies them with the
//    matching pieces of the M hidden rows held in its registers using v_dot2 (bf16 pairs,
//    fp32 accumulate), and the 64 lane partials are combined by a transpose-reduction.
//  * lmhead_mfma  (M large): a real dense contraction; 128x128 output tiles on bf16 MFMA
//    (v_mfma_f32_32x32x16_bf16) with LDS double buffering, weight rows gathered through
//    keep_ids while staging the tile.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "softmax_impl.hpp"
#include "vt_common.hpp"

namespace vt {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float dot8(const uint4 &w, const uint4 &h, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.x), __builtin_bit_cast(bf16x2, h.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.y), __builtin_bit_cast(bf16x2, h.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.z), __builtin_bit_cast(bf16x2, h.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.w), __builtin_bit_cast(bf16x2, h.w), acc, false);
  return acc;
}

__device__ __forceinline__ uint4 load_nt(const uint4 *p) {
  uint4 r;
  r.x = __builtin_nontemporal_load(&reinterpret_cast<const unsigned int *>(p)[0]);
  r.y = __builtin_nontemporal_load(&reinterpret_cast<const unsigned int *>(p)[1]);
  r.z = __builtin_nontemporal_load(&reinterpret_cast<const unsigned int *>(p)[2]);
  r.w = __builtin_nontemporal_load(&reinterpret_cast<const unsigned int *>(p)[3]);
  return r;
}

// Reduction over each half-wave (lanes 0..31 and 32..63), the result in every lane of the half:
// quad steps (lane ^ 1, ^ 2), then the mirrors within 8 and 16 lanes (after each step a lane's
// partner holds the other half of its group), then lane ^ 16 -- all DPP / permlane moves, no LDS.
template <typename Op>
__device__ __forceinline__ float half_wave_reduce(float v, Op op) {
  v = op(v, dpp<kDppXor1>(v));
  v = op(v, dpp<kDppXor2>(v));
  v = op(v, dpp<kDppHalfMirror>(v));
  v = op(v, dpp<kDppMirror>(v));
  float a = v, b = v;
  swap16(a, b);
  return op(a, b);
}

// One step of a reduce-scatter over a half-wave: the lanes at one distance (16: row swap; 8:
// rotation of the row by 8; 4: mirror of each group of 8, whose lanes hold the same entries by
// then; 2 and 1: quad permutations) pair up and each keeps the half of its N entries that its
// partner gives up, reduced with the partner's copy.
template <int CTRL, int BIT, int H, typename Op, int N>
__device__ __forceinline__ void scatter_step(float (&v)[N], Op op) {
  const bool up = (lane_id() & BIT) != 0;
#pragma unroll
  for (int k = 0; k < H; ++k) {
    const float send = up ? v[k] : v[k + H];
    const float keep = up ? v[k + H] : v[k];
    v[k] = op(keep, lane_swap<CTRL>(send));
  }
}
// The movement of scatter_step reversed: each lane ends with its own H entries and its partner's.
template <int CTRL, int BIT, int H, int N>
__device__ __forceinline__ void gather_step(float (&v)[N]) {
  const bool up = (lane_id() & BIT) != 0;
#pragma unroll
  for (int k = 0; k < H; ++k) {
    const float mine = v[k];
    const float other = lane_swap<CTRL>(mine);
    v[k] = up ? other : mine;
    v[k + H] = up ? mine : other;
  }
}

// Reduce-scatter of 16 per-lane entries over each half-wave: steps at lane distances 16 (the row
// swap of v_permlane16_swap), 8, 4 and 2 (scatter_step), each halving what a lane carries, then a
// plain reduction with the lane at distance 1; afterwards v[0] holds the reduction over the
// half's 32 lanes of entry (lane & 31) >> 1.  16 exchanges instead of 5 for each of 16 entries.
template <typename Op>
__device__ __forceinline__ void half_reduce_scatter16(float (&v)[16], Op op) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float a = v[k], b = v[k + 8];
    swap16(a, b);
    v[k] = op(a, b);
  }
  scatter_step<kDppRor8, 8, 4>(v, op);
  scatter_step<kDppHalfMirror, 4, 2>(v, op);
  scatter_step<kDppXor2, 2, 1>(v, op);
  v[0] = op(v[0], lane_swap<kDppXor1>(v[0]));
}

// The movement of half_reduce_scatter16 reversed: from v[0] = entry (lane & 31) >> 1, every lane
// of the half ends with all 16 entries in order.  15 exchanges.
__device__ __forceinline__ void half_all_gather16(float (&v)[16]) {
  gather_step<kDppXor2, 2, 1>(v);
  gather_step<kDppHalfMirror, 4, 2>(v);
  gather_step<kDppRor8, 8, 4>(v);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float a = v[k], b = v[k];
    swap16(a, b);
    v[k] = a;
    v[k + 8] = b;
  }
}

// Argmax over each half-wave of 16 per-lane (value, index) entries, by the same steps as
// half_reduce_scatter16 with the pair moved together: afterwards (v[0], ix[0]) is the largest
// value of entry (lane & 31) >> 1 over the half's 32 lanes, the lowest index among equal values.
template <int CTRL, int BIT, int H>
__device__ __forceinline__ void argmax_step(float (&v)[16], int (&ix)[16]) {
  const bool up = (lane_id() & BIT) != 0;
#pragma unroll
  for (int k = 0; k < H; ++k) {
    const float sv = up ? v[k] : v[k + H], kv = up ? v[k + H] : v[k];
    const int si = up ? ix[k] : ix[k + H], ki = up ? ix[k + H] : ix[k];
    const float ov = lane_swap<CTRL>(sv);
    const int oi = lane_swap<CTRL>(si);
    const bool take = argmax_better(ov, oi, kv, ki);
    v[k] = take ? ov : kv;
    ix[k] = take ? oi : ki;
  }
}
__device__ __forceinline__ void half_argmax_scatter16(float (&v)[16], int (&ix)[16]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float a = v[k], b = v[k + 8];
    float ia = __int_as_float(ix[k]), ib = __int_as_float(ix[k + 8]);
    swap16(a, b);
    swap16(ia, ib);
    const bool take = argmax_better(b, __float_as_int(ib), a, __float_as_int(ia));
    v[k] = take ? b : a;
    ix[k] = take ? __float_as_int(ib) : __float_as_int(ia);
  }
  argmax_step<kDppRor8, 8, 4>(v, ix);
  argmax_step<kDppHalfMirror, 4, 2>(v, ix);
  argmax_step<kDppXor2, 2, 1>(v, ix);
  const float ov = lane_swap<kDppXor1>(v[0]);
  const int oi = lane_swap<kDppXor1>(ix[0]);
  if (argmax_better(ov, oi, v[0], ix[0])) {
    v[0] = ov;
    ix[0] = oi;
  }
}

// Transpose-reduction of NP (1, 2, 4 or 8) per-lane partial sums over the 64 lanes.  The steps
// at lane distance 32, 16 and 8 halve the number of values each lane carries (each lane keeps
// the half its partner gives up), the remaining steps add within groups of 64/NP lanes.  On
// return lane l holds the complete sum of value index l / (64 / NP).  About NP + 6 exchanges
// instead of 6 * NP for NP separate reductions.
template <int NP>
__device__ __forceinline__ float transpose_reduce(float (&v)[NP]) {
  if constexpr (NP >= 2) {
#pragma unroll
    for (int k = 0; k < NP / 2; ++k) {
      float a = v[k], b = v[k + NP / 2];
      swap32(a, b);
      v[k] = a + b;
    }
  } else {
    float a = v[0], b = v[0];
    swap32(a, b);
    v[0] = a + b;
  }
  if constexpr (NP >= 4) {
#pragma unroll
    for (int k = 0; k < NP / 4; ++k) {
      float a = v[k], b = v[k + NP / 4];
      swap16(a, b);
      v[k] = a + b;
    }
  } else {
    float a = v[0], b = v[0];
    swap16(a, b);
    v[0] = a + b;
  }
  if constexpr (NP >= 8) {
    const bool up = (lane_id() & 8) != 0;
#pragma unroll
    for (int k = 0; k < NP / 8; ++k) {
      const float send = up ? v[k] : v[k + NP / 8];
      const float keep = up ? v[k + NP / 8] : v[k];
      v[k] = keep + dpp<kDppRor8>(send);
    }
  } else {
    v[0] += dpp<kDppRor8>(v[0]);
  }
  v[0] += dpp<kDppHalfMirror>(v[0]);
  v[0] += dpp<kDppXor2>(v[0]);
  v[0] += dpp<kDppXor1>(v[0]);
  return v[0];
}

template <int N>
struct Pow2Ceil {
  static constexpr int value = N <= 1 ? 1 : 2 * Pow2Ceil<(N + 1) / 2>::value;
};
template <>
struct Pow2Ceil<1> {
  static constexpr int value = 1;
};

// Row of the full head behind kept row j: keep_ids[j], clamped into [0, vrows) so that an id out of
// range (a violated precondition) gives unspecified logits but never a read outside the head.
__device__ __forceinline__ int64_t kept_row(const int32_t *__restrict__ keep, int j, int vrows) {
  return static_cast<int64_t>(min(static_cast<uint32_t>(keep[j]), static_cast<uint32_t>(vrows - 1)));
}

constexpr int kGemvPrefetch = 2;  // weight rows in flight per wavefront beyond the one in use

// Rows per workgroup block: the head is cut into contiguous blocks of `per` rows (a multiple of 4,
// one block per workgroup), sized for one workgroup per CU of a 256-CU device.  The size depends
// only on Vt, so results never depend on the device or on the batch.
inline int gemv_rows_per_block(int64_t Vt) {
  const int64_t per = (Vt + 255) / 256;
  return static_cast<int>((per + kWavesPerBlock - 1) / kWavesPerBlock * kWavesPerBlock);
}
inline int gemv_blocks(int64_t Vt) {
  const int per = gemv_rows_per_block(Vt);
  return static_cast<int>((Vt + per - 1) / per);
}

// Draft softmax partials produced by the GEMV epilogue (optional): for every hidden row m and
// workgroup block k, (max_j x_mj, sum_j exp((x_mj - max) / T)) over the block's rows j, written
// to part[m * nblocks + k] (k2 = log2(e) / T).
// The batch-1 block also hands the GEMV launch the target rows' first softmax pass: workgroups
// past the head's row blocks each take one (row, 4096-chunk) of the target logits (tsel: 0 none,
// 1 fp32 16-byte loads, 2 fp32 element loads, 3 bf16 16-byte loads, 4 bf16 element loads), so
// that pass overlaps the head instead of preceding it.
struct GemvParts {
  float2 *part;
  float k2;
  SmParams tgt;
  int tsel;
};

__device__ __forceinline__ void target_partial_chunk(const GemvParts &parts, int64_t t) {
  switch (parts.tsel) {
    case 1: partial_chunk<float, true>(parts.tgt, t); break;
    case 2: partial_chunk<float, false>(parts.tgt, t); break;
    case 3: partial_chunk<uint16_t, true>(parts.tgt, t); break;
    case 4: partial_chunk<uint16_t, false>(parts.tgt, t); break;
    default: break;
  }
}

// Workgroup k owns head rows [k * per, (k + 1) * per); its four wavefronts take every fourth row of
// the block, so the workgroup streams one contiguous region of the head (measured ~10% faster than
// a grid-stride walk).  A ring of PD + 1 register buffers keeps PD rows in flight while one is
// multiplied.  Every load is unconditional and in bounds (row indices past the wave's last row
// repeat the last row, pieces past H repeat the last piece and are masked), so the compiler can
// wait for exactly the oldest row (vmcnt(N)) instead of draining the queue.  FULL: H is a multiple
// of 512 (no masking at all).  TRIM: rows are gathered through keep_ids.  PARTS = kPartsSoftmax:
// also produce the draft softmax partials of the block (online max / sum per hidden row, combined
// over the four wavefronts through LDS), so the softmax never re-reads the logits for its first
// pass; kPartsArgmax: the block's (max, lowest index of the max) per hidden row instead, for
// argmax drafts.
constexpr int kPartsNone = 0, kPartsSoftmax = 1, kPartsArgmax = 2;

template <int M, int NIT, int PD, bool FULL, bool TRIM, int PARTS>
__global__ __launch_bounds__(kBlock) void lmhead_gemv(const uint16_t *__restrict__ hidden,
                                                      const uint16_t *__restrict__ weight,
                                                      const int32_t *__restrict__ keep, int vrows, int H, int Vt,
                                                      int per, float *__restrict__ logits, GemvParts parts) {
  constexpr int NP = Pow2Ceil<M>::value;
  constexpr int kGroup = kWave / NP;
  const int nblk = (Vt + per - 1) / per;
  if constexpr (PARTS != kPartsNone) {
    if (static_cast<int>(blockIdx.x) >= nblk) {
      target_partial_chunk(parts, static_cast<int64_t>(blockIdx.x) - nblk);
      return;
    }
  }
  const int lane = lane_id();
  const int pieces = H >> 3;  // 16-byte pieces per row
  auto piece = [&](int it) -> int {
    const int p = it * kWave + lane;
    return (FULL || it < NIT - 1) ? p : min(p, pieces - 1);
  };
  auto live = [&](int it) -> bool { return FULL || it < NIT - 1 || it * kWave + lane < pieces; };

  uint4 h[M][NIT];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const uint4 v = reinterpret_cast<const uint4 *>(hidden + static_cast<int64_t>(m) * H)[piece(it)];
      h[m][it] = live(it) ? v : make_uint4(0, 0, 0, 0);
    }

  const int wid = __builtin_amdgcn_readfirstlane(wave_id());
  const int base = static_cast<int>(blockIdx.x) * per;
  const int wv = base + wid;
  const int end = min(Vt, base + per);
  const int nrows = wv < end ? (end - 1 - wv) / kWavesPerBlock + 1 : 0;
  auto row_of = [&](int t) { return wv + t * kWavesPerBlock; };
  const int mrow = lane / kGroup;  // hidden row whose sum this lane holds after the reduction
  float pmax = kNegInf, psum = 0.f;
  int pidx = kNoIndex;

  auto fetch = [&](int t, uint4(&dst)[NIT]) {
    const int j = row_of(min(t, nrows - 1));  // wave-uniform
    int64_t r = j;
    if constexpr (TRIM) r = kept_row(keep, j, vrows);
    const uint4 *src = reinterpret_cast<const uint4 *>(weight + r * H);
#pragma unroll
    for (int it = 0; it < NIT; ++it) dst[it] = load_nt(src + piece(it));
  };
  auto consume = [&](int t, const uint4(&src)[NIT]) {
    float acc[NP];
#pragma unroll
    for (int m = 0; m < NP; ++m) acc[m] = 0.f;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const uint4 wv4 = live(it) ? src[it] : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m] = dot8(wv4, h[m][it], acc[m]);
    }
    const float sum = transpose_reduce<NP>(acc);
    if ((lane % kGroup) == 0 && mrow < M) logits[static_cast<int64_t>(mrow) * Vt + row_of(t)] = sum;
    if constexpr (PARTS == kPartsSoftmax) {
      const float nm = fmaxf(pmax, sum);
      psum = psum * __builtin_amdgcn_exp2f((pmax - nm) * parts.k2) + __builtin_amdgcn_exp2f((sum - nm) * parts.k2);
      pmax = nm;
    } else if constexpr (PARTS == kPartsArgmax) {
      if (argmax_better(sum, row_of(t), pmax, pidx)) {
        pmax = sum;
        pidx = row_of(t);
      }
    }
  };

  if (nrows > 0) {
    uint4 w[PD + 1][NIT];
#pragma unroll
    for (int s = 0; s < PD; ++s) fetch(s, w[s]);
    // whole groups of PD + 1 rows: straight-line code, so each multiply waits only for its own row
    int t0 = 0;
    for (; t0 + PD < nrows; t0 += PD + 1) {
#pragma unroll
      for (int s = 0; s <= PD; ++s) {
        fetch(t0 + s + PD, w[(s + PD) % (PD + 1)]);
        consume(t0 + s, w[s]);
      }
    }
    // the last rows (fewer than PD + 1) are already in flight
#pragma unroll
    for (int s = 0; s < PD; ++s)
      if (t0 + s < nrows) consume(t0 + s, w[s]);
  }

  if constexpr (PARTS == kPartsArgmax) {
    __shared__ float2 wbest[kWavesPerBlock][NP];
    if ((lane % kGroup) == 0) wbest[wid][mrow] = make_float2(pmax, __int_as_float(pidx));
    __syncthreads();
    if (threadIdx.x < M) {
      const int m = threadIdx.x;
      float bv = kNegInf;
      int bi = kNoIndex;
#pragma unroll
      for (int w = 0; w < kWavesPerBlock; ++w) {
        const float2 v = wbest[w][m];
        if (argmax_better(v.x, __float_as_int(v.y), bv, bi)) {
          bv = v.x;
          bi = __float_as_int(v.y);
        }
      }
      parts.part[static_cast<int64_t>(m) * nblk + blockIdx.x] = make_float2(bv, __int_as_float(bi));
    }
  }
  if constexpr (PARTS == kPartsSoftmax) {
    __shared__ float2 wpart[kWavesPerBlock][NP];
    if ((lane % kGroup) == 0) wpart[wid][mrow] = make_float2(pmax, psum);
    __syncthreads();
    if (threadIdx.x < M) {
      const int m = threadIdx.x;
      float mx = kNegInf;
#pragma unroll
      for (int w = 0; w < kWavesPerBlock; ++w) mx = fmaxf(mx, wpart[w][m].x);
      float sx = 0.f;
#pragma unroll
      for (int w = 0; w < kWavesPerBlock; ++w) {
        const float2 v = wpart[w][m];
        if (v.x != kNegInf) sx += v.y * __builtin_amdgcn_exp2f((v.x - mx) * parts.k2);
      }
      parts.part[static_cast<int64_t>(m) * nblk + blockIdx.x] = make_float2(mx, sx);
    }
  }
}

// ------------------------------------------------------------------------------ MFMA path
constexpr int kBM = 128, kBN = 128, kBK = 32, kLdsPad = 8;
constexpr int kLdsRow = kBK + kLdsPad;  // bf16 elements per LDS row (80 bytes)

__global__ __launch_bounds__(kBlock) void lmhead_mfma(const uint16_t *__restrict__ hidden,
                                                      const uint16_t *__restrict__ weight,
                                                      const int32_t *__restrict__ keep, int vrows, int M, int H,
                                                      int Vt, float *__restrict__ logits) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kBM * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kBN * kLdsRow];

  const int nbm = (M + kBM - 1) / kBM;
  const int nbn = (Vt + kBN - 1) / kBN;
  const int tile = static_cast<int>(xcd_remap(blockIdx.x, static_cast<int64_t>(nbm) * nbn));
  const int bm = tile % nbm, bn = tile / nbm;
  const int m0 = bm * kBM, n0 = bn * kBN;

  const int tid = threadIdx.x;
  // staging: 128 rows x 4 pieces of 8 bf16 per operand = 512 pieces, 2 per thread each
  int a_row[2], b_row[2], piece[2];
  const uint16_t *a_src[2];
  const uint16_t *b_src[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int c = tid + s * kBlock;
    a_row[s] = c >> 2;
    b_row[s] = c >> 2;
    piece[s] = c & 3;
    const int gm = m0 + a_row[s];
    a_src[s] = gm < M ? hidden + static_cast<int64_t>(gm) * H : nullptr;
    const int gn = n0 + b_row[s];
    if (gn < Vt) {
      const int64_t r = keep ? kept_row(keep, gn, vrows) : static_cast<int64_t>(gn);
      b_src[s] = weight + r * H;
    } else {
      b_src[s] = nullptr;
    }
  }
  auto fetch = [&](int k0, uint4 (&ra)[2], uint4 (&rb)[2]) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int k = k0 + piece[s] * 8;
      const bool kin = k < H;
      ra[s] = (a_src[s] && kin) ? *reinterpret_cast<const uint4 *>(a_src[s] + k) : make_uint4(0, 0, 0, 0);
      rb[s] = (b_src[s] && kin) ? *reinterpret_cast<const uint4 *>(b_src[s] + k) : make_uint4(0, 0, 0, 0);
    }
  };
  auto stage = [&](int buf, const uint4 (&ra)[2], const uint4 (&rb)[2]) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      *reinterpret_cast<uint4 *>(&sA[buf][a_row[s] * kLdsRow + piece[s] * 8]) = ra[s];
      *reinterpret_cast<uint4 *>(&sB[buf][b_row[s] * kLdsRow + piece[s] * 8]) = rb[s];
    }
  };

  // 4 waves in a 2x2 arrangement, each owning a 64x64 output block = 2x2 MFMA tiles of 32x32
  const int w = wave_id();
  const int wm = (w >> 1) * 64, wn = (w & 1) * 64;
  const int lane = lane_id();
  const int lr = lane & 31, lk = (lane >> 5) * 8;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][jj][v] = 0.f;

  uint4 ra[2], rb[2];
  fetch(0, ra, rb);
  stage(0, ra, rb);
  __syncthreads();
  const int nk = (H + kBK - 1) / kBK;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) fetch((kt + 1) * kBK, ra, rb);
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 16) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8 *>(&sA[cur][(wm + i * 32 + lr) * kLdsRow + kk + lk]);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        b[jj] = *reinterpret_cast<const bf16x8 *>(&sB[cur][(wn + jj * 32 + lr) * kLdsRow + kk + lk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[jj], acc[i][jj], 0, 0, 0);
    }
    if (kt + 1 < nk) stage(cur ^ 1, ra, rb);
    __syncthreads();
  }

  // 32x32 accumulator layout: lane l holds column l % 32; register v holds row
  // 8 * (v / 4) + 4 * (l / 32) + v % 4.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int gn = n0 + wn + jj * 32 + lr;
      if (gn >= Vt) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int gm = m0 + wm + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (gm < M) logits[static_cast<int64_t>(gm) * Vt + gn] = acc[i][jj][v];
      }
    }
}

// ------------------------------------------------------------------------------ dispatch
using GemvFn = void (*)(const uint16_t *, const uint16_t *, const int32_t *, int, int, int, int, float *, GemvParts);

constexpr int kGemvMaxM = 8;
constexpr int kGemvMaxNit = 8;
constexpr int kGemvMaxRegs = 48;  // M * NIT: the hidden slice lives in 4 * M * NIT VGPRs

template <int M, int NIT, int PARTS>
GemvFn gemv_entry(bool full, bool trim) {
  if constexpr (M * NIT > kGemvMaxRegs) {
    return nullptr;
  } else {
    constexpr int PD = kGemvPrefetch;
    if (full)
      return trim ? &lmhead_gemv<M, NIT, PD, true, true, PARTS> : &lmhead_gemv<M, NIT, PD, true, false, PARTS>;
    return trim ? &lmhead_gemv<M, NIT, PD, false, true, PARTS> : &lmhead_gemv<M, NIT, PD, false, false, PARTS>;
  }
}

template <int M, int PARTS>
GemvFn gemv_for_nit(int nit, bool full, bool trim) {
  switch (nit) {
    case 1: return gemv_entry<M, 1, PARTS>(full, trim);
    case 2: return gemv_entry<M, 2, PARTS>(full, trim);
    case 3: return gemv_entry<M, 3, PARTS>(full, trim);
    case 4: return gemv_entry<M, 4, PARTS>(full, trim);
    case 5: return gemv_entry<M, 5, PARTS>(full, trim);
    case 6: return gemv_entry<M, 6, PARTS>(full, trim);
    case 7: return gemv_entry<M, 7, PARTS>(full, trim);
    case 8: return gemv_entry<M, 8, PARTS>(full, trim);
    default: return nullptr;
  }
}

// The GEMV kernel for (M, H), or nullptr when the shape needs the MFMA kernel.
template <int PARTS>
GemvFn pick_gemv(int64_t M, int64_t H, bool trim) {
  const int nit = static_cast<int>((H + 511) / 512);
  const bool full = H % 512 == 0;
  if (nit > kGemvMaxNit || M > kGemvMaxM || M * nit > kGemvMaxRegs) return nullptr;
  switch (M) {
    case 1: return gemv_for_nit<1, PARTS>(nit, full, trim);
    case 2: return gemv_for_nit<2, PARTS>(nit, full, trim);
    case 3: return gemv_for_nit<3, PARTS>(nit, full, trim);
    case 4: return gemv_for_nit<4, PARTS>(nit, full, trim);
    case 5: return gemv_for_nit<5, PARTS>(nit, full, trim);
    case 6: return gemv_for_nit<6, PARTS>(nit, full, trim);
    case 7: return gemv_for_nit<7, PARTS>(nit, full, trim);
    case 8: return gemv_for_nit<8, PARTS>(nit, full, trim);
    default: return nullptr;
  }
}

// ---------------------------------------------------------- batches past the GEMV (MFMA tiles)
//
// 256 x 256 output tiles (hidden rows x head rows), K in steps of 64, one workgroup of four waves
// per CU (the double-buffered tiles take 144 KB of LDS).  Each wave owns a 128 x 128 quarter as
// 4 x 4 v_mfma_f32_32x32x16_bf16 accumulators, so every 16-deep slice reads 4 + 4 fragments from
// LDS for 16 MFMAs (half the LDS traffic per MFMA of a 64 x 64 wave tile).  The next K step is
// fetched into registers while the current one is multiplied.  Loads are unconditional: rows past
// M or Vt repeat the last row (their outputs are never stored) and pieces past H are zeroed.
// PARTS: the epilogue also emits the draft softmax partials of the tile's 256 columns per hidden
// row (max and sum of 2^((x - max) k2)), combined across the two waves that share rows.
constexpr int kBigBM = 256, kBigBN = 256, kBigBK = 64, kBigPad = 8;
constexpr int kBigRow = kBigBK + kBigPad;  // bf16 per LDS row: 144 bytes
constexpr int kBigMinM = 129;  // with H % 32 != 0: register-staged 256 x 256 tiles from here, 128 x 128 below

// Tile order of the 256 x 256 kernels.  Each XCD works through one contiguous range of logical
// tiles (xcd_remap); logical tiles are ordered in groups of kTileGroup hidden-row blocks, walked
// head-block-major inside a group, so the 32 tiles an XCD runs at once span about three hidden-row
// blocks and eleven head-row blocks and share both in its L2.  Measured on the large-drafter
// shape (9 x 256 tiles) against groups of 1, 2, 4 and 9 rows: 3 is the fastest (about 5% over 9).
constexpr int kTileGroup = 3;
__device__ __forceinline__ void big_tile_of(int tile, int nbm, int nbn, int &bm, int &bn) {
  const int group = tile / (kTileGroup * nbn);
  const int in = tile - group * kTileGroup * nbn;
  const int rows = min(kTileGroup, nbm - group * kTileGroup);
  bm = group * kTileGroup + in % rows;
  bn = in / rows;
}

// Epilogue of a TM x BN tile (TM hidden rows x BN head rows) whose waves hold MI x NJ
// accumulator blocks of 32 x 32 each: the logits, and per hidden row the draft partials of the
// tile's BN columns: with PARTS = kPartsSoftmax the max and sum of 2^((x - max) k2), with
// kPartsArgmax the max and the lowest column index holding it (for argmax drafts).  Per row block
// of a wave the 16 row maxima over the wave's 32 NJ columns are reduce-scattered over the
// half-wave (a lane holds 16 rows of its half in each block), gathered back for the exponentials,
// and the sums reduce-scattered: 47 lane exchanges per block, 16 maxima and sums in registers at a
// time.  The BN / (32 NJ) waves that cover the same rows merge through LDS.  All threads of the
// workgroup must call (at least TM of them).
// wpart: LDS scratch of kSlots x TM float2 that the caller no longer needs (its operand tiles), so
// that the kernel keeps a single LDS object (a second one makes the compiler wait for every
// outstanding direct-to-LDS load before any LDS read in the main loop).
template <int PARTS, int MI, int NJ, int TM, int BN = kBigBN>
__device__ __forceinline__ void tile_store(const f32x16 (&acc)[MI][NJ], int M, int Vt, int m0, int n0, int wm,
                                           int wn, int nbn, int bn, float *__restrict__ logits,
                                           const GemvParts &parts, float2 (*wpart)[TM]) {
  constexpr int kSlots = BN / (32 * NJ);  // waves covering the same tile rows
  const int tid = threadIdx.x, lane = lane_id(), lr = lane & 31;
  const int slot = wn / (32 * NJ);
  // 32x32 accumulator layout: lane l holds column l % 32; register v holds row
  // 8 * (v / 4) + 4 * (l / 32) + v % 4.
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int gm = m0 + wm + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (gm < M) {
        float *dst = logits + static_cast<int64_t>(gm) * Vt;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int gn = n0 + wn + j * 32 + lr;
          if (gn < Vt) __builtin_nontemporal_store(acc[i][j][v], dst + gn);  // streamed out, not re-read here
        }
      }
    }
  if constexpr (PARTS == kPartsArgmax) {
    // per row: the wave's best (value, column) over its 32 NJ columns, reduce-scattered over the
    // half-wave, then merged across the waves that cover the same rows
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      float bv[16];
      int bi[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        bv[v] = kNegInf;
        bi[v] = kNoIndex;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int gn = n0 + wn + j * 32 + lr;
          if (gn < Vt && argmax_better(acc[i][j][v], gn, bv[v], bi[v])) {
            bv[v] = acc[i][j][v];
            bi[v] = gn;
          }
        }
      }
      half_argmax_scatter16(bv, bi);
      if ((lane & 1) == 0) {  // lanes l and l ^ 1 hold the same row
        const int e = lr >> 1;
        wpart[slot][wm + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)] = make_float2(bv[0], __int_as_float(bi[0]));
      }
    }
    __syncthreads();
    const int r = tid;
    const int gm = m0 + r;
    if (r < TM && gm < M) {
      float v = kNegInf;
      int ix = kNoIndex;
#pragma unroll
      for (int k = 0; k < kSlots; ++k) {
        const float2 p = wpart[k][r];
        if (argmax_better(p.x, __float_as_int(p.y), v, ix)) {
          v = p.x;
          ix = __float_as_int(p.y);
        }
      }
      parts.part[static_cast<int64_t>(gm) * nbn + bn] = make_float2(v, __int_as_float(ix));
    }
  }
  if constexpr (PARTS == kPartsSoftmax) {
    bool cin[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) cin[j] = n0 + wn + j * 32 + lr < Vt;
    const auto fmax_op = [](float a, float b) { return fmaxf(a, b); };
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      float mx[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float m = cin[0] ? acc[i][0][v] : kNegInf;
#pragma unroll
        for (int j = 1; j < NJ; ++j) m = fmaxf(m, cin[j] ? acc[i][j][v] : kNegInf);
        mx[v] = m;
      }
      half_reduce_scatter16(mx, fmax_op);
      const float own_m = mx[0];
      half_all_gather16(mx);
      float sm[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        // a row with no column in range has max -inf: reference 0 there, so every term is exp2(-inf) = 0
        const float ref = mx[v] == kNegInf ? 0.f : mx[v];
        float t = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) t += __builtin_amdgcn_exp2f(((cin[j] ? acc[i][j][v] : kNegInf) - ref) * parts.k2);
        sm[v] = t;
      }
      half_reduce_scatter16(sm, [](float a, float b) { return a + b; });
      if ((lane & 1) == 0) {  // lanes l and l ^ 1 hold the same row
        const int e = lr >> 1;
        wpart[slot][wm + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)] = make_float2(own_m, sm[0]);
      }
    }
    __syncthreads();
    const int r = tid;  // one thread per row of the tile
    const int gm = m0 + r;
    if (r < TM && gm < M) {
      float mx = kNegInf;
#pragma unroll
      for (int k = 0; k < kSlots; ++k) mx = fmaxf(mx, wpart[k][r].x);
      float sm = 0.f;
#pragma unroll
      for (int k = 0; k < kSlots; ++k) {
        const float2 p = wpart[k][r];
        if (p.x != kNegInf) sm += p.y * __builtin_amdgcn_exp2f((p.x - mx) * parts.k2);
      }
      parts.part[static_cast<int64_t>(gm) * nbn + bn] = make_float2(mx, sm);
    }
  }
}


template <bool TRIM, int PARTS, bool KFULL>
__global__ __launch_bounds__(kBlock, 1) void lmhead_mfma_big(const uint16_t *__restrict__ hidden,
                                                             const uint16_t *__restrict__ weight,
                                                             const int32_t *__restrict__ keep, int vrows, int M, int H,
                                                             int Vt, float *__restrict__ logits, GemvParts parts) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2][(kBigBM + kBigBN) * kBigRow];
  const int nbm = (M + kBigBM - 1) / kBigBM;
  const int nbn = (Vt + kBigBN - 1) / kBigBN;
  const int tile = static_cast<int>(xcd_remap(blockIdx.x, static_cast<int64_t>(nbm) * nbn));
  int bm, bn;
  big_tile_of(tile, nbm, nbn, bm, bn);
  const int m0 = bm * kBigBM, n0 = bn * kBigBN;
  const int tid = threadIdx.x;

  // staging: thread t moves 16-byte piece (t & 7) of rows (t >> 3) + 32 i, i < 8, of both operands
  const int piece = tid & 7, r0 = tid >> 3;
  int arow[8], brow[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    arow[i] = min(m0 + r0 + 32 * i, M - 1);
    const int n = min(n0 + r0 + 32 * i, Vt - 1);
    brow[i] = TRIM ? static_cast<int>(kept_row(keep, n, vrows)) : n;
  }
  uint4 ra[8], rb[8];
  uint32_t keepk = 0xffffffffu;  // all ones while the fetched pieces lie inside H; pieces past H are zeroed
  auto fetch = [&](int k0) {
    const int k = k0 + piece * 8;
    const bool kin = KFULL || k < H;
    const int kc = kin ? k : 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ra[i] = *reinterpret_cast<const uint4 *>(hidden + static_cast<int64_t>(arow[i]) * H + kc);
      rb[i] = *reinterpret_cast<const uint4 *>(weight + static_cast<int64_t>(brow[i]) * H + kc);
    }
    if (!KFULL) keepk = kin ? 0xffffffffu : 0u;
  };
  // the masking happens here, when the data are written to LDS, so that nothing waits for the
  // global loads before then
  auto stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint4 x = ra[i], y = rb[i];
      if (!KFULL) {
        x = make_uint4(x.x & keepk, x.y & keepk, x.z & keepk, x.w & keepk);
        y = make_uint4(y.x & keepk, y.y & keepk, y.z & keepk, y.w & keepk);
      }
      *reinterpret_cast<uint4 *>(&smem[buf][(r0 + 32 * i) * kBigRow + piece * 8]) = x;
      *reinterpret_cast<uint4 *>(&smem[buf][(kBigBM + r0 + 32 * i) * kBigRow + piece * 8]) = y;
    }
  };

  const int w = wave_id();
  const int wm = (w >> 1) * 128, wn = (w & 1) * 128;
  const int lane = lane_id();
  const int lr = lane & 31, lk = (lane >> 5) * 8;
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  fetch(0);
  stage(0);
  __syncthreads();
  const int nk = (H + kBigBK - 1) / kBigBK;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const uint16_t *sa = smem[cur] + (wm + lr) * kBigRow + lk;
    const uint16_t *sb = smem[cur] + (kBigBM + wn + lr) * kBigRow + lk;
    // fragments double-buffered in registers: the slice kk + 16 is read from LDS while the 16
    // MFMAs of slice kk run.  The next K step is fetched unconditionally (the last step re-reads
    // itself) so the whole iteration is one scheduling region.
    bf16x8 a[2][4], b[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[0][i] = *reinterpret_cast<const bf16x8 *>(sa + i * 32 * kBigRow);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[0][j] = *reinterpret_cast<const bf16x8 *>(sb + j * 32 * kBigRow);
    fetch(min(kt + 1, nk - 1) * kBigBK);
#pragma unroll
    for (int s4 = 0; s4 < kBigBK / 16; ++s4) {
      const int c = s4 & 1;
      if (s4 + 1 < kBigBK / 16) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a[c ^ 1][i] = *reinterpret_cast<const bf16x8 *>(sa + i * 32 * kBigRow + (s4 + 1) * 16);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          b[c ^ 1][j] = *reinterpret_cast<const bf16x8 *>(sb + j * 32 * kBigRow + (s4 + 1) * 16);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c][i], b[c][j], acc[i][j], 0, 0, 0);
    }
    stage(cur ^ 1);
    // issue order for the iteration: the first fragments and the next step's global loads, then
    // each slice's MFMAs interleaved with the LDS reads of the following slice, and the last
    // slice's MFMAs interleaved with the LDS writes of the next step
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 16, 0);
#pragma unroll
    for (int q = 0; q < kBigBK / 16 - 1; ++q) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    }
    __syncthreads();
  }

  tile_store<PARTS, 4, 4, kBigBM>(acc, M, Vt, m0, n0, wm, wn, nbn, bn, logits, parts,
                        reinterpret_cast<float2(*)[kBigBM]>(&smem[0][0]));
}

// Direct-to-LDS operand staging for 256 x 256 tiles: the load units write each lane's 16 bytes
// straight into LDS (global_load_lds_dwordx4: lane L's piece lands at LDS base + 16 L), through a
// ring of four K steps of 32, so a load has two to three steps of MFMA work to arrive and no
// register staging or LDS write instructions are needed.  A wave's 64 pieces fill 16 rows x 64
// bytes contiguously, so rows cannot be padded; instead piece p of tile row r is stored at slot
// p ^ f(r), f(r) = ((r >> 1) ^ (r >> 3)) & 3, which spreads the 16 rows of a fragment read over
// all banks.  Needs H % 32 == 0 (a piece past H cannot be zeroed on the way into LDS).
constexpr int kDmaBK = 32;
static_assert(kDmaBK == kTileK && kBigBM == kTileRows && kBigBN == kTileRows, "K-tiled operand layout");
constexpr int kDmaStages = 4;                           // ring depth: loads get kDmaStages - 2 steps to land
constexpr int kDmaRowBytes = kDmaBK * 2;                // 64
constexpr int kDmaOperandBytes = kBigBM * kDmaRowBytes;  // 16 KB per operand per step
constexpr int kDmaStageBytes = 2 * kDmaOperandBytes;    // 32 KB
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int dma_swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

// s_waitcnt with vmcnt = n and the other counters left alone (gfx9 encoding: vmcnt[3:0],
// expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] in bits [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The same 256 x 256 tile and LDS ring with eight waves (two per SIMD): wave w computes rows
// 128 (w / 4) .. +127 and columns 64 (w % 4) .. +63 of the tile, 4 x 2 accumulator blocks (128
// AGPRs), so each SIMD holds two waves and one issues MFMAs while the other waits on LDS or the
// barrier.  Each wave loads two 1 KB chunks of each operand per K step.
constexpr int kDma8Block = 512;

// ATILED: the hidden rows come K-tiled (hidden_tiles below): each K step's 256 x 32 slice of a
// hidden-row block is one contiguous 16 KB run instead of 256 rows 8 KB apart.  Measured on the
// large-drafter shape, the kernel's loads then take about 15% less time and the kernel 4-6% less;
// the products and their summation order are unchanged, so the logits are the same bits.
// BTILED: the head rows come from a K-tiled W^Trim (vt_trim_head_tiled) instead of being
// gathered from the full head through keep; again the same products in the same order.
template <bool TRIM, int PARTS, bool ATILED = false, bool BTILED = false>
__global__ __launch_bounds__(kDma8Block, 1) void lmhead_mfma_dma8(const uint16_t *__restrict__ hidden,
                                                                  const uint16_t *__restrict__ weight,
                                                                  const int32_t *__restrict__ keep, int vrows, int M,
                                                                  int H, int Vt, float *__restrict__ logits,
                                                                  GemvParts parts) {
  // with the K-tiled hidden rows a five-slot ring (the whole 160 KB of LDS) gives the loads three
  // steps to land: ~3% faster on the large-drafter shape; row-major rows keep four slots
  constexpr int kStages = ATILED ? 5 : kDmaStages;
  static_assert(!(BTILED && TRIM), "a K-tiled head is already trimmed");
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kDmaStageBytes];
  const int nbm = (M + kBigBM - 1) / kBigBM;
  const int nbn = (Vt + kBigBN - 1) / kBigBN;
  const int tile = static_cast<int>(xcd_remap(blockIdx.x, static_cast<int64_t>(nbm) * nbn));
  int bm, bn;
  big_tile_of(tile, nbm, nbn, bm, bn);
  const int m0 = bm * kBigBM, n0 = bn * kBigBN;
  const int w = wave_id(), lane = lane_id();

  // loads: wave w fills 1 KB chunks q = 2 w + j (j < 2) of each operand, i.e. tile rows
  // 16 q .. 16 q + 15; lane L writes row 16 q + L / 4, slot L % 4, and fetches piece slot ^ f(row)
  const uint16_t *asrc[2], *bsrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 16 * (2 * w + j) + (lane >> 2);
    const int piece = (lane & 3) ^ dma_swz(r);
    const int am = min(m0 + r, M - 1);
    const int n = min(n0 + r, Vt - 1);
    const int64_t brow = TRIM ? kept_row(keep, n, vrows) : static_cast<int64_t>(n);
    asrc[j] = ATILED ? hidden + (static_cast<int64_t>(bm) * (H / kDmaBK) * kBigBM + r) * kDmaBK + piece * 8
                     : hidden + static_cast<int64_t>(am) * H + piece * 8;
    bsrc[j] = BTILED ? weight + (static_cast<int64_t>(bn) * (H / kDmaBK) * kBigBN + r) * kDmaBK + piece * 8
                     : weight + brow * H + piece * 8;
  }
  const int nk = H / kDmaBK;
  auto issue = [&](int kstep, int slot) {
    const int k0 = min(kstep, nk - 1) * kDmaBK;
    const int64_t kt = static_cast<int64_t>(min(kstep, nk - 1)) * kBigBM * kDmaBK;  // K-tiled step offset
    const int64_t ka = ATILED ? kt : k0;
    const int64_t kb = BTILED ? kt : k0;
    char *base = smem + slot * kDmaStageBytes;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_global_load_lds(asrc[j] + ka, (lds_void *)(base + (2 * w + j) * 1024), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_global_load_lds(bsrc[j] + kb, (lds_void *)(base + kDmaOperandBytes + (2 * w + j) * 1024),
                                       16, 0, 0);
  };

  const int wm = (w >> 2) * 128, wn = (w & 3) * 64;
  const int lr = lane & 31;
  const int sw = dma_swz(lr);
  const int off0 = lr * kDmaRowBytes + (((lane >> 5) ^ sw) << 4);
  const int off1 = lr * kDmaRowBytes + (((2 + (lane >> 5)) ^ sw) << 4);
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  auto frags = [&](int slot, int off, bf16x8(&a)[4], bf16x8(&b)[2]) {
    const char *sa = smem + slot * kDmaStageBytes + wm * kDmaRowBytes + off;
    const char *sb = smem + slot * kDmaStageBytes + kDmaOperandBytes + wn * kDmaRowBytes + off;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const bf16x8 *>(sa + i * 32 * kDmaRowBytes);
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = *reinterpret_cast<const bf16x8 *>(sb + j * 32 * kDmaRowBytes);
  };
  auto mfmas = [&](const bf16x8(&a)[4], const bf16x8(&b)[2]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  };
  auto interleave = [&]() {  // 6 LDS reads spread over the first 6 of 8 MFMAs
#pragma unroll
    for (int r = 0; r < 6; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  };

  // Each step k: the MFMAs of its first 16-deep slice run while the second slice's fragments are
  // read; then (wait + barrier) step k + 1 is complete in LDS and the slot of step k - 1 is free,
  // the loads of step k + 3 go into it, and the second slice's MFMAs run while the first slice of
  // step k + 1 is read.  LDS reads never wait on an idle MFMA pipe; loads have two steps to land.
  // The waits are explicit: before the barrier of step k a thread waits until at most the loads
  // of the steps after k + 1 are outstanding (k + 2 and k + 3 with four slots, k + 2 .. k + 4 with
  // five); steps past the last re-fetch the last step into the free slot (never read), so every
  // step issues the same 4 loads per wave.
  bf16x8 a0[4], b0[2], a1[4], b1[2];
  constexpr int kAhead = kStages - 1;
#pragma unroll
  for (int s = 0; s < kAhead; ++s) issue(s, s);
  wait_vmcnt<4 * (kAhead - 1)>();
  __builtin_amdgcn_s_barrier();
  frags(0, off0, a0, b0);
  for (int kt = 0; kt < nk; ++kt) {
    const int slot = kt % kStages;
    frags(slot, off1, a1, b1);
    mfmas(a0, b0);
    interleave();
    wait_vmcnt<4 * (kAhead - 2)>();
    __builtin_amdgcn_s_barrier();
    issue(kt + kAhead, (kt + kAhead) % kStages);
    frags((kt + 1) % kStages, off0, a0, b0);  // past the last step: unused reads of a re-fetch
    mfmas(a1, b1);
    __builtin_amdgcn_sched_group_barrier(0x020, 4, 0);
    interleave();
  }
  wait_vmcnt<0>();
  __syncthreads();
  tile_store<PARTS, 4, 2, kBigBM>(acc, M, Vt, m0, n0, wm, wn, nbn, bn, logits, parts,
                           reinterpret_cast<float2(*)[kBigBM]>(smem));
}

// 384 x 256 output tiles (384 hidden rows x 256 head rows) for batches whose hidden rows fill
// 384-row blocks at least as tightly as 256-row ones (the large-drafter shape: 2304 = 6 x 384).
// Per K step a CU loads 640 rows x 64 bytes for 384 x 256 x 32 multiply-adds, a sixth fewer
// bytes per flop than the 256 x 256 tile, which is what bounds the loop.  Eight waves of 96 x 128
// (3 x 4 accumulator blocks, 192 registers), so the fragments of a 16-deep slice are read into a
// single buffer (a second one spills); the other wave on the SIMD covers the read latency.  The
// hidden rows come K-tiled in 384-row blocks (hidden_tiles with kTallBM rows); the head rows
// either gathered through keep or K-tiled (BTILED); a four-slot ring of 40 KB slices fills the
// 160 KB of LDS.  Each output element sums the same products in the same K order as the 256 x
// 256 kernels, so the logits are the same bits.
constexpr int kTallBM = 384;
constexpr int kTallStages = 4;
constexpr int kTallStageBytes = (kTallBM + kBigBN) * kDmaRowBytes;  // 40 KB

template <bool TRIM, int PARTS, bool BTILED>
__global__ __launch_bounds__(kDma8Block, 1) void lmhead_mfma_tall(const uint16_t *__restrict__ hidden,
                                                                  const uint16_t *__restrict__ weight,
                                                                  const int32_t *__restrict__ keep, int vrows, int M,
                                                                  int H, int Vt, float *__restrict__ logits,
                                                                  GemvParts parts) {
  static_assert(!(BTILED && TRIM), "a K-tiled head is already trimmed");
  constexpr int kMI = 3, kNJ = 4;           // accumulator blocks per wave
  constexpr int kLA = kTallBM / 128;        // 1 KB hidden-row loads per wave per step
  constexpr int kLoads = kLA + 2;           // and two of head rows
  constexpr int kOpA = kTallBM * kDmaRowBytes;
  __shared__ __attribute__((aligned(1024))) char smem[kTallStages * kTallStageBytes];
  const int nbm = (M + kTallBM - 1) / kTallBM;
  const int nbn = (Vt + kBigBN - 1) / kBigBN;
  const int tile = static_cast<int>(xcd_remap(blockIdx.x, static_cast<int64_t>(nbm) * nbn));
  int bm, bn;
  big_tile_of(tile, nbm, nbn, bm, bn);
  const int m0 = bm * kTallBM, n0 = bn * kBigBN;
  const int w = wave_id(), lane = lane_id();
  const int nk = H / kDmaBK;

  // loads: wave w fills hidden chunks 3 w + j (tile rows 16 (3 w + j) + lane / 4) and head chunks
  // 2 w + j.  Rows r and r + 32 share their swizzle, r + 16 does not: the hidden rows take one
  // source pointer (at row ra, with the swizzle of row ra + 16 p) for the even chunks and one for
  // the odd chunk, offset by 16 j rows when issued; each head chunk has its own.
  const int ra = 16 * (kLA * w) + (lane >> 2), rb = 16 * (2 * w) + (lane >> 2);
  const uint16_t *asrc[2], *bsrc[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    asrc[p] = hidden + (static_cast<int64_t>(bm) * nk * kTallBM + ra) * kDmaBK +
              ((lane & 3) ^ dma_swz(ra + 16 * p)) * 8;
    const int q = rb + 16 * p;
    const int piece = (lane & 3) ^ dma_swz(q);
    if (BTILED) {
      bsrc[p] = weight + (static_cast<int64_t>(bn) * nk * kBigBN + q) * kDmaBK + piece * 8;
    } else {
      const int n = min(n0 + q, Vt - 1);
      const int64_t brow = TRIM ? kept_row(keep, n, vrows) : static_cast<int64_t>(n);
      bsrc[p] = weight + brow * H + piece * 8;
    }
  }
  auto issue = [&](int kstep, int slot) {
    const int k = min(kstep, nk - 1);
    const int64_t ka = static_cast<int64_t>(k) * kTallBM * kDmaBK;
    const int64_t kb = BTILED ? static_cast<int64_t>(k) * kBigBN * kDmaBK : static_cast<int64_t>(k) * kDmaBK;
    char *base = smem + slot * kTallStageBytes;
#pragma unroll
    for (int j = 0; j < kLA; ++j)
      __builtin_amdgcn_global_load_lds(asrc[j & 1] + ka + j * 16 * kDmaBK, (lds_void *)(base + (kLA * w + j) * 1024),
                                       16, 0, 0);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_global_load_lds(bsrc[j] + kb, (lds_void *)(base + kOpA + (2 * w + j) * 1024), 16, 0, 0);
  };

  const int wm = (w >> 1) * 96, wn = (w & 1) * 128;
  const int lr = lane & 31;
  const int sw = dma_swz(lr);
  const int off0 = lr * kDmaRowBytes + (((lane >> 5) ^ sw) << 4);
  const int off1 = lr * kDmaRowBytes + (((2 + (lane >> 5)) ^ sw) << 4);
  f32x16 acc[kMI][kNJ];
#pragma unroll
  for (int i = 0; i < kMI; ++i)
#pragma unroll
    for (int j = 0; j < kNJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  bf16x8 a[kMI], b[kNJ];
  auto slice = [&](int slot, int off) {
    const char *sa = smem + slot * kTallStageBytes + wm * kDmaRowBytes + off;
    const char *sb = smem + slot * kTallStageBytes + kOpA + wn * kDmaRowBytes + off;
#pragma unroll
    for (int i = 0; i < kMI; ++i) a[i] = *reinterpret_cast<const bf16x8 *>(sa + i * 32 * kDmaRowBytes);
#pragma unroll
    for (int j = 0; j < kNJ; ++j) b[j] = *reinterpret_cast<const bf16x8 *>(sb + j * 32 * kDmaRowBytes);
#pragma unroll
    for (int i = 0; i < kMI; ++i)
#pragma unroll
      for (int j = 0; j < kNJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  };

  // step k: both 16-deep slices of slot k % 4; then (wait + barrier) step k + 1 is in LDS and the
  // slot of step k - 1 is free, and the loads of step k + 3 go into it; past the last step the last
  // step is fetched again into the free slot (never read), so every step issues the same loads
  constexpr int kAhead = kTallStages - 1;
#pragma unroll
  for (int s = 0; s < kAhead; ++s) issue(s, s);
  wait_vmcnt<kLoads * (kAhead - 1)>();
  __builtin_amdgcn_s_barrier();
  for (int kt = 0; kt < nk; ++kt) {
    const int slot = kt % kTallStages;
    slice(slot, off0);
    slice(slot, off1);
    wait_vmcnt<kLoads * (kAhead - 2)>();
    __builtin_amdgcn_s_barrier();
    issue(kt + kAhead, (kt + kAhead) % kTallStages);
  }
  wait_vmcnt<0>();
  __syncthreads();
  tile_store<PARTS, kMI, kNJ, kTallBM>(acc, M, Vt, m0, n0, wm, wn, nbn, bn, logits, parts,
                         reinterpret_cast<float2(*)[kTallBM]>(smem));
}

// Up to rows_max(Vt) hidden rows (decode batches of a few to a few dozen sequences): the head is
// bound by streaming W^Trim once, so a tile holds every hidden row, padded only to the next
// multiple of 32, against BN head rows: one workgroup per BN head rows streams its share of the
// head once while the hidden rows come from L2.  The 256-row tiles would multiply up to 256 rows
// whatever M is.  BN / 32 waves: for an odd number MB of 32-row blocks wave w holds all 32 MB tile
// rows against head columns 32 w .. 32 w + 31 (MB accumulator blocks); for an even one the waves
// form two rows, each wave holding half the tile rows against 64 columns (MB / 2 x 2 blocks, fewer
// fragment reads per MFMA); the epilogue merges the column slots per row.  BN = 256 (eight waves,
// one workgroup per CU and 160 KB of LDS) when the head has at least kCUs blocks of 256 rows,
// else BN = 128 (four waves and 80 KB, so up to two workgroups per CU), so that a 32768-row head
// still spreads over every CU.  The loads of a K step are two 1 KB chunks (16 rows x 64 bytes,
// swizzled as in the 256 x 256 kernel) per 32-row block of hidden rows and BN / 16 of head rows,
// dealt out to the waves in turn; a wave with fewer distinct chunks fetches one of the others
// again, which writes the same bytes to the same place, so every wave issues the same number of
// loads per step and one wait count serves all.  The ring holds as many K steps as fit the
// workgroup's LDS, at most eight.  Each output sums the same products in the same K order as the
// other direct-to-LDS kernels: the same logits bits.  Up to 192 rows (six blocks) in general; with
// 128-column blocks, where the 256 x 256 tiles would leave CUs idle, up to 256 (seven or eight
// blocks, each workgroup then taking the whole 160 KB of LDS), and up to 384 in two row blocks of
// at most six (two workgroups per CU, one of each block).
constexpr int kRowsMaxMB = 6, kRowsMaxMB128 = 8;
constexpr int kRowsMaxM = 32 * kRowsMaxMB;
constexpr int kCUs = 256;  // compute units of the part

template <int MB, int BN>
struct RowsTile {
  static constexpr int kTM = 32 * MB;
  static constexpr int kWaves = BN / 32;
  static constexpr int kThreads = kWave * kWaves;
  static constexpr int kChunks = 2 * MB + BN / 16;  // 1 KB loads per K step
  static constexpr int kLoads = (kChunks + kWaves - 1) / kWaves;  // per wave
  static constexpr int kStageBytes = kChunks * 1024;
  static constexpr int kLdsBytes = MB > kRowsMaxMB ? 160 * 1024 : 160 * 1024 / (256 / BN);
  static constexpr int kFit = kLdsBytes / kStageBytes;
  static constexpr int kStages = kFit < 8 ? kFit : 8;
  static_assert(BN == 128 || BN == 256, "tile widths");
  static_assert(MB <= (BN == 128 ? kRowsMaxMB128 : kRowsMaxMB), "row blocks");
  static_assert(kStages >= 3 && kLoads * (kStages - 2) < 64, "ring and wait counts");
};

// One lane's 16-byte direct-to-LDS load (the wave's 64 lanes fill dst .. dst + 1 KB).  A plain
// device function, so that the builtin's operands never depend on a kernel's template parameters
// (the host pass checks such a call against its own target and rejects the 16-byte size).
__device__ __forceinline__ void lds_load16(const uint16_t *src, char *dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void *)dst, 16, 0, 0);
}

template <int MB, int BN, bool TRIM, int PARTS, bool ATILED, bool BTILED>
__global__ __launch_bounds__(kWave * (BN / 32)) void lmhead_mfma_rows(const uint16_t *__restrict__ hidden,
                                                                      const uint16_t *__restrict__ weight,
                                                                      const int32_t *__restrict__ keep, int vrows,
                                                                      int M, int H, int Vt, float *__restrict__ logits,
                                                                      GemvParts parts) {
  static_assert(!(BTILED && TRIM), "a K-tiled head is already trimmed");
  using G = RowsTile<MB, BN>;
  constexpr int kTM = G::kTM, kS = G::kStages, kL = G::kLoads, kW = G::kWaves, kOpA = kTM * kDmaRowBytes;
  // even row-block counts: waves in two rows of kW / 2, each holding half the rows against 64
  // columns (fewer fragment reads per MFMA); odd: one row of kW waves against 32 columns each
  constexpr int kWM = MB % 2 == 0 ? 2 : 1, kNJ = kWM, kMI = MB / kWM, kWN = kW / kWM;
  __shared__ __attribute__((aligned(1024))) char smem[kS * G::kStageBytes];
  const int nbm = (M + kTM - 1) / kTM;
  const int nbn = (Vt + BN - 1) / BN;
  const int tile = static_cast<int>(xcd_remap(blockIdx.x, static_cast<int64_t>(nbm) * nbn));
  int bm, bn;
  big_tile_of(tile, nbm, nbn, bm, bn);
  const int m0 = bm * kTM, n0 = bn * BN;
  const int w = wave_id(), lane = lane_id();
  const int nk = H / kDmaBK;

  // load j of wave w: chunk q = w + kW j (wrapped), lane L writing row 16 q + L / 4 of the stage,
  // slot L % 4, with piece slot ^ f(row) of that row; per K step the source advances by step[j].
  // The K-tiled W^Trim comes in 256-row blocks: a 128-row tile is one half of one.
  const uint16_t *src[kL];
  int64_t step[kL];
  int dst[kL];
#pragma unroll
  for (int j = 0; j < kL; ++j) {
    int q = w + kW * j;
    if (q >= G::kChunks) q -= G::kChunks;
    dst[j] = q * 1024;
    if (q < 2 * MB) {
      const int r = 16 * q + (lane >> 2);
      const int piece = (lane & 3) ^ dma_swz(r);
      if (ATILED) {
        src[j] = hidden + (static_cast<int64_t>(bm) * nk * kTM + r) * kDmaBK + piece * 8;
        step[j] = static_cast<int64_t>(kTM) * kDmaBK;
      } else {
        src[j] = hidden + static_cast<int64_t>(min(m0 + r, M - 1)) * H + piece * 8;
        step[j] = kDmaBK;
      }
    } else {
      const int r = 16 * (q - 2 * MB) + (lane >> 2);
      const int piece = (lane & 3) ^ dma_swz(r);
      if (BTILED) {
        src[j] = weight + (static_cast<int64_t>(n0 / kTileRows) * nk * kTileRows + n0 % kTileRows + r) * kDmaBK +
                 piece * 8;
        step[j] = static_cast<int64_t>(kTileRows) * kDmaBK;
      } else {
        const int n = min(n0 + r, Vt - 1);
        const int64_t brow = TRIM ? kept_row(keep, n, vrows) : static_cast<int64_t>(n);
        src[j] = weight + brow * H + piece * 8;
        step[j] = kDmaBK;
      }
    }
  }
  auto issue = [&](int kstep, int slot) {
    const int64_t k = min(kstep, nk - 1);
    char *base = smem + slot * G::kStageBytes;
#pragma unroll
    for (int j = 0; j < kL; ++j) lds_load16(src[j] + k * step[j], base + dst[j]);
  };

  const int wn = (w % kWN) * 32 * kNJ, wm = (w / kWN) * 32 * kMI;
  const int lr = lane & 31;
  const int sw = dma_swz(lr);
  const int off0 = lr * kDmaRowBytes + (((lane >> 5) ^ sw) << 4);
  const int off1 = lr * kDmaRowBytes + (((2 + (lane >> 5)) ^ sw) << 4);
  f32x16 acc[kMI][kNJ];
#pragma unroll
  for (int i = 0; i < kMI; ++i)
#pragma unroll
    for (int j = 0; j < kNJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  auto slice = [&](int slot, int off) {
    const char *sa = smem + slot * G::kStageBytes + wm * kDmaRowBytes + off;
    const char *sb = smem + slot * G::kStageBytes + kOpA + wn * kDmaRowBytes + off;
    bf16x8 a[kMI], b[kNJ];
#pragma unroll
    for (int j = 0; j < kNJ; ++j) b[j] = *reinterpret_cast<const bf16x8 *>(sb + j * 32 * kDmaRowBytes);
#pragma unroll
    for (int i = 0; i < kMI; ++i) a[i] = *reinterpret_cast<const bf16x8 *>(sa + i * 32 * kDmaRowBytes);
#pragma unroll
    for (int i = 0; i < kMI; ++i)
#pragma unroll
      for (int j = 0; j < kNJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  };

  // step k: both 16-deep slices of slot k % kS; then (wait + barrier) step k + 1 is in LDS and the
  // slot of step k - 1 is free for the loads of step k + kS - 1; past the last step the last step
  // is fetched again into the free slot (never read), so every step issues the same loads
  constexpr int kAhead = kS - 1;
#pragma unroll
  for (int s = 0; s < kAhead; ++s) issue(s, s);
  wait_vmcnt<kL * (kAhead - 1)>();
  __builtin_amdgcn_s_barrier();
  for (int kt = 0; kt < nk; ++kt) {
    const int slot = kt % kS;
    slice(slot, off0);
    slice(slot, off1);
    wait_vmcnt<kL * (kAhead - 2)>();
    __builtin_amdgcn_s_barrier();
    issue(kt + kAhead, (kt + kAhead) % kS);
  }
  wait_vmcnt<0>();
  __syncthreads();
  tile_store<PARTS, kMI, kNJ, kTM, BN>(acc, M, Vt, m0, n0, wm, wn, nbn, bn, logits, parts,
                                       reinterpret_cast<float2(*)[kTM]>(smem));
}

typedef void (*HeadKernel)(const uint16_t *, const uint16_t *, const int32_t *, int, int, int, int, float *,
                           GemvParts);

template <int BN, bool TRIM, int PARTS, bool ATILED, bool BTILED>
HeadKernel pick_rows_bn(int mb) {
  switch (mb) {
    case 1: return &lmhead_mfma_rows<1, BN, TRIM, PARTS, ATILED, BTILED>;
    case 2: return &lmhead_mfma_rows<2, BN, TRIM, PARTS, ATILED, BTILED>;
    case 3: return &lmhead_mfma_rows<3, BN, TRIM, PARTS, ATILED, BTILED>;
    case 4: return &lmhead_mfma_rows<4, BN, TRIM, PARTS, ATILED, BTILED>;
    case 5: return &lmhead_mfma_rows<5, BN, TRIM, PARTS, ATILED, BTILED>;
    case 6: return &lmhead_mfma_rows<6, BN, TRIM, PARTS, ATILED, BTILED>;
    case 7:
      if constexpr (BN == 128) return &lmhead_mfma_rows<7, BN, TRIM, PARTS, ATILED, BTILED>;
      return nullptr;
    case 8:
      if constexpr (BN == 128) return &lmhead_mfma_rows<8, BN, TRIM, PARTS, ATILED, BTILED>;
      return nullptr;
    default: return nullptr;
  }
}
static_assert(kRowsMaxMB == 6 && kRowsMaxMB128 == 8, "pick_rows_bn covers the row blocks");

template <bool TRIM, int PARTS, bool ATILED, bool BTILED>
HeadKernel pick_rows(int mb, int bn) {
  return bn == 128 ? pick_rows_bn<128, TRIM, PARTS, ATILED, BTILED>(mb)
                   : pick_rows_bn<256, TRIM, PARTS, ATILED, BTILED>(mb);
}

inline int64_t mfma_big_tiles_n(int64_t Vt) { return (Vt + kBigBN - 1) / kBigBN; }

// Rows per hidden-row block of the 256-column heads that read a K-tiled copy: 384 (the tall
// tiles) or 256, whichever needs fewer hidden rows per CU: one tile per CU at a time, so a launch
// of t tiles of R rows takes about ceil(t / kCUs) R row-steps (2304 rows and 256 head blocks: 6
// waves of 384 against 9 of 256, a tie, and the tall tiles move fewer bytes per flop; 384 rows
// and 128 head blocks: one wave of 128 tall tiles, 384 row-steps on half the CUs, against one of
// 256 square tiles, 256).
inline int big_tile_rows(int64_t M, int64_t Vt) {
  const int64_t nbn = mfma_big_tiles_n(Vt);
  const int64_t t384 = (M + kTallBM - 1) / kTallBM * nbn, t256 = (M + kBigBM - 1) / kBigBM * nbn;
  return (t384 + kCUs - 1) / kCUs * kTallBM <= (t256 + kCUs - 1) / kCUs * kBigBM ? kTallBM : kBigBM;
}

// Hidden rows up to which the all-rows kernel runs: 256 when its column blocks are 128 rows (fewer
// than kCUs blocks of 256 head rows), else 192.
inline int64_t rows_max(int64_t Vt) { return mfma_big_tiles_n(Vt) < kCUs ? 32 * kRowsMaxMB128 : kRowsMaxM; }

// Whether the all-rows kernel takes M rows: in one block up to rows_max(Vt), and on heads of fewer
// than kCUs blocks of 256 rows in two blocks of at most kRowsMaxM rows (the batched shape's head
// at 264 to 384 rows: 88-93 us against 101-104 us on 256 x 256 tiles).  rows_block: its rows per
// block.
inline bool rows_kernel(int64_t M, int64_t Vt) {
  return M <= rows_max(Vt) || (mfma_big_tiles_n(Vt) < kCUs && M <= 2 * kRowsMaxM);
}
inline int rows_block(int64_t M, int64_t Vt) {
  const int64_t per = M <= rows_max(Vt) ? M : (M + 1) / 2;
  return static_cast<int>((per + 31) / 32 * 32);
}

// Rows per hidden-row block of the direct-to-LDS heads: rows_block(M, Vt) for the all-rows kernel,
// else big_tile_rows(M, Vt).
inline int head_tile_rows(int64_t M, int64_t Vt) {
  return rows_kernel(M, Vt) ? rows_block(M, Vt) : big_tile_rows(M, Vt);
}

// Head rows per column block of the MFMA heads with whole 32-column K steps, which is also the
// chunk of their draft partials: 128 for the all-rows kernel when fewer than kCUs blocks of 256
// head rows would leave CUs idle, else 256.
inline int head_tile_cols(int64_t M, int64_t H, int64_t Vt) {
  return H % kDmaBK == 0 && rows_kernel(M, Vt) && mfma_big_tiles_n(Vt) < kCUs ? 128 : kBigBN;
}

// K-tiled copy of the hidden rows for the direct-to-LDS heads (lmhead_mfma_rows, _dma8 and _tall
// with ATILED), in blocks of R = head_tile_rows(M, Vt) rows: out[bm][ks][r][32] = hidden[min(R bm + r,
// M - 1)][32 ks .. 32 ks + 31] (rows past M repeat the last row; their logits are never stored).
// One thread moves one 16-byte piece; a wave reads 16 rows x 64 bytes and writes 1 KB
// contiguously.  Needs H % 32 == 0.
// Bytes of the K-tiled hidden copy (0 when H % 32 != 0: the direct-to-LDS kernels do not run).
inline size_t hidden_tiles_bytes(int64_t M, int64_t H, int64_t Vt) {
  if (H % kDmaBK != 0) return 0;
  const int64_t R = head_tile_rows(M, Vt);
  return static_cast<size_t>((M + R - 1) / R) * R * static_cast<size_t>(H) * 2;
}

struct TileParams {
  const uint16_t *hidden;
  uint16_t *out;
  int64_t pieces;
  int M, H, rows;  // rows: rows per block of the copy
};

// Workgroup `blk` of the copy (kBlock pieces).
__device__ __forceinline__ void hidden_tiles_block(const TileParams &T, int64_t blk) {
  const uint16_t *__restrict__ hidden = T.hidden;
  const int M = T.M, H = T.H;
  const int64_t q = blk * kBlock + threadIdx.x;  // piece index in out
  if (q >= T.pieces) return;
  const int p = static_cast<int>(q & 3);
  const int64_t rr = q >> 2;  // (bm, ks, r) flattened
  const int r = static_cast<int>(rr % T.rows);
  const int64_t bk = rr / T.rows;
  const int nk = H / kDmaBK;
  const int ks = static_cast<int>(bk % nk);
  const int bm = static_cast<int>(bk / nk);
  const int m = min(bm * T.rows + r, M - 1);
  const uint4 v = *reinterpret_cast<const uint4 *>(hidden + static_cast<int64_t>(m) * H + ks * kDmaBK + p * 8);
  *reinterpret_cast<uint4 *>(T.out + q * 8) = v;
}

inline TileParams hidden_tiles_params(const uint16_t *hidden, int64_t M, int64_t H, int64_t Vt, uint16_t *out) {
  TileParams T{};
  T.hidden = hidden;
  T.out = out;
  T.M = static_cast<int>(M);
  T.H = static_cast<int>(H);
  T.rows = head_tile_rows(M, Vt);
  T.pieces = static_cast<int64_t>(hidden_tiles_bytes(M, H, Vt) / 16);
  return T;
}

inline int64_t hidden_tiles_blocks(const TileParams &T) { return (T.pieces + kBlock - 1) / kBlock; }

__global__ __launch_bounds__(kBlock) void hidden_tiles(TileParams T) { hidden_tiles_block(T, blockIdx.x); }

// The target rows' softmax partials (one workgroup per (row, 4096-chunk)) with the K-tiled copy of
// the hidden rows in extra workgroups past them: both only read inputs of the block, so the copy
// rides in the launch that precedes the head instead of taking one of its own.
template <typename Tin, bool kVec>
__global__ __launch_bounds__(kBlock) void softmax_partial_tiles(SmParams P, TileParams T) {
  const int64_t nparts = P.rows * P.nchunk;
  const int64_t bid = blockIdx.x;
  if (bid < nparts)
    partial_chunk<Tin, kVec>(P, bid);
  else
    hidden_tiles_block(T, bid - nparts);
}




// The MFMA heads with whole 32-column K steps (any M), or with M >= kBigMinM (any H).
// PARTS = kPartsNone (the separate LM-head call): the hidden rows as given; the all-rows kernel
// where rows_kernel(M, Vt) (blocks of rows_block(M, Vt) rows, head_tile_cols(M, H, Vt) head rows
// per workgroup), else 256 x 256 tiles.  kPartsSoftmax / kPartsArgmax (the fused block's head, with its draft partials per
// head_tile_cols(M, H, Vt) head rows): when H % 32 == 0 hidden_tiled must hold the K-tiled copy
// of the hidden rows made by hidden_tiles, in blocks of head_tile_rows(M, Vt) rows, which select
// the kernel (all-rows blocks, 384-row tall tiles or 256 x 256 tiles); weight_tiled: NULL, or
// the K-tiled trimmed head of vt_trim_head_tiled (weight and keep are then not read by the
// kernel).  Other H take the register-staged kernel on the rows as given.
template <int PARTS>
inline hipError_t launch_mfma_head(const uint16_t *hidden, const uint16_t *weight, const int32_t *keep, int vrows,
                                   int64_t M, int64_t H, int64_t Vt, float *logits, GemvParts parts,
                                   hipStream_t stream, const uint16_t *hidden_tiled = nullptr,
                                   const uint16_t *weight_tiled = nullptr) {
  const int64_t tiles = ((M + kBigBM - 1) / kBigBM) * mfma_big_tiles_n(Vt);
  const int iM = static_cast<int>(M), iH = static_cast<int>(H), iV = static_cast<int>(Vt);
  if (H % kDmaBK == 0 && rows_kernel(M, Vt)) {
    const int tm = rows_block(M, Vt), mb = tm / 32, bn = head_tile_cols(M, H, Vt);
    const int64_t nbm = (M + tm - 1) / tm;
    const dim3 grid(static_cast<unsigned>(nbm * ((Vt + bn - 1) / bn))), block(static_cast<unsigned>(kWave * (bn / 32)));
    if constexpr (PARTS == kPartsNone) {
      if (hidden_tiled || weight_tiled) return hipErrorInvalidValue;
      const HeadKernel f =
          keep ? pick_rows<true, PARTS, false, false>(mb, bn) : pick_rows<false, PARTS, false, false>(mb, bn);
      return launch(f, grid, block, 0, stream, hidden, weight, keep, vrows, iM, iH, iV, logits, parts);
    } else {
      if (!hidden_tiled) return hipErrorInvalidValue;
      const HeadKernel f = weight_tiled ? pick_rows<false, PARTS, true, true>(mb, bn)
                                        : (keep ? pick_rows<true, PARTS, true, false>(mb, bn)
                                                : pick_rows<false, PARTS, true, false>(mb, bn));
      return launch(f, grid, block, 0, stream, hidden_tiled, weight_tiled ? weight_tiled : weight, keep, vrows, iM, iH,
                    iV, logits, parts);
    }
  }
  if (H % kDmaBK == 0) {
    if constexpr (PARTS == kPartsNone) {
      if (hidden_tiled || weight_tiled) return hipErrorInvalidValue;
      auto fd = keep ? &lmhead_mfma_dma8<true, PARTS> : &lmhead_mfma_dma8<false, PARTS>;
      return launch(fd, dim3(static_cast<unsigned>(tiles)), dim3(kDma8Block), 0, stream, hidden, weight, keep, vrows,
                    iM, iH, iV, logits, parts);
    } else {
      if (!hidden_tiled) return hipErrorInvalidValue;
      if (big_tile_rows(M, Vt) == kTallBM) {
        const unsigned tall = static_cast<unsigned>(((M + kTallBM - 1) / kTallBM) * mfma_big_tiles_n(Vt));
        auto f = weight_tiled ? &lmhead_mfma_tall<false, PARTS, true>
                              : (keep ? &lmhead_mfma_tall<true, PARTS, false> : &lmhead_mfma_tall<false, PARTS, false>);
        return launch(f, dim3(tall), dim3(kDma8Block), 0, stream, hidden_tiled, weight_tiled ? weight_tiled : weight,
                      keep, vrows, iM, iH, iV, logits, parts);
      }
      auto ft = weight_tiled ? &lmhead_mfma_dma8<false, PARTS, true, true>
                             : (keep ? &lmhead_mfma_dma8<true, PARTS, true> : &lmhead_mfma_dma8<false, PARTS, true>);
      return launch(ft, dim3(static_cast<unsigned>(tiles)), dim3(kDma8Block), 0, stream, hidden_tiled,
                    weight_tiled ? weight_tiled : weight, keep, vrows, iM, iH, iV, logits, parts);
    }
  }
  if (hidden_tiled || weight_tiled) return hipErrorInvalidValue;
  auto fn = H % kBigBK == 0 ? (keep ? &lmhead_mfma_big<true, PARTS, true> : &lmhead_mfma_big<false, PARTS, true>)
                            : (keep ? &lmhead_mfma_big<true, PARTS, false> : &lmhead_mfma_big<false, PARTS, false>);
  return launch(fn, dim3(static_cast<unsigned>(tiles)), dim3(kBlock), 0, stream, hidden, weight, keep, vrows, iM, iH,
                iV, logits, parts);
}

// extra: workgroups past the head's row blocks (target partial chunks; PARTS kernels only).
inline hipError_t launch_gemv(GemvFn fn, const uint16_t *hidden, const uint16_t *weight, const int32_t *keep,
                              int vrows, int64_t H, int64_t Vt, float *logits, GemvParts parts, hipStream_t stream,
                              int64_t extra = 0) {
  return launch(fn, dim3(static_cast<unsigned>(gemv_blocks(Vt) + extra)), dim3(kBlock), 0, stream, hidden, weight, keep,
                vrows, static_cast<int>(H), static_cast<int>(Vt), gemv_rows_per_block(Vt), logits, parts);
}

// Whether the MFMA head for M hidden rows is one of launch_mfma_head's kernels (else the 128 x
// 128 tiles).
inline bool mfma_head_direct(int64_t M, int64_t H) { return H % kDmaBK == 0 || M >= kBigMinM; }

inline hipError_t launch_mfma(const uint16_t *hidden, const uint16_t *weight, const int32_t *keep, int vrows,
                              int64_t M, int64_t H, int64_t Vt, float *logits, hipStream_t stream) {
  if (mfma_head_direct(M, H))
    return launch_mfma_head<kPartsNone>(hidden, weight, keep, vrows, M, H, Vt, logits, GemvParts{}, stream);
  const int64_t tiles = ((M + kBM - 1) / kBM) * ((Vt + kBN - 1) / kBN);
  return launch(lmhead_mfma, dim3(static_cast<unsigned>(tiles)), dim3(kBlock), 0, stream, hidden, weight, keep,
                vrows, static_cast<int>(M), static_cast<int>(H), static_cast<int>(Vt), logits);
}

}  // namespace
}  // namespace vt


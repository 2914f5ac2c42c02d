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
#include <hip/hip_runtime.h>

#include <cstdint>

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

// Transpose-reduction of N (power of two) per-lane values across the wavefront.  Each step
// exchanges half of the remaining values with the partner lane (lane ^ offset) and keeps the
// sums of the other half, so the whole reduction costs about N + log2(64/N) shuffles instead of
// 6N.  On return lane l holds the full 64-lane sum of value index (l >> (6 - log2 N)).
template <int N>
__device__ __forceinline__ float transpose_reduce(float (&v)[N]) {
  const int lane = lane_id();
  int n = N;
  int off = kWave / 2;
#pragma unroll
  for (int step = 0; step < 6; ++step) {
    if (n > 1) {
      const bool upper = (lane & off) != 0;
      const int h = n / 2;
#pragma unroll
      for (int k = 0; k < N / 2; ++k) {
        if (k < h) {
          const float send = upper ? v[k] : v[k + h];
          const float keep = upper ? v[k + h] : v[k];
          v[k] = keep + __shfl_xor(send, off, kWave);
        }
      }
      n = h;
    } else {
      v[0] += __shfl_xor(v[0], off, kWave);
    }
    off >>= 1;
  }
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

// One wavefront per weight row at a time; the next row's loads are issued before the current
// row is reduced (register double buffering).  NIT = ceil(H / 512): lane l covers the 16-byte
// pieces l + 64 * it of a row.
template <int M, int NIT>
__global__ __launch_bounds__(kBlock) void lmhead_gemv(const uint16_t *__restrict__ hidden,
                                                      const uint16_t *__restrict__ weight,
                                                      const int32_t *__restrict__ keep, int H, int Vt,
                                                      float *__restrict__ logits) {
  constexpr int NP = Pow2Ceil<M>::value;
  const int lane = lane_id();
  const int pieces = H >> 3;  // 16-byte pieces per row
  uint4 h[M][NIT];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int p = it * kWave + lane;
      h[m][it] = p < pieces ? reinterpret_cast<const uint4 *>(hidden + static_cast<int64_t>(m) * H)[p]
                            : make_uint4(0, 0, 0, 0);
    }

  const int nwaves = gridDim.x * kWavesPerBlock;
  int j = blockIdx.x * kWavesPerBlock + wave_id();
  if (j >= Vt) return;

  auto row_ptr = [&](int jj) -> const uint4 * {
    const int64_t r = keep ? static_cast<int64_t>(keep[jj]) : static_cast<int64_t>(jj);
    return reinterpret_cast<const uint4 *>(weight + r * H);
  };
  uint4 w[NIT];
  {
    const uint4 *src = row_ptr(j);
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int p = it * kWave + lane;
      w[it] = p < pieces ? load_nt(src + p) : make_uint4(0, 0, 0, 0);
    }
  }
  for (; j < Vt; j += nwaves) {
    const int jn = j + nwaves;
    uint4 wn[NIT];
    if (jn < Vt) {
      const uint4 *src = row_ptr(jn);
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int p = it * kWave + lane;
        wn[it] = p < pieces ? load_nt(src + p) : make_uint4(0, 0, 0, 0);
      }
    }
    float acc[NP];
#pragma unroll
    for (int m = 0; m < NP; ++m) acc[m] = 0.f;
#pragma unroll
    for (int it = 0; it < NIT; ++it)
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m] = dot8(w[it], h[m][it], acc[m]);
    const float s = transpose_reduce<NP>(acc);
    // lane l holds the sum for hidden row l / (64 / NP)
    constexpr int kGroup = kWave / NP;
    const int m = lane / kGroup;
    if ((lane % kGroup) == 0 && m < M) logits[static_cast<int64_t>(m) * Vt + j] = s;
    if (jn < Vt) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) w[it] = wn[it];
    }
  }
}

// ------------------------------------------------------------------------------ MFMA path
constexpr int kBM = 128, kBN = 128, kBK = 32, kLdsPad = 8;
constexpr int kLdsRow = kBK + kLdsPad;  // bf16 elements per LDS row (80 bytes)

// Workgroups are handed to the 8 XCDs round-robin; remap so that each XCD works on a
// contiguous range of logical tiles (consecutive tiles share a weight tile in that XCD's L2).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcd = 8;
  const int per = (nblocks + kXcd - 1) / kXcd;
  const int tall = nblocks % kXcd == 0 ? kXcd : nblocks % kXcd;
  const int xcd = bid % kXcd, local = bid / kXcd;
  return xcd < tall ? xcd * per + local : tall * per + (xcd - tall) * (per - 1) + local;
}

__global__ __launch_bounds__(kBlock) void lmhead_mfma(const uint16_t *__restrict__ hidden,
                                                      const uint16_t *__restrict__ weight,
                                                      const int32_t *__restrict__ keep, int M, int H, int Vt,
                                                      float *__restrict__ logits) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kBM * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kBN * kLdsRow];

  const int nbm = (M + kBM - 1) / kBM;
  const int nbn = (Vt + kBN - 1) / kBN;
  const int tile = xcd_remap(blockIdx.x, nbm * nbn);
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
      const int64_t r = keep ? static_cast<int64_t>(keep[gn]) : static_cast<int64_t>(gn);
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
using GemvFn = void (*)(const uint16_t *, const uint16_t *, const int32_t *, int, int, float *);

template <int M, int NIT>
constexpr GemvFn gemv_entry() {
  return &lmhead_gemv<M, NIT>;
}

constexpr int kGemvMaxM = 8;
constexpr int kGemvMaxNit = 8;
constexpr int kGemvMaxRegs = 48;  // M * NIT: hidden slice kept in 4 * M * NIT VGPRs

template <int M>
GemvFn gemv_for_nit(int nit) {
  switch (nit) {
    case 1: return gemv_entry<M, 1>();
    case 2: return gemv_entry<M, 2>();
    case 3: return gemv_entry<M, 3>();
    case 4: return gemv_entry<M, 4>();
    case 5: return M * 5 <= kGemvMaxRegs ? gemv_entry<M, 5>() : nullptr;
    case 6: return M * 6 <= kGemvMaxRegs ? gemv_entry<M, 6>() : nullptr;
    case 7: return M * 7 <= kGemvMaxRegs ? gemv_entry<M, 7>() : nullptr;
    case 8: return M * 8 <= kGemvMaxRegs ? gemv_entry<M, 8>() : nullptr;
    default: return nullptr;
  }
}

GemvFn pick_gemv(int64_t M, int64_t H) {
  const int nit = static_cast<int>((H + 511) / 512);
  if (nit > kGemvMaxNit || M > kGemvMaxM || M * nit > kGemvMaxRegs) return nullptr;
  switch (M) {
    case 1: return gemv_for_nit<1>(nit);
    case 2: return gemv_for_nit<2>(nit);
    case 3: return gemv_for_nit<3>(nit);
    case 4: return gemv_for_nit<4>(nit);
    case 5: return gemv_for_nit<5>(nit);
    case 6: return gemv_for_nit<6>(nit);
    case 7: return gemv_for_nit<7>(nit);
    case 8: return gemv_for_nit<8>(nit);
    default: return nullptr;
  }
}

}  // namespace
}  // namespace vt

extern "C" vt_status_t vt_lmhead_trimmed(const uint16_t *hidden, const uint16_t *weight, const int32_t *keep_ids,
                                         int64_t M, int64_t H, int64_t Vt, int64_t V_rows, float *logits,
                                         hipStream_t stream) {
  using namespace vt;
  if (!hidden || !weight || !logits) return VT_ERR_INVALID_ARG;
  if (M <= 0 || H <= 0 || Vt <= 0 || V_rows <= 0) return VT_ERR_INVALID_ARG;
  if (!keep_ids && Vt > V_rows) return VT_ERR_INVALID_ARG;
  if (M > INT32_MAX || H > INT32_MAX || Vt > INT32_MAX) return VT_ERR_UNSUPPORTED;
  if (H % 8 != 0 || !aligned16(hidden) || !aligned16(weight)) return VT_ERR_UNSUPPORTED;

  const GemvFn gemv = pick_gemv(M, H);
  if (gemv) {
    // enough wavefronts to keep every CU streaming, each walking rows with a stride
    const int64_t rows_per_block = kWavesPerBlock;
    int64_t blocks = (Vt + rows_per_block - 1) / rows_per_block;
    const int64_t kMaxBlocks = 256 * 4;  // 256 CUs x 4 workgroups
    if (blocks > kMaxBlocks) blocks = kMaxBlocks;
    return hip_status(launch(gemv, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, stream, hidden, weight,
                             keep_ids, static_cast<int>(H), static_cast<int>(Vt), logits));
  }
  const int64_t tiles = ((M + kBM - 1) / kBM) * ((Vt + kBN - 1) / kBN);
  if (tiles > INT32_MAX) return VT_ERR_UNSUPPORTED;
  return hip_status(launch(lmhead_mfma, dim3(static_cast<unsigned>(tiles)), dim3(kBlock), 0, stream, hidden, weight,
                           keep_ids, static_cast<int>(M), static_cast<int>(H), static_cast<int>(Vt), logits));
}

// Shared device helpers for the gfx950 kernels: 64-wide wavefront reductions and scans,
// 256-thread workgroup reductions and scans through LDS, bf16 decoding, host-side status glue.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <tuple>
#include <utility>

#include "vt.h"

namespace vt {

constexpr int kWave = 64;
constexpr int kBlock = 256;             // threads per workgroup in the row kernels
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kChunk = 4096;            // elements per chunk of a row (fixed: results never depend on B)
constexpr int kPerThread = kChunk / kBlock;  // 16 contiguous elements per thread

static_assert(kPerThread == 16, "chunk geometry");

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return static_cast<int>(threadIdx.x) / kWave; }

// ---- cross-lane moves without LDS: DPP within 16-lane rows, v_permlane16/32_swap across rows.
// (Shuffles with a computed lane index compile to ds_bpermute, an LDS round trip with a wait;
// these are plain VALU operations.)
// DPP controls: quad permutations that swap neighbours (lane ^ 1) and pairs (lane ^ 2), mirror
// within 8 and 16 lanes, rotate a row by 8, shift a row right by 1, 2, 4, 8, broadcast lane 15 of
// each row to the next row and lane 31 to the upper half, and shift the whole wave right by 1.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140, kDppRor8 = 0x128;
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143, kDppWaveShr1 = 0x138;

// x from the DPP source lane; lanes without one (or in rows outside ROWMASK) get `old`.
template <int CTRL, int ROWMASK = 0xF, typename T>
__device__ __forceinline__ T lane_move(T x, T old) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(
        T, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, x), CTRL, ROWMASK, 0xF,
                                       false));
  } else {
    const int2 xv = __builtin_bit_cast(int2, x), ov = __builtin_bit_cast(int2, old);
    int2 r;
    r.x = __builtin_amdgcn_update_dpp(ov.x, xv.x, CTRL, ROWMASK, 0xF, false);
    r.y = __builtin_amdgcn_update_dpp(ov.y, xv.y, CTRL, ROWMASK, 0xF, false);
    return __builtin_bit_cast(T, r);
  }
}
// x from the DPP source lane for patterns in which every lane has one (quad permutations,
// mirrors, rotations).  Written with bound_ctrl and no old value, so the compiler can fold the
// move into the consuming VALU operation (one v_*_dpp instead of a copy, a wait state and a move).
template <int CTRL, typename T>
__device__ __forceinline__ T lane_swap(T x) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
  } else {
    int2 v = __builtin_bit_cast(int2, x);
    v.x = __builtin_amdgcn_mov_dpp(v.x, CTRL, 0xF, 0xF, true);
    v.y = __builtin_amdgcn_mov_dpp(v.y, CTRL, 0xF, 0xF, true);
    return __builtin_bit_cast(T, v);
  }
}
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return lane_swap<CTRL>(x);
}

// v_permlane32_swap: lanes 32..63 of the first operand trade places with lanes 0..31 of the
// second; v_permlane16_swap does the same for the odd 16-lane rows of the first operand and the
// even rows of the second.  With both operands equal, each lane then holds its own value and its
// partner's at lane ^ 32 (^ 16), one in each result.
__device__ __forceinline__ void swap32(float &x, float &y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(float &x, float &y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}
template <bool k32, typename T>
__device__ __forceinline__ void swap_rows(T &x, T &y) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  constexpr int W = sizeof(T) / 4;
  uint32_t xa[W], ya[W];
  __builtin_memcpy(xa, &x, sizeof(T));
  __builtin_memcpy(ya, &y, sizeof(T));
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const auto r = k32 ? __builtin_amdgcn_permlane32_swap(xa[w], ya[w], false, false)
                       : __builtin_amdgcn_permlane16_swap(xa[w], ya[w], false, false);
    xa[w] = r[0];
    ya[w] = r[1];
  }
  __builtin_memcpy(&x, xa, sizeof(T));
  __builtin_memcpy(&y, ya, sizeof(T));
}

// Reduction of a commutative, associative op over the 64 lanes, the result in every lane: quad
// steps, the mirrors within 8 and 16 lanes (after each step a lane's partner holds the other
// half of its group), then lane ^ 16 and lane ^ 32.
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  v = op(v, lane_swap<kDppXor1>(v));
  v = op(v, lane_swap<kDppXor2>(v));
  v = op(v, lane_swap<kDppHalfMirror>(v));
  v = op(v, lane_swap<kDppMirror>(v));
  T a = v, b = v;
  swap_rows<false>(a, b);
  v = op(a, b);
  a = v;
  b = v;
  swap_rows<true>(a, b);
  return op(a, b);
}

__device__ __forceinline__ float wave_sum(float v) { return wave_reduce(v, [](float a, float b) { return a + b; }); }
__device__ __forceinline__ float wave_max(float v) { return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); }); }
__device__ __forceinline__ int wave_min_int(int v) { return wave_reduce(v, [](int a, int b) { return min(a, b); }); }
__device__ __forceinline__ int wave_max_int(int v) { return wave_reduce(v, [](int a, int b) { return max(a, b); }); }

// Inclusive prefix sum across the 64 lanes: shifts by 1, 2, 4, 8 inside each 16-lane row, then
// the last lane of each row is added to the next row and lane 31 to the upper half.
template <typename T>
__device__ __forceinline__ T wave_scan_incl(T v) {
  const T z = T(0);
  // row shifts: bound_ctrl gives 0 to the lanes without a source
  v = v + lane_swap<kDppRowShr1>(v);
  v = v + lane_swap<kDppRowShr2>(v);
  v = v + lane_swap<kDppRowShr4>(v);
  v = v + lane_swap<kDppRowShr8>(v);
  v = v + lane_move<kDppRowBcast15, 0xA>(v, z);
  v = v + lane_move<kDppRowBcast31, 0xC>(v, z);
  return v;
}
__device__ __forceinline__ float wave_inclusive_scan(float v) { return wave_scan_incl(v); }

// The previous lane's value (`first` in lane 0).
template <typename T>
__device__ __forceinline__ T wave_prev(T v, T first) {
  return lane_move<kDppWaveShr1>(v, first);
}

// Lane k's value in every lane (k uniform across the wave).
template <typename T>
__device__ __forceinline__ T lane_value(T v, int k) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), k));
  } else {
    int2 x = __builtin_bit_cast(int2, v);
    x.x = __builtin_amdgcn_readlane(x.x, k);
    x.y = __builtin_amdgcn_readlane(x.y, k);
    return __builtin_bit_cast(T, x);
  }
}

// Workgroup-wide reductions (all kBlock threads must call; result broadcast to every thread).
// `red` is LDS scratch of at least kWavesPerBlock floats/ints.
__device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  __syncthreads();
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kWavesPerBlock; ++w) t += red[w];
  return t;
}

__device__ __forceinline__ float block_max(float v, float *red) {
  v = wave_max(v);
  __syncthreads();
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  float t = red[0];
#pragma unroll
  for (int w = 1; w < kWavesPerBlock; ++w) t = fmaxf(t, red[w]);
  return t;
}

__device__ __forceinline__ int block_min_int(int v, int *red) {
  v = wave_min_int(v);
  __syncthreads();
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  int t = red[0];
#pragma unroll
  for (int w = 1; w < kWavesPerBlock; ++w) t = min(t, red[w]);
  return t;
}

__device__ __forceinline__ int block_max_int(int v, int *red) {
  v = wave_max_int(v);
  __syncthreads();
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  int t = red[0];
#pragma unroll
  for (int w = 1; w < kWavesPerBlock; ++w) t = max(t, red[w]);
  return t;
}

// Workgroups are handed to the 8 XCDs of the device round-robin (workgroup i runs on XCD i % 8).
// xcd_remap returns a logical index such that each XCD works through one contiguous range of
// logical indices, so workgroups that share data (a weight tile, a sequence's rows) can be given
// neighbouring logical indices and meet in one XCD's L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t nblocks) {
  constexpr int64_t kXcd = 8;
  const int64_t per = (nblocks + kXcd - 1) / kXcd;
  const int64_t tall = nblocks % kXcd == 0 ? kXcd : nblocks % kXcd;
  const int64_t xcd = bid % kXcd, local = bid / kXcd;
  return xcd < tall ? xcd * per + local : tall * per + (xcd - tall) * (per - 1) + local;
}

// K-tiled layout of a matrix of rows of H bf16 values (the trimmed head made by
// vt_trim_head_tiled; the MFMA heads' hidden-row copy takes the same layout with blocks of their
// own tile rows): block b of kTileRows rows and K step s of kTileK columns sit at
// out[b][s][r][kTileK], so each (b, s) slice is one contiguous 16 KB run.  Rows past the matrix's
// end fill out its last block.
constexpr int kTileRows = 256, kTileK = 32;
inline size_t tiled_rows_bytes(int64_t rows, int64_t H) {
  return static_cast<size_t>((rows + kTileRows - 1) / kTileRows) * kTileRows * static_cast<size_t>(H) * 2;
}

// Argmax with ties to the lowest index (padding carries index INT_MAX, so it never wins a tie).
constexpr int kNoIndex = 0x7fffffff;
__device__ __forceinline__ bool argmax_better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

struct ValIdx {
  float v;
  int i;
};
__device__ __forceinline__ void wave_argmax(float &v, int &i) {
  const uint64_t best = wave_reduce(__builtin_bit_cast(uint64_t, ValIdx{v, i}), [](uint64_t a, uint64_t b) {
    const ValIdx x = __builtin_bit_cast(ValIdx, a), y = __builtin_bit_cast(ValIdx, b);
    return argmax_better(y.v, y.i, x.v, x.i) ? b : a;
  });
  const ValIdx r = __builtin_bit_cast(ValIdx, best);
  v = r.v;
  i = r.i;
}

// Workgroup argmax (all threads call; result broadcast).  redv/redi: LDS scratch of 4 entries.
__device__ __forceinline__ void block_argmax(float &v, int &i, float *redv, int *redi) {
  wave_argmax(v, i);
  __syncthreads();
  if (lane_id() == 0) {
    redv[wave_id()] = v;
    redi[wave_id()] = i;
  }
  __syncthreads();
  v = redv[0];
  i = redi[0];
#pragma unroll
  for (int w = 1; w < kWavesPerBlock; ++w)
    if (argmax_better(redv[w], redi[w], v, i)) {
      v = redv[w];
      i = redi[w];
    }
}

// Inclusive prefix over the workgroup's threads in thread order.  Returns this thread's
// inclusive value; *prev receives the previous thread's inclusive value (0 for thread 0) and
// *total the last thread's, each formed by the very same floating-point operations as the value
// that thread returns, so comparisons against them are mutually consistent.
__device__ __forceinline__ float block_inclusive_scan(float v, float *red, float *prev, float *total) {
  const int lane = lane_id(), w = wave_id();
  const float inc = wave_inclusive_scan(v);
  const float up = wave_prev(inc, 0.f);
  __syncthreads();
  if (lane == kWave - 1) red[w] = inc;
  __syncthreads();
  float before = 0.f;
#pragma unroll
  for (int k = 0; k < kWavesPerBlock; ++k)
    if (k < w) before += red[k];
  float all = 0.f;
#pragma unroll
  for (int k = 0; k < kWavesPerBlock; ++k) all += red[k];
  *prev = lane == 0 ? before : before + up;
  *total = all;
  return before + inc;
}

// The N contiguous elements [base + N t, base + N t + N) of a row as fp32 (t = thread index);
// -inf past n.  kVec: the row start is 16-byte aligned and n a multiple of 8 (bf16) or 4 (fp32).
template <typename Tin, bool kVec, int N>
__device__ __forceinline__ void load_run(const Tin *__restrict__ row, int64_t n, int64_t base, float (&v)[N]) {
  static_assert(N % 4 == 0, "whole 4-element pieces");
  const int64_t e0 = base + static_cast<int64_t>(threadIdx.x) * N;
  if (kVec && e0 + N <= n) {
    if constexpr (sizeof(Tin) == 4) {
      const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(row) + e0);
#pragma unroll
      for (int q = 0; q < N / 4; ++q) {
        const float4 f = p[q];
        v[4 * q + 0] = f.x;
        v[4 * q + 1] = f.y;
        v[4 * q + 2] = f.z;
        v[4 * q + 3] = f.w;
      }
    } else if constexpr (N % 8 == 0) {
      const uint4 *p = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(row) + e0);
#pragma unroll
      for (int q = 0; q < N / 8; ++q) {
        const uint4 b = p[q];
        const unsigned int wds[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[8 * q + 2 * k + 0] = __uint_as_float(wds[k] << 16);
          v[8 * q + 2 * k + 1] = __uint_as_float(wds[k] & 0xffff0000u);
        }
      }
    } else {
      const uint2 *p = reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(row) + e0);
#pragma unroll
      for (int q = 0; q < N / 4; ++q) {
        const uint2 b = p[q];
        v[4 * q + 0] = __uint_as_float(b.x << 16);
        v[4 * q + 1] = __uint_as_float(b.x & 0xffff0000u);
        v[4 * q + 2] = __uint_as_float(b.y << 16);
        v[4 * q + 3] = __uint_as_float(b.y & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int64_t e = e0 + j;
      if (e < n) {
        if constexpr (sizeof(Tin) == 4)
          v[j] = reinterpret_cast<const float *>(row)[e];
        else
          v[j] = bf16_to_f32(reinterpret_cast<const uint16_t *>(row)[e]);
      } else {
        v[j] = kNegInf;
      }
    }
  }
}

template <typename Tin, bool kVec>
__device__ __forceinline__ void load16(const Tin *__restrict__ row, int64_t n, int64_t base, float (&v)[16]) {
  load_run<Tin, kVec, kPerThread>(row, n, base, v);
}

// Launch with an explicit status: arguments are converted to the kernel's parameter types and
// handed to hipLaunchKernel, whose return value reports this launch alone.
template <typename... KArgs, typename Tuple, size_t... I>
inline hipError_t launch_packed(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t stream,
                                Tuple &packed, std::index_sequence<I...>) {
  void *ptrs[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1] = {static_cast<void *>(&std::get<I>(packed))...};
  return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, ptrs, shmem, stream);
}

template <typename... KArgs, typename... Args>
inline hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t stream,
                         Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  std::tuple<KArgs...> packed(static_cast<KArgs>(args)...);
  return launch_packed(kernel, grid, block, shmem, stream, packed, std::index_sequence_for<KArgs...>{});
}

inline vt_status_t hip_status(hipError_t e) { return e == hipSuccess ? VT_OK : VT_ERR_HIP; }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool finite_positive(float t) { return t > 0.f && t <= 3.4028234663852886e38f; }

}  // namespace vt

// Keep-set construction: token histogram, kept-set selection, trimmed-head row gather.
//
// [VT] §3: the trimmed vocabulary is Top-K of a token-frequency counter (Algorithm 1, Eq. 1), with
// Top-P and a minimum frequency as alternative rules; W^Trim is the matching slice of W's rows.
//
// Histogram: the counter (V uint32, 513 KB at V = 128256) does not fit one CU's LDS, so the
// vocabulary is cut into slabs of kSlabBins bins (128 KB of LDS each).  Workgroup (g, s) counts
// the tokens of corpus segment g that fall in slab s with LDS atomics, then stores its slab of
// partial counts; a second launch sums the partials per id (no global atomics, deterministic).
// The S workgroups of one segment get neighbouring logical indices on one XCD, so the segment is
// fetched from HBM once and re-read by the other slabs from that XCD's L2.
#include "vt_common.hpp"
#include "vt_keepset.h"

namespace vt {
namespace {

constexpr int kHistThreads = 1024;
constexpr int kSlabBins = 32064;           // 4 slabs cover V = 128256 exactly
constexpr int64_t kMinTokensPerGroup = 1 << 16;
constexpr int kTargetWorkgroups = 256;     // one resident workgroup per CU (LDS-limited)

struct HistPlan {
  int slabs, groups;
  int64_t seg;  // tokens per group, a multiple of 4
};

HistPlan hist_plan(int64_t n, int64_t V) {
  HistPlan p{};
  p.slabs = static_cast<int>((V + kSlabBins - 1) / kSlabBins);
  const int64_t gmax = std::max<int64_t>(1, kTargetWorkgroups / p.slabs);
  const int64_t g = std::min<int64_t>(gmax, std::max<int64_t>(1, (n + kMinTokensPerGroup - 1) / kMinTokensPerGroup));
  p.groups = static_cast<int>(g);
  p.seg = ((n + g - 1) / g + 3) / 4 * 4;
  return p;
}

size_t hist_ws_bytes(const HistPlan &p, int64_t V) {
  return p.groups > 1 ? static_cast<size_t>(p.groups) * static_cast<size_t>(V) * sizeof(uint32_t) : 0;
}

// The slab bin holding the most counts so far (lowest index on ties); all threads call.
__device__ __forceinline__ int hottest_bin(const uint32_t *bins, int len, uint32_t *redc, int *redi) {
  uint32_t bc = 0;
  int bi = 0;
  for (int i = threadIdx.x; i < len; i += kHistThreads)
    if (bins[i] > bc) {
      bc = bins[i];
      bi = i;
    }
  // (count, -index) ordered as one 64-bit key: the wave maximum is the hottest, lowest bin
  const uint64_t key = wave_reduce((static_cast<uint64_t>(bc) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(bi)),
                                   [](uint64_t a, uint64_t b) { return a > b ? a : b; });
  bc = static_cast<uint32_t>(key >> 32);
  bi = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key));
  if (lane_id() == 0) {
    redc[wave_id()] = bc;
    redi[wave_id()] = bi;
  }
  __syncthreads();
  bc = redc[0];
  bi = redi[0];
  for (int w = 1; w < kHistThreads / kWave; ++w)
    if (redc[w] > bc || (redc[w] == bc && redi[w] < bi)) {
      bc = redc[w];
      bi = redi[w];
    }
  return bi;
}

// Counts tokens [g*seg, min(n, (g+1)*seg)) that fall in slab s.  With one group the slab is
// written (or added) to counts directly; otherwise to part[g][.] for hist_sum.
// Token frequencies are heavy-tailed, and lanes of one LDS atomic that hit the same bin are
// serialised; so after the first 64K tokens of the segment the slab's most frequent bin so far
// is counted in a register per lane instead, and folded in once at the end.
template <bool kVec>
__global__ __launch_bounds__(kHistThreads) void hist_slab(const int32_t *__restrict__ tokens, int64_t n, int64_t seg,
                                                          int V, int slabs, int accumulate, uint32_t *__restrict__ counts,
                                                          uint32_t *__restrict__ part) {
  __shared__ uint32_t bins[kSlabBins];
  __shared__ uint32_t redc[kHistThreads / kWave];
  __shared__ int redi[kHistThreads / kWave];
  const int64_t L = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t g = L / slabs;
  const int s = static_cast<int>(L - g * slabs);
  const int lo = s * kSlabBins;
  const int len = min(kSlabBins, V - lo);
  for (int i = threadIdx.x; i < kSlabBins; i += kHistThreads) bins[i] = 0u;
  __syncthreads();

  const int64_t b0 = g * seg;
  const int64_t b1 = min(n, b0 + seg);
  uint32_t hot = 0, hot_n = 0;
  bool use_hot = false;
  auto add = [&](int32_t t) {
    const uint32_t u = static_cast<uint32_t>(t - lo);  // negative ids and ids past the slab fail
    if (use_hot && u == hot)
      ++hot_n;
    else if (u < static_cast<uint32_t>(len))
      atomicAdd(&bins[u], 1u);
  };
  constexpr int kU = 4;
  auto run = [&](const int4 *t4, int64_t q, int64_t q1) {
    for (; q + (kU - 1) * kHistThreads < q1; q += kU * kHistThreads) {
      int4 v[kU];
#pragma unroll
      for (int r = 0; r < kU; ++r) v[r] = t4[q + r * kHistThreads];  // plain loads: the other slabs re-read them from L2
#pragma unroll
      for (int r = 0; r < kU; ++r) {
        add(v[r].x);
        add(v[r].y);
        add(v[r].z);
        add(v[r].w);
      }
    }
    for (; q < q1; q += kHistThreads) {
      const int4 v = t4[q];
      add(v.x);
      add(v.y);
      add(v.z);
      add(v.w);
    }
  };
  int64_t tail = b0;
  if (kVec && b1 > b0) {
    // b0 is a multiple of 4 and tokens is 16-byte aligned: whole int4 groups up to b1 & ~3
    const int4 *t4 = reinterpret_cast<const int4 *>(tokens);
    const int64_t q0 = b0 / 4, q1 = b1 / 4;
    const int64_t qa = min(q1, q0 + 16 * kHistThreads);
    run(t4, q0 + threadIdx.x, qa);
    if (qa < q1) {
      __syncthreads();
      hot = static_cast<uint32_t>(hottest_bin(bins, len, redc, redi));
      use_hot = true;
      run(t4, qa + threadIdx.x, q1);
    }
    tail = q1 * 4;
  }
  for (int64_t i = tail + threadIdx.x; i < b1; i += kHistThreads) add(tokens[i]);
  if (use_hot) {
    hot_n = wave_reduce(hot_n, [](uint32_t a, uint32_t b) { return a + b; });
    if (lane_id() == 0 && hot_n) atomicAdd(&bins[hot], hot_n);
  }
  __syncthreads();

  if (part == nullptr) {
    for (int i = threadIdx.x; i < len; i += kHistThreads)
      counts[lo + i] = (accumulate ? counts[lo + i] : 0u) + bins[i];
  } else {
    uint32_t *dst = part + g * static_cast<int64_t>(V) + lo;
    for (int i = threadIdx.x; i < len; i += kHistThreads) dst[i] = bins[i];
  }
}

__global__ __launch_bounds__(kBlock) void hist_sum(const uint32_t *__restrict__ part, int groups, int V,
                                                   int accumulate, uint32_t *__restrict__ counts) {
  const int v = blockIdx.x * kBlock + threadIdx.x;
  if (v >= V) return;
  uint32_t s = accumulate ? counts[v] : 0u;
  for (int g = 0; g < groups; ++g) s += part[static_cast<int64_t>(g) * V + v];
  counts[v] = s;
}

// ---------------------------------------------------------------- selection (one workgroup)
//
// The counts (513 KB at V = 128256) are walked in tiles of 16384: thread t owns the 16 contiguous
// ids [tile + 16 t, tile + 16 t + 16), fetched with 16-byte loads, so every pass is a handful of
// wide loads per thread rather than a latency-bound loop.

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kSelPer = 16;
constexpr int kSelTile = kSelThreads * kSelPer;
constexpr int kDigitBits = 11;
constexpr int kDigits = 1 << kDigitBits;   // 2048 buckets, two per thread

template <typename T>
__device__ __forceinline__ T wave_sum_t(T v) {
  return wave_reduce(v, [](T a, T b) { return a + b; });
}

// Exclusive prefix over the 1024 threads in thread order; *total gets the sum of all.
template <typename T>
__device__ __forceinline__ T sel_exclusive_scan(T v, T *red, T *total) {
  const int lane = lane_id(), w = wave_id();
  const T inc = wave_scan_incl(v);
  __syncthreads();
  if (lane == kWave - 1) red[w] = inc;
  __syncthreads();
  T before = 0, all = 0;
#pragma unroll
  for (int k = 0; k < kSelWaves; ++k) {
    if (k < w) before += red[k];
    all += red[k];
  }
  *total = all;
  return before + inc - v;
}

struct SelParams {
  const uint32_t *counts;
  int V;
  int rule;
  int64_t k;
  double p;
  uint32_t min_count;
  int32_t *keep;
  int32_t *f2t;
  int32_t *num_kept;
};

// This thread's 16 counts of the tile starting at id `tile`, loaded without a branch, at
// indices clamped into [0, V) (kVec is chosen only when V is a multiple of 4, so V >= 4 and each
// 16-byte piece lies wholly inside or wholly past the end); entries past
// V hold repeats and must be masked by the caller (tile_valid).  Loading the next tile this way
// while the current one is processed keeps the loads in flight: a branch around them would make
// the compiler wait for them at the join.
template <bool kVec>
__device__ __forceinline__ void load_tile_raw(const SelParams &P, int tile, uint32_t (&c)[kSelPer]) {
  const int e0 = tile + static_cast<int>(threadIdx.x) * kSelPer;
  if constexpr (kVec) {
    const uint4 *p4 = reinterpret_cast<const uint4 *>(P.counts);
    const int last = P.V / 4 - 1;
#pragma unroll
    for (int q = 0; q < kSelPer / 4; ++q) {
      const uint4 v = p4[min(e0 / 4 + q, last)];
      c[4 * q] = v.x;
      c[4 * q + 1] = v.y;
      c[4 * q + 2] = v.z;
      c[4 * q + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kSelPer; ++j) c[j] = P.counts[min(e0 + j, P.V - 1)];
  }
}

__device__ __forceinline__ int tile_valid(const SelParams &P, int tile) {
  return max(0, min(kSelPer, P.V - tile - static_cast<int>(threadIdx.x) * kSelPer));
}

// Radix descent for the threshold count.  by_mass = false: `want` counts ids (the k-th largest
// count); by_mass = true: `want` is a summed count.  Returns the threshold c* and leaves in *rest
// what the ids with count == c* must still contribute (ids or count).  Each thread folds runs of
// equal digits among its 16 ids before touching LDS, and each wavefront merges the bucket of its
// first contributing lane into a single atomic: heavy-tailed counts put most ids in one bucket.
template <bool kVec>
__device__ uint32_t radix_threshold(const SelParams &P, bool by_mass, uint64_t want, uint64_t *hist, uint64_t *red,
                                    uint64_t *rest) {
  __shared__ uint32_t sh_digit;
  __shared__ uint64_t sh_above;
  const int lane = lane_id();
  uint32_t prefix = 0, mask = 0;
  const int shifts[3] = {21, 10, 0};
  const uint32_t dmasks[3] = {2047u, 2047u, 1023u};
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = shifts[pass];
    const uint32_t dm = dmasks[pass];
    for (int i = threadIdx.x; i < kDigits; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    uint32_t c[kSelPer], cn[kSelPer];
    load_tile_raw<kVec>(P, 0, c);
    for (int tile = 0; tile < P.V; tile += kSelTile) {
      load_tile_raw<kVec>(P, tile + kSelTile, cn);  // the next tile (clamped, unused past the end)
      const int nv = tile_valid(P, tile);
      int cur = -1;
      uint64_t acc = 0;
#pragma unroll
      for (int j = 0; j < kSelPer; ++j) {
        if (j < nv && (c[j] & mask) == prefix) {
          const int d = static_cast<int>((c[j] >> sh) & dm);
          const uint64_t v = by_mass ? c[j] : 1u;
          if (d == cur) {
            acc += v;
          } else {
            if (cur >= 0) atomicAdd(reinterpret_cast<unsigned long long *>(&hist[cur]), acc);
            cur = d;
            acc = v;
          }
        }
      }
      const unsigned long long has = __ballot(cur >= 0);
      if (has) {
        const int leader = __ffsll(static_cast<long long>(has)) - 1;
        const int d0 = lane_value(cur, leader);
        const bool same = cur >= 0 && cur == d0;
        const uint64_t tot = wave_sum_t<uint64_t>(same ? acc : 0);
        if (lane == leader) atomicAdd(reinterpret_cast<unsigned long long *>(&hist[d0]), tot);
        if (cur >= 0 && !same) atomicAdd(reinterpret_cast<unsigned long long *>(&hist[cur]), acc);
      }
#pragma unroll
      for (int j = 0; j < kSelPer; ++j) c[j] = cn[j];
    }
    __syncthreads();
    // thread t owns digits hi = 2047 - 2t and hi - 1, so thread order is descending digit order
    const int hi = kDigits - 1 - 2 * static_cast<int>(threadIdx.x);
    const uint64_t hh = hist[hi], hl = hist[hi - 1];
    uint64_t tot;
    const uint64_t before = sel_exclusive_scan<uint64_t>(hh + hl, red, &tot);
    if (before < want && want <= before + hh + hl) {
      if (want <= before + hh) {
        sh_digit = static_cast<uint32_t>(hi);
        sh_above = before;
      } else {
        sh_digit = static_cast<uint32_t>(hi - 1);
        sh_above = before + hh;
      }
    }
    __syncthreads();
    want -= sh_above;
    prefix |= sh_digit << sh;
    mask |= dm << sh;
    __syncthreads();
  }
  *rest = want;
  return prefix;
}

template <bool kVec>
__global__ __launch_bounds__(kSelThreads) void keep_select(SelParams P) {
  __shared__ uint64_t hist[kDigits];
  __shared__ uint64_t red64[kSelWaves];
  __shared__ int red32[kSelWaves];

  // threshold count and how many ids at exactly that count are kept (lowest ids first)
  uint32_t thr = 0;
  int64_t need = 0;
  if (P.rule == VT_SELECT_MIN_FREQ) {
    thr = P.min_count;
    need = INT64_MAX;
  } else {
    uint64_t want = static_cast<uint64_t>(P.k);
    bool by_mass = false;
    if (P.rule == VT_SELECT_TOP_P) {
      uint64_t s = 0;
      uint32_t c[kSelPer], cn[kSelPer];
      load_tile_raw<kVec>(P, 0, c);
      for (int tile = 0; tile < P.V; tile += kSelTile) {
        load_tile_raw<kVec>(P, tile + kSelTile, cn);
        const int nv = tile_valid(P, tile);
#pragma unroll
        for (int j = 0; j < kSelPer; ++j) {
          s += j < nv ? c[j] : 0u;
          c[j] = cn[j];
        }
      }
      uint64_t total;
      (void)sel_exclusive_scan<uint64_t>(s, red64, &total);
      want = static_cast<uint64_t>(ceil(P.p * static_cast<double>(total)));
      by_mass = want > 0;
      if (!by_mass) want = 1;  // nothing counted: keep one id
    }
    uint64_t rest;
    thr = radix_threshold<kVec>(P, by_mass, want, hist, red64, &rest);
    // by mass, ties are taken until their count covers the rest: ceil(rest / thr) of them
    need = by_mass ? static_cast<int64_t>((rest + thr - 1) / thr) : static_cast<int64_t>(rest);
  }

  // ordered compaction, tile by tile, carrying the tie and kept counts across tiles.  full_to_trim
  // goes out as 16-byte stores of each thread's 16 ids; the tile's kept ids are staged in LDS and
  // written contiguously by consecutive lanes.
  __shared__ int32_t kbuf[kSelTile];
  int tie_carry = 0, keep_carry = 0;
  uint32_t c[kSelPer], cn[kSelPer];
  load_tile_raw<kVec>(P, 0, c);
  for (int tile = 0; tile < P.V; tile += kSelTile) {
    load_tile_raw<kVec>(P, tile + kSelTile, cn);
    const int nv = tile_valid(P, tile);
    int above = 0, ties = 0;
#pragma unroll
    for (int j = 0; j < kSelPer; ++j) {
      above += j < nv && c[j] > thr;
      ties += j < nv && c[j] == thr;
    }
    int tie_total;
    const int tie_base = tie_carry + sel_exclusive_scan<int>(ties, red32, &tie_total);
    const int take = static_cast<int>(min<int64_t>(ties, max<int64_t>(0, need - tie_base)));
    int kept_total;
    const int local = sel_exclusive_scan<int>(above + take, red32, &kept_total);
    const int e0 = tile + static_cast<int>(threadIdx.x) * kSelPer;
    int pos = local, tie_rank = tie_base;
    int32_t f[kSelPer];
#pragma unroll
    for (int j = 0; j < kSelPer; ++j) {
      bool kept = j < nv && c[j] > thr;
      if (j < nv && c[j] == thr) {
        kept = tie_rank < need;
        ++tie_rank;
      }
      f[j] = kept ? keep_carry + pos : -1;
      if (kept) kbuf[pos++] = e0 + j;
    }
    if (kVec && nv == kSelPer) {
      int4 *f4 = reinterpret_cast<int4 *>(P.f2t + e0);
#pragma unroll
      for (int q = 0; q < kSelPer / 4; ++q) f4[q] = make_int4(f[4 * q], f[4 * q + 1], f[4 * q + 2], f[4 * q + 3]);
    } else {
#pragma unroll
      for (int j = 0; j < kSelPer; ++j)
        if (j < nv) P.f2t[e0 + j] = f[j];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kept_total; i += kSelThreads) P.keep[keep_carry + i] = kbuf[i];
    __syncthreads();
    tie_carry += tie_total;
    keep_carry += kept_total;
#pragma unroll
    for (int j = 0; j < kSelPer; ++j) c[j] = cn[j];
  }
  if (threadIdx.x == 0) *P.num_kept = keep_carry;
}

// ---------------------------------------------------------------- trimmed head

constexpr int kRowsPerBlock = 4;  // one wave per row

__global__ __launch_bounds__(kBlock) void trim_rows(const uint16_t *__restrict__ weight, int V_rows, int H,
                                                    const int32_t *__restrict__ keep, int k, uint16_t *__restrict__ out) {
  const int r = blockIdx.x * kRowsPerBlock + wave_id();
  if (r >= k) return;
  const int id = keep[r];
  const int n16 = H / 8;  // 16-byte groups per row
  uint4 *dst = reinterpret_cast<uint4 *>(out + static_cast<int64_t>(r) * H);
  if (id < 0 || id >= V_rows) {
    for (int i = lane_id(); i < n16; i += kWave) dst[i] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  const uint4 *src = reinterpret_cast<const uint4 *>(weight + static_cast<int64_t>(id) * H);
  for (int i = lane_id(); i < n16; i += kWave) dst[i] = src[i];
}

// K-tiled trimmed head: one thread per 16-byte piece of the output, out[b][s][r][32] = row
// 256 b + r of W^Trim, columns 32 s .. 32 s + 31 (a wave reads 16 rows x 64 bytes and writes 1 KB
// contiguously).  Rows past k and rows whose id lies outside [0, V_rows) are zeros.
__global__ __launch_bounds__(kBlock) void trim_tiles(const uint16_t *__restrict__ weight, int V_rows, int H,
                                                     const int32_t *__restrict__ keep, int k, int64_t pieces,
                                                     uint16_t *__restrict__ out) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (q >= pieces) return;
  const int p = static_cast<int>(q & 3);
  const int64_t rr = q >> 2;
  const int r = static_cast<int>(rr % kTileRows);
  const int64_t bs = rr / kTileRows;
  const int nk = H / kTileK;
  const int s = static_cast<int>(bs % nk);
  const int j = static_cast<int>(bs / nk) * kTileRows + r;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (j < k) {
    const int id = keep ? keep[j] : j;
    if (id >= 0 && id < V_rows)
      v = *reinterpret_cast<const uint4 *>(weight + static_cast<int64_t>(id) * H + s * kTileK + p * 8);
  }
  *reinterpret_cast<uint4 *>(out + q * 8) = v;
}

}  // namespace
}  // namespace vt

extern "C" size_t vt_token_histogram_workspace_bytes(int64_t n, int64_t V) {
  if (n < 0 || V <= 0 || V > INT32_MAX) return 0;
  const vt::HistPlan p = vt::hist_plan(n, V);
  return vt::hist_ws_bytes(p, V);
}

extern "C" vt_status_t vt_token_histogram(const int32_t *tokens, int64_t n, int64_t V, int accumulate,
                                          uint32_t *counts, void *workspace, size_t workspace_bytes,
                                          hipStream_t stream) {
  using namespace vt;
  if (!counts || n < 0 || V <= 0 || (n > 0 && !tokens)) return VT_ERR_INVALID_ARG;
  if (V > INT32_MAX || (reinterpret_cast<uintptr_t>(tokens) & 3u) != 0) return VT_ERR_UNSUPPORTED;
  const HistPlan p = hist_plan(n, V);
  const size_t need = hist_ws_bytes(p, V);
  if (need > 0 && (!workspace || workspace_bytes < need)) return VT_ERR_WORKSPACE;
  uint32_t *part = need > 0 ? static_cast<uint32_t *>(workspace) : nullptr;
  const int acc = accumulate ? 1 : 0;
  const unsigned grid = static_cast<unsigned>(p.groups) * static_cast<unsigned>(p.slabs);
  const bool vec = aligned16(tokens);
  hipError_t e = vec ? launch(hist_slab<true>, dim3(grid), dim3(kHistThreads), 0, stream, tokens, n, p.seg,
                              static_cast<int>(V), p.slabs, acc, counts, part)
                     : launch(hist_slab<false>, dim3(grid), dim3(kHistThreads), 0, stream, tokens, n, p.seg,
                              static_cast<int>(V), p.slabs, acc, counts, part);
  if (e != hipSuccess || part == nullptr) return hip_status(e);
  e = launch(hist_sum, dim3(static_cast<unsigned>((V + kBlock - 1) / kBlock)), dim3(kBlock), 0, stream,
             static_cast<const uint32_t *>(part), p.groups, static_cast<int>(V), acc, counts);
  return hip_status(e);
}

extern "C" vt_status_t vt_keep_select(const uint32_t *counts, int64_t V, vt_select_t rule, int64_t k, double p,
                                      uint32_t min_count, int32_t *keep_ids, int32_t *full_to_trim,
                                      int32_t *num_kept, hipStream_t stream) {
  using namespace vt;
  if (!counts || !keep_ids || !full_to_trim || !num_kept || V <= 0) return VT_ERR_INVALID_ARG;
  if (rule != VT_SELECT_TOP_K && rule != VT_SELECT_TOP_P && rule != VT_SELECT_MIN_FREQ) return VT_ERR_INVALID_ARG;
  if (rule == VT_SELECT_TOP_K && (k < 1 || k > V)) return VT_ERR_INVALID_ARG;
  if (rule == VT_SELECT_TOP_P && !(p > 0.0 && p <= 1.0)) return VT_ERR_INVALID_ARG;
  if (V > INT32_MAX) return VT_ERR_UNSUPPORTED;
  const SelParams P{counts, static_cast<int>(V), static_cast<int>(rule), k, p, min_count, keep_ids, full_to_trim,
                    num_kept};
  // 16-byte loads need aligned buffers and whole 4-count pieces (load_tile_raw clamps piece indices)
  return hip_status(aligned16(counts) && aligned16(full_to_trim) && V % 4 == 0
                        ? launch(keep_select<true>, dim3(1), dim3(kSelThreads), 0, stream, P)
                                      : launch(keep_select<false>, dim3(1), dim3(kSelThreads), 0, stream, P));
}

extern "C" vt_status_t vt_trim_head(const uint16_t *weight, int64_t V_rows, int64_t H, const int32_t *keep_ids,
                                    int64_t k, uint16_t *trimmed, hipStream_t stream) {
  using namespace vt;
  if (!weight || !keep_ids || !trimmed || V_rows <= 0 || H <= 0 || k <= 0) return VT_ERR_INVALID_ARG;
  if (H % 8 != 0 || !aligned16(weight) || !aligned16(trimmed)) return VT_ERR_UNSUPPORTED;
  if (k > INT32_MAX || V_rows > INT32_MAX || H > INT32_MAX) return VT_ERR_UNSUPPORTED;
  const unsigned grid = static_cast<unsigned>((k + kRowsPerBlock - 1) / kRowsPerBlock);
  return hip_status(launch(trim_rows, dim3(grid), dim3(kBlock), 0, stream, weight, static_cast<int>(V_rows),
                           static_cast<int>(H), keep_ids, static_cast<int>(k), trimmed));
}

extern "C" size_t vt_trim_head_tiled_bytes(int64_t k, int64_t H) {
  if (k <= 0 || H <= 0 || H % vt::kTileK != 0) return 0;
  return vt::tiled_rows_bytes(k, H);
}

extern "C" vt_status_t vt_trim_head_tiled(const uint16_t *weight, int64_t V_rows, int64_t H, const int32_t *keep_ids,
                                          int64_t k, uint16_t *tiled, hipStream_t stream) {
  using namespace vt;
  if (!weight || !tiled || V_rows <= 0 || H <= 0 || k <= 0 || (!keep_ids && k > V_rows)) return VT_ERR_INVALID_ARG;
  if (H % kTileK != 0 || !aligned16(weight) || !aligned16(tiled)) return VT_ERR_UNSUPPORTED;
  if (k > INT32_MAX || V_rows > INT32_MAX || H > INT32_MAX) return VT_ERR_UNSUPPORTED;
  const int64_t pieces = static_cast<int64_t>(tiled_rows_bytes(k, H) / 16);
  const int64_t grid = (pieces + kBlock - 1) / kBlock;
  if (grid > INT32_MAX) return VT_ERR_UNSUPPORTED;
  return hip_status(launch(trim_tiles, dim3(static_cast<unsigned>(grid)), dim3(kBlock), 0, stream, weight,
                           static_cast<int>(V_rows), static_cast<int>(H), keep_ids, static_cast<int>(k), pieces,
                           tiled));
}

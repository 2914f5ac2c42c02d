// Generation loop for table models ("A rejection rule keeps speculative decoding's output exact",
// section "Extending the rule from one token to a drafted run"; "VocabTrim", Appendix C.1,
// Algorithm 2).  One wavefront runs one sequence's whole loop: lane j holds token j of the row in
// use, so a softmax row, its running sum and an inverse-CDF draw are wave-wide operations with
// no LDS traffic.  Both tables (at most 65 x 64 fp32 each) and their per-row log-normalisers live
// in LDS; each workgroup loads them once and its four waves then take sequences grid-stride.
#include "vt_generate.h"
#include "verify_impl.hpp"

namespace vt {
namespace {

constexpr int kGenMaxV = kWave;
constexpr int kGenMaxRows = kGenMaxV + 1;
constexpr int kGenMaxBlocks = 2048;

struct GenParams {
  const float *tt;
  const float *dt;
  int V;
  double Tt, Td;
  float k2t, k2d;
  int gamma;
  int64_t B;
  int L;
  const float *u;
  int32_t *tokens;
  int32_t *stats;
};

__device__ __forceinline__ double wave_max_d(double v) {
  return wave_reduce(v, [](double a, double b) { return fmax(a, b); });
}

__device__ __forceinline__ double wave_sum_d(double v) {
  return wave_reduce(v, [](double a, double b) { return a + b; });
}

// Inverse-CDF draw over lanes 0..V-1 (token order) from weights w (0 on lanes >= V): the first
// lane whose inclusive running sum reaches u * Z, Z the running sum at lane V-1; else the last
// lane with positive weight; lane 0 if there is none.
__device__ __forceinline__ int wave_draw(float w, float u, int V) {
  const int lane = lane_id();
  const float C = wave_inclusive_scan(w);
  const float Z = lane_value(C, V - 1);
  const float t = u * Z;
  const unsigned long long hit = __ballot(lane < V && t <= C);
  if (hit) return __ffsll(static_cast<long long>(hit)) - 1;
  const unsigned long long pos = __ballot(lane < V && w > 0.f);
  return pos ? 63 - __clzll(static_cast<long long>(pos)) : 0;
}

__global__ __launch_bounds__(kBlock) void markov_generate(GenParams P) {
  __shared__ float tl[kGenMaxRows * kGenMaxV];
  __shared__ float dl[kGenMaxRows * kGenMaxV];
  __shared__ double tlse[kGenMaxRows];
  __shared__ double dlse[kGenMaxRows];
  const int V = P.V, rows = V + 1, g = P.gamma;
  const int lane = lane_id();
  const bool on = lane < V;
  for (int i = threadIdx.x; i < rows * V; i += kBlock) {
    tl[i] = P.tt[i];
    dl[i] = P.dt[i];
  }
  __syncthreads();
  // per-row log-normalisers of logits / T, in float64
  for (int r = wave_id(); r < 2 * rows; r += kWavesPerBlock) {
    const bool tgt = r < rows;
    const int row = tgt ? r : r - rows;
    const double T = tgt ? P.Tt : P.Td;
    const double x = on ? static_cast<double>((tgt ? tl : dl)[row * V + lane]) / T : -__builtin_inf();
    const double m = wave_max_d(x);
    const double s = wave_sum_d(on ? exp(x - m) : 0.0);
    if (lane == 0) (tgt ? tlse : dlse)[row] = m + log(s);
  }
  __syncthreads();

  const int64_t nw = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
  for (int64_t b = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave_id(); b < P.B; b += nw) {
    int ctx = 0, count = 0, blk = 0, tests = 0, accepted = 0, emitted = 0;
    int32_t *out = P.tokens + b * P.L;
    while (count < P.L) {
      const float *ub = P.u + (b * P.L + blk) * static_cast<int64_t>(2 * g + 1);
      // drafts: lane i keeps draft i and the table row it was drawn at
      int cur = ctx, myx = 0, myrow = 0;
      for (int i = 0; i < g; ++i) {
        const RowExp qe = make_row_exp(dlse[cur], P.Td, P.k2d);
        const float q = on ? qe(dl[cur * V + lane]) : 0.f;
        const int x = wave_draw(q, ub[i], V);
        if (lane == i) {
          myx = x;
          myrow = cur;
        }
        cur = x + 1;
      }
      // accept tests on lanes 0..gamma-1, fp64 ratios; n = first rejection, else gamma
      bool ok = true;
      if (lane < g) {
        const double a = static_cast<double>(tl[myrow * V + myx]) / P.Tt - tlse[myrow];
        const double d = static_cast<double>(dl[myrow * V + myx]) / P.Td - dlse[myrow];
        ok = static_cast<double>(ub[g + lane]) <= fmin(1.0, exp(a - d));
      }
      const unsigned long long rej = __ballot(lane < g && !ok);
      const int n = rej ? __ffsll(static_cast<long long>(rej)) - 1 : g;
      // final token: residual max(0, p_n - q_n) after a rejection, p_gamma after g acceptances
      const int rn = n < g ? lane_value(myrow, n) : cur;
      const RowExp pe = make_row_exp(tlse[rn], P.Tt, P.k2t);
      const float p = on ? pe(tl[rn * V + lane]) : 0.f;
      float w = p;
      if (n < g) {
        const RowExp qe = make_row_exp(dlse[rn], P.Td, P.k2d);
        const float q = on ? qe(dl[rn * V + lane]) : 0.f;
        w = fmaxf(p - q, 0.f);
        const float z = lane_value(wave_inclusive_scan(w), V - 1);
        if (!(z > 0.f)) w = p;
      }
      const int fin = wave_draw(w, ub[2 * g], V);
      if (lane < n && count + lane < P.L) out[count + lane] = myx;
      if (lane == 0 && count + n < P.L) out[count + n] = fin;
      tests += n < g ? n + 1 : g;
      accepted += n;
      emitted += n + 1;
      count += n + 1;
      ctx = fin + 1;
      ++blk;
    }
    if (P.stats && lane < 4) {
      const int v = lane == 0 ? blk : lane == 1 ? tests : lane == 2 ? accepted : emitted;
      P.stats[b * 4 + lane] = v;
    }
  }
}

}  // namespace
}  // namespace vt

extern "C" vt_status_t vt_spec_generate_markov(const float *target_table, const float *draft_table, int64_t V,
                                               float target_T, float draft_T, int64_t gamma, int64_t B,
                                               int64_t n_tokens, const float *u, int32_t *out_tokens,
                                               int32_t *out_stats, hipStream_t stream) {
  using namespace vt;
  if (!target_table || !draft_table || !u || !out_tokens) return VT_ERR_INVALID_ARG;
  if (V < 1 || gamma < 1 || B < 1 || n_tokens < 1) return VT_ERR_INVALID_ARG;
  if (!finite_positive(target_T) || !finite_positive(draft_T)) return VT_ERR_INVALID_ARG;
  if (V > kGenMaxV || gamma > kWave || n_tokens > INT32_MAX) return VT_ERR_UNSUPPORTED;
  GenParams P{};
  P.tt = target_table;
  P.dt = draft_table;
  P.V = static_cast<int>(V);
  P.Tt = target_T;
  P.Td = draft_T;
  P.k2t = static_cast<float>(kLog2e / static_cast<double>(target_T));
  P.k2d = static_cast<float>(kLog2e / static_cast<double>(draft_T));
  P.gamma = static_cast<int>(gamma);
  P.B = B;
  P.L = static_cast<int>(n_tokens);
  P.u = u;
  P.tokens = out_tokens;
  P.stats = out_stats;
  const int64_t blocks = std::min<int64_t>(kGenMaxBlocks, (B + kWavesPerBlock - 1) / kWavesPerBlock);
  return hip_status(launch(markov_generate, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, stream, P));
}

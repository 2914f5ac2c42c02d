// C entry points of the temperature softmax; the kernels live in softmax_impl.hpp.
#include "softmax_impl.hpp"

extern "C" size_t vt_softmax_temp_workspace_bytes(int64_t rows, int64_t n) {
  if (rows <= 0 || n <= 0) return 0;
  return vt::sm_ws_layout(rows, (n + vt::kChunk - 1) / vt::kChunk).bytes;
}

extern "C" vt_status_t vt_softmax_temp(const void *logits, vt_dtype_t dtype, int64_t rows, int64_t n, int64_t ld,
                                       float temperature, double *lse, float *probs, const float *u, int32_t *sampled,
                                       void *workspace, size_t workspace_bytes, hipStream_t stream) {
  using namespace vt;
  if (!logits || !lse) return VT_ERR_INVALID_ARG;
  if (dtype != VT_F32 && dtype != VT_BF16) return VT_ERR_INVALID_ARG;
  if (rows <= 0 || n <= 0 || ld < n) return VT_ERR_INVALID_ARG;
  const bool greedy = temperature == 0.f;
  if (!greedy && !finite_positive(temperature)) return VT_ERR_INVALID_ARG;
  if (!greedy && (u == nullptr) != (sampled == nullptr)) return VT_ERR_INVALID_ARG;
  if (n > INT32_MAX) return VT_ERR_UNSUPPORTED;
  const int64_t nchunk = (n + kChunk - 1) / kChunk;
  if (nchunk > INT32_MAX || rows > INT64_MAX / nchunk || rows * nchunk > static_cast<int64_t>(UINT32_MAX))
    return VT_ERR_UNSUPPORTED;
  const SMWsLayout L = sm_ws_layout(rows, nchunk);
  if (L.bytes > 0 && (!workspace || workspace_bytes < L.bytes)) return VT_ERR_WORKSPACE;

  SmParams P{};
  P.logits = logits;
  P.rows = rows;
  P.n = n;
  P.ld = ld;
  P.greedy = greedy;
  P.T = greedy ? 1.0 : static_cast<double>(temperature);
  P.invT = 1.0 / P.T;
  P.k2 = greedy ? 0.f : static_cast<float>(1.4426950408889634 / static_cast<double>(temperature));
  P.lse = lse;
  P.probs = probs;
  P.u = greedy ? nullptr : u;
  P.sampled = sampled;
  P.nchunk = static_cast<int>(nchunk);
  P.chunk = kChunk;
  if (L.bytes > 0) {
    char *ws = static_cast<char *>(workspace);
    P.rowstat = reinterpret_cast<float2 *>(ws + L.rowstat);
    P.part = reinterpret_cast<float2 *>(ws + L.part);
  }
  const size_t esize = dtype == VT_F32 ? 4 : 2;
  const int64_t vec_elems = 16 / static_cast<int64_t>(esize);
  const bool vec = aligned16(logits) && ld % vec_elems == 0;
  const hipError_t e = dtype == VT_F32 ? sm_launch_dtype<float>(P, vec, stream) : sm_launch_dtype<uint16_t>(P, vec, stream);
  return hip_status(e);
}

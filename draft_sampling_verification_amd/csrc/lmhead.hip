// C entry point of the trimmed LM head; the kernels live in lmhead_impl.hpp.
#include "lmhead_impl.hpp"

extern "C" vt_status_t vt_lmhead_trimmed(const uint16_t *hidden, const uint16_t *weight, const int32_t *keep_ids,
                                         int64_t M, int64_t H, int64_t Vt, int64_t V_rows, float *logits,
                                         hipStream_t stream) {
  using namespace vt;
  if (!hidden || !weight || !logits) return VT_ERR_INVALID_ARG;
  if (M <= 0 || H <= 0 || Vt <= 0 || V_rows <= 0) return VT_ERR_INVALID_ARG;
  if (!keep_ids && Vt > V_rows) return VT_ERR_INVALID_ARG;
  if (M > INT32_MAX || H > INT32_MAX || Vt > INT32_MAX || V_rows > INT32_MAX) return VT_ERR_UNSUPPORTED;
  if (H % 8 != 0 || !aligned16(hidden) || !aligned16(weight)) return VT_ERR_UNSUPPORTED;

  const GemvFn gemv = pick_gemv<kPartsNone>(M, H, keep_ids != nullptr);
  const int vrows = static_cast<int>(V_rows);
  if (gemv) return hip_status(launch_gemv(gemv, hidden, weight, keep_ids, vrows, H, Vt, logits, GemvParts{}, stream));
  const int64_t tiles = ((M + kBM - 1) / kBM) * ((Vt + kBN - 1) / kBN);
  if (tiles > INT32_MAX) return VT_ERR_UNSUPPORTED;
  return hip_status(launch_mfma(hidden, weight, keep_ids, vrows, M, H, Vt, logits, stream));
}

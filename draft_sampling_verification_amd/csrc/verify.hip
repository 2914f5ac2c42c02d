// C entry points of the verifier; the kernels live in verify_impl.hpp.
#include "verify_impl.hpp"

extern "C" size_t vt_spec_verify_workspace_bytes(int64_t B, int64_t gamma, int64_t V) {
  if (B <= 0 || gamma <= 0 || V <= 0) return 0;
  return vt::vf_ws_layout(B, gamma, (V + vt::kChunk - 1) / vt::kChunk).bytes;
}

extern "C" vt_status_t vt_spec_verify(int64_t B, int64_t gamma, int64_t V, int64_t Vt, const void *target_logits,
                                      vt_dtype_t target_dtype, const double *target_lse, float target_T,
                                      const float *draft_logits, int64_t R, const double *draft_lse, float draft_T,
                                      const int32_t *draft_ids, const int32_t *keep_ids, const int32_t *full_to_trim,
                                      const float *u_accept, const float *u_final, int32_t *out_tokens,
                                      int32_t *out_num_accepted, void *workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  using namespace vt;
  const bool greedy = target_T == 0.f;
  if (!target_logits || !draft_ids || !out_tokens || !out_num_accepted) return VT_ERR_INVALID_ARG;
  if (!greedy && (!target_lse || !draft_logits || !draft_lse || !u_accept || !u_final)) return VT_ERR_INVALID_ARG;
  if (target_dtype != VT_F32 && target_dtype != VT_BF16) return VT_ERR_INVALID_ARG;
  if (B <= 0 || gamma <= 0 || V <= 0 || Vt <= 0 || Vt > V || R < gamma) return VT_ERR_INVALID_ARG;
  if (!greedy && (!finite_positive(target_T) || !finite_positive(draft_T))) return VT_ERR_INVALID_ARG;
  if ((keep_ids == nullptr) != (full_to_trim == nullptr)) return VT_ERR_INVALID_ARG;
  if (!keep_ids && Vt != V) return VT_ERR_INVALID_ARG;
  if (gamma > kWave) return VT_ERR_UNSUPPORTED;
  if (V > INT32_MAX) return VT_ERR_UNSUPPORTED;
  const int64_t nchunk = (V + kChunk - 1) / kChunk;
  if (B > static_cast<int64_t>(UINT32_MAX) / nchunk) return VT_ERR_UNSUPPORTED;
  const VFWsLayout L = vf_ws_layout(B, gamma, nchunk);
  if (L.bytes > 0 && (!workspace || workspace_bytes < L.bytes)) return VT_ERR_WORKSPACE;

  VfParams P{};
  P.target = target_logits;
  P.tlse = target_lse;
  P.draft = draft_logits;
  P.dlse = draft_lse;
  P.ids = draft_ids;
  P.keep = keep_ids;
  P.f2t = full_to_trim;
  P.uacc = u_accept;
  P.ufin = u_final;
  P.out_tokens = out_tokens;
  P.out_n = out_num_accepted;
  P.V = V;
  P.Vt = Vt;
  P.R = R;
  P.greedy = greedy;
  P.Tt = greedy ? 1.0 : target_T;
  P.Td = greedy ? 1.0 : draft_T;
  P.invTt = 1.0 / P.Tt;
  P.invTd = 1.0 / P.Td;
  P.k2t = greedy ? 0.f : static_cast<float>(kLog2e / static_cast<double>(target_T));
  P.k2d = greedy ? 0.f : static_cast<float>(kLog2e / static_cast<double>(draft_T));
  P.gamma = static_cast<int>(gamma);
  P.nchunk = static_cast<int>(nchunk);
  if (L.bytes > 0) {
    char *ws = static_cast<char *>(workspace);
    P.nbuf = reinterpret_cast<int *>(ws + L.nbuf);
    P.part = reinterpret_cast<float2 *>(ws + L.part);
  }
  const int64_t vec_elems = target_dtype == VT_F32 ? 4 : 8;
  const bool vec = aligned16(target_logits) && V % vec_elems == 0;
  const hipError_t e = target_dtype == VT_F32 ? launch_verify<float>(P, vec, B, stream)
                                              : launch_verify<uint16_t>(P, vec, B, stream);
  return hip_status(e);
}

extern "C" const char *vt_status_string(vt_status_t s) {
  switch (s) {
    case VT_OK: return "ok";
    case VT_ERR_INVALID_ARG: return "invalid argument";
    case VT_ERR_UNSUPPORTED: return "unsupported argument combination";
    case VT_ERR_WORKSPACE: return "workspace missing or too small";
    case VT_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

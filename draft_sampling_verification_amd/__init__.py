"""Python binding of libvt.so, the MI355X (gfx950) draft-sampling / verification library.

Argument marshalling only: every function here checks tensor dtypes/shapes, passes device
pointers and the current HIP stream to the C ABI declared in include/vt.h, and raises VtError
on a non-OK status.  All arithmetic runs in the library's kernels.  There is no CPU fallback:
importing works anywhere, but calling a function without the built library (or without a GPU)
raises.

Entry points (same names as the C ABI):
  vt_lmhead_trimmed(hidden, weight, keep_ids, logits)
  vt_softmax_temp(logits, temperature, lse, probs=None, u=None, sampled=None, workspace=None, n=None)
  vt_spec_verify(target_logits, target_lse, target_T, draft_logits, draft_lse, draft_T, draft_ids,
                 keep_ids, full_to_trim, u_accept, u_final, out_tokens, out_num_accepted, workspace=None)
  vt_spec_block(hidden, weight, keep_ids, full_to_trim, target_logits, target_T, draft_T, u_draft, u_accept,
                u_final, draft_logits, draft_lse, draft_ids, target_lse, out_tokens, out_num_accepted,
                workspace=None, lmhead_events=None)
  vt_spec_block_noalloc(... the same without workspace ...): the library's fixed device scratch instead
Keep-set construction (include/vt_keepset.h):
  vt_token_histogram(tokens, V, counts, accumulate=False, workspace=None)
  vt_keep_select(counts, rule, keep_ids, full_to_trim, num_kept, k=0, p=0.0, min_count=0)
  vt_trim_head(weight, keep_ids, trimmed)
Generation loop for table models (include/vt_generate.h):
  vt_spec_generate_markov(target_table, draft_table, target_T, draft_T, gamma, u, out_tokens, out_stats=None)
Helpers: softmax_workspace(rows, n), verify_workspace(B, gamma, V), block_workspace(...), lib() (the raw ctypes handle).
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libvt.so")

VT_OK, VT_ERR_INVALID_ARG, VT_ERR_UNSUPPORTED, VT_ERR_WORKSPACE, VT_ERR_HIP = range(5)
VT_F32, VT_BF16 = 0, 1

_lib = None


class VtError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib().vt_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{fn} failed: {msg} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded libvt.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m draft_sampling_verification_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, F, I, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
        L.vt_lmhead_trimmed.argtypes = [P, P, P, I64, I64, I64, I64, P, P]
        L.vt_lmhead_trimmed.restype = I
        L.vt_softmax_temp.argtypes = [P, I, I64, I64, I64, F, P, P, P, P, P, SZ, P]
        L.vt_softmax_temp.restype = I
        L.vt_softmax_temp_workspace_bytes.argtypes = [I64, I64]
        L.vt_softmax_temp_workspace_bytes.restype = SZ
        L.vt_spec_verify.argtypes = [I64, I64, I64, I64, P, I, P, F, P, I64, P, F, P, P, P, P, P, P, P, P, SZ, P]
        L.vt_spec_verify.restype = I
        L.vt_spec_verify_workspace_bytes.argtypes = [I64, I64, I64]
        L.vt_spec_verify_workspace_bytes.restype = SZ
        L.vt_spec_block.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, I64, P, I, F, F, P, P, P, P, P, P, P, P,
                                    P, P, P, P, SZ, P]
        L.vt_spec_block.restype = I
        L.vt_spec_block_noalloc.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, I64, P, I, F, F, P, P, P, P, P,
                                            P, P, P, P, P, P, P]
        L.vt_spec_block_noalloc.restype = I
        L.vt_spec_block_workspace_bytes.argtypes = [I64, I64, I64, I64, I64, I64]
        L.vt_spec_block_workspace_bytes.restype = SZ
        L.vt_token_histogram.argtypes = [P, I64, I64, I, P, P, SZ, P]
        L.vt_token_histogram.restype = I
        L.vt_token_histogram_workspace_bytes.argtypes = [I64, I64]
        L.vt_token_histogram_workspace_bytes.restype = SZ
        L.vt_keep_select.argtypes = [P, I64, I, I64, ctypes.c_double, ctypes.c_uint32, P, P, P, P]
        L.vt_keep_select.restype = I
        L.vt_trim_head.argtypes = [P, I64, I64, P, I64, P, P]
        L.vt_trim_head.restype = I
        L.vt_trim_head_tiled.argtypes = [P, I64, I64, P, I64, P, P]
        L.vt_trim_head_tiled.restype = I
        L.vt_trim_head_tiled_bytes.argtypes = [I64, I64]
        L.vt_trim_head_tiled_bytes.restype = SZ
        L.vt_spec_generate_markov.argtypes = [P, P, I64, F, F, I64, I64, I64, P, P, P, P]
        L.vt_spec_generate_markov.restype = I
        L.vt_status_string.argtypes = [I]
        L.vt_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


EXPORTED = ("vt_lmhead_trimmed", "vt_softmax_temp", "vt_softmax_temp_workspace_bytes", "vt_spec_verify",
            "vt_spec_verify_workspace_bytes", "vt_spec_block", "vt_spec_block_workspace_bytes",
            "vt_spec_block_noalloc", "vt_status_string",
            "vt_token_histogram", "vt_token_histogram_workspace_bytes", "vt_keep_select", "vt_trim_head",
            "vt_trim_head_tiled", "vt_trim_head_tiled_bytes", "vt_spec_generate_markov")

VT_SELECT_TOP_K, VT_SELECT_TOP_P, VT_SELECT_MIN_FREQ = range(3)


def _torch():
    import torch
    return torch


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t, what, dtype=None, numel=None):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{what}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{what}: dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{what}: {t.numel()} elements, need {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _check(fn, status):
    if status != VT_OK:
        raise VtError(fn, status)


def _bits16(t, what):
    """bf16 tensors are passed as their bit patterns (uint16 storage)."""
    torch = _torch()
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{what}: expected bfloat16 (or its 16-bit patterns), got {t.dtype}")
    return t


def softmax_workspace(rows: int, n: int, device="cuda"):
    """A workspace for vt_softmax_temp (None when the shape needs none)."""
    nbytes = lib().vt_softmax_temp_workspace_bytes(rows, n)
    return _torch().empty(nbytes, dtype=_torch().uint8, device=device) if nbytes else None


def verify_workspace(B: int, gamma: int, V: int, device="cuda"):
    """A workspace for vt_spec_verify (None when the shape needs none)."""
    nbytes = lib().vt_spec_verify_workspace_bytes(B, gamma, V)
    return _torch().empty(nbytes, dtype=_torch().uint8, device=device) if nbytes else None


def vt_lmhead_trimmed(hidden, weight, keep_ids, logits):
    """logits[M, Vt] = hidden[M, H] @ weight[keep_ids].T (bf16 in, fp32 out); keep_ids may be None."""
    torch = _torch()
    _bits16(hidden, "hidden")
    _bits16(weight, "weight")
    M, H = hidden.shape
    V_rows = weight.shape[0]
    Vt = keep_ids.numel() if keep_ids is not None else logits.shape[1]
    if weight.shape[1] != H or tuple(logits.shape) != (M, Vt):
        raise ValueError("vt_lmhead_trimmed: shape mismatch")
    st = lib().vt_lmhead_trimmed(_ptr(hidden, "hidden"), _ptr(weight, "weight"),
                                 _ptr(keep_ids, "keep_ids", torch.int32), M, H, Vt, V_rows,
                                 _ptr(logits, "logits", torch.float32), _stream())
    _check("vt_lmhead_trimmed", st)
    return logits


def vt_softmax_temp(logits, temperature, lse, probs=None, u=None, sampled=None, workspace=None, n=None):
    """Row-wise temperature softmax of logits[rows, ld] (first n columns; default all).

    lse: float64 [rows]; probs: optional float32 [rows, n]; u / sampled: optional float32 / int32
    [rows] (draw).  logits may be float32 or bfloat16.  workspace: from softmax_workspace().
    """
    torch = _torch()
    rows, ld = logits.shape
    n = ld if n is None else n
    if logits.dtype == torch.float32:
        dt = VT_F32
    else:
        _bits16(logits, "logits")
        dt = VT_BF16
    if workspace is None:
        workspace = softmax_workspace(rows, n, logits.device)
    wsb = workspace.numel() if workspace is not None else 0
    st = lib().vt_softmax_temp(_ptr(logits, "logits"), dt, rows, n, ld, float(temperature),
                               _ptr(lse, "lse", torch.float64, rows), _ptr(probs, "probs", torch.float32, rows * n),
                               _ptr(u, "u", torch.float32, rows), _ptr(sampled, "sampled", torch.int32, rows),
                               _ptr(workspace, "workspace"), wsb, _stream())
    _check("vt_softmax_temp", st)
    return lse


def vt_spec_verify(target_logits, target_lse, target_T, draft_logits, draft_lse, draft_T, draft_ids, keep_ids,
                   full_to_trim, u_accept, u_final, out_tokens, out_num_accepted, workspace=None):
    """Modified rejection sampling; shapes: target [B, gamma+1, V], draft [B, R, Vt], ids [B, R].
    target_T = 0: greedy verification (target_lse, draft_logits, draft_lse, u_accept, u_final may be None)."""
    torch = _torch()
    B, g1, V = target_logits.shape
    gamma = g1 - 1
    if draft_logits is not None:
        Bd, R, Vt = draft_logits.shape
    else:  # greedy verification (target_T = 0) reads no draft logits
        Bd, R = draft_ids.shape
        Vt = keep_ids.numel() if keep_ids is not None else V
    if Bd != B or tuple(draft_ids.shape) != (B, R) or tuple(out_tokens.shape) != (B, g1):
        raise ValueError("vt_spec_verify: shape mismatch")
    if target_logits.dtype == torch.float32:
        dt = VT_F32
    else:
        _bits16(target_logits, "target_logits")
        dt = VT_BF16
    if workspace is None:
        workspace = verify_workspace(B, gamma, V, target_logits.device)
    wsb = workspace.numel() if workspace is not None else 0
    st = lib().vt_spec_verify(B, gamma, V, Vt, _ptr(target_logits, "target_logits"), dt,
                              _ptr(target_lse, "target_lse", torch.float64, B * g1), float(target_T),
                              _ptr(draft_logits, "draft_logits", torch.float32), R,
                              _ptr(draft_lse, "draft_lse", torch.float64, B * R), float(draft_T or 0.0),
                              _ptr(draft_ids, "draft_ids", torch.int32), _ptr(keep_ids, "keep_ids", torch.int32),
                              _ptr(full_to_trim, "full_to_trim", torch.int32, V),
                              _ptr(u_accept, "u_accept", torch.float32, B * gamma),
                              _ptr(u_final, "u_final", torch.float32, B),
                              _ptr(out_tokens, "out_tokens", torch.int32),
                              _ptr(out_num_accepted, "out_num_accepted", torch.int32, B),
                              _ptr(workspace, "workspace"), wsb, _stream())
    _check("vt_spec_verify", st)
    return out_tokens, out_num_accepted


def block_workspace(B: int, gamma: int, R: int, H: int, Vt: int, V: int, device="cuda"):
    """A workspace for vt_spec_block (None when the shape needs none)."""
    nbytes = lib().vt_spec_block_workspace_bytes(B, gamma, R, H, Vt, V)
    return _torch().empty(nbytes, dtype=_torch().uint8, device=device) if nbytes else None


def _weight_tiled(weight_tiled, Vt, H, fn):
    if weight_tiled is None:
        return None
    _bits16(weight_tiled, "weight_tiled")
    need = lib().vt_trim_head_tiled_bytes(Vt, H) // 2
    if need == 0 or weight_tiled.numel() != need:
        raise ValueError(f"{fn}: weight_tiled must hold the K-tiled W^Trim of {Vt} rows ({need} values)")
    return _ptr(weight_tiled, "weight_tiled")


def vt_spec_block(hidden, weight, keep_ids, full_to_trim, target_logits, target_T, draft_T, u_draft, u_accept,
                  u_final, draft_logits, draft_lse, draft_ids, target_lse, out_tokens, out_num_accepted,
                  workspace=None, lmhead_events=None, weight_tiled=None):
    """One whole block.  hidden [B*R, H] bf16, weight [V, H] bf16, target [B, gamma+1, V];
    outputs draft_logits [B*R, Vt] f32, draft_lse [B*R] f64, draft_ids [B*R] i32, target_lse
    [B*(gamma+1)] f64, out_tokens [B, gamma+1] i32, out_num_accepted [B] i32.
    lmhead_events: optional (start, end) torch.cuda.Event pair recorded around the LM-head kernel.
    weight_tiled: optional K-tiled W^Trim from vt_trim_head_tiled(weight, keep_ids), read by the
    MFMA head instead of gathering rows of weight (same logits).
    target_T = 0: greedy verification (target_lse, u_accept, u_final may be None); draft_T = 0 (with
    target_T = 0): argmax drafts (u_draft may be None)."""
    torch = _torch()
    _bits16(hidden, "hidden")
    _bits16(weight, "weight")
    B, g1, V = target_logits.shape
    gamma = g1 - 1
    M, H = hidden.shape
    R = M // B
    Vt = draft_logits.shape[1]
    if M != B * R or weight.shape != (V, H) or tuple(draft_logits.shape) != (M, Vt) or \
            tuple(out_tokens.shape) != (B, g1):
        raise ValueError("vt_spec_block: shape mismatch")
    if target_logits.dtype == torch.float32:
        dt = VT_F32
    else:
        _bits16(target_logits, "target_logits")
        dt = VT_BF16
    if workspace is None:
        workspace = block_workspace(B, gamma, R, H, Vt, V, target_logits.device)
    wsb = workspace.numel() if workspace is not None else 0
    ev0 = ev1 = None
    if lmhead_events is not None:
        ev0, ev1 = (ctypes.c_void_p(e.cuda_event) for e in lmhead_events)
    wt = _weight_tiled(weight_tiled, Vt, H, "vt_spec_block")
    st = lib().vt_spec_block(_ptr(hidden, "hidden"), _ptr(weight, "weight"), wt,
                             _ptr(keep_ids, "keep_ids", torch.int32),
                             _ptr(full_to_trim, "full_to_trim", torch.int32, V), B, gamma, R, H, Vt, V,
                             _ptr(target_logits, "target_logits"), dt, float(target_T), float(draft_T),
                             _ptr(u_draft, "u_draft", torch.float32, M), _ptr(u_accept, "u_accept", torch.float32, B * gamma),
                             _ptr(u_final, "u_final", torch.float32, B), _ptr(draft_logits, "draft_logits", torch.float32),
                             _ptr(draft_lse, "draft_lse", torch.float64, M), _ptr(draft_ids, "draft_ids", torch.int32, M),
                             _ptr(target_lse, "target_lse", torch.float64, B * g1),
                             _ptr(out_tokens, "out_tokens", torch.int32), _ptr(out_num_accepted, "out_num_accepted",
                                                                                torch.int32, B),
                             ev0, ev1, _ptr(workspace, "workspace"), wsb, _stream())
    _check("vt_spec_block", st)
    return out_tokens, out_num_accepted


def vt_spec_block_noalloc(hidden, weight, keep_ids, full_to_trim, target_logits, target_T, draft_T, u_draft,
                          u_accept, u_final, draft_logits, draft_lse, draft_ids, target_lse, out_tokens,
                          out_num_accepted, lmhead_events=None, weight_tiled=None):
    """vt_spec_block with the library's fixed per-device scratch instead of a workspace (nothing is
    allocated; shapes needing more than 64 MiB of workspace are rejected).  Calls that overlap on
    one device race on that scratch."""
    torch = _torch()
    _bits16(hidden, "hidden")
    _bits16(weight, "weight")
    B, g1, V = target_logits.shape
    gamma = g1 - 1
    M, H = hidden.shape
    R = M // B
    Vt = draft_logits.shape[1]
    if M != B * R or weight.shape != (V, H) or tuple(draft_logits.shape) != (M, Vt) or \
            tuple(out_tokens.shape) != (B, g1):
        raise ValueError("vt_spec_block_noalloc: shape mismatch")
    if target_logits.dtype == torch.float32:
        dt = VT_F32
    else:
        _bits16(target_logits, "target_logits")
        dt = VT_BF16
    ev0 = ev1 = None
    if lmhead_events is not None:
        ev0, ev1 = (ctypes.c_void_p(e.cuda_event) for e in lmhead_events)
    wt = _weight_tiled(weight_tiled, Vt, H, "vt_spec_block_noalloc")
    st = lib().vt_spec_block_noalloc(
        _ptr(hidden, "hidden"), _ptr(weight, "weight"), wt, _ptr(keep_ids, "keep_ids", torch.int32),
        _ptr(full_to_trim, "full_to_trim", torch.int32, V), B, gamma, R, H, Vt, V, _ptr(target_logits, "target_logits"),
        dt, float(target_T), float(draft_T), _ptr(u_draft, "u_draft", torch.float32, M),
        _ptr(u_accept, "u_accept", torch.float32, B * gamma), _ptr(u_final, "u_final", torch.float32, B),
        _ptr(draft_logits, "draft_logits", torch.float32), _ptr(draft_lse, "draft_lse", torch.float64, M),
        _ptr(draft_ids, "draft_ids", torch.int32, M), _ptr(target_lse, "target_lse", torch.float64, B * g1),
        _ptr(out_tokens, "out_tokens", torch.int32), _ptr(out_num_accepted, "out_num_accepted", torch.int32, B),
        ev0, ev1, _stream())
    _check("vt_spec_block_noalloc", st)
    return out_tokens, out_num_accepted


# ---------------------------------------------------------------- keep-set construction

def histogram_workspace(n: int, V: int, device="cuda"):
    """A workspace for vt_token_histogram (None when the shape needs none)."""
    nbytes = lib().vt_token_histogram_workspace_bytes(n, V)
    return _torch().empty(nbytes, dtype=_torch().uint8, device=device) if nbytes else None


def vt_token_histogram(tokens, V: int, counts, accumulate: bool = False, workspace=None):
    """counts[V] (uint32 storage: int32 or uint32 tensor) = (counts +) occurrences of each id in tokens."""
    torch = _torch()
    n = tokens.numel()
    if workspace is None:
        workspace = histogram_workspace(n, V, tokens.device)
    if counts.numel() != V or counts.dtype not in (torch.int32, torch.uint32):
        raise ValueError("vt_token_histogram: counts must hold V 32-bit entries")
    ws = _ptr(workspace, "workspace") if workspace is not None else None
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().vt_token_histogram(_ptr(tokens, "tokens", torch.int32) if n else None, n, V, 1 if accumulate else 0,
                                  _ptr(counts, "counts"), ws, wsb, _stream())
    _check("vt_token_histogram", st)
    return counts


def vt_keep_select(counts, rule: int, keep_ids, full_to_trim, num_kept, k: int = 0, p: float = 0.0,
                   min_count: int = 0):
    """Kept ids (ascending) into keep_ids[:K], the inverse map into full_to_trim, K into num_kept[0]."""
    torch = _torch()
    V = counts.numel()
    if counts.dtype not in (torch.int32, torch.uint32):
        raise TypeError("vt_keep_select: counts must be 32-bit")
    st = lib().vt_keep_select(_ptr(counts, "counts"), V, rule, k, p, min_count,
                              _ptr(keep_ids, "keep_ids", torch.int32, V),
                              _ptr(full_to_trim, "full_to_trim", torch.int32, V),
                              _ptr(num_kept, "num_kept", torch.int32, 1), _stream())
    _check("vt_keep_select", st)
    return num_kept


def vt_trim_head(weight, keep_ids, trimmed):
    """trimmed[k, H] = weight[keep_ids] (bf16 rows)."""
    torch = _torch()
    _bits16(weight, "weight")
    _bits16(trimmed, "trimmed")
    V_rows, H = weight.shape
    k = keep_ids.numel()
    if tuple(trimmed.shape) != (k, H):
        raise ValueError("vt_trim_head: shape mismatch")
    st = lib().vt_trim_head(_ptr(weight, "weight"), V_rows, H, _ptr(keep_ids, "keep_ids", torch.int32), k,
                            _ptr(trimmed, "trimmed"), _stream())
    _check("vt_trim_head", st)
    return trimmed


def vt_trim_head_tiled(weight, keep_ids, k=None, tiled=None):
    """W^Trim = weight[keep_ids] (or rows 0..k-1 when keep_ids is None) in the K-tiled layout
    [ceil(k/256)][H/32][256][32] of vt_trim_head_tiled, as a flat bf16-bits tensor (allocated when
    tiled is None)."""
    torch = _torch()
    _bits16(weight, "weight")
    V_rows, H = weight.shape
    if keep_ids is not None:
        k = keep_ids.numel()
    elif k is None:
        raise ValueError("vt_trim_head_tiled: give keep_ids or the row count k")
    nbytes = lib().vt_trim_head_tiled_bytes(k, H)
    if nbytes == 0:
        raise ValueError(f"vt_trim_head_tiled: no K-tiled layout for k={k}, H={H} (needs k > 0 and H % 32 == 0)")
    if tiled is None:
        tiled = torch.empty(nbytes // 2, dtype=weight.dtype, device=weight.device)
    _bits16(tiled, "tiled")
    if tiled.numel() * 2 != nbytes:
        raise ValueError("vt_trim_head_tiled: tiled must hold vt_trim_head_tiled_bytes(k, H) bytes")
    st = lib().vt_trim_head_tiled(_ptr(weight, "weight"), V_rows, H, _ptr(keep_ids, "keep_ids", torch.int32), k,
                                  _ptr(tiled, "tiled"), _stream())
    _check("vt_trim_head_tiled", st)
    return tiled


# ---------------------------------------------------------------- generation loop

def vt_spec_generate_markov(target_table, draft_table, target_T: float, draft_T: float, gamma: int, u, out_tokens,
                            out_stats=None):
    """Chained speculative blocks for B sequences of order-1 table models (tables fp32 [V+1, V],
    u fp32 [B, n_tokens, 2*gamma+1]) -> out_tokens int32 [B, n_tokens], out_stats int32 [B, 4]."""
    torch = _torch()
    rows, V = target_table.shape
    B, L = out_tokens.shape
    if rows != V + 1 or tuple(draft_table.shape) != (V + 1, V):
        raise ValueError("vt_spec_generate_markov: tables must be [V+1, V]")
    if tuple(u.shape) != (B, L, 2 * gamma + 1):
        raise ValueError("vt_spec_generate_markov: u must be [B, n_tokens, 2*gamma+1]")
    if out_stats is not None and tuple(out_stats.shape) != (B, 4):
        raise ValueError("vt_spec_generate_markov: out_stats must be [B, 4]")
    st = lib().vt_spec_generate_markov(_ptr(target_table, "target_table", torch.float32),
                                       _ptr(draft_table, "draft_table", torch.float32), V, target_T, draft_T, gamma,
                                       B, L, _ptr(u, "u", torch.float32), _ptr(out_tokens, "out_tokens", torch.int32),
                                       _ptr(out_stats, "out_stats", torch.int32), _stream())
    _check("vt_spec_generate_markov", st)
    return out_tokens

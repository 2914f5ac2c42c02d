"""Helpers for the GPU parity tests: run one block of the path through the C ABI on the GPU, run
the oracle on the same seeded inputs, and compare them.

Comparison rules:
  * integer outputs (draft ids, accept counts, tokens) are compared exactly; they may differ only
    at a decision the oracle itself places within BAND of the uniform that decides it
    (|u - ratio| for an accept test, |u - C[i]/Z| at the CDF boundaries around a draw), where fp32
    rounding settles it; such a mismatch is counted and the rest of that sequence is skipped;
  * log-normalisers and probabilities are compared with explicit tolerances.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import draft_sampling_verification_amd as vt
from oracle import ref
from workloads import Workload, make_workload

BAND = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.array(bits, copy=True, order="C").view(np.int16)).view(torch.bfloat16).cuda()


def dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.array(x, copy=True, order="C")).cuda()


def target_tensor(wl: Workload) -> torch.Tensor:
    return dev(wl.target) if wl.cfg.target_dtype == "f32" else dev_bf16(wl.target)


def gpu_block(wl: Workload, probs: bool = False, device_inputs=None) -> dict:
    """One block (LM head -> draft softmax + draw -> target softmax -> verify) through the ABI."""
    cfg = wl.cfg
    B, R, g = wl.B, cfg.R, cfg.gamma
    d = device_inputs or {}
    keep = d.get("keep") if "keep" in d else (dev(wl.keep_ids) if wl.keep_ids is not None else None)
    f2t = d.get("f2t") if "f2t" in d else (dev(wl.full_to_trim) if wl.full_to_trim is not None else None)
    if wl.draft_logits is None:
        weight = d.get("weight")
        if weight is None:
            weight = dev_bf16(wl.weight)
        hidden = dev_bf16(wl.hidden)
        logits = torch.empty(B * R, cfg.Vt, dtype=torch.float32, device="cuda")
        vt.vt_lmhead_trimmed(hidden, weight, keep, logits)
    else:
        logits = dev(wl.draft_logits)
    dlse = torch.empty(B * R, dtype=torch.float64, device="cuda")
    dids = torch.empty(B * R, dtype=torch.int32, device="cuda")
    dprobs = torch.empty(B * R, cfg.Vt, dtype=torch.float32, device="cuda") if probs else None
    vt.vt_softmax_temp(logits, wl.T, dlse, dprobs, dev(wl.u_draft.reshape(-1)), dids)
    target = target_tensor(wl)
    tlse = torch.empty(B * (g + 1), dtype=torch.float64, device="cuda")
    tprobs = torch.empty(B * (g + 1), cfg.V, dtype=torch.float32, device="cuda") if probs else None
    vt.vt_softmax_temp(target.view(B * (g + 1), cfg.V), wl.T, tlse, tprobs)
    tokens = torch.empty(B, g + 1, dtype=torch.int32, device="cuda")
    nacc = torch.empty(B, dtype=torch.int32, device="cuda")
    vt.vt_spec_verify(target, tlse, wl.T, logits.view(B, R, cfg.Vt), dlse, wl.T, dids.view(B, R), keep, f2t,
                      dev(wl.u_acc), dev(wl.u_fin), tokens, nacc)
    torch.cuda.synchronize()
    out = dict(draft_logits=logits.cpu().numpy(), draft_lse=dlse.cpu().numpy(),
               draft_ids=dids.cpu().numpy().reshape(B, R), target_lse=tlse.cpu().numpy().reshape(B, g + 1),
               tokens=tokens.cpu().numpy(), n=nacc.cpu().numpy())
    if probs:
        out["draft_probs"] = dprobs.cpu().numpy()
        out["target_probs"] = tprobs.cpu().numpy()
    return out


def gpu_block_fused(wl: Workload, events=None, tiled: bool = False) -> dict:
    """The same block through the single fused call vt_spec_block (tiled: with the K-tiled W^Trim
    of vt_trim_head_tiled, which the MFMA heads read instead of gathering rows)."""
    cfg = wl.cfg
    B, R, g = wl.B, cfg.R, cfg.gamma
    keep = dev(wl.keep_ids) if wl.keep_ids is not None else None
    f2t = dev(wl.full_to_trim) if wl.full_to_trim is not None else None
    weight = dev_bf16(wl.weight)
    wt = vt.vt_trim_head_tiled(weight, keep, k=cfg.Vt) if tiled else None
    logits = torch.empty(B * R, cfg.Vt, dtype=torch.float32, device="cuda")
    dlse = torch.empty(B * R, dtype=torch.float64, device="cuda")
    dids = torch.empty(B * R, dtype=torch.int32, device="cuda")
    tlse = torch.empty(B * (g + 1), dtype=torch.float64, device="cuda")
    tokens = torch.empty(B, g + 1, dtype=torch.int32, device="cuda")
    nacc = torch.empty(B, dtype=torch.int32, device="cuda")
    vt.vt_spec_block(dev_bf16(wl.hidden), weight, keep, f2t, target_tensor(wl), wl.T, wl.T,
                     dev(wl.u_draft.reshape(-1)), dev(wl.u_acc), dev(wl.u_fin), logits, dlse, dids, tlse, tokens, nacc,
                     lmhead_events=events, weight_tiled=wt)
    torch.cuda.synchronize()
    return dict(draft_logits=logits.cpu().numpy(), draft_lse=dlse.cpu().numpy(),
                draft_ids=dids.cpu().numpy().reshape(B, R), target_lse=tlse.cpu().numpy().reshape(B, g + 1),
                tokens=tokens.cpu().numpy(), n=nacc.cpu().numpy())


def oracle_block(wl: Workload) -> dict:
    cfg = wl.cfg
    return ref.block(wl.hidden, wl.weight, wl.keep_ids, wl.draft_logits, wl.target, cfg.target_dtype, wl.T,
                     wl.u_draft, wl.u_acc, wl.u_fin, cfg.gamma, cfg.R)


def compare_tokens(gpu: dict, orc: dict, wl: Workload) -> dict:
    """Exact comparison of draft ids, n and tokens.

    A GPU result may differ from the oracle's only at a decision the oracle itself places within
    BAND of its uniform; such a mismatch is counted as excused and the rest of that sequence (which
    depends on it) is not compared.  Agreement inside the band is simply agreement.
    """
    cfg = wl.cfg
    g, R = cfg.gamma, cfg.R
    st = dict(sequences=wl.B, full_match=0, excused_draft=0, excused_accept=0, excused_final=0)
    for b in range(wl.B):
        stop = False
        for i in range(R):
            if gpu["draft_ids"][b, i] != orc["draft_ids"][b, i]:
                assert orc["draft_margins"][b, i] < BAND, (
                    "draft draw differs outside the band", b, i, gpu["draft_ids"][b], orc["draft_ids"][b],
                    orc["draft_margins"][b, i])
                st["excused_draft"] += 1
                if i < g:
                    stop = True
                    break
        if stop:
            continue
        n_g, n_o = int(gpu["n"][b]), int(orc["n"][b])
        if n_g != n_o:
            k = min(n_g, n_o)  # the first test on which the two disagree
            r = orc["accept_ratios"][b][k]
            assert abs(float(wl.u_acc[b, k]) - r) < BAND, ("accept count differs outside the band", b, n_g, n_o,
                                                            float(wl.u_acc[b, k]), r)
            st["excused_accept"] += 1
            continue
        n = n_o
        assert np.array_equal(gpu["tokens"][b, :n], orc["tokens"][b, :n]), b
        assert np.all(gpu["tokens"][b, n + 1:] == -1), b
        if gpu["tokens"][b, n] != orc["tokens"][b, n]:
            assert orc["final_margin"][b] < BAND, ("final token differs outside the band", b, n, gpu["tokens"][b],
                                                   orc["tokens"][b], orc["final_margin"][b])
            st["excused_final"] += 1
            continue
        st["full_match"] += 1
    return st


def lmhead_error_bound(hidden_bits, weight_bits, keep_ids):
    """Recursive-summation bound H * 2^-24 * sum_k |h_k w_k| per logit (plus fp32 rounding of the result)."""
    h = np.abs(ref.bf16_to_f64(hidden_bits))
    rows = weight_bits if keep_ids is None else np.asarray(weight_bits)[np.asarray(keep_ids)]
    w = np.abs(ref.bf16_to_f64(rows))
    H = h.shape[1]
    return H * 2.0 ** -24 * (h @ w.T)


def sequences_workload(cfg, seqs, **kw) -> Workload:
    """One workload holding the listed sequences of a config (each sequence's inputs are those it
    has in the full batch: hidden rows, target rows and uniforms are seeded per sequence)."""
    parts = [make_workload(cfg, B=1, b0=int(s), **kw) for s in seqs]
    wl = parts[0]
    out = Workload(cfg=cfg, b0=-1, B=len(parts), T=wl.T, weight=wl.weight, keep_ids=wl.keep_ids,
                   full_to_trim=wl.full_to_trim)
    for k in ("hidden", "target", "draft_logits", "u_draft", "u_acc", "u_fin"):
        if getattr(wl, k) is not None:
            setattr(out, k, np.concatenate([getattr(p, k) for p in parts]))
    return out


def beta_z(gpu: dict, wl: Workload):
    """z-score of the number of sequences whose first draft was accepted against its expectation
    sum_b beta_b, beta_b = sum_x min(p_0(x), q_0(x)) ("A rejection rule keeps speculative
    decoding's output exact", "What draft accuracy buys": beta is the chance that a draft survives),
    with variance sum_b beta_b (1 - beta_b).  p_0 from the target row, q_0 from the GPU's own draft
    logits (q = 0 off the kept set)."""
    from oracle import stats

    cfg = wl.cfg
    B, R = wl.B, cfg.R
    t = ref.as_f64(wl.target, cfg.target_dtype)[:, 0, :]
    _, p0 = ref.softmax_temp(t, wl.T)
    d = gpu["draft_logits"].reshape(B, R, cfg.Vt)[:, 0, :].astype(np.float64)
    _, q0 = ref.softmax_temp(d, wl.T)
    beta = np.empty(B)
    for b in range(B):
        qf = np.zeros(cfg.V)
        if wl.keep_ids is None:
            qf[:] = q0[b]
        else:
            qf[wl.keep_ids] = q0[b]
        beta[b] = stats.beta(p0[b], qf)
    acc = float((np.asarray(gpu["n"]) >= 1).sum())
    var = float((beta * (1 - beta)).sum())
    return (acc - beta.sum()) / np.sqrt(max(var, 1e-12)), acc, float(beta.sum())

"""GPU parity of whole blocks (LM head -> draft softmax + draw -> target softmax -> verify) and of
vt_spec_verify's special cases against the oracle, at sizes the oracle finishes in seconds that
still span several chunks and ragged tails; plus the glossary page's worked example on a grid,
the toy workload's 1e5-trial Monte Carlo, determinism and batch-size independence."""
import math

import numpy as np
import pytest
import torch

import draft_sampling_verification_amd as vt
from oracle import ref
from tests.gpu_harness import (BAND, compare_tokens, dev, gpu_block, oracle_block, say, target_tensor)
from workloads import CONFIGS, counter_uniforms, make_workload

pytestmark = pytest.mark.gpu

SCALED = {
    "c2-full-head": CONFIGS[2].scaled(V=20000, Vt=20000, H=512),
    "c3-trimmed": CONFIGS[3].scaled(V=20000, Vt=5000, H=512),
    "c4-batched": CONFIGS[4].scaled(B=24, V=20000, Vt=5000, H=256),
    "c5-mfma": CONFIGS[5].scaled(B=16, V=13000, Vt=6000, H=256),
    "c4-ragged": CONFIGS[4].scaled(B=10, V=9001, Vt=4097, H=264, gamma=3),
}


def _check_block(wl, probs=True):
    gpu = gpu_block(wl, probs=probs)
    orc = oracle_block(wl)
    cfg = wl.cfg
    d_err = np.abs(gpu["draft_lse"] - orc["draft_lse_flat"]).max()
    t_err = np.abs(gpu["target_lse"] - orc["target_lse"]).max()
    say(f"  max |draft lse err| {d_err:.2e}  max |target lse err| {t_err:.2e}")
    assert t_err <= 2e-6
    assert d_err <= (2e-6 if wl.draft_logits is not None else 1e-4)
    if probs:
        _, tp = ref.softmax_temp(ref.as_f64(wl.target, cfg.target_dtype).reshape(-1, cfg.V), wl.T)
        assert np.all(np.abs(gpu["target_probs"] - tp) <= 1e-5 * tp + 1.2e-38)
        qp = orc["draft_probs"]
        tol = 1e-5 if wl.draft_logits is not None else 2e-2  # bf16-weight logits
        rel = np.abs(gpu["draft_probs"] - qp) / np.maximum(qp, 1.2e-38)
        say(f"  max draft prob rel err {rel.max():.2e} (tolerance {tol})")
        assert np.all(np.abs(gpu["draft_probs"] - qp) <= tol * qp + 1.2e-38)
    st = compare_tokens(gpu, orc, wl)
    say(f"  {st}; mean accepted {orc['n'].mean():.2f}")
    assert st["full_match"] >= 0.95 * wl.B
    return gpu, orc, st


@pytest.mark.parametrize("name", list(SCALED))
def test_block_parity_scaled(name):
    say(f"block parity {name}")
    _check_block(make_workload(SCALED[name]))


@pytest.mark.parametrize("name", ["c3-trimmed", "c4-batched", "c5-mfma", "c4-ragged"])
def test_block_parity_aligned_scaled(name):
    # draft = target at the kept ids: many deep accepts, bonus tokens, residuals off the kept set
    say(f"aligned block parity {name}")
    wl = make_workload(SCALED[name], aligned=True)
    gpu, orc, _ = _check_block(wl)
    kept = np.zeros(wl.cfg.V, bool)
    kept[wl.keep_ids] = True
    for b in range(wl.B):
        n = int(gpu["n"][b])
        if n < wl.cfg.gamma:
            assert not kept[gpu["tokens"][b, n]]  # every residual token lies off the kept set
    assert (gpu["n"] == wl.cfg.gamma).any() and (gpu["n"] > 0).mean() > 0.5


def _verify_only(target, T, draft, ids, u_acc, u_fin, keep=None, f2t=None):
    """Run softmax (lse) + vt_spec_verify on given float32 logits [B, g+1, V] / [B, R, Vt]."""
    B, g1, V = target.shape
    _, R, Vt = draft.shape
    tt, dd = dev(target), dev(draft)
    tl = torch.empty(B * g1, dtype=torch.float64, device="cuda")
    dl = torch.empty(B * R, dtype=torch.float64, device="cuda")
    vt.vt_softmax_temp(tt.view(B * g1, V), T, tl)
    vt.vt_softmax_temp(dd.view(B * R, Vt), T, dl)
    tok = torch.empty(B, g1, dtype=torch.int32, device="cuda")
    nacc = torch.empty(B, dtype=torch.int32, device="cuda")
    vt.vt_spec_verify(tt, tl, T, dd, dl, T, dev(ids.astype(np.int32)), keep, f2t, dev(u_acc), dev(u_fin), tok, nacc)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), nacc.cpu().numpy()


def test_block_parity_longest_draft():
    # gamma = 64 through the separate calls (draft = target at the kept ids: deep accepts,
    # full acceptance with the bonus draw from row 64)
    say("aligned block parity gamma=64")
    wl = make_workload(CONFIGS[4].scaled(B=4, gamma=64, R=65, V=6000, Vt=2500, H=256), aligned=True)
    _, orc, _ = _check_block(wl)
    assert (orc["n"] == 64).any()


def test_worked_example_grid_on_gpu():
    # glossary two-token example (A 0.6 / B 0.4 target, 0.8 / 0.2 draft), 40 x 40 grid of
    # (u_draft, u_accept) as 1600 sequences: 960 keep A, 320 keep B, 320 are rejected -> B
    G = 40
    mid = ((np.arange(G) + 0.5) / G).astype(np.float32)
    ud, ua = np.meshgrid(mid, mid, indexing="ij")
    B = G * G
    draft = np.log(np.array([0.8, 0.2]))[None, None, :].repeat(B, 0).astype(np.float32)
    target = np.log(np.array([0.6, 0.4]))[None, None, :].repeat(B, 0).repeat(2, 1).astype(np.float32)
    dd = dev(draft)
    dl = torch.empty(B, dtype=torch.float64, device="cuda")
    ids = torch.empty(B, dtype=torch.int32, device="cuda")
    vt.vt_softmax_temp(dd.view(B, 2), 1.0, dl, None, dev(ud.reshape(-1).copy()), ids)
    ids = ids.cpu().numpy().reshape(B, 1)
    for uf in (0.01, 0.5, 0.99):
        tok, n = _verify_only(target, 1.0, draft, ids, ua.reshape(B, 1).copy(), np.full(B, uf, np.float32))
        keep_a = ((n == 1) & (tok[:, 0] == 0)).sum()
        keep_b = ((n == 1) & (tok[:, 0] == 1)).sum()
        rej = n == 0
        assert (keep_a, keep_b, rej.sum()) == (960, 320, 320)
        assert np.all(tok[rej, 0] == 1)  # the residual always returns B
        assert (tok[:, 0] == 0).sum() * 5 == B * 3  # final A mass 0.6


@pytest.mark.parametrize("B,g,V", [(12, 5, 9000), (3, 64, 3000)])  # 64: the longest run taken
def test_identical_draft_accepts_everything(B, g, V):
    rng = np.random.default_rng(1)
    target = (1.5 * rng.standard_normal((B, g + 1, V))).astype(np.float32)
    draft = target.copy()  # q == p bitwise at every position (R = gamma + 1)
    u_d = counter_uniforms(7, 4, B, g + 1)
    dd = dev(draft)
    dl = torch.empty(B * (g + 1), dtype=torch.float64, device="cuda")
    ids = torch.empty(B * (g + 1), dtype=torch.int32, device="cuda")
    vt.vt_softmax_temp(dd.view(-1, V), 1.0, dl, None, dev(u_d.reshape(-1)), ids)
    ids = ids.cpu().numpy().reshape(B, g + 1)
    u_acc, u_fin = counter_uniforms(7, 5, B, g), counter_uniforms(7, 6, B, 1)[:, 0].copy()
    tok, n = _verify_only(target, 1.0, draft, ids, u_acc, u_fin)
    assert np.all(n == g)
    assert np.array_equal(tok[:, :g], ids[:, :g])
    _, p = ref.softmax_temp(target[:, g].astype(np.float64), 1.0)
    for b in range(B):
        idx, margin = ref.draw(p[b], float(u_fin[b]))
        assert tok[b, g] == idx or margin < BAND


def test_disjoint_supports_reject_first():
    B, g, V = 8, 3, 6000
    rng = np.random.default_rng(2)
    target = np.full((B, g + 1, V), -np.inf, np.float32)
    draft = np.full((B, g, V), -np.inf, np.float32)
    target[:, :, 1::2] = rng.standard_normal((B, g + 1, V // 2))  # p on odd ids
    draft[:, :, 0::2] = rng.standard_normal((B, g, V // 2))  # q on even ids
    ids = np.zeros((B, g), np.int32)
    ids[:, :] = 2 * rng.integers(0, V // 2, size=(B, g))
    u_fin = counter_uniforms(8, 6, B, 1)[:, 0].copy()
    tok, n = _verify_only(target, 1.0, draft, ids, np.full((B, g), 2.0 ** -24, np.float32), u_fin)
    assert np.all(n == 0) and np.all(tok[:, 1:] == -1)
    _, p0 = ref.softmax_temp(target[:, 0].astype(np.float64), 1.0)
    for b in range(B):
        idx, margin = ref.draw(p0[b], float(u_fin[b]))
        assert tok[b, 0] % 2 == 1
        assert tok[b, 0] == idx or margin < BAND


def test_one_hot_target_is_greedy():
    B, g, V = 6, 4, 5000
    rng = np.random.default_rng(3)
    argmax = rng.integers(0, V, size=(B, g + 1))
    target = np.full((B, g + 1, V), -np.inf, np.float32)
    for b in range(B):
        for i in range(g + 1):
            target[b, i, argmax[b, i]] = 0.0
    draft = rng.standard_normal((B, g, V)).astype(np.float32)
    ids = argmax[:, :g].copy()
    for b in range(B):  # sequence b drafts the argmax up to position b, then a wrong token
        if b < g:
            ids[b, b] = (argmax[b, b] + 1) % V
    tok, n = _verify_only(target, 1.0, draft, ids.astype(np.int32), np.ones((B, g), np.float32),
                          np.full(B, 0.5, np.float32))
    for b in range(B):
        want_n = b if b < g else g
        assert n[b] == want_n and tok[b, want_n] == argmax[b, want_n]


def test_invalid_draft_id_flags_sequence():
    B, g, V = 4, 3, 5000
    rng = np.random.default_rng(4)
    target = rng.standard_normal((B, g + 1, V)).astype(np.float32)
    draft = rng.standard_normal((B, g, V)).astype(np.float32)
    ids = rng.integers(0, V, size=(B, g)).astype(np.int32)
    ids[1, 2] = V  # out of range
    ids[3, 0] = -5
    tok, n = _verify_only(target, 1.0, draft, ids, np.full((B, g), 0.5, np.float32), np.full(B, 0.5, np.float32))
    assert n[1] == -1 and n[3] == -1 and np.all(tok[1] == -1) and np.all(tok[3] == -1)
    assert n[0] >= 0 and n[2] >= 0


def _toy_gpu(wl):
    """The order-1 toy on the GPU: the harness evaluates the table "models" (row lookups) and the
    path runs the draft draws, the target log-normalisers and the verification."""
    cfg = wl.cfg
    B, g = wl.B, cfg.gamma
    Q = dev(wl.toy.draft_logits)
    P = dev(wl.toy.target_logits)
    ud = dev(wl.u_draft)
    ctx = torch.zeros(B, dtype=torch.long, device="cuda")
    rows, lses, ids, ctxs = [], [], [], [ctx]
    for i in range(g):
        r = Q[ctx].contiguous()
        lse = torch.empty(B, dtype=torch.float64, device="cuda")
        s = torch.empty(B, dtype=torch.int32, device="cuda")
        vt.vt_softmax_temp(r, wl.T, lse, None, ud[:, i].contiguous(), s)
        rows.append(r)
        lses.append(lse)
        ids.append(s)
        ctx = s.long() + 1
        ctxs.append(ctx)
    target = torch.stack([P[c] for c in ctxs], 1).contiguous()
    tl = torch.empty(B * (g + 1), dtype=torch.float64, device="cuda")
    vt.vt_softmax_temp(target.view(-1, cfg.V), wl.T, tl)
    draft = torch.stack(rows, 1).contiguous()
    dl = torch.stack(lses, 1).contiguous()
    di = torch.stack(ids, 1).contiguous()
    tok = torch.empty(B, g + 1, dtype=torch.int32, device="cuda")
    nacc = torch.empty(B, dtype=torch.int32, device="cuda")
    vt.vt_spec_verify(target, tl, wl.T, draft, dl, wl.T, di, None, None, dev(wl.u_acc), dev(wl.u_fin), tok, nacc)
    torch.cuda.synchronize()
    return dict(tokens=tok.cpu().numpy(), n=nacc.cpu().numpy(), draft_ids=di.cpu().numpy())


def test_toy_monte_carlo_and_parity():
    """Config 1 at 1e5 trials: exact parity with the oracle outside the band, and the first
    emitted token follows p(. | start) within 3 sigma for every token."""
    cfg = CONFIGS[1]
    N = 100_000
    say("toy MC 1e5")
    wl = make_workload(cfg, B=N)
    gpu = _toy_gpu(wl)
    orc = ref.toy_block(wl.toy.target_logits, wl.toy.draft_logits, wl.T, cfg.gamma, wl.u_draft, wl.u_acc, wl.u_fin)
    st = compare_tokens(dict(gpu, draft_ids=gpu["draft_ids"]), orc, wl)
    say(f"  {st}")
    assert st["full_match"] >= N - 10
    _, Ptab = ref.softmax_temp(wl.toy.target_logits.astype(np.float64), 1.0)
    freq = np.bincount(gpu["tokens"][:, 0], minlength=cfg.V) / N
    sig = np.sqrt(Ptab[0] * (1 - Ptab[0]) / N)
    say(f"  max |freq - p| / sigma = {(np.abs(freq - Ptab[0]) / sig).max():.2f}")
    assert np.all(np.abs(freq - Ptab[0]) < 3 * sig)


def test_determinism_and_batch_independence():
    """Two runs give identical bits; a sequence's results do not depend on the batch it is in:
    the LM head's value for a row does not depend on M within one kernel (checked on sub-batches
    that stay on the MFMA path), and the softmax/draw/verify calls give a sequence the same bits
    alone as inside the batch."""
    cfg = SCALED["c4-batched"]
    wl = make_workload(cfg)
    a = gpu_block(wl)
    b = gpu_block(wl)
    for k in ("draft_logits", "draft_lse", "draft_ids", "target_lse", "tokens", "n"):
        assert np.array_equal(a[k], b[k]), k
    R = cfg.R
    for s in (0, 6, cfg.B - 2):  # sub-batch of 2 sequences: M = 16 rows, still the MFMA kernel
        two = gpu_block(make_workload(cfg, B=2, b0=s))
        assert np.array_equal(two["draft_logits"], a["draft_logits"][s * R:(s + 2) * R])
        assert np.array_equal(two["tokens"], a["tokens"][s:s + 2])
    for s in (0, 7, cfg.B - 1):  # one sequence alone, fed the batch's draft logits
        one = make_workload(cfg, B=1, b0=s)
        one.draft_logits = a["draft_logits"][s * R:(s + 1) * R]
        r1 = gpu_block(one)
        assert np.array_equal(r1["draft_lse"], a["draft_lse"][s * R:(s + 1) * R])
        assert np.array_equal(r1["draft_ids"][0], a["draft_ids"][s])
        assert np.array_equal(r1["target_lse"][0], a["target_lse"][s])
        assert np.array_equal(r1["tokens"][0], a["tokens"][s]) and r1["n"][0] == a["n"][s]


def test_workspace_reuse_across_calls():
    # a workspace carries nothing between calls: reuse one buffer for differently shaped calls
    wsz = vt.verify_workspace(64, 7, 20000)
    cfg = SCALED["c3-trimmed"]
    for B in (3, 1, 5):
        wl = make_workload(cfg.scaled(B=B), aligned=True)
        g = gpu_block(wl)
        target = target_tensor(wl)
        tl = torch.empty(B * (cfg.gamma + 1), dtype=torch.float64, device="cuda")
        vt.vt_softmax_temp(target.view(-1, cfg.V), wl.T, tl)
        dd = dev(wl.draft_logits)
        dl = torch.empty(B * cfg.R, dtype=torch.float64, device="cuda")
        vt.vt_softmax_temp(dd, wl.T, dl)
        tok = torch.empty(B, cfg.gamma + 1, dtype=torch.int32, device="cuda")
        nacc = torch.empty(B, dtype=torch.int32, device="cuda")
        vt.vt_spec_verify(target, tl, wl.T, dd.view(B, cfg.R, cfg.Vt), dl, wl.T,
                          dev(g["draft_ids"].astype(np.int32)), dev(wl.keep_ids), dev(wl.full_to_trim),
                          dev(wl.u_acc), dev(wl.u_fin), tok, nacc, workspace=wsz)
        torch.cuda.synchronize()
        assert np.array_equal(tok.cpu().numpy(), g["tokens"]) and np.array_equal(nacc.cpu().numpy(), g["n"])

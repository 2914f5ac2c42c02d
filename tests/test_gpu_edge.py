"""Edge cases of the verification kernels on the GPU:

* the residual that rounds to zero after a rejection ("Speculative decoding" glossary, "Why a
  rejection needs a special draw": the residual is a distribution after normalisation, so in exact
  arithmetic a rejection leaves it positive mass; reading R5 draws from p_n when it is zero);
* greedy verification with the longest draft (gamma = 64) on a vocabulary of at most 64 ids, where
  the bonus row has no lane of its own;
* batch independence: a sequence's outputs do not depend on the batch around it, even though the
  LM head's kernel (and with it the fp32 summation order of the logits) depends on the number of
  hidden rows.
"""
import numpy as np
import pytest
import torch

import draft_sampling_verification_amd as vt
from oracle import ref
from tests.gpu_harness import BAND, compare_tokens, dev, gpu_block_fused, oracle_block, say
from workloads import CONFIGS, counter_uniforms, make_workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("V,B,gamma", [(18, 37, 4), (3000, 24, 3), (20000, 16, 5), (20000, 64, 5)])
def test_zero_residual_draws_from_p(V, B, gamma):
    """Draft rows equal to the target rows, but draft_lse = target_lse - delta: then q = p e^delta
    at every id, every accept ratio is e^-delta < 1, u = 1 rejects draft 0, and the fp32 residual
    max(0, p - q) is zero everywhere, so the final token is drawn from p_0 (verify_wave for V <= 64,
    verify_single for one chunk, verify_partial + verify_final otherwise, also at 64 sequences).
    The oracle's verify_sequence is fed the same q."""
    say(f"zero residual V={V} B={B} gamma={gamma}")
    rng = np.random.default_rng(V)
    T = np.float32(0.9)
    delta = 1e-3
    target = (rng.standard_normal((B, gamma + 1, V)) * 2).astype(np.float32)
    R = gamma + 1
    draft = np.ascontiguousarray(target[:, :R, :])  # untrimmed head, Vt = V
    t_lse, p = ref.softmax_temp(ref.as_f64(target, "f32"), T)
    ids = rng.integers(0, V, size=(B, R)).astype(np.int32)
    u_acc = counter_uniforms(9, 5, B, gamma)
    u_acc[:, 0] = 1.0
    u_fin = counter_uniforms(9, 6, B, 1)[:, 0].copy()
    tok = torch.full((B, gamma + 1), -9, dtype=torch.int32, device="cuda")
    nacc = torch.full((B,), -9, dtype=torch.int32, device="cuda")
    vt.vt_spec_verify(dev(target), dev(t_lse.reshape(-1)), float(T), dev(draft),
                      dev((t_lse[:, :R] - delta).reshape(-1)), float(T), dev(ids), None, None, dev(u_acc), dev(u_fin),
                      tok, nacc)
    torch.cuda.synchronize()
    tok, nacc = tok.cpu().numpy(), nacc.cpu().numpy()
    assert np.all(nacc == 0)
    excused = 0
    for b in range(B):
        q_rows = p[b, :R] * np.exp(delta)
        want, n, ratios, margin = ref.verify_sequence(p[b], q_rows, ids[b], None, u_acc[b], u_fin[b], gamma)
        assert n == 0 and abs(ratios[0] - np.exp(-delta)) < 1e-12
        # the fallback: the oracle's final token is the inverse-CDF draw from p_0 itself
        assert want[0] == ref.draw(p[b, 0], float(u_fin[b]))[0]
        if tok[b, 0] != want[0]:
            assert margin < BAND, (b, tok[b], want)
            excused += 1
        assert np.all(tok[b, 1:] == -1)
    assert excused <= max(1, B // 20)


@pytest.mark.parametrize("V", [18, 50, 64])
def test_greedy_longest_draft_small_vocab(V):
    """gamma = 64, drafts equal to the target argmaxes for a prefix of random length (0..64): the
    bonus token after 64 accepted drafts is the argmax of target row 64."""
    rng = np.random.default_rng(64 + V)
    g, B = 64, 24
    target = rng.standard_normal((B, g + 1, V)).astype(np.float32)
    amax = target.astype(np.float64).argmax(axis=2)
    ids = rng.integers(0, V, size=(B, g + 1)).astype(np.int32)
    for b in range(B):
        k = g if b < B // 2 else int(rng.integers(0, g))
        ids[b, :k] = amax[b, :k]
    tok = torch.full((B, g + 1), -9, dtype=torch.int32, device="cuda")
    nacc = torch.full((B,), -9, dtype=torch.int32, device="cuda")
    vt.vt_spec_verify(dev(target), None, 0.0, None, None, None, dev(ids), None, None, None, None, tok, nacc)
    torch.cuda.synchronize()
    want_tok, want_n = ref.greedy_verify(target.astype(np.float64), ids, None, g)
    assert (want_n == g).sum() >= B // 2
    assert np.array_equal(nacc.cpu().numpy(), want_n)
    assert np.array_equal(tok.cpu().numpy(), want_tok)


def _merge(parts):
    return {k: np.concatenate([p[k] for p in parts]) for k in ("tokens", "n", "draft_ids")}


@pytest.mark.parametrize("c,B,follow", [(4, 40, 0.5), (5, 32, 0.5), (4, 40, 0.0), (4, 64, 0.5)])
def test_batch_independence_across_head_kernels(c, B, follow):
    """The same sequences alone (B = 1: the GEMV head and the three-launch path for 8 draft rows,
    a one-block MFMA head for 9), in batches of at most 128 hidden rows (one block of all rows) and
    in a batch of 256+ hidden rows (two all-rows blocks for 320 and 288 rows, 256 x 256 tiles for
    512).
    The MFMA kernels sum in one order, the GEMV in another, and the draft running sums are chunked
    by the head's blocks, so a decision may differ only where the oracle places it within the
    band; every other output must be the same, and each run must match the oracle."""
    cfg = CONFIGS[c].scaled(B=B, V=20000, Vt=6000, H=512)
    assert cfg.B * cfg.R >= 256
    say(f"batch independence config {c}: B={B} (M={cfg.B * cfg.R}), follow={follow}")
    big = make_workload(cfg, follow=follow)
    gbig = gpu_block_fused(big)
    orc = oracle_block(big)
    st = compare_tokens(gbig, orc, big)
    say(f"  batch of {B}: {st}")
    assert st["full_match"] >= 0.95 * B
    mb = 128 // cfg.R
    gmid = _merge([gpu_block_fused(make_workload(cfg.scaled(B=min(mb, B - b0)), b0=b0, follow=follow))
                   for b0 in range(0, B, mb)])
    st = compare_tokens(gmid, orc, big)
    say(f"  batches of {mb}: {st}")
    assert st["full_match"] >= 0.95 * B
    one = cfg.scaled(B=1)
    singles = [gpu_block_fused(make_workload(one, b0=b, follow=follow)) for b in range(B)]
    gone = {k: np.concatenate([s[k] for s in singles]) for k in ("tokens", "n", "draft_ids")}
    st = compare_tokens(gone, orc, big)
    say(f"  one at a time: {st}")
    assert st["full_match"] >= 0.95 * B
    same = (gone["tokens"] == gbig["tokens"]).all(axis=1) & (gone["n"] == gbig["n"])
    say(f"  identical outputs alone and in the batch: {same.sum()} of {B}")
    # compare_tokens has already asserted that every difference from the oracle lies at a decision
    # the oracle places within the band, so the two runs can differ only at such decisions
    assert same.sum() >= B - 2 * max(1, B // 20)

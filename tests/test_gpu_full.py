"""Full-size parity for configs 2-5 in the launch configuration the benchmark times (the same four
calls on the same shapes).  The oracle recomputes every sequence of configs 2-4 and 32 sequences
spread over config 5's batch (their hidden rows through the whole trimmed head, their target rows
over the full vocabulary); every sequence is checked for properties that hold at any size, and the
first-draft acceptances of the whole batch against sum_b beta_b.  Whole 256 x 256 tiles of the
large-batch heads are checked logit by logit against the recursive-summation bound.  The aligned
variants (draft = target at the kept ids) exercise deep accepts, bonus tokens and off-set residual
draws at full size."""
import numpy as np
import pytest

from oracle import ref
from tests.gpu_harness import (beta_z, compare_tokens, gpu_block, lmhead_error_bound, oracle_block, say,
                               sequences_workload)
from workloads import CONFIGS, make_workload

pytestmark = pytest.mark.gpu

SAMPLE = {2: [0], 3: [0], 4: list(range(64)), 5: sorted(set(np.linspace(0, 255, 32).round().astype(int).tolist()))}


def _properties(gpu, wl):
    cfg = wl.cfg
    n = gpu["n"]
    assert np.all((n >= 0) & (n <= cfg.gamma))
    for b in range(wl.B):
        t = gpu["tokens"][b]
        assert np.all(t[: n[b] + 1] >= 0) and np.all(t[: n[b] + 1] < cfg.V)
        assert np.all(t[n[b] + 1:] == -1)
        if wl.keep_ids is not None:
            ids = gpu["draft_ids"][b, : n[b]]
            assert np.array_equal(t[: n[b]], wl.keep_ids[ids])
    assert np.all(np.isfinite(gpu["draft_lse"])) and np.all(np.isfinite(gpu["target_lse"]))
    assert np.all((gpu["draft_ids"] >= 0) & (gpu["draft_ids"] < cfg.Vt))


_RUNS = {}


def _run(c):
    """The recipe's full-size block of config c on the GPU (kept for the tests that follow)."""
    if c not in _RUNS:
        _RUNS.clear()
        wl = make_workload(CONFIGS[c])
        _RUNS[c] = (wl, gpu_block(wl))
    return _RUNS[c]


def _rows(seqs, R):
    return (np.asarray(seqs)[:, None] * R + np.arange(R)[None, :]).reshape(-1)


@pytest.mark.parametrize("c", [2, 3, 4, 5])
def test_full_size_block(c):
    cfg = CONFIGS[c]
    say(f"full-size block config {c}: {cfg.name}")
    wl, gpu = _run(c)
    _properties(gpu, wl)
    z, acc, exp = beta_z(gpu, wl)
    say(f"  first drafts accepted {acc:.0f}, expected sum beta {exp:.2f}, z = {z:.2f}")
    assert abs(z) < 4.5
    R, seqs = cfg.R, SAMPLE[c]
    say(f"  oracle on {len(seqs)} sequences")
    sub_wl = sequences_workload(cfg, seqs)
    orc = oracle_block(sub_wl)
    sel = np.asarray(seqs)
    sub = dict(draft_ids=gpu["draft_ids"][sel], n=gpu["n"][sel], tokens=gpu["tokens"][sel])
    st = compare_tokens(sub, orc, sub_wl)
    rows = _rows(seqs, R)
    dl = np.abs(gpu["draft_lse"][rows] - orc["draft_lse_flat"]).max()
    tl = np.abs(gpu["target_lse"][sel] - orc["target_lse"]).max()
    bound = lmhead_error_bound(sub_wl.hidden, sub_wl.weight, sub_wl.keep_ids)
    lerr = np.abs(gpu["draft_logits"][rows] - orc["draft_logits"])
    say(f"  {st}; |logit err| / bound {np.max(lerr / bound):.3f}; |draft lse err| {dl:.2e} "
        f"|target lse err| {tl:.2e}")
    assert st["full_match"] >= 0.95 * len(seqs)
    assert tl <= 2e-6 and dl <= 1e-4
    assert np.all(lerr <= bound)


@pytest.mark.parametrize("c,tile", [(4, (0, 0)), (4, (1, 127)), (5, (0, 0)), (5, (8, 255)), (5, (4, 100))])
def test_full_size_head_tile(c, tile):
    """One whole 256 x 256 output tile of the large-batch head (hidden-row block, head-row block),
    every logit within H 2^-24 sum_k |h_k w_k| of the float64 head."""
    bm, bn = tile
    say(f"full-size head tile config {c}, tile {tile}")
    wl, gpu = _run(c)
    r = slice(256 * bm, 256 * (bm + 1))
    cols = slice(256 * bn, 256 * (bn + 1))
    keep = wl.keep_ids[cols]
    want = ref.lm_head(wl.hidden[r], wl.weight, keep)
    bound = lmhead_error_bound(wl.hidden[r], wl.weight, keep)
    err = np.abs(gpu["draft_logits"][r, cols] - want)
    say(f"  max |err| {err.max():.2e}, max err / bound {np.max(err / bound):.3f}")
    assert err.shape == (256, 256) and np.all(err <= bound)


@pytest.mark.parametrize("c", [3, 4, 5])
def test_full_size_aligned(c):
    cfg = CONFIGS[c]
    say(f"full-size aligned config {c}")
    wl = make_workload(cfg, aligned=True)
    gpu = gpu_block(wl)
    _properties(gpu, wl)
    kept = np.zeros(cfg.V, bool)
    kept[wl.keep_ids] = True
    for b in range(wl.B):
        n = gpu["n"][b]
        if n < cfg.gamma:
            assert not kept[gpu["tokens"][b, n]]
    say(f"  mean accepted {gpu['n'].mean():.2f}, bonus blocks {(gpu['n'] == cfg.gamma).sum()} of {wl.B}")
    z, acc, exp = beta_z(gpu, wl)
    say(f"  first drafts accepted {acc:.0f}, expected sum beta {exp:.2f}, z = {z:.2f}")
    assert abs(z) < 4.5
    orc = oracle_block(wl)
    st = compare_tokens(gpu, orc, wl)
    say(f"  {st}")
    assert st["full_match"] >= 0.95 * wl.B

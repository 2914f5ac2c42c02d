"""Full-size parity for configs 2-5 in the launch configuration the benchmark times (the same four
calls on the same shapes).  The oracle recomputes sampled sequences one by one (their hidden rows
through the whole trimmed head, their target rows over the full vocabulary); every sequence is
checked for properties that hold at any size.  The aligned variants (draft = target at the kept
ids) exercise deep accepts, bonus tokens and off-set residual draws at full size."""
import numpy as np
import pytest

from tests.gpu_harness import compare_tokens, gpu_block, oracle_block, say
from workloads import CONFIGS, make_workload

pytestmark = pytest.mark.gpu

SAMPLE = {2: [0], 3: [0], 4: [0, 17, 63], 5: [0, 128, 255]}


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


@pytest.mark.parametrize("c", [2, 3, 4, 5])
def test_full_size_block(c):
    cfg = CONFIGS[c]
    say(f"full-size block config {c}: {cfg.name}")
    wl = make_workload(cfg)
    gpu = gpu_block(wl)
    _properties(gpu, wl)
    R = cfg.R
    for s in SAMPLE[c]:
        one = make_workload(cfg, B=1, b0=s)
        orc = oracle_block(one)
        sub = dict(draft_ids=gpu["draft_ids"][s:s + 1], n=gpu["n"][s:s + 1], tokens=gpu["tokens"][s:s + 1])
        st = compare_tokens(sub, orc, one)
        dl = np.abs(gpu["draft_lse"][s * R:(s + 1) * R] - orc["draft_lse_flat"]).max()
        tl = np.abs(gpu["target_lse"][s] - orc["target_lse"][0]).max()
        lg = np.abs(gpu["draft_logits"][s * R:(s + 1) * R] - orc["draft_logits"]).max()
        say(f"  seq {s}: {st}; |logit err| {lg:.2e} |draft lse err| {dl:.2e} |target lse err| {tl:.2e}")
        assert tl <= 2e-6 and dl <= 1e-4 and lg <= 1e-3


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
    orc = oracle_block(wl)
    st = compare_tokens(gpu, orc, wl)
    say(f"  {st}")
    assert st["full_match"] >= 0.95 * wl.B

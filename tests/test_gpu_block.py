"""GPU parity of the fused single-call block (vt_spec_block) against the oracle, and its
agreement with the four separate calls: the LM-head logits and the target log-normalisers are
the same bits; draft draws may differ only where the oracle puts a CDF boundary within the band
(the fused path chunks the draft running sums by the LM head's row blocks)."""
import numpy as np
import pytest
import torch

from tests.gpu_harness import compare_tokens, gpu_block, gpu_block_fused, oracle_block, say
from workloads import CONFIGS, make_workload

pytestmark = pytest.mark.gpu

SCALED = {
    "c2-full-head": CONFIGS[2].scaled(V=20000, Vt=20000, H=512),
    "c3-trimmed": CONFIGS[3].scaled(V=20000, Vt=5000, H=512),
    "c3-ragged": CONFIGS[3].scaled(V=9001, Vt=1234, H=520),
    "c4-batched-mfma": CONFIGS[4].scaled(B=24, V=20000, Vt=5000, H=256),
    "c5-mfma": CONFIGS[5].scaled(B=16, V=13000, Vt=6000, H=256),
    "c4-big-tiles": CONFIGS[4].scaled(B=40, V=20000, Vt=5000, H=520),  # M = 320: fused 256x256 tiles
    "c5-big-tiles": CONFIGS[5].scaled(B=32, V=13000, Vt=6001, H=256),  # M = 288, ragged Vt
    "c3-one-chunk-target": CONFIGS[3].scaled(V=4000, Vt=1500, H=256),
}


def _check(wl):
    gpu = gpu_block_fused(wl)
    orc = oracle_block(wl)
    t_err = np.abs(gpu["target_lse"] - orc["target_lse"]).max()
    d_err = np.abs(gpu["draft_lse"] - orc["draft_lse_flat"]).max()
    say(f"  |target lse err| {t_err:.2e}  |draft lse err| {d_err:.2e}")
    assert t_err <= 2e-6 and d_err <= (2e-6 if wl.draft_logits is not None else 1e-4)
    st = compare_tokens(gpu, orc, wl)
    say(f"  {st}; mean accepted {orc['n'].mean():.2f}")
    assert st["full_match"] >= 0.95 * wl.B
    return gpu, orc


@pytest.mark.parametrize("name", list(SCALED))
def test_fused_block_parity_scaled(name):
    say(f"fused block parity {name}")
    _check(make_workload(SCALED[name]))


@pytest.mark.parametrize("name", ["c3-trimmed", "c3-ragged", "c5-mfma"])
def test_fused_block_rank_ordered_keep_set(name):
    # kept ids stored best-ranked first instead of ascending: the gathers are no longer monotone
    say(f"fused block parity {name}, keep set in rank order")
    _check(make_workload(SCALED[name], keep_order="rank"))


@pytest.mark.parametrize("name", ["c3-trimmed", "c4-batched-mfma", "c4-big-tiles"])
def test_fused_matches_separate_calls(name):
    wl = make_workload(SCALED[name])
    a = gpu_block(wl)
    b = gpu_block_fused(wl)
    assert np.array_equal(a["draft_logits"], b["draft_logits"])
    assert np.array_equal(a["target_lse"], b["target_lse"])
    assert np.abs(a["draft_lse"] - b["draft_lse"]).max() < 1e-6
    same = (a["tokens"] == b["tokens"]).all(axis=1) & (a["n"] == b["n"])
    assert same.mean() >= 0.95, same.mean()


@pytest.mark.parametrize("c,order", [(2, "id"), (3, "id"), (4, "id"), (5, "id"), (3, "rank")])
def test_fused_block_full_size(c, order):
    cfg = CONFIGS[c]
    say(f"fused block full size config {c}, keep order {order}")
    wl = make_workload(cfg, keep_order=order)
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for e in ev:
        e.record()  # materialise the events
    torch.cuda.synchronize()
    gpu = gpu_block_fused(wl, events=ev)
    say(f"  LM head inside the call: {ev[0].elapsed_time(ev[1]) * 1e3:.1f} us")
    assert ev[0].elapsed_time(ev[1]) > 0
    R = cfg.R
    for s in ([0] if cfg.B == 1 else [0, cfg.B - 1]):
        one = make_workload(cfg, B=1, b0=s, keep_order=order)
        orc = oracle_block(one)
        sub = dict(draft_ids=gpu["draft_ids"][s:s + 1], n=gpu["n"][s:s + 1], tokens=gpu["tokens"][s:s + 1])
        st = compare_tokens(sub, orc, one)
        say(f"  seq {s}: {st}")
        assert np.abs(gpu["target_lse"][s] - orc["target_lse"][0]).max() <= 2e-6
        assert np.abs(gpu["draft_lse"][s * R:(s + 1) * R] - orc["draft_lse_flat"]).max() <= 1e-4

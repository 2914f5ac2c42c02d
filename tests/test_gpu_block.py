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
    "c4-big-tiles": CONFIGS[4].scaled(B=40, V=20000, Vt=5000, H=520),  # M = 320: register-staged tiles
    "c5-big-tiles": CONFIGS[5].scaled(B=32, V=13000, Vt=6001, H=256),  # M = 288: two all-rows blocks, ragged Vt
    "c3-one-chunk-target": CONFIGS[3].scaled(V=4000, Vt=1500, H=256),
    # untrimmed head at 288 hidden rows: K-tiled hidden copy, no keep set
    "c2-untrimmed-big-tiles": CONFIGS[2].scaled(B=48, V=6000, Vt=6000, H=256),
    # 288 hidden rows with a one-chunk target row: the hidden copy takes a launch of its own
    "c5-big-tiles-one-chunk-target": CONFIGS[5].scaled(B=32, V=4000, Vt=1500, H=256),
    # the head's row blocks: 756 hidden rows against 126 head blocks take 384-row tiles (two
    # blocks, the second ragged: 252 tiles, one per CU, against 378 of 256 rows), 512 rows take
    # 256-row tiles (two blocks)
    "c5-tall-two-blocks": CONFIGS[5].scaled(B=84, V=40000, Vt=32001, H=256),
    "c4-square-two-blocks": CONFIGS[4].scaled(B=64, V=20000, Vt=5000, H=256),
    # 2250 hidden rows against 128 head blocks: 768 tall tiles in three waves (six row blocks, the
    # last ragged; ragged Vt)
    "c5-tall-ragged": CONFIGS[5].scaled(B=250, V=34000, Vt=32700, H=128),
    # past the GEMV sizes: one block of all rows padded to a multiple of 32 (9 rows: one 32-row
    # block; 96: three; 128, 129: four, five; 192: six) per 256 head rows (66000 head rows) up to
    # 192 rows, or per 128 (fewer than 256 blocks of 256) up to 256 rows (194: seven; 256:
    # eight) and in two blocks up to 384 (258: two of 160), then 256 x 256 tiles; with
    # H % 32 != 0 below 129 rows, 128 x 128 tiles and a separate draft softmax
    "rows-9": CONFIGS[4].scaled(B=3, gamma=2, R=3, V=20000, Vt=5000, H=256),
    "rows-96": CONFIGS[4].scaled(B=12, V=20000, Vt=5000, H=256),
    "rows-128": CONFIGS[4].scaled(B=16, V=20000, Vt=5000, H=256),
    "rows-129": CONFIGS[4].scaled(B=43, gamma=2, R=3, V=20000, Vt=5000, H=256),
    "rows-192": CONFIGS[4].scaled(B=24, V=20000, Vt=5000, H=256),
    "rows-194-seven-blocks": CONFIGS[4].scaled(B=97, gamma=1, R=2, V=20000, Vt=5000, H=256),
    "rows-256-eight-blocks": CONFIGS[4].scaled(B=32, V=20000, Vt=5000, H=256),
    "rows-258-two-blocks": CONFIGS[4].scaled(B=129, gamma=1, R=2, V=20000, Vt=5000, H=256),
    "rows-36-wide-head": CONFIGS[5].scaled(B=4, V=70000, Vt=66000, H=256),
    # up to 32 hidden rows of at most 8 per sequence the MFMA head is followed by the two-pass
    # verification (chunk pass and final pass) instead of the combine and verify launches
    "rows-32-two-pass": CONFIGS[4].scaled(B=4, V=20000, Vt=5000, H=256),
    # more than 8 draft rows per sequence: each chunk-pass wavefront draws two rows (9 and 16 rows,
    # the latter with 16 target rows)
    "rows-18-two-pass-9-rows": CONFIGS[5].scaled(B=2, V=20000, Vt=5000, H=256),
    "rows-32-two-pass-16-rows": CONFIGS[4].scaled(B=2, gamma=15, R=16, V=20000, Vt=5000, H=256),
    # a 64-row head past the GEMV sizes (one partial per draft row) and H = 32 (one K step)
    "rows-tiny-head": CONFIGS[4].scaled(B=8, V=3000, Vt=64, H=256),
    "rows-one-k-step": CONFIGS[4].scaled(B=6, V=5000, Vt=1500, H=32),
    "small-batch-odd-H": CONFIGS[4].scaled(B=4, V=9001, Vt=1234, H=520),
}


# Decode-sized blocks (B*R <= 8, both sides sampled) run the three-launch path: each case reaches
# a branch of it the configs above do not.
SMALL = {
    "b1-wide-vocab": CONFIGS[3].scaled(V=300000, Vt=20000, H=256),        # > 64 target chunks
    "b1-gamma8": CONFIGS[3].scaled(gamma=8, R=8, V=20000, Vt=5000, H=256),  # target row 8 on wave 0
    "b1-bf16-target": CONFIGS[4].scaled(B=1, gamma=5, R=6, V=20000, Vt=5000, H=256),
    "b1-bf16-ragged": CONFIGS[4].scaled(B=1, gamma=4, R=5, V=9001, Vt=1234, H=520),  # element loads
    "b2-r4": CONFIGS[3].scaled(B=2, gamma=3, R=4, V=20000, Vt=5000, H=256),
    "b1-rows-past-gamma": CONFIGS[3].scaled(gamma=3, R=6, V=20000, Vt=5000, H=256),
    "b1-cold": CONFIGS[3].scaled(T=0.3, V=20000, Vt=5000, H=256),
    "b1-tiny-head": CONFIGS[3].scaled(V=3000, Vt=64, H=256),  # 4-row head blocks, one chunk
    "b1-full-head": CONFIGS[2].scaled(V=20000, Vt=20000, H=512),  # untrimmed: no full_to_trim
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


def test_fused_block_longest_draft():
    # gamma = 64, the longest run the path takes (one lane per draft position), with a drafter that
    # follows the target closely: runs of every length up to full acceptance and its bonus token
    cfg = CONFIGS[4].scaled(B=6, gamma=64, R=65, V=6000, Vt=2500, H=256)
    say("fused block parity gamma=64, following drafter")
    _, orc = _check(make_workload(cfg, follow=0.03))
    assert (orc["n"] == 64).any() and (orc["n"] < 64).any()


@pytest.mark.parametrize("name", list(SMALL))
def test_fused_block_parity_small_batch(name):
    say(f"fused block parity {name} (three-launch path)")
    _check(make_workload(SMALL[name]))


@pytest.mark.parametrize("name", list(SMALL))
def test_fused_block_small_batch_long_runs(name):
    # a drafter that follows the target: accepted runs of every length, rejections at every
    # position and full acceptance (the bonus draw from p_gamma) over six seeds
    say(f"fused block parity {name}, following drafter")
    seen = set()
    for b0 in range(6):
        _, orc = _check(make_workload(SMALL[name], b0=b0, follow=0.5))
        seen.update(int(x) for x in orc["n"])
    say(f"  accepted counts seen: {sorted(seen)}")
    assert len(seen) >= 2 and max(seen) > 0


@pytest.mark.parametrize("name", ["c4-batched-mfma", "c4-big-tiles", "c5-mfma", "c5-big-tiles", "rows-32-two-pass",
                                  "rows-18-two-pass-9-rows"])
def test_fused_block_following_drafter(name):
    say(f"fused block parity {name}, following drafter")
    _, orc = _check(make_workload(SCALED[name], follow=0.5))
    say(f"  accepted counts: {np.bincount(orc['n'], minlength=SCALED[name].gamma + 1).tolist()}")
    assert orc["n"].max() > 0


def test_two_pass_sixteen_draft_rows_following_drafter():
    # two sequences of 16 draft rows whose drafts the oracle accepts in part (sequences 8 and 9 of
    # the recipe: 1 and 3 accepted), so the chunk pass's second row per wavefront feeds a residual
    cfg = SCALED["rows-32-two-pass-16-rows"]
    say("fused block parity rows-32-two-pass-16-rows, following drafter, sequences 8 and 9")
    _, orc = _check(make_workload(cfg, follow=0.5, b0=8))
    say(f"  accepted: {orc['n'].tolist()}")
    assert orc["n"].max() > 0


@pytest.mark.parametrize("name", ["b1-wide-vocab", "b1-bf16-target", "b1-bf16-ragged"])
def test_small_batch_matches_separate_calls(name):
    wl = make_workload(SMALL[name])
    a = gpu_block(wl)
    b = gpu_block_fused(wl)
    assert np.array_equal(a["draft_logits"], b["draft_logits"])
    assert np.array_equal(a["target_lse"], b["target_lse"])  # same operations, same bits
    assert np.abs(a["draft_lse"] - b["draft_lse"]).max() < 1e-6
    assert (a["tokens"] == b["tokens"]).all() and (a["n"] == b["n"]).all()


@pytest.mark.parametrize("name", ["c3-trimmed", "c3-ragged", "c5-mfma"])
def test_fused_block_rank_ordered_keep_set(name):
    # kept ids stored best-ranked first instead of ascending: the gathers are no longer monotone
    say(f"fused block parity {name}, keep set in rank order")
    _check(make_workload(SCALED[name], keep_order="rank"))


@pytest.mark.parametrize("name", ["c3-trimmed", "c4-batched-mfma", "c4-big-tiles", "c5-big-tiles",
                                  "c5-tall-two-blocks", "c4-square-two-blocks", "c5-tall-ragged"])
def test_fused_matches_separate_calls(name):
    # c5-big-tiles (M = 288, H = 256) and c5-tall-two-blocks (M = 756): the fused call's head runs
    # 384 x 256 tiles on a K-tiled copy of the hidden rows, the separate call 256 x 256 tiles on
    # the rows as given; c4-square-two-blocks (M = 512): 256 x 256 tiles on both; the logits must
    # be the same bits
    wl = make_workload(SCALED[name])
    a = gpu_block(wl)
    b = gpu_block_fused(wl)
    assert np.array_equal(a["draft_logits"], b["draft_logits"])
    assert np.array_equal(a["target_lse"], b["target_lse"])
    assert np.abs(a["draft_lse"] - b["draft_lse"]).max() < 1e-6
    same = (a["tokens"] == b["tokens"]).all(axis=1) & (a["n"] == b["n"])
    assert same.mean() >= 0.95, same.mean()


@pytest.mark.parametrize("name,order", [("c5-big-tiles", "id"), ("c5-big-tiles", "rank"),
                                        ("c2-untrimmed-big-tiles", "id"), ("c5-big-tiles-one-chunk-target", "id"),
                                        ("c5-tall-two-blocks", "id"), ("c4-square-two-blocks", "id"),
                                        ("c5-tall-ragged", "id"), ("c5-tall-ragged", "rank")])
def test_tiled_head_gives_the_same_block(name, order):
    # the K-tiled W^Trim holds the same rows as the gather through keep_ids: every output, the
    # logits included, must be the same bits (M = 288, ragged Vt = 6001 in the first two)
    wl = make_workload(SCALED[name], keep_order=order)
    say(f"tiled head vs gathered rows: {name}, keep order {order}")
    a = gpu_block_fused(wl)
    b = gpu_block_fused(wl, tiled=True)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("c", [4, 5])
def test_tiled_head_gives_the_same_block_full_size(c):
    # the benchmark's launch configuration (config 5: 384 x 256 tiles on the K-tiled W^Trim;
    # config 4: 256 x 256) against the same call gathering rows, and its logits and target
    # log-normalisers against the separate calls (256 x 256 tiles on the rows as given)
    wl = make_workload(CONFIGS[c])
    say(f"tiled head vs gathered rows and separate calls: full size config {c}")
    a = gpu_block_fused(wl)
    b = gpu_block_fused(wl, tiled=True)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    sep = gpu_block(wl)
    assert np.array_equal(b["draft_logits"], sep["draft_logits"])
    assert np.array_equal(b["target_lse"], sep["target_lse"])


@pytest.mark.parametrize("c,order,follow", [(2, "id", 0.0), (3, "id", 0.0), (4, "id", 0.0), (5, "id", 0.0),
                                            (3, "rank", 0.0), (3, "id", 0.5)])
def test_fused_block_full_size(c, order, follow):
    # configs 4 and 5 run as the benchmark times them: with the K-tiled W^Trim
    cfg = CONFIGS[c]
    tiled = c in (4, 5)
    say(f"fused block full size config {c}, keep order {order}, following drafter {follow}, tiled head {tiled}")
    wl = make_workload(cfg, keep_order=order, follow=follow)
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for e in ev:
        e.record()  # materialise the events
    torch.cuda.synchronize()
    gpu = gpu_block_fused(wl, events=ev, tiled=tiled)
    say(f"  LM head inside the call: {ev[0].elapsed_time(ev[1]) * 1e3:.1f} us")
    assert ev[0].elapsed_time(ev[1]) > 0
    R = cfg.R
    for s in ([0] if cfg.B == 1 else [0, cfg.B - 1]):
        one = make_workload(cfg, B=1, b0=s, keep_order=order, follow=follow)
        orc = oracle_block(one)
        sub = dict(draft_ids=gpu["draft_ids"][s:s + 1], n=gpu["n"][s:s + 1], tokens=gpu["tokens"][s:s + 1])
        st = compare_tokens(sub, orc, one)
        say(f"  seq {s}: {st}")
        assert np.abs(gpu["target_lse"][s] - orc["target_lse"][0]).max() <= 2e-6
        assert np.abs(gpu["draft_lse"][s * R:(s + 1) * R] - orc["draft_lse_flat"]).max() <= 1e-4

"""GPU parity of greedy mode (temperature 0): vt_softmax_temp's argmax draws (lowest id on ties,
lse = row max, one-hot probabilities) and vt_spec_verify's greedy verification, against the
oracle.  All outputs are decided by exact comparisons, so they must match bit for bit."""
import numpy as np
import pytest
import torch

import draft_sampling_verification_amd as vt
from oracle import ref
from tests.gpu_harness import dev, dev_bf16, say
from workloads import CONFIGS, bf16_round, make_workload

pytestmark = pytest.mark.gpu


def _rows_with_ties(rows, n, seed, dtype):
    rng = np.random.default_rng(seed)
    x = np.round(rng.normal(size=(rows, n)) * 4) / 4  # coarse values: many exact ties
    for r in range(rows):                          # force a tie for the maximum in half the rows
        if r % 2 == 0:
            j = rng.choice(n, size=2, replace=False)
            x[r, j] = x[r].max() + 1
    x = x.astype(np.float32)
    return x if dtype == "f32" else bf16_round(x)


@pytest.mark.parametrize("rows,n,dtype", [(9, 18, "f32"), (7, 4096, "f32"), (5, 9000, "bf16"), (6, 128256, "f32"),
                                          (40, 5000, "bf16")])
def test_softmax_greedy(rows, n, dtype):
    store = _rows_with_ties(rows, n, rows + n, dtype)
    x64 = ref.as_f64(store, dtype)
    xs = dev(store) if dtype == "f32" else dev_bf16(store)
    lse = torch.empty(rows, dtype=torch.float64, device="cuda")
    pr = torch.empty(rows, n, dtype=torch.float32, device="cuda")
    samp = torch.empty(rows, dtype=torch.int32, device="cuda")
    vt.vt_softmax_temp(xs, 0.0, lse, pr, None, samp)
    torch.cuda.synchronize()
    want = np.array([ref.argmax_lowest(x64[r]) for r in range(rows)])
    assert np.array_equal(samp.cpu().numpy(), want)
    assert np.array_equal(lse.cpu().numpy(), x64.max(axis=1))
    onehot = np.zeros((rows, n), np.float32)
    onehot[np.arange(rows), want] = 1
    assert np.array_equal(pr.cpu().numpy(), onehot)


def _greedy_gpu(target_store, dtype, ids, keep, f2t):
    B, g1, V = target_store.shape
    t = dev(target_store) if dtype == "f32" else dev_bf16(target_store)
    tok = torch.empty(B, g1, dtype=torch.int32, device="cuda")
    nacc = torch.empty(B, dtype=torch.int32, device="cuda")
    vt.vt_spec_verify(t, None, 0.0, None, None, None, dev(ids.astype(np.int32)),
                      dev(keep) if keep is not None else None, dev(f2t) if f2t is not None else None,
                      None, None, tok, nacc)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), nacc.cpu().numpy()


@pytest.mark.parametrize("name,cfg,dtype", [
    ("toy", CONFIGS[1], "f32"),
    ("c3-scaled", CONFIGS[3].scaled(B=32, V=20000, Vt=5000, H=64), "f32"),
    ("c4-scaled", CONFIGS[4].scaled(B=48, V=9001, Vt=3000, H=64), "bf16"),
    ("c4-full", CONFIGS[4], "bf16"),
])
def test_greedy_verify(name, cfg, dtype):
    say(f"greedy verify {name}")
    B, g, V = (64, cfg.gamma, cfg.V) if cfg.H == 0 else (cfg.B, cfg.gamma, cfg.V)
    rng = np.random.default_rng(7)
    if cfg.H == 0:
        target = _rows_with_ties(B * (g + 1), V, 1, "f32").reshape(B, g + 1, V)
        keep = f2t = None
    else:
        wl = make_workload(cfg, aligned=True)
        target, keep, f2t = wl.target, wl.keep_ids, wl.full_to_trim
    t64 = ref.as_f64(target, dtype)
    amax = t64.argmax(axis=2)  # first maximum = lowest id
    # drafts: the target's argmax (mapped into trimmed ids when kept) for a random prefix, then noise
    inv = {int(k): j for j, k in enumerate(keep)} if keep is not None else None
    R = g + 1
    ids = rng.integers(0, cfg.Vt, size=(B, R))
    for b in range(B):
        k = rng.integers(0, g + 1)
        for i in range(k):
            a = int(amax[b, i])
            if inv is None:
                ids[b, i] = a
            elif a in inv:
                ids[b, i] = inv[a]
    tok, n = _greedy_gpu(target, dtype, ids, keep, f2t)
    want_tok, want_n = ref.greedy_verify(t64, ids, keep, g)
    say(f"  mean accepted {want_n.mean():.2f}, full blocks {(want_n == g).sum()} of {B}")
    assert np.array_equal(n, want_n) and np.array_equal(tok, want_tok)


def test_greedy_flags_bad_ids():
    target = np.random.default_rng(0).normal(size=(3, 4, 5000)).astype(np.float32)
    ids = np.zeros((3, 3), np.int32)
    ids[1, 2] = 5000
    tok, n = _greedy_gpu(target, "f32", ids, None, None)
    assert n[1] == -1 and (tok[1] == -1).all() and n[0] >= 0 and n[2] >= 0


def _block_greedy(wl, draft_T, tiled=False):
    cfg = wl.cfg
    B, R, g = wl.B, cfg.R, cfg.gamma
    keep = dev(wl.keep_ids) if wl.keep_ids is not None else None
    f2t = dev(wl.full_to_trim) if wl.full_to_trim is not None else None
    target = dev(wl.target) if cfg.target_dtype == "f32" else dev_bf16(wl.target)
    logits = torch.empty(B * R, cfg.Vt, dtype=torch.float32, device="cuda")
    dlse = torch.empty(B * R, dtype=torch.float64, device="cuda")
    dids = torch.empty(B * R, dtype=torch.int32, device="cuda")
    tok = torch.full((B, g + 1), -9, dtype=torch.int32, device="cuda")
    nacc = torch.empty(B, dtype=torch.int32, device="cuda")
    ud = dev(wl.u_draft.reshape(-1)) if draft_T > 0 else None
    weight = dev_bf16(wl.weight)
    wt = vt.vt_trim_head_tiled(weight, keep, k=cfg.Vt) if tiled else None
    vt.vt_spec_block(dev_bf16(wl.hidden), weight, keep, f2t, target, 0.0, draft_T, ud, None, None,
                     logits, dlse, dids, None, tok, nacc, weight_tiled=wt)
    torch.cuda.synchronize()
    return (logits.cpu().numpy(), dlse.cpu().numpy(), dids.cpu().numpy().reshape(B, R), tok.cpu().numpy(),
            nacc.cpu().numpy())


@pytest.mark.parametrize("name,cfg,draft_T", [
    ("c3-scaled argmax drafts", CONFIGS[3].scaled(B=4, V=20000, Vt=5000, H=512), 0.0),
    ("c3-scaled sampled drafts", CONFIGS[3].scaled(B=4, V=20000, Vt=5000, H=512), 1.0),
    ("c4-scaled argmax drafts", CONFIGS[4].scaled(B=24, V=9001, Vt=3000, H=256), 0.0),
    ("c4 big tiles argmax drafts", CONFIGS[4].scaled(B=40, V=20000, Vt=5000, H=256), 0.0),
    # argmax partials from the all-rows blocks (96, 192 and 225 rows), and with H % 32 != 0 at 32
    # rows a separate argmax pass after 128 x 128 tiles
    ("rows 96 argmax drafts", CONFIGS[4].scaled(B=12, V=20000, Vt=5000, H=256), 0.0),
    ("rows 192 argmax drafts", CONFIGS[4].scaled(B=24, V=20000, Vt=5000, H=256), 0.0),
    ("rows 225 argmax drafts", CONFIGS[4].scaled(B=75, gamma=2, R=3, V=20000, Vt=5000, H=256), 0.0),
    ("odd H 32 rows argmax drafts", CONFIGS[4].scaled(B=4, V=9001, Vt=1234, H=520), 0.0),
    # argmax partials from the large-batch heads' epilogues: 512 hidden rows on 256 x 256 tiles,
    # 756 on 384 x 256 tiles (two row blocks, ragged Vt), H = 520 on the register-staged tiles
    ("c4 square tiles argmax drafts", CONFIGS[4].scaled(B=64, V=20000, Vt=5000, H=256), 0.0),
    ("c5 tall tiles argmax drafts", CONFIGS[5].scaled(B=84, V=40000, Vt=32001, H=256), 0.0),
    # 2250 rows against 128 head blocks: three waves of tall tiles, ragged rows and head
    ("c5 ragged tall tiles argmax drafts", CONFIGS[5].scaled(B=250, V=34000, Vt=32700, H=128), 0.0),
    ("c4 register-staged tiles argmax drafts", CONFIGS[4].scaled(B=40, V=20000, Vt=5000, H=520), 0.0),
    ("c5 full size argmax drafts, K-tiled head", CONFIGS[5], 0.0),
    ("c5-scaled sampled drafts", CONFIGS[5].scaled(B=32, V=13000, Vt=6001, H=256), 0.8),
    ("c2 full size argmax drafts", CONFIGS[2], 0.0),
    ("c3-scaled argmax drafts, following drafter", CONFIGS[3].scaled(B=4, V=20000, Vt=5000, H=512), 0.0),
    ("c4-scaled argmax drafts, following drafter", CONFIGS[4].scaled(B=24, V=9001, Vt=3000, H=256), 0.0),
    ("c5-scaled sampled drafts, following drafter", CONFIGS[5].scaled(B=32, V=13000, Vt=6001, H=256), 0.8),
])
def test_block_greedy(name, cfg, draft_T):
    """vt_spec_block with target_T = 0: argmax drafts (draft_T = 0) decided on the call's own fp32
    logits, or sampled drafts; the greedy verification is then exact against the oracle.  The
    following drafter (draft argmax mostly the target's) reaches long accepted runs."""
    say(f"fused block, greedy target: {name}")
    wl = make_workload(cfg, follow=0.5 if "following" in name else 0.0)
    logits, dlse, ids, tok, n = _block_greedy(wl, draft_T, tiled="K-tiled" in name)
    B, R, g = wl.B, cfg.R, cfg.gamma
    if draft_T == 0.0:
        want_ids = np.array([ref.argmax_lowest(row) for row in logits]).reshape(B, R)
        assert np.array_equal(ids, want_ids)
        assert np.array_equal(dlse, logits.max(axis=1).astype(np.float64))
    else:
        assert np.all((ids >= 0) & (ids < cfg.Vt))
    t64 = ref.as_f64(wl.target, cfg.target_dtype)
    want_tok, want_n = ref.greedy_verify(t64, ids, wl.keep_ids, g)
    say(f"  mean accepted {want_n.mean():.2f}")
    assert np.array_equal(n, want_n) and np.array_equal(tok, want_tok)
    if "following" in name:
        assert want_n.max() > 0


# Decode-sized greedy blocks (B*R <= 8, both temperatures 0) take the two-launch path: argmax
# partials from the GEMV head launch, then one reduce-and-compare workgroup per sequence.
@pytest.mark.parametrize("name,cfg,b0,follow", [
    ("c3 batch 1, random head", CONFIGS[3].scaled(B=1, V=20000, Vt=5000, H=512), 0, 0.0),
    ("c3 batch 1, following drafter", CONFIGS[3].scaled(B=1, V=20000, Vt=5000, H=512), 1, 0.5),
    ("c4 bf16 batch 1, 8 draft rows, following drafter", CONFIGS[4].scaled(B=1, gamma=7, R=8, V=9001, Vt=3000, H=256),
     2, 0.5),
    ("two sequences, 300000-id vocabulary, following drafter",
     CONFIGS[3].scaled(B=2, gamma=3, R=4, V=300000, Vt=20000, H=256), 0, 0.5),
    ("c2 full size, following drafter", CONFIGS[2], 0, 0.5),
])
def test_block_greedy_small(name, cfg, b0, follow):
    say(f"fused block, greedy, decode-sized: {name}")
    wl = make_workload(cfg, b0=b0, follow=follow)
    logits, dlse, ids, tok, n = _block_greedy(wl, 0.0)
    B, R, g = wl.B, cfg.R, cfg.gamma
    want_ids = np.array([ref.argmax_lowest(row) for row in logits]).reshape(B, R)
    assert np.array_equal(ids, want_ids)
    assert np.array_equal(dlse, logits.max(axis=1).astype(np.float64))
    t64 = ref.as_f64(wl.target, cfg.target_dtype)
    want_tok, want_n = ref.greedy_verify(t64, ids, wl.keep_ids, g)
    say(f"  accepted {want_n.tolist()}")
    assert np.array_equal(n, want_n) and np.array_equal(tok, want_tok)
    if follow > 0:
        assert want_n.max() > 0

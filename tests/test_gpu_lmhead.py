"""GPU parity of vt_lmhead_trimmed against the oracle's float64 LM head (VocabTrim §3 Eq. 1).

Tolerance: |gpu - oracle| <= H * 2^-24 * sum_k |h_k w_k| per logit (the recursive-summation
bound for fp32 accumulation of exact bf16 products) -- the observed error is also reported.
Shapes cover the dot2 GEMV (M <= 8) and the MFMA kernels (M > 8 or large H: all rows in one
block up to 192 rows, or on heads of fewer than 256 blocks of 256 rows in one block up to 256
and two up to 384, 256 x 256 tiles beyond; 128 x 128 and register-staged tiles when H is not a multiple of 32), ragged row and K
tails, trimmed and untrimmed heads."""
import numpy as np
import pytest
import torch

import draft_sampling_verification_amd as vt
from oracle import ref
from tests.gpu_harness import dev, dev_bf16, lmhead_error_bound, say
from workloads import bf16_round

pytestmark = pytest.mark.gpu


def _inputs(M, H, V, Vt, trim, seed):
    rng = np.random.default_rng(seed)
    h = bf16_round(rng.standard_normal((M, H), dtype=np.float32))
    w = bf16_round(rng.standard_normal((V, H), dtype=np.float32) * np.float32(0.02))
    keep = rng.permutation(V)[:Vt].astype(np.int32) if trim else None
    return h, w, keep


def _run(h, w, keep, Vt):
    out = torch.empty(h.shape[0], Vt, dtype=torch.float32, device="cuda")
    vt.vt_lmhead_trimmed(dev_bf16(h), dev_bf16(w), dev(keep) if keep is not None else None, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


CASES = [
    (6, 3072, 5000, 5000, False),   # GEMV, untrimmed head (configs 2/3 row shape)
    (6, 3072, 5000, 1234, True),    # GEMV, trimmed, ragged row count
    (1, 520, 3001, 3001, False),    # GEMV, H with a 16-byte tail past 512
    (8, 1024, 777, 300, True),
    (3, 4096, 2000, 999, True),     # GEMV at H = 4096
    (9, 520, 1000, 513, True),      # MFMA (M > 8), K tail inside a 32-wide step
    (130, 256, 1500, 1300, True),   # MFMA, all rows in one block (160), ragged
    (33, 512, 3001, 2500, True),    # one block of 64 rows, ragged rows and head rows
    (64, 1024, 3000, 3000, False),  # one block of exactly 64 rows, untrimmed
    (96, 256, 2000, 777, True),     # 96 rows
    (192, 512, 1200, 1100, True),   # six row blocks
    (224, 512, 1200, 1100, True),   # seven and eight row blocks: only on 128-column blocks
    (256, 512, 1200, 1100, True),
    (257, 512, 1200, 1100, True),   # one row past them: two all-rows blocks of 160
    (385, 512, 1200, 1100, True),   # past two blocks of 192: 256 x 256 tiles
    (193, 256, 70000, 66000, True), # 256 x 256 tiles past 192 rows when the head has 256+ blocks
    (100, 520, 1000, 700, True),    # H % 32 != 0 at 100 rows: 128 x 128 tiles
    (40, 256, 70000, 66000, True),  # all rows per 256 head rows (258 blocks of 256: one per CU)
    (40, 256, 3000, 64, True),      # a head of 64 rows: one 128-column block, half of it past Vt
    (70, 32, 500, 300, True),       # H = 32: a single K step (the ring re-fetches it)
    (512, 3072, 2000, 1000, True),  # MFMA at config 4's M and H
    (7, 8192, 700, 700, False),     # M * ceil(H/512) too large for registers: MFMA
    (2304, 512, 300, 257, True),    # MFMA at config 5's M
    (256, 520, 900, 512, True),     # 256 x 256 tiles: one row tile, K tail inside a 64-wide step
    (300, 1024, 700, 700, False),   # 256 x 256 tiles, ragged rows and columns, untrimmed
    (512, 3072, 40000, 32768, True),  # config 4's shape on the 256 x 256 tiles
]


@pytest.mark.parametrize("M,H,V,Vt,trim", CASES)
def test_lmhead_parity(M, H, V, Vt, trim):
    say(f"lmhead parity M={M} H={H} V={V} Vt={Vt} trim={trim}")
    h, w, keep = _inputs(M, H, V, Vt, trim, seed=M * 7 + H)
    got = _run(h, w, keep, Vt)
    want = ref.lm_head(h, w, keep)
    bound = lmhead_error_bound(h, w, keep) + np.abs(want) * 2.0 ** -24
    err = np.abs(got - want)
    say(f"  max |err| {err.max():.3e}, max err/bound {(err / bound).max():.3e}")
    assert np.all(err <= bound)


@pytest.mark.parametrize("M,H", [(6, 3072), (200, 1024), (260, 520)])
def test_trimmed_equals_full_gathered_bitwise(M, H):
    # trimmed logits are the untrimmed logits at the kept ids, bit for bit (row-independent order)
    say(f"trimmed == full[:, keep] M={M} H={H}")
    V, Vt = 3000, 1111
    h, w, keep = _inputs(M, H, V, Vt, True, seed=5)
    full = _run(h, w, None, V)
    trim = _run(h, w, keep, Vt)
    assert np.array_equal(trim, full[:, keep])


def test_pre_gathered_head_equals_gather():
    # passing W^Trim itself (keep_ids = NULL) gives the same logits as gathering through keep_ids
    h, w, keep = _inputs(6, 3072, 4000, 1500, True, seed=9)
    a = _run(h, w, keep, 1500)
    b = _run(h, np.ascontiguousarray(w[keep]), None, 1500)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("H,V,Vt,rows", [(1024, 2500, 2100, (9, 40, 96, 130, 192, 193, 256)),
                                        (256, 70000, 66000, (9, 100, 192, 193, 256)),
                                        (520, 2500, 2100, (9, 100, 128, 129, 256))])
def test_mfma_kernels_sum_in_one_order(H, V, Vt, rows):
    # every MFMA kernel sums a logit's products in the same K order, so a hidden row's logits are
    # the same bits whatever the batch's row count selects (H % 32 == 0: all-rows blocks of 32 ..
    # 256 rows per 128 head rows or 32 .. 192 per 256, 256 x 256 tiles; other H: 128 x 128 and register-staged
    # 256 x 256 tiles); only the GEMV (M <= 8) sums differently
    h, w, keep = _inputs(300, H, V, Vt, True, seed=13)
    want = _run(h, w, keep, Vt)
    for M in rows:
        say(f"rows 0..{M - 1} alone against the 300-row call")
        assert np.array_equal(_run(np.ascontiguousarray(h[:M]), w, keep, Vt), want[:M])

"""The stratified grid of tests/test_oracle_grid.py on the GPU: every one of the 8^5 grid points of
a gamma = 2 block (V = 4, three kept ids in rank order, T = 0.5) through the fused call
vt_spec_block (large-batch path: MFMA head, combine, verify) and through the four separate calls,
and a sample of the points through the batch-1 fused path (GEMV head, chunk pass, final pass).
Every grid point must give exactly the oracle's tokens: the oracle places every decision 1/16
away from its uniform, so no decision is settled by rounding.  The oracle's grid frequencies are
themselves equal to the exact block distribution (tests/test_oracle_grid.py).

The drafter's logits come out of the LM head: hidden row (b, i) is the unit vector e_i, so the
head returns column i of the weight, which holds position i's draft logits (bf16; the oracle reads
the same bits)."""
import numpy as np
import pytest
import torch

import draft_sampling_verification_amd as vt
from oracle import ref
from tests.gpu_harness import dev, dev_bf16, say
from tests.test_oracle_grid import GAMMA, KEEP, P_ROWS, Q_FULL, R, T, V, block_inputs, logits_of
from workloads import bf16_round

pytestmark = pytest.mark.gpu

H = 32  # the MFMA head's direct-to-LDS staging needs H % 32 == 0


def grid_case():
    _, target, u_draft, u_acc, u_fin = block_inputs()
    B = u_fin.shape[0]
    weight = np.zeros((V, H), dtype=np.float32)
    for i in range(R):
        weight[:, i] = logits_of(Q_FULL[i])  # -inf at the off-set id 1: never gathered
    weight[1, :] = 0.0
    w_bits = bf16_round(weight)
    hid = np.zeros((B * R, H), dtype=np.float32)
    hid[np.arange(B * R), np.tile(np.arange(R), B)] = 1.0
    h_bits = bf16_round(hid)
    full_to_trim = np.full(V, -1, dtype=np.int32)
    full_to_trim[KEEP] = np.arange(len(KEEP), dtype=np.int32)
    return dict(h=h_bits, w=w_bits, target=target, u_draft=u_draft, u_acc=u_acc, u_fin=u_fin, f2t=full_to_trim, B=B)


@pytest.fixture(scope="module")
def case():
    c = grid_case()
    c["orc"] = ref.block(c["h"], c["w"], KEEP, None, c["target"], "f32", np.float32(T), c["u_draft"], c["u_acc"],
                         c["u_fin"], GAMMA, R)
    assert np.all(c["orc"]["final_margin"] > 1e-3) and np.all(c["orc"]["draft_margins"] > 1e-3)
    return c


def fused(c, rows):
    B = len(rows)
    sel = np.asarray(rows)
    hrows = (sel[:, None] * R + np.arange(R)[None, :]).reshape(-1)
    logits = torch.empty(B * R, len(KEEP), dtype=torch.float32, device="cuda")
    dlse = torch.empty(B * R, dtype=torch.float64, device="cuda")
    dids = torch.empty(B * R, dtype=torch.int32, device="cuda")
    tlse = torch.empty(B * (GAMMA + 1), dtype=torch.float64, device="cuda")
    tok = torch.full((B, GAMMA + 1), -9, dtype=torch.int32, device="cuda")
    nacc = torch.full((B,), -9, dtype=torch.int32, device="cuda")
    vt.vt_spec_block(dev_bf16(c["h"][hrows]), dev_bf16(c["w"]), dev(KEEP), dev(c["f2t"]), dev(c["target"][sel]),
                     float(np.float32(T)), float(np.float32(T)), dev(c["u_draft"][sel].reshape(-1)),
                     dev(c["u_acc"][sel]), dev(c["u_fin"][sel]), logits, dlse, dids, tlse, tok, nacc)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), nacc.cpu().numpy(), dids.cpu().numpy().reshape(B, R)


def check(c, tok, n, ids, rows):
    orc = c["orc"]
    assert np.array_equal(ids, orc["draft_ids"][rows])
    assert np.array_equal(n, orc["n"][rows])
    assert np.array_equal(tok, orc["tokens"][rows])


def test_grid_fused_large_batch(case):
    say(f"grid of {case['B']} points through vt_spec_block (large-batch path)")
    rows = np.arange(case["B"])
    tok, n, ids = fused(case, rows)
    check(case, tok, n, ids, rows)


def test_grid_separate_calls(case):
    say(f"grid of {case['B']} points through the four separate calls")
    c, B = case, case["B"]
    logits = torch.empty(B * R, len(KEEP), dtype=torch.float32, device="cuda")
    vt.vt_lmhead_trimmed(dev_bf16(c["h"]), dev_bf16(c["w"]), dev(KEEP), logits)
    dlse = torch.empty(B * R, dtype=torch.float64, device="cuda")
    dids = torch.empty(B * R, dtype=torch.int32, device="cuda")
    Tf = float(np.float32(T))
    vt.vt_softmax_temp(logits, Tf, dlse, None, dev(c["u_draft"].reshape(-1)), dids)
    target = dev(c["target"])
    tlse = torch.empty(B * (GAMMA + 1), dtype=torch.float64, device="cuda")
    vt.vt_softmax_temp(target.view(-1, V), Tf, tlse)
    tok = torch.full((B, GAMMA + 1), -9, dtype=torch.int32, device="cuda")
    nacc = torch.full((B,), -9, dtype=torch.int32, device="cuda")
    vt.vt_spec_verify(target, tlse, Tf, logits.view(B, R, len(KEEP)), dlse, Tf, dids.view(B, R), dev(KEEP),
                      dev(c["f2t"]), dev(c["u_acc"]), dev(c["u_fin"]), tok, nacc)
    torch.cuda.synchronize()
    check(c, tok.cpu().numpy(), nacc.cpu().numpy(), dids.cpu().numpy().reshape(B, R), np.arange(B))


def test_grid_batch_one_fused_path(case):
    """Batch 1 (three rows of the head: the GEMV head with the softmax partials, the chunk pass,
    the final pass), one grid point per call, 256 points spread over the grid."""
    rng = np.random.default_rng(11)
    pts = rng.choice(case["B"], size=256, replace=False)
    say("256 grid points through vt_spec_block at batch 1")
    for b in pts:
        tok, n, ids = fused(case, [b])
        check(case, tok, n, ids, [b])

"""The generation loop on the GPU (vt_spec_generate_markov) with the rejection-rule article's own
toy, rebuilt from the corpus it prints ("A target and a draft small enough to print in full"):
parity with the oracle's chained blocks on sampled sequences, and the measured acceptance and
tokens per target call against the values the article reports at gamma = 4 ("What draft accuracy
buys, measured in tokens per call"; tests/golden/rr_toy.json), within the tolerances it states
(0.004 for acceptance, 0.01 for tokens per call)."""
import json
import os

import numpy as np
import pytest
import torch

import draft_sampling_verification_amd as vt
from oracle import ref, stats
from tests.gpu_harness import BAND, dev, say
from workloads import article_toy, counter_uniforms

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def page():
    with open(os.path.join(HERE, "golden", "rr_toy.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("w", [0.0, 0.9])
def test_article_toy_generation(w):
    m, tol, g = page()["measured"], page()["tolerance"], page()["gamma"]
    t = article_toy(w)
    B, L = 2048, 2048  # long chains: the start context weighs 1/700 of the blocks
    u = counter_uniforms(1, 80 + int(10 * w), B, L * (2 * g + 1)).reshape(B, L, 2 * g + 1)
    tok = torch.full((B, L), -7, dtype=torch.int32, device="cuda")
    st = torch.full((B, 4), -7, dtype=torch.int32, device="cuda")
    say(f"article toy w={w}: {B} sequences x {L} tokens")
    vt.vt_spec_generate_markov(dev(t.target_logits), dev(t.draft_logits), 1.0, 1.0, g, dev(u), tok, st)
    torch.cuda.synchronize()
    tok, st = tok.cpu().numpy(), st.cpu().numpy()
    assert np.all((tok >= 0) & (tok < 18))
    # parity with the oracle on sampled sequences (exact, up to the first decision in the band)
    rows = [0, 1, 2, 3, 777, 1500, B - 1]
    orc = ref.toy_generate(t.target_logits, t.draft_logits, 1.0, 1.0, g, L, u[rows], band=BAND)
    full = 0
    for k, b in enumerate(rows):
        cut = orc["tie_token"][k]
        assert np.array_equal(tok[b, :cut], orc["tokens"][k, :cut]), (b, cut)
        if orc["tie_block"][k] == L:
            assert np.array_equal(tok[b], orc["tokens"][k])
            assert st[b].tolist() == [orc["blocks"][k], orc["tests"][k], orc["accepted"][k], orc["emitted"][k]]
            full += 1
    assert full >= len(rows) - 1
    a_exact = stats.alpha_toy(t.target_logits, t.draft_logits, 1.0, 1.0)
    a_hat = st[:, 2].sum() / st[:, 1].sum()
    tau = st[:, 3].sum() / st[:, 0].sum()
    say(f"  measured acceptance {a_hat:.5f} (exact alpha {a_exact:.5f}), tokens per call {tau:.4f}")
    assert abs(a_hat - a_exact) <= tol["acceptance"]
    if w == 0.0:
        assert abs(a_hat - m["acceptance_w0"]) <= tol["acceptance"]
        assert abs(tau - m["tokens_per_call_w0"]) <= tol["tokens_per_call"]
    else:
        assert abs(tau - m["tokens_per_call_w0.9"]) <= tol["tokens_per_call"]

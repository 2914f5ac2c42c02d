"""The rejection-rule article's own toy, rebuilt from the corpus it prints, pins the oracle's
acceptance statistics and generation loop to the numbers the article measured
(tests/golden/rr_toy.json: "A target and a draft small enough to print in full", "What draft
accuracy buys, measured in tokens per call", "Acceptance rate has to beat cost").

The page's values are Monte-Carlo measurements over 200000 generated tokens; the page states that
its measured acceptance stays within 0.004 of the exact value and its tokens per step within 0.01
of the closed form, so those are the tolerances here."""
import json
import os

import numpy as np
import pytest

from oracle import ref, stats
from workloads import article_toy, article_toy_counts, counter_uniforms

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def page():
    with open(os.path.join(HERE, "golden", "rr_toy.json")) as f:
        return json.load(f)


def alpha(w):
    t = article_toy(w)
    return stats.alpha_toy(t.target_logits, t.draft_logits, 1.0, 1.0)


def test_corpus_and_vocabulary(page):
    """An 80-character corpus whose next-character distributions are tables of eighteen numbers."""
    vocab, bigram, unigram = article_toy_counts()
    assert len(page["corpus"]) == 80 and len(vocab) == page["vocabulary_size"] == 18
    assert vocab == "".join(sorted(vocab)) and vocab[0] == " "
    # Laplace smoothing: one pseudo-count per pair, then one count per transition (80 of them,
    # the first from the start context)
    assert bigram.min() >= 1 and bigram.sum() == 19 * 18 + 80 and bigram[0].sum() == 18 + 1
    assert unigram.sum() == 18 + 80
    t = article_toy(0.3)
    for tab in (t.target_logits, t.draft_logits):
        assert np.all(np.isfinite(tab))
        assert np.allclose(np.exp(tab.astype(np.float64)).sum(axis=1), 1.0, atol=1e-6)


def test_alpha_and_tokens_per_call_match_the_page(page):
    m, tol = page["measured"], page["tolerance"]
    g = page["gamma"]
    a0, a9 = alpha(0.0), alpha(0.9)
    assert abs(a0 - m["acceptance_w0"]) <= tol["acceptance"], a0
    assert abs(stats.expected_tokens(a0, g) - m["tokens_per_call_w0"]) <= tol["tokens_per_call"]
    assert abs(stats.expected_tokens(a9, g) - m["tokens_per_call_w0.9"]) <= tol["tokens_per_call"]
    # at w = 1 the draft is the target: every token survives and a call yields gamma + 1 tokens
    assert alpha(1.0) == pytest.approx(1.0, abs=1e-6)
    assert stats.expected_tokens(alpha(1.0), g) == pytest.approx(m["tokens_per_call_w1"], abs=1e-5)
    # acceptance rises with the draft weight
    assert a0 < alpha(0.3) < alpha(0.6) < a9 < 1.0


def test_walltime_projections_match_the_page(page):
    m, g = page["measured"], page["gamma"]
    for w, key in ((0.0, "w0"), (0.9, "w0.9")):
        e = stats.expected_tokens(alpha(w), g)
        for c in (0.1, 0.25):
            assert abs(stats.walltime_improvement(e, g, c) - m[f"speedup_{key}_c{c}"]) < 0.01, (w, c)


@pytest.mark.slow
@pytest.mark.parametrize("w", [0.0, 0.9])
def test_generation_loop_measures_the_page_values(page, w):
    """The oracle's generation loop on the page's tables, 600000 tokens: measured acceptance within
    0.004 of the page's 72.6% (w = 0) and of the exact alpha; tokens per block within 0.01 of the
    page's 2.92 / 4.7336."""
    m, tol, g = page["measured"], page["tolerance"], page["gamma"]
    t = article_toy(w)
    L, B = 2000, 300
    u = counter_uniforms(1, 77, B, L * (2 * g + 1)).reshape(B, L, 2 * g + 1)
    r = ref.toy_generate(t.target_logits, t.draft_logits, 1.0, 1.0, g, L, u)
    a_hat = r["accepted"].sum() / r["tests"].sum()
    tau = r["emitted"].sum() / r["blocks"].sum()
    assert abs(a_hat - alpha(w)) <= tol["acceptance"], (a_hat, alpha(w))
    want = m["tokens_per_call_w0"] if w == 0.0 else m["tokens_per_call_w0.9"]
    assert abs(tau - want) <= tol["tokens_per_call"], (tau, want)
    if w == 0.0:
        assert abs(a_hat - m["acceptance_w0"]) <= tol["acceptance"]

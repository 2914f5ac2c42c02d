"""Pins of the chained generation loop (oracle.ref.toy_generate) and of the closed-form
acceptance statistics (oracle.stats): closed forms, the page's printed projections, an
independent autoregressive sampler for the always-reject case, and Monte Carlo against the exact
target joint and against alpha / E[#tokens]."""
import math

import numpy as np
import pytest

from oracle import ref, stats
from workloads import CONFIGS, counter_uniforms, toy_tables


def uniforms(B, L, gamma, stream=12):
    return counter_uniforms(1, stream, B, L * (2 * gamma + 1)).reshape(B, L, 2 * gamma + 1)


def test_stationary_two_state_closed_form():
    a, b = 0.3, 0.05
    P = np.array([[1 - a, a], [b, 1 - b]])
    pi = stats.stationary(P)
    assert np.allclose(pi, [b / (a + b), a / (a + b)], atol=1e-12)


def test_stationary_of_the_toy_is_invariant():
    t = toy_tables(CONFIGS[1], 0.5)
    P = stats.transition_matrix(t.target_logits, 1.0)
    pi = stats.stationary(P)
    assert abs(pi.sum() - 1) < 1e-12 and np.all(pi > 0)
    assert np.abs(pi @ P - pi).max() < 1e-14


def test_expected_tokens_closed_form():
    assert stats.expected_tokens(0.0, 4) == 1.0
    assert stats.expected_tokens(1.0, 4) == 5.0
    for al in (0.2, 0.726, 0.95):
        assert math.isclose(stats.expected_tokens(al, 4), sum(al ** k for k in range(5)), rel_tol=1e-12)
    assert round(stats.expected_tokens(0.726, 4), 3) == 2.914  # the page's w = 0 figure, 2.92 per call


def test_walltime_projection_matches_printed_values():
    # [RR] "Acceptance rate has to beat cost": 4.7336 tokens per call at gamma = 4 projects to
    # 3.381x at c = 0.1 and 2.367x at c = 0.25; 2.912 tokens give 2.080x and 1.456x
    assert round(stats.walltime_improvement(4.7336, 4, 0.1), 3) == 3.381
    assert round(stats.walltime_improvement(4.7336, 4, 0.25), 3) == 2.367
    assert round(stats.walltime_improvement(2.912, 4, 0.1), 3) == 2.080
    assert round(stats.walltime_improvement(2.912, 4, 0.25), 3) == 1.456


def test_beta_extremes():
    p = np.array([0.2, 0.3, 0.5, 0.0])
    assert stats.beta(p, p) == pytest.approx(1.0)
    assert stats.beta(p, np.array([0, 0, 0, 1.0])) == 0.0
    t = toy_tables(CONFIGS[1], 1.0)
    assert stats.alpha_toy(t.target_logits, t.draft_logits, 1.0, 1.0) == pytest.approx(1.0, abs=1e-6)


def test_draft_equal_to_target_accepts_everything():
    t = toy_tables(CONFIGS[1], 0.5)
    g, L, B = 4, 23, 6
    r = ref.toy_generate(t.target_logits, t.target_logits, 1.0, 1.0, g, L, uniforms(B, L, g))
    blocks = math.ceil(L / (g + 1))
    assert np.all(r["blocks"] == blocks)
    assert np.all(r["tests"] == g * blocks) and np.all(r["accepted"] == g * blocks)
    assert np.all(r["emitted"] == (g + 1) * blocks)
    assert np.all((r["tokens"] >= 0) & (r["tokens"] < 18))


def test_deterministic_cycle_follows_the_contexts():
    # p(.|previous = a) and q(.|previous = a) put all mass on (a + 1) mod V, and the start row on
    # token 0: every draft survives and the output is 0, 1, 2, ... whatever the uniforms
    V, g, L, B = 7, 3, 25, 3
    tab = np.full((V + 1, V), -np.inf, dtype=np.float32)
    tab[0, 0] = 0.0
    for a in range(V):
        tab[a + 1, (a + 1) % V] = 0.0
    r = ref.toy_generate(tab, tab, 1.0, 1.0, g, L, uniforms(B, L, g, stream=16))
    assert np.all(r["tokens"] == np.arange(L) % V)
    assert np.all(r["accepted"] == g * r["blocks"])


def test_disjoint_draft_is_the_autoregressive_sampler():
    # the draft only proposes tokens the target never emits: every block rejects its first draft
    # and draws from p(.|context) with the block's final uniform, so the chain must reproduce a
    # plain token-by-token sampler fed the same uniforms
    rng = np.random.default_rng(5)
    V, g, L, B = 10, 3, 30, 8
    tt = rng.standard_normal((V + 1, V)).astype(np.float32)
    dt = rng.standard_normal((V + 1, V)).astype(np.float32)
    tt[:, V // 2:] = -np.inf
    dt[:, : V // 2] = -np.inf
    u = uniforms(B, L, g, stream=13)
    r = ref.toy_generate(tt, dt, 0.8, 1.3, g, L, u)
    assert np.all(r["blocks"] == L) and np.all(r["tests"] == L) and np.all(r["accepted"] == 0)
    _, P = ref.softmax_temp(tt.astype(np.float64), 0.8)
    for b in range(B):
        prev = 0
        for j in range(L):
            w = P[prev]
            C = np.cumsum(w)
            tok = int(np.nonzero(float(u[b, j, 2 * g]) * C[-1] <= C)[0][0])
            assert r["tokens"][b, j] == tok
            prev = tok + 1


@pytest.mark.slow
def test_two_token_joint_matches_the_target():
    # [RR]: two tokens from the start context, gamma = 2, w = 0.3, 200000 runs; the page reports a
    # total-variation distance of 0.01523 over the 324 pairs for its tables
    t = toy_tables(CONFIGS[1], 0.3)
    g, B = 2, 200_000
    r = ref.toy_generate(t.target_logits, t.draft_logits, 1.0, 1.0, g, 2, uniforms(B, 2, g, stream=14))
    _, P = ref.softmax_temp(t.target_logits.astype(np.float64), 1.0)
    emp = np.zeros((18, 18))
    np.add.at(emp, (r["tokens"][:, 0], r["tokens"][:, 1]), 1.0 / B)
    exact_joint = P[0][:, None] * P[1:]
    tv = 0.5 * np.abs(emp - exact_joint).sum()
    assert tv < 0.03, tv


@pytest.mark.slow
@pytest.mark.parametrize("w", [0.0, 0.5, 0.9])
def test_measured_acceptance_matches_alpha(w):
    # [RR] "What draft accuracy buys": the measured acceptance tracks alpha within 0.004 and
    # tokens per block track (1 - alpha^(gamma+1)) / (1 - alpha) within 0.01 (600000 tokens here,
    # so that 0.01 is over three standard errors of the tokens-per-block mean)
    t = toy_tables(CONFIGS[1], w)
    g, L, B = 4, 2000, 300
    r = ref.toy_generate(t.target_logits, t.draft_logits, 1.0, 1.0, g, L, uniforms(B, L, g, stream=15))
    a = stats.alpha_toy(t.target_logits, t.draft_logits, 1.0, 1.0)
    a_hat = r["accepted"].sum() / r["tests"].sum()
    tau = r["emitted"].sum() / r["blocks"].sum()
    assert abs(a_hat - a) < 0.004, (a_hat, a)
    assert abs(tau - stats.expected_tokens(a, g)) < 0.01, (tau, stats.expected_tokens(a, g))

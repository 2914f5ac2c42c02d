"""Pins for the greedy verification oracle: hand-worked cases, the tie rule, agreement with the
sampling rule on one-hot targets (where the two must coincide for any uniforms), and the
temperature -> 0 limit of the sampling rule on well-separated logits."""
import numpy as np
import pytest

from oracle import ref


def test_greedy_hand_cases():
    # V = 4, gamma = 3; target argmaxes per position: 2, 0, 3, 1
    t = np.full((1, 4, 4), -1.0)
    for i, a in enumerate([2, 0, 3, 1]):
        t[0, i, a] = 5.0
    cases = {(2, 0, 3): ([2, 0, 3, 1], 3), (2, 1, 3): ([2, 0, -1, -1], 1), (1, 0, 3): ([2, -1, -1, -1], 0),
             (2, 0, 0): ([2, 0, 3, -1], 2)}
    for drafts, (want_tok, want_n) in cases.items():
        tok, n = ref.greedy_verify(t, np.array([drafts]), None, 3)
        assert tok[0].tolist() == want_tok and n[0] == want_n


def test_greedy_ties_go_to_lowest_id_and_remap():
    t = np.array([[[1.0, 3.0, 3.0, 0.0], [2.0, 2.0, 2.0, 2.0]]])
    keep = np.array([2, 1, 3], dtype=np.int32)  # trimmed id 1 -> full id 1, 0 -> 2
    tok, n = ref.greedy_verify(t, np.array([[1]]), keep, 1)   # draft full id 1 = lowest argmax
    assert n[0] == 1 and tok[0].tolist() == [1, 0]            # bonus: all tie -> id 0
    tok, n = ref.greedy_verify(t, np.array([[0]]), keep, 1)   # draft full id 2: tied but not lowest
    assert n[0] == 0 and tok[0].tolist() == [1, -1]


@pytest.mark.parametrize("seed", range(10))
def test_greedy_equals_sampling_rule_on_one_hot_targets(seed):
    rng = np.random.default_rng(seed)
    V, g = 7, 4
    argmax = rng.integers(0, V, size=g + 1)
    p = np.zeros((g + 1, V))
    p[np.arange(g + 1), argmax] = 1.0
    logits = np.where(p > 0, 0.0, -np.inf)[None]
    q = rng.dirichlet(np.ones(V), size=g)
    drafts = np.where(rng.random(g) < 0.7, argmax[:g], rng.integers(0, V, size=g))
    tok_g, n_g = ref.greedy_verify(logits, drafts[None], None, g)
    for _ in range(20):
        u = 1.0 - rng.random(g + 1)
        tok_s, n_s, _, _ = ref.verify_sequence(p, q, drafts, None, u[:g], u[g], g)
        assert n_s == n_g[0] and np.array_equal(tok_s, tok_g[0])


def test_greedy_is_the_low_temperature_limit_of_sampling():
    # as T -> 0 both distributions become one-hot at their argmax; the draft's own draw is then its
    # argmax and the sampling rule reduces to greedy matching (any uniforms in (0, 1))
    rng = np.random.default_rng(3)
    B, g, V = 20, 3, 50
    t = rng.normal(size=(B, g + 1, V)) * 3
    d = rng.normal(size=(B, g, V)) * 3
    d[:10] = t[:10, :g]                        # half the sequences' drafters agree with the target
    ids = d.argmax(axis=2)                     # the drafter's T -> 0 draws
    tok_g, n_g = ref.greedy_verify(t, ids, None, g)
    T = 1e-3                                   # gaps between the top logits are >> T here
    out = ref.verify(t, T, d, T, ids, None, np.full((B, g), 0.5), np.full(B, 0.5), g)
    assert np.array_equal(out["n"], n_g) and np.array_equal(out["tokens"], tok_g)
    assert (n_g[:10] == g).all() and (n_g[10:] < g).any()

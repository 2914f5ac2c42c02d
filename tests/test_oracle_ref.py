"""Pins for the float64 oracle run with explicit uniforms: the worked example on an exact grid
of uniforms, the naive-redraw negative control, Monte-Carlo agreement with the exact
enumerator, the special cases, the toy workload's Monte-Carlo p-match and the VocabTrim-aligned
variant's closed-form acceptance."""
import math
from fractions import Fraction as F

import numpy as np
import pytest

from oracle import exact, ref
from workloads import CONFIGS, make_workload


def _mid(G):
    return [(k + 0.5) / G for k in range(G)]


def test_worked_example_grid():
    # glossary two-token example: A 0.6 / B 0.4 target, 0.8 / 0.2 draft, gamma = 1
    p_rows = np.array([[0.6, 0.4], [0.6, 0.4]])
    q_rows = np.array([[0.8, 0.2]])
    G = 40
    acc_a = acc_b = rej = 0
    for ud in _mid(G):
        x, _ = ref.draw(q_rows[0], ud)
        for ua in _mid(G):
            tok, n, _, _ = ref.verify_sequence(p_rows, q_rows, [x], None, [ua], 0.5, 1)
            if n == 1:
                acc_a += tok[0] == 0
                acc_b += tok[0] == 1
                continue
            rej += 1
            for uf in _mid(G):
                tok, n, _, _ = ref.verify_sequence(p_rows, q_rows, [x], None, [ua], uf, 1)
                assert n == 0 and tok[0] == 1 and tok[1] == -1, "the residual must always return B"
    assert (acc_a, acc_b, rej) == (960, 320, 320)
    assert F(acc_a, G * G) == F(3, 5)
    assert F(acc_b + rej, G * G) == F(2, 5)


def test_worked_example_naive_grid_gives_072():
    p_rows = np.array([[0.6, 0.4], [0.6, 0.4]])
    q_rows = np.array([[0.8, 0.2]])
    G = 40
    a = 0
    for ud in _mid(G):
        x, _ = ref.draw(q_rows[0], ud)
        for ua in _mid(G):
            for uf in _mid(G):
                tok, *_ = ref.verify_sequence(p_rows, q_rows, [x], None, [ua], uf, 1, correction="naive")
                a += tok[0] == 0
    assert F(a, G ** 3) == F(18, 25)


def _rows_from_fracs(rows):
    return np.array([[float(x) for x in r] for r in rows])


@pytest.mark.parametrize("seed,gamma,V", [(0, 1, 3), (1, 2, 3), (2, 2, 4), (3, 3, 2)])
def test_monte_carlo_matches_exact_block_distribution(seed, gamma, V):
    rng = np.random.default_rng(seed)
    ps = [tuple(F(int(x), 100) for x in _split(rng, V)) for _ in range(gamma + 1)]
    qs = [tuple(F(int(x), 100) for x in _split(rng, V)) for _ in range(gamma)]
    want = exact.block_distribution(lambda c: ps[len(c)], lambda c: qs[len(c)], gamma)
    p_rows, q_rows = _rows_from_fracs(ps), _rows_from_fracs(qs)
    N = 40000
    u = 1.0 - rng.random((N, 2 * gamma + 1))  # (0, 1]
    counts = {}
    for t in range(N):
        ids = [ref.draw(q_rows[i], u[t, i])[0] for i in range(gamma)]
        tok, n, _, _ = ref.verify_sequence(p_rows, q_rows, ids, None, u[t, gamma:2 * gamma], u[t, -1], gamma)
        key = tuple(int(x) for x in tok[: n + 1])
        counts[key] = counts.get(key, 0) + 1
    assert set(counts) <= set(want)
    for key, pr in want.items():
        pr = float(pr)
        sig = math.sqrt(pr * (1 - pr) / N)
        assert abs(counts.get(key, 0) / N - pr) <= 4.5 * sig + 1e-12, key


def _split(rng, V):
    """V positive integer weights summing to 100."""
    cuts = np.sort(rng.choice(np.arange(1, 100), size=V - 1, replace=False))
    return np.diff(np.concatenate([[0], cuts, [100]]))


def test_identical_rows_accept_all_and_bonus_from_last():
    rng = np.random.default_rng(3)
    p_rows = rng.dirichlet(np.ones(6), size=4)
    for t in range(200):
        u = 1.0 - rng.random(7)
        ids = [ref.draw(p_rows[i], u[i])[0] for i in range(3)]
        tok, n, _, _ = ref.verify_sequence(p_rows, p_rows[:3], ids, None, u[3:6], u[6], 3)
        assert n == 3
        assert tok[3] == ref.draw(p_rows[3], u[6])[0]
        assert list(tok[:3]) == ids


def test_disjoint_supports_final_is_target_draw():
    p = np.array([[0.0, 0.25, 0.75, 0.0]] * 3)
    q = np.array([[0.5, 0.0, 0.0, 0.5]] * 2)
    for uf in _mid(16):
        tok, n, _, _ = ref.verify_sequence(p, q, [0, 3], None, [1e-7, 1e-7], uf, 2)
        assert n == 0 and tok[0] == ref.draw(p[0], uf)[0] and list(tok[1:]) == [-1, -1]


def test_one_hot_target_is_greedy():
    # one-hot p (the greedy limit): accept iff the draft equals the argmax; the final is the argmax
    argmax = [2, 0, 1, 3]
    p = np.eye(4)[argmax]
    q = np.full((3, 4), 0.25)
    for drafts in [(2, 0, 1), (2, 1, 1), (0, 0, 0), (2, 0, 3)]:
        tok, n, _, _ = ref.verify_sequence(p, q, list(drafts), None, [1.0, 1.0, 1.0], 0.5, 3)
        want_n = next((i for i in range(3) if drafts[i] != argmax[i]), 3)
        assert n == want_n and tok[n] == argmax[n]


def test_identity_keep_ids_equals_full_head():
    rng = np.random.default_rng(4)
    p = rng.dirichlet(np.ones(9), size=3)
    q = rng.dirichlet(np.ones(9), size=2)
    keep = np.arange(9, dtype=np.int32)
    for t in range(100):
        u = 1.0 - rng.random(5)
        ids = [ref.draw(q[i], u[i])[0] for i in range(2)]
        a = ref.verify_sequence(p, q, ids, None, u[2:4], u[4], 2)
        b = ref.verify_sequence(p, q, ids, keep, u[2:4], u[4], 2)
        assert np.array_equal(a[0], b[0]) and a[1] == b[1]


def test_trimmed_remap_and_zero_draft_mass_off_set():
    # kept set {5, 1, 7} in rank order: trimmed id 0 -> 5, 1 -> 1, 2 -> 7
    keep = np.array([5, 1, 7], dtype=np.int32)
    p = np.full((2, 8), 1 / 8)
    q = np.array([[0.2, 0.3, 0.5]])
    tok, n, _, _ = ref.verify_sequence(p, q, [2], keep, [1e-7], 0.5, 1)
    assert n == 1 and tok[0] == 7  # accepted draft is reported as its full id
    # a rejected draft of trimmed id 2 (full 7): residual is p - q with q = 0 off the kept set
    tok, n, _, _ = ref.verify_sequence(p, q, [2], keep, [1.0], 2.0 ** -24, 1)
    assert n == 0 and tok[0] == 0  # first full id with positive residual is 0 (not kept)
    w = np.maximum(p[0] - np.array([0, .3, 0, 0, 0, .2, 0, .5]), 0)
    for uf in _mid(50):
        assert ref.verify_sequence(p, q, [2], keep, [1.0], uf, 1)[0][0] == ref.draw(w, uf)[0]


@pytest.mark.slow
def test_toy_monte_carlo_first_token_matches_target():
    """Config 1 at 1e5 trials: the first emitted token follows p(. | start) within 3 sigma per
    token, and the first draft's acceptance rate matches beta = sum min(p, q) (z < 3)."""
    cfg = CONFIGS[1]
    N = 100_000
    wl = make_workload(cfg, B=N)
    out = ref.toy_block(wl.toy.target_logits, wl.toy.draft_logits, wl.T, cfg.gamma,
                        wl.u_draft, wl.u_acc, wl.u_fin)
    _, P = ref.softmax_temp(wl.toy.target_logits.astype(np.float64), 1.0)
    _, Q = ref.softmax_temp(wl.toy.draft_logits.astype(np.float64), 1.0)
    freq = np.bincount(out["tokens"][:, 0], minlength=cfg.V) / N
    sig = np.sqrt(P[0] * (1 - P[0]) / N)
    assert np.all(np.abs(freq - P[0]) < 3 * sig), np.abs(freq - P[0]) / sig
    beta = np.minimum(P[0], Q[0]).sum()
    acc = (out["n"] >= 1).mean()
    assert abs(acc - beta) / math.sqrt(beta * (1 - beta) / N) < 3


def test_aligned_variant_properties_scaled():
    """Draft logits = target logits at the kept ids (same T): acceptance probability at a
    position is p(kept) and every residual token lies off the kept set."""
    cfg = CONFIGS[4].scaled(B=48, V=3000, Vt=700, gamma=3)
    wl = make_workload(cfg, aligned=True)
    out = ref.block(None, None, wl.keep_ids, wl.draft_logits, wl.target, cfg.target_dtype, wl.T,
                    wl.u_draft, wl.u_acc, wl.u_fin, cfg.gamma, cfg.R)
    kept = np.zeros(cfg.V, bool)
    kept[wl.keep_ids] = True
    for b in range(cfg.B):
        n = out["n"][b]
        toks = out["tokens"][b]
        assert all(kept[t] for t in toks[:n])
        if n < cfg.gamma:
            assert not kept[toks[n]]
    # every test performed has ratio p_i(kept set) exactly (q >= p on the kept set)
    _, p = ref.softmax_temp(ref.as_f64(wl.target, cfg.target_dtype), wl.T)
    pk = p[:, :, wl.keep_ids].sum(axis=2)
    for b in range(cfg.B):
        for i, r in enumerate(out["accept_ratios"][b]):
            assert math.isclose(r, pk[b, i], rel_tol=1e-12)
    assert out["n"].mean() > 0.0


def test_block_shapes_and_remap_scaled():
    cfg = CONFIGS[3].scaled(V=2000, Vt=300, H=64)
    wl = make_workload(cfg)
    out = ref.block(wl.hidden, wl.weight, wl.keep_ids, None, wl.target, cfg.target_dtype, wl.T,
                    wl.u_draft, wl.u_acc, wl.u_fin, cfg.gamma, cfg.R)
    assert out["draft_logits"].shape == (cfg.M, cfg.Vt)
    assert out["tokens"].shape == (cfg.B, cfg.gamma + 1)
    n = out["n"][0]
    assert list(out["tokens"][0, :n]) == [int(wl.keep_ids[z]) for z in out["draft_ids"][0, :n]]
    assert np.all(out["tokens"][0, n + 1:] == -1)


def test_zero_residual_falls_back_to_p():
    """Reading R5: after a rejection the residual max(0, p_n - q_n) has positive mass in exact
    arithmetic ("Speculative decoding" glossary, "Why a rejection needs a special draw": it is a
    real distribution once normalised), but rounding can leave q_n >= p_n at every id.  Then the
    final token is drawn from p_n itself.  Here q_n = p_n except at id 0, where q_n is larger, so
    draft 0 is rejected with ratio 2/3 when u = 1 and the residual is zero everywhere; the draw
    must follow p_n's running sum (0.1, 0.3, 0.6, 1.0), not q_n's (0.15, 0.35, 0.65, 1.05)/1.05."""
    p = np.array([[0.1, 0.2, 0.3, 0.4], [0.25, 0.25, 0.25, 0.25]])
    q = np.array([[0.15, 0.2, 0.3, 0.4]])
    for uf, want in [(0.05, 0), (0.12, 1), (0.29, 1), (0.45, 2), (0.62, 3), (0.8, 3), (1.0, 3)]:
        tok, n, ratios, _ = ref.verify_sequence(p, q, [0], None, [1.0], uf, 1)
        assert n == 0 and abs(ratios[0] - 2 / 3) < 1e-15
        assert tok[0] == want and tok[1] == -1, (uf, tok)
    # a ratio of exactly 1 (p = q at the drafted id) always accepts, even at u = 1
    tok, n, ratios, _ = ref.verify_sequence(p, q, [2], None, [1.0], 0.5, 1)
    assert n == 1 and ratios[0] == 1.0 and tok[0] == 2

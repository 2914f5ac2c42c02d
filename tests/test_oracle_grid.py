"""Pins of the oracle's whole-block compositions (ref.block, ref.draft_draws, ref.toy_block) against
the exact output distribution of a block (oracle/exact.py, fractions), over a stratified grid of
every uniform the block consumes.

Every probability in the tables below (draft rows, target rows, accept ratios min(1, p/q), the
normalised residual max(0, p - q) / (1 - beta), and every running sum of them) is a multiple of
1/8.  On a grid of 8 midpoints (k + 1/2) / 8 per uniform, an inverse-CDF draw or an accept test
then selects each outcome on exactly 8 x (its probability) of the points, and since every step of
a block reads its own uniform, the number of grid points on which a block emits a token tuple is
exactly 8^(2 gamma + 1) times the tuple's probability.  So the grid frequencies of the oracle must
EQUAL the exact block distribution, fraction for fraction; no tolerance is involved.

Pages: "Speculative decoding" glossary, "Why a rejection needs a special draw" (residual draw);
"A rejection rule keeps speculative decoding's output exact", "Extending the rule from one token
to a drafted run" (draft gamma tokens, verify left to right, bonus after full acceptance);
"VocabTrim" §3 (the trimmed drafter puts no mass off the kept set) and Appendix C.1,
Algorithm 2 (drafts in the trimmed id space, mapped back to full ids).
"""
from __future__ import annotations

import itertools
from collections import Counter
from fractions import Fraction as F

import numpy as np
import pytest

from oracle import exact, ref

G = 8  # grid points per uniform
T = 0.5  # a temperature far enough from 1 that a softmax formed at the wrong temperature moves a
#          draft boundary across a grid point


def midpoints():
    return (np.arange(G, dtype=np.float64) + 0.5) / G


def logits_of(probs, temperature=T):
    """float32 logits whose temperature softmax is `probs` (up to fp32 rounding of the logits)."""
    p = np.asarray([float(x) for x in probs], dtype=np.float64)
    with np.errstate(divide="ignore"):
        return (temperature * np.log(p)).astype(np.float32)


# ------------------------------------------------------------------ rows that do not depend on the drafts
# V = 4 full ids, kept set {2, 0, 3} stored in that (rank) order, id 1 off the kept set.
KEEP = np.array([2, 0, 3], dtype=np.int32)
V = 4
GAMMA = 2
R = GAMMA + 1
# draft rows over the full ids (0 off the kept set); row 2 is drawn but never verified
Q_FULL = [
    [F(1, 4), F(0), F(1, 2), F(1, 4)],
    [F(1, 2), F(0), F(1, 4), F(1, 4)],
    [F(1, 4), F(0), F(1, 4), F(1, 2)],
]
# target rows at positions 0..gamma
P_ROWS = [
    [F(3, 8), F(3, 8), F(1, 8), F(1, 8)],  # residual after a rejection at 0: (1/4, 3/4, 0, 0)
    [F(1, 4), F(1, 8), F(3, 8), F(1, 4)],  # residual after a rejection at 1: (0, 1/2, 1/2, 0)
    [F(1, 8), F(1, 4), F(1, 2), F(1, 8)],  # bonus row
]


def test_tables_are_grid_aligned():
    """The premise of the exact comparison: every threshold the block compares a uniform with is a
    multiple of 1/G (kept-order running sums of q, accept ratios, residual and bonus running sums)."""
    def aligned(x):
        return (x * G).denominator == 1

    for i in range(R):
        assert sum(Q_FULL[i]) == 1 and Q_FULL[i][1] == 0
        c = F(0)
        for x in KEEP:
            c += Q_FULL[i][x]
            assert aligned(c)
    for i in range(GAMMA + 1):
        assert sum(P_ROWS[i]) == 1
        assert all(aligned(c) for c in itertools.accumulate(P_ROWS[i]))
    for i in range(GAMMA):
        for x in range(V):
            if Q_FULL[i][x]:
                assert aligned(exact.accept_prob(P_ROWS[i][x], Q_FULL[i][x]))
        assert all(aligned(c) for c in itertools.accumulate(exact.residual(P_ROWS[i], Q_FULL[i])))


def grid_uniforms(n_dims):
    """All G^n_dims points of the midpoint grid, one row per point."""
    m = midpoints()
    pts = np.array(list(itertools.product(range(G), repeat=n_dims)), dtype=np.int64)
    return m[pts].astype(np.float32), pts


def exact_fixed_rows():
    return exact.block_distribution(lambda ctx: P_ROWS[len(ctx)], lambda ctx: Q_FULL[len(ctx)], GAMMA)


def emitted_counts(tokens, n):
    c = Counter()
    for b in range(tokens.shape[0]):
        c[tuple(int(t) for t in tokens[b, : n[b] + 1])] += 1
    return c


def assert_equals_exact(counts, dist, total):
    assert set(counts) <= {k for k, v in dist.items() if v}, set(counts) - set(dist)
    for k, v in dist.items():
        assert F(counts.get(k, 0), total) == v, (k, counts.get(k, 0), total, v)


def block_inputs():
    """Grid over (u_draft[0], u_draft[1], u_acc[0], u_acc[1], u_final); the third draft row's uniform
    is fixed (its draw is never verified)."""
    u, _ = grid_uniforms(2 * GAMMA + 1)
    B = u.shape[0]
    u_draft = np.concatenate([u[:, :GAMMA], np.full((B, 1), 0.3, np.float32)], axis=1)
    u_acc = np.ascontiguousarray(u[:, GAMMA:2 * GAMMA])
    u_fin = np.ascontiguousarray(u[:, 2 * GAMMA])
    d_rows = np.stack([logits_of([Q_FULL[i][x] for x in KEEP]) for i in range(R)])  # [R, Vt] in keep order
    t_rows = np.stack([logits_of(P_ROWS[i]) for i in range(GAMMA + 1)])  # [gamma+1, V]
    draft_logits = np.ascontiguousarray(np.broadcast_to(d_rows, (B, R, len(KEEP))).reshape(B * R, len(KEEP)))
    target = np.ascontiguousarray(np.broadcast_to(t_rows, (B, GAMMA + 1, V)))
    return draft_logits, target, u_draft, u_acc, u_fin


@pytest.fixture(scope="module")
def block_grid():
    draft_logits, target, u_draft, u_acc, u_fin = block_inputs()
    out = ref.block(None, None, KEEP, draft_logits, target, "f32", np.float32(T), u_draft, u_acc, u_fin, GAMMA, R)
    return out, u_draft


def test_block_grid_frequencies_equal_exact_distribution(block_grid):
    """ref.block over the whole grid emits every token tuple on exactly the fraction of grid points
    that the exact distribution gives it (the trimmed drafter, rank-ordered kept ids, T != 1)."""
    out, _ = block_grid
    dist = exact_fixed_rows()
    assert_equals_exact(emitted_counts(out["tokens"], out["n"]), dist, G ** (2 * GAMMA + 1))
    # and, as the exactness argument requires, the first emitted token follows p_0 exactly
    first = exact.first_token_marginal(dist, V)
    assert first == tuple(P_ROWS[0])


def test_block_draft_ids_follow_kept_order(block_grid):
    """ref.draft_draws inside ref.block: draft i is the inverse-CDF draw of row i over the kept ids
    in keep_ids order with the sequence's own uniform u_draft[b, i]: the grid points with uniform
    in (C[j-1], C[j]] draw kept index j."""
    out, u_draft = block_grid
    for i in range(R):
        cdf = np.cumsum([float(Q_FULL[i][x]) for x in KEEP])
        want = np.searchsorted(cdf, u_draft[:, i].astype(np.float64), side="left")
        assert np.array_equal(out["draft_ids"][:, i], want), i


def test_block_draws_with_the_sequence_own_uniforms():
    """Sequences are independent: a sequence's outputs are those it gets alone (B = 1), whatever
    the batch around it."""
    draft_logits, target, u_draft, u_acc, u_fin = block_inputs()
    full = ref.block(None, None, KEEP, draft_logits, target, "f32", np.float32(T), u_draft, u_acc, u_fin, GAMMA, R)
    rng = np.random.default_rng(5)
    for b in rng.choice(u_fin.shape[0], size=40, replace=False):
        one = ref.block(None, None, KEEP, draft_logits[b * R:(b + 1) * R], target[b:b + 1], "f32", np.float32(T),
                        u_draft[b:b + 1], u_acc[b:b + 1], u_fin[b:b + 1], GAMMA, R)
        assert np.array_equal(one["tokens"][0], full["tokens"][b]) and one["n"][0] == full["n"][b], b


def test_block_lm_head_path_matches_given_logits():
    """ref.block's own LM head (hidden x trimmed weight rows) feeds the same steps: one-hot hidden
    rows pick one column of the head, so the head gives the draft rows above (as bf16 logits) and
    the block's grid frequencies stay within the bf16 rounding of the exact ones -- here equal,
    since every threshold lies 1/16 away from every midpoint."""
    from workloads import bf16_round

    d_rows = np.stack([logits_of([Q_FULL[i][x] for x in range(V)]) for i in range(R)])  # [R, V] by full id
    H = 8
    weight = np.zeros((V, H), dtype=np.float32)
    weight[:, :R] = d_rows.T  # column i holds position i's draft logits
    w_bits = bf16_round(weight)
    draft_logits, target, u_draft, u_acc, u_fin = block_inputs()
    B = u_fin.shape[0]
    hid = np.zeros((B * R, H), dtype=np.float32)
    hid[np.arange(B * R), np.tile(np.arange(R), B)] = 1.0
    out = ref.block(bf16_round(hid), w_bits, KEEP, None, target, "f32", np.float32(T), u_draft, u_acc, u_fin,
                    GAMMA, R)
    assert_equals_exact(emitted_counts(out["tokens"], out["n"]), exact_fixed_rows(), G ** (2 * GAMMA + 1))


# ------------------------------------------------------------------ the order-1 toy: rows follow the drafts
# V = 3 tokens; table row 0 is the start context, row r the context "previous token r - 1".
TOY_Q = [
    [F(1, 2), F(1, 4), F(1, 4)],
    [F(1, 4), F(1, 2), F(1, 4)],
    [F(1, 4), F(1, 4), F(1, 2)],
    [F(1, 8), F(3, 8), F(1, 2)],
]
TOY_P = [
    [F(1, 4), F(3, 8), F(3, 8)],  # residual (0, 1/2, 1/2)
    [F(1, 2), F(1, 4), F(1, 4)],
    [F(1, 8), F(5, 8), F(1, 4)],
    [F(1, 4), F(1, 2), F(1, 4)],  # residual (1/2, 1/2, 0)
]
TOY_V = 3


def toy_row(table, ctx):
    return table[0] if not ctx else table[ctx[-1] + 1]


def test_toy_tables_are_grid_aligned():
    for c in range(TOY_V + 1):
        for row in (TOY_P[c], TOY_Q[c]):
            assert sum(row) == 1 and all((s * G).denominator == 1 for s in itertools.accumulate(row))
        for x in range(TOY_V):
            assert (exact.accept_prob(TOY_P[c][x], TOY_Q[c][x]) * G).denominator == 1
        assert all((s * G).denominator == 1 for s in itertools.accumulate(exact.residual(TOY_P[c], TOY_Q[c])))


@pytest.fixture(scope="module")
def toy_grid():
    u, _ = grid_uniforms(2 * GAMMA + 1)
    tt = np.stack([logits_of(r) for r in TOY_P])
    dt = np.stack([logits_of(r) for r in TOY_Q])
    out = ref.toy_block(tt, dt, np.float32(T), GAMMA, np.ascontiguousarray(u[:, :GAMMA]),
                        np.ascontiguousarray(u[:, GAMMA:2 * GAMMA]), np.ascontiguousarray(u[:, 2 * GAMMA]))
    return out, u


def test_toy_block_grid_frequencies_equal_exact_distribution(toy_grid):
    """ref.toy_block: the draft chain x_{i+1} ~ q(. | x_i) from the start context and the target rows
    along it give, over the grid, exactly the exact distribution of the whole emitted tuple."""
    out, _ = toy_grid
    dist = exact.block_distribution(lambda ctx: toy_row(TOY_P, ctx), lambda ctx: toy_row(TOY_Q, ctx), GAMMA)
    assert_equals_exact(emitted_counts(out["tokens"], out["n"]), dist, G ** (2 * GAMMA + 1))


def test_toy_block_draft_chain(toy_grid):
    """Draft i of the toy is drawn from the row of the context "previous token = draft i - 1" with
    the uniform u_draft[b, i]."""
    out, u = toy_grid
    ids = out["draft_ids"]
    for i in range(GAMMA):
        ctx_rows = np.zeros(len(ids), dtype=np.int64) if i == 0 else ids[:, i - 1] + 1
        for c in range(TOY_V + 1):
            sel = ctx_rows == c
            cdf = np.cumsum([float(x) for x in TOY_Q[c]])
            want = np.searchsorted(cdf, u[sel, i].astype(np.float64), side="left")
            assert np.array_equal(ids[sel, i], want), (i, c)


def test_toy_generate_first_block_is_toy_block(toy_grid):
    """The generation loop's first block reads u[b, 0] as (drafts, accept tests, final) and emits
    what toy_block emits with the same uniforms."""
    out, u = toy_grid
    tt = np.stack([logits_of(r) for r in TOY_P])
    dt = np.stack([logits_of(r) for r in TOY_Q])
    sel = np.arange(0, u.shape[0], 97)
    gen = ref.toy_generate(tt, dt, np.float32(T), np.float32(T), GAMMA, 1, u[sel][:, None, :])
    assert np.array_equal(gen["tokens"][:, 0], out["tokens"][sel, 0])
    assert np.array_equal(gen["accepted"], out["n"][sel])

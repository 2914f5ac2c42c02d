"""Pins for the oracle's building blocks: bf16 decoding, the trimmed LM head, the temperature
softmax and the inverse-CDF draw.  Each check comes from a closed form, a textbook special case
or brute force on tiny inputs, never from the oracle re-run against itself."""
import math

import numpy as np
import pytest

from oracle import ref


# ------------------------------------------------------------------ bf16 decoding

@pytest.mark.parametrize("bits,value", [
    (0x3F80, 1.0), (0xBF80, -1.0), (0x4000, 2.0), (0xC040, -3.0), (0x3F81, 1.0 + 2.0 ** -7),
    (0x0000, 0.0), (0x3E80, 0.25), (0x7F7F, (2 - 2.0 ** -7) * 2.0 ** 127), (0x0001, 2.0 ** -133),
])
def test_bf16_decode_known_patterns(bits, value):
    assert ref.bf16_to_f64(np.array([bits], dtype=np.uint16))[0] == value


# ------------------------------------------------------------------ LM head (VocabTrim Eq. 1)

def _bf16_of_small_ints(a):
    """bf16 bit patterns of small integers (exact), built without the code under test."""
    out = np.empty(a.shape, dtype=np.uint16)
    for idx, v in np.ndenumerate(a):
        out[idx] = np.array([float(v)], dtype=np.float32).view(np.uint32)[0] >> 16
    return out


def test_lm_head_brute_force_tiny():
    rng = np.random.default_rng(11)
    M, H, V = 3, 5, 7
    h = rng.integers(-4, 5, size=(M, H))
    W = rng.integers(-4, 5, size=(V, H))
    keep = np.array([5, 0, 3, 6], dtype=np.int32)
    got = ref.lm_head(_bf16_of_small_ints(h), _bf16_of_small_ints(W), keep)
    assert got.shape == (M, len(keep))
    for m in range(M):
        for j, row in enumerate(keep):
            want = sum(int(h[m, k]) * int(W[row, k]) for k in range(H))
            assert got[m, j] == want


def test_lm_head_unit_probe_catches_transpose():
    # hidden = unit vector e_k picks column k of the gathered head: logits[m, j] = W[keep[j], k]
    rng = np.random.default_rng(12)
    H, V = 6, 9
    W = rng.integers(-8, 9, size=(V, H))
    keep = np.array([8, 2, 4], dtype=np.int32)
    eye = np.eye(H, dtype=np.int64)
    got = ref.lm_head(_bf16_of_small_ints(eye), _bf16_of_small_ints(W), keep)
    assert np.array_equal(got, W[keep].T.astype(np.float64))


def test_trimmed_head_equals_full_head_gathered():
    # VocabTrim §3 Eq. 1: W^Trim is W's kept rows, so trimmed logits are full logits at keep_ids.
    rng = np.random.default_rng(13)
    h = rng.integers(0, 1 << 16, size=(4, 32), dtype=np.uint16) & 0x3FFF
    W = rng.integers(0, 1 << 16, size=(50, 32), dtype=np.uint16) & 0xBFFF
    keep = rng.permutation(50)[:17].astype(np.int32)
    full = ref.lm_head(h, W, None)
    trim = ref.lm_head(h, W, keep)
    assert np.array_equal(trim, full[:, keep])


# ------------------------------------------------------------------ temperature softmax

def test_softmax_constant_row():
    lse, p = ref.softmax_temp(np.full((1, 37), 3.0), 0.5)
    assert np.allclose(p, 1.0 / 37, rtol=0, atol=1e-15)
    assert math.isclose(lse[0], 3.0 / 0.5 + math.log(37), rel_tol=1e-15)


@pytest.mark.parametrize("a,b,T", [(1.0, 0.0, 1.0), (2.5, -1.0, 0.7), (-3.0, 4.0, 0.25)])
def test_softmax_two_element_closed_form(a, b, T):
    lse, p = ref.softmax_temp(np.array([[a, b]]), T)
    p0 = 1.0 / (1.0 + math.exp(-(a - b) / T))
    assert math.isclose(p[0, 0], p0, rel_tol=1e-14)
    assert math.isclose(p[0, 1], 1.0 - p0, rel_tol=1e-13, abs_tol=1e-16)
    assert math.isclose(lse[0], math.log(math.exp(a / T) + math.exp(b / T)), rel_tol=1e-14)


def test_softmax_shift_and_temperature_scaling():
    rng = np.random.default_rng(14)
    x = rng.normal(size=(3, 100)) * 4
    _, p1 = ref.softmax_temp(x, 0.8)
    _, p2 = ref.softmax_temp(x + 123.0, 0.8)
    _, p3 = ref.softmax_temp(x / 0.8, 1.0)
    assert np.allclose(p1, p2, rtol=1e-12, atol=0)
    assert np.allclose(p1, p3, rtol=1e-12, atol=0)
    assert np.allclose(p1.sum(axis=1), 1.0, rtol=0, atol=1e-14)


def test_softmax_large_logits_do_not_overflow():
    lse, p = ref.softmax_temp(np.array([[1e4, 1e4 - 1.0, -1e4]]), 1.0)
    e = math.exp(-1.0)
    # lse ~ 1e4 carries an ulp of 1.8e-12, which bounds the accuracy of exp(x - lse)
    assert math.isclose(p[0, 0], 1 / (1 + e), rel_tol=1e-11)
    assert math.isclose(p[0, 1], e / (1 + e), rel_tol=1e-11)
    assert p[0, 2] == 0.0
    assert math.isclose(lse[0], 1e4 + math.log1p(e), rel_tol=1e-15)


# ------------------------------------------------------------------ inverse-CDF draw

@pytest.mark.parametrize("u,idx", [
    (0.05, 0), (0.1, 0), (0.1000001, 1), (0.3, 1), (0.31, 2), (0.6, 2), (0.61, 3), (1.0, 3),
])
def test_draw_boundaries(u, idx):
    # weights 1,2,3,4: CDF boundaries at 0.1, 0.3, 0.6; a uniform on a boundary goes to the left
    assert ref.draw(np.array([1.0, 2.0, 3.0, 4.0]), u)[0] == idx


def test_draw_unnormalised_weights_scale_free():
    w = np.array([1.0, 2.0, 3.0, 4.0])
    for u in np.linspace(0.01, 1.0, 97):
        assert ref.draw(w, u)[0] == ref.draw(w * 7.5, u)[0]


def test_draw_never_returns_zero_weight():
    w = np.array([0.0, 1.0, 0.0, 1.0, 0.0])
    assert ref.draw(w, 2.0 ** -24)[0] == 1
    assert ref.draw(w, 0.5)[0] == 1
    assert ref.draw(w, 0.5 + 2.0 ** -24)[0] == 3
    assert ref.draw(w, 1.0)[0] == 3


def test_draw_margin():
    w = np.array([1.0, 2.0, 3.0, 4.0])
    idx, m = ref.draw(w, 0.35)
    assert idx == 2 and math.isclose(m, 0.05, rel_tol=1e-12)
    idx, m = ref.draw(w, 0.9)  # last token: only the lower boundary 0.6 counts
    assert idx == 3 and math.isclose(m, 0.3, rel_tol=1e-12)
    idx, m = ref.draw(np.array([0.0, 5.0]), 0.4)  # C = (0, 5): no interior boundary
    assert idx == 1 and m == math.inf


def test_draw_frequencies_match_weights():
    # a uniform grid of u reproduces the weights exactly when boundaries are grid-aligned
    w = np.array([3.0, 0.0, 5.0, 2.0])
    G = 100
    counts = np.zeros(4, dtype=int)
    for k in range(G):
        counts[ref.draw(w, (k + 0.5) / G)[0]] += 1
    assert counts.tolist() == [30, 0, 50, 20]

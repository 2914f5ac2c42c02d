"""GPU parity of the generation loop (vt_spec_generate_markov) against the oracle's chained
blocks on the order-1 toy, and its statistics against the closed forms.

Integer outputs are compared exactly.  A sequence may depart from the oracle only from the first
block holding a decision the oracle places within BAND of its uniform (fp32 rounding decides it;
every later block then starts from another context): such sequences are compared up to that
block, and at least 95% of the sequences must match in full."""
import numpy as np
import pytest
import torch

import draft_sampling_verification_amd as vt
from oracle import ref, stats
from tests.gpu_harness import BAND, dev, say
from workloads import CONFIGS, counter_uniforms, toy_tables

pytestmark = pytest.mark.gpu


def uniforms(B, L, gamma, stream):
    return counter_uniforms(1, stream, B, L * (2 * gamma + 1)).reshape(B, L, 2 * gamma + 1)


def run_gpu(tt, dt, Tt, Td, g, u):
    B, L = u.shape[:2]
    tok = torch.full((B, L), -7, dtype=torch.int32, device="cuda")
    st = torch.full((B, 4), -7, dtype=torch.int32, device="cuda")
    vt.vt_spec_generate_markov(dev(tt), dev(dt), Tt, Td, g, dev(u), tok, st)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), st.cpu().numpy()


def compare(tt, dt, Tt, Td, g, u, rows=None):
    tok, st = run_gpu(tt, dt, Tt, Td, g, u)
    rows = np.arange(u.shape[0]) if rows is None else np.asarray(rows)
    orc = ref.toy_generate(tt, dt, Tt, Td, g, u.shape[1], u[rows], band=BAND)
    full = 0
    for k, b in enumerate(rows):
        cut = orc["tie_token"][k]
        assert np.array_equal(tok[b, :cut], orc["tokens"][k, :cut]), (b, cut)
        if orc["tie_block"][k] == u.shape[1]:
            assert np.array_equal(tok[b], orc["tokens"][k]), b
            want = [orc["blocks"][k], orc["tests"][k], orc["accepted"][k], orc["emitted"][k]]
            assert st[b].tolist() == want, (b, st[b], want)
            full += 1
    say(f"  {full} of {len(rows)} sequences compared in full")
    assert full >= 0.95 * len(rows)
    return tok, st


def f32(x):
    return float(np.float32(x))


@pytest.mark.parametrize("w,g,B,L", [
    (0.5, 4, 1027, 64),   # B not a multiple of the four sequences per workgroup
    (0.0, 4, 512, 40),
    (0.9, 6, 512, 40),
    (0.3, 1, 300, 50),
    (0.7, 8, 256, 1),     # one token: the first block only
    (0.5, 2, 64, 1000),   # long chains
])
def test_toy_generation_matches_oracle(w, g, B, L):
    say(f"toy generate w={w} gamma={g} B={B} L={L}")
    t = toy_tables(CONFIGS[1], w)
    compare(t.target_logits, t.draft_logits, 1.0, 1.0, g, uniforms(B, L, g, stream=20 + g))


def test_identical_tables_accept_everything():
    t = toy_tables(CONFIGS[1], 0.5)
    g, B, L = 4, 200, 33
    tok, st = compare(t.target_logits, t.target_logits, 1.0, 1.0, g, uniforms(B, L, g, stream=30))
    assert np.all(st[:, 2] == g * st[:, 0]) and np.all(st[:, 3] == (g + 1) * st[:, 0])


def test_wide_vocabulary_trimmed_draft_and_temperatures():
    # V = 64 (every lane), draft trimmed to 40 ids (-inf elsewhere), T_t != T_d
    rng = np.random.default_rng(40)
    V, g, B, L = 64, 5, 400, 48
    tt = (rng.standard_normal((V + 1, V)) * 1.5).astype(np.float32)
    dt = (0.6 * tt + 0.8 * rng.standard_normal((V + 1, V))).astype(np.float32)
    dt[:, rng.choice(V, V - 40, replace=False)] = -np.inf
    compare(tt, dt, f32(0.7), f32(1.3), g, uniforms(B, L, g, stream=41))


def test_disjoint_draft_equals_autoregressive_sampling():
    rng = np.random.default_rng(50)
    V, g, B, L = 12, 3, 128, 40
    tt = rng.standard_normal((V + 1, V)).astype(np.float32)
    dt = rng.standard_normal((V + 1, V)).astype(np.float32)
    tt[:, ::2] = -np.inf
    dt[:, 1::2] = -np.inf
    tok, st = compare(tt, dt, 1.0, 1.0, g, uniforms(B, L, g, stream=51))
    assert np.all(st[:, 0] == L) and np.all(st[:, 2] == 0)


def test_two_token_joint_on_the_gpu():
    # [RR]: 200000 two-token generations from the start context, gamma = 2, w = 0.3
    t = toy_tables(CONFIGS[1], 0.3)
    g, B = 2, 200_000
    tok, _ = run_gpu(t.target_logits, t.draft_logits, 1.0, 1.0, g, uniforms(B, 2, g, stream=60))
    _, P = ref.softmax_temp(t.target_logits.astype(np.float64), 1.0)
    emp = np.zeros((18, 18))
    np.add.at(emp, (tok[:, 0], tok[:, 1]), 1.0 / B)
    tv = 0.5 * np.abs(emp - P[0][:, None] * P[1:]).sum()
    say(f"  two-token joint TV {tv:.5f}")
    assert tv < 0.03


@pytest.mark.parametrize("w", [0.0, 0.5, 0.9])
def test_statistics_at_scale(w):
    """The measured workload: 16384 sequences x 256 tokens.  Sampled sequences against the
    oracle; acceptance and tokens per block against the closed forms (4.2M tokens)."""
    t = toy_tables(CONFIGS[1], w)
    g, B, L = 4, 16384, 256
    u = uniforms(B, L, g, stream=70)
    say(f"toy generate at scale w={w}")
    compare(t.target_logits, t.draft_logits, 1.0, 1.0, g, u, rows=[0, 1, 4097, 13333, B - 1])
    tok, st = run_gpu(t.target_logits, t.draft_logits, 1.0, 1.0, g, u)
    assert np.all((tok >= 0) & (tok < 18))
    a = stats.alpha_toy(t.target_logits, t.draft_logits, 1.0, 1.0)
    a_hat = st[:, 2].sum() / st[:, 1].sum()
    tau = st[:, 3].sum() / st[:, 0].sum()
    say(f"  alpha {a:.5f} measured {a_hat:.5f}; tokens/block {tau:.5f} closed form {stats.expected_tokens(a, g):.5f}")
    assert abs(a_hat - a) < 0.004
    assert abs(tau - stats.expected_tokens(a, g)) < 0.01

"""GPU parity of vt_softmax_temp: log-normalisers, probabilities and inverse-CDF draws against the
oracle (float64 softmax of the same stored logits, float64 sequential running sum for the draw).

Tolerances: |lse| error <= 2e-6 (fp32 reduction, fp64 output); probabilities within rel 1e-5
(plus FLT_MIN absolute, for entries that underflow fp32); draws exact unless the oracle's
uniform lies within 1e-6 of a CDF boundary of the drawn token."""
import numpy as np
import pytest
import torch

import draft_sampling_verification_amd as vt
from oracle import ref
from tests.gpu_harness import BAND, dev, dev_bf16, say
from workloads import bf16_round, counter_uniforms

pytestmark = pytest.mark.gpu
FLT_MIN = np.float32(1.1754944e-38)


def _logits(rows, n, kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "zipf":  # target-like: Zipf bias of a random ranking plus N(0, 2)
        rank = rng.permutation(n) + 1
        x = -1.1 * np.log(rank)[None, :] + 2.0 * rng.standard_normal((rows, n))
    else:  # draft-like: N(0, 1.1)
        x = 1.1 * rng.standard_normal((rows, n))
    return x.astype(np.float32)


def _run(x_store, dtype, rows, n, ld, T, u, probs=True):
    xs = dev(x_store) if dtype == "f32" else dev_bf16(x_store)
    lse = torch.empty(rows, dtype=torch.float64, device="cuda")
    pr = torch.empty(rows, n, dtype=torch.float32, device="cuda") if probs else None
    samp = torch.empty(rows, dtype=torch.int32, device="cuda")
    vt.vt_softmax_temp(xs.view(rows, ld), T, lse, pr, dev(u), samp, n=n)
    torch.cuda.synchronize()
    return lse.cpu().numpy(), (pr.cpu().numpy() if probs else None), samp.cpu().numpy()


CASES = [
    (7, 18, "f32", 1.0, "draft"),       # toy width: one partial chunk, scalar path
    (5, 4096, "f32", 0.7, "zipf"),      # exactly one chunk
    (5, 4097, "bf16", 0.8, "zipf"),     # one element into a second chunk
    (9, 12345, "f32", 1.0, "draft"),    # ragged last chunk
    (3, 128256, "bf16", 0.7, "zipf"),   # full vocabulary, bf16 target rows
    (6, 128256, "f32", 1.0, "draft"),   # configs 2/3 draft rows
    (300, 1000, "f32", 0.8, "zipf"),    # many short rows
    (4, 32768, "f32", 0.7, "draft"),    # trimmed draft width
]


@pytest.mark.parametrize("rows,n,dtype,T,kind", CASES)
def test_softmax_parity(rows, n, dtype, T, kind):
    say(f"softmax parity rows={rows} n={n} {dtype} T={T} {kind}")
    x = _logits(rows, n, kind, seed=rows + n)
    store = x if dtype == "f32" else bf16_round(x)
    x64 = ref.as_f64(store, dtype)
    u = counter_uniforms(99, n % 1000, rows, 1)[:, 0].copy()
    lse, pr, samp = _run(store, dtype, rows, n, n, T, u)
    olse, opr = ref.softmax_temp(x64, T)
    say(f"  max |lse err| {np.abs(lse - olse).max():.3e}")
    assert np.all(np.abs(lse - olse) <= 2e-6)
    rel = np.abs(pr - opr) / np.maximum(opr, FLT_MIN)
    say(f"  max prob rel err {rel.max():.3e}")
    assert np.all(np.abs(pr - opr) <= 1e-5 * opr + FLT_MIN)
    excused = 0
    for r in range(rows):
        idx, margin = ref.draw(opr[r], float(u[r]))
        assert opr[r, samp[r]] > 0
        if samp[r] != idx:
            assert margin < BAND, (r, samp[r], idx, margin)
            excused += 1
    say(f"  draws exact, {excused} mismatches excused by the band of {rows}")


def test_softmax_strided_rows_scalar_path():
    rows, n, ld = 6, 5000, 5003  # row stride not a multiple of 4: element-wise loads
    x = _logits(rows, ld, "zipf", seed=3)
    u = counter_uniforms(98, 0, rows, 1)[:, 0].copy()
    lse, _, samp = _run(x, "f32", rows, n, ld, 0.9, u, probs=False)
    olse, opr = ref.softmax_temp(x[:, :n].astype(np.float64), 0.9)
    assert np.all(np.abs(lse - olse) <= 2e-6)
    for r in range(rows):
        idx, margin = ref.draw(opr[r], float(u[r]))
        assert samp[r] == idx or margin < BAND


def test_draw_grid_reproduces_weights_exactly():
    # weights 1:2:3:4 at T = 1 (logits ln w); a 100-point grid of uniforms lands 10/20/30/40
    x = np.log(np.array([1.0, 2.0, 3.0, 4.0]))[None, :].repeat(100, 0).astype(np.float32)
    u = ((np.arange(100) + 0.5) / 100).astype(np.float32)
    _, _, samp = _run(x, "f32", 100, 4, 4, 1.0, u, probs=False)
    assert np.bincount(samp, minlength=4).tolist() == [10, 20, 30, 40]


def test_masked_entries_never_drawn_and_u_one():
    # -inf logits have zero weight: never drawn; u = 1 returns the last positive-weight entry
    n = 9000
    x = np.full((3, n), -np.inf, dtype=np.float32)
    x[0, [5, 4100, 8999]] = [0.0, 1.0, 2.0]
    x[1, [0, 1]] = [3.0, 3.0]
    x[2, 4096:4200] = 0.5
    u = np.array([1.0, 1.0, 2.0 ** -24], dtype=np.float32)
    lse, pr, samp = _run(x, "f32", 3, n, n, 1.0, u)
    assert samp.tolist() == [8999, 1, 4096]
    assert np.all(pr[np.isinf(x)] == 0)
    want0 = np.log(np.exp(0) + np.exp(1) + np.exp(2))
    assert abs(lse[0] - want0) < 1e-6


def test_extreme_logits_do_not_overflow():
    x = np.array([[1e4, 1e4 - 1.0, -1e4] + [-1e4] * 5000], dtype=np.float32)
    u = np.array([0.5], dtype=np.float32)
    lse, pr, samp = _run(x, "f32", 1, x.shape[1], x.shape[1], 1.0, u)
    e = np.exp(-1.0)
    assert abs(pr[0, 0] - 1 / (1 + e)) < 1e-6 and abs(pr[0, 1] - e / (1 + e)) < 1e-6
    assert abs(lse[0] - (1e4 + np.log1p(e))) < 2e-3  # lse ~ 1e4: fp32 ulp 1e-3
    assert samp[0] == 0

"""GPU parity of keep-set construction (VocabTrim §3: Algorithm 1, Eq. 1, Top-P / minimum
frequency) against the oracle: token counts, kept ids, inverse map and the trimmed head must
match bit for bit."""
import functools

import numpy as np
import pytest
import torch

import draft_sampling_verification_amd as vt
from oracle import keepset
from tests.gpu_harness import dev, dev_bf16, say
from workloads import bf16_round, token_stream

pytestmark = pytest.mark.gpu

V_FULL = 128256


def gpu_counts(tokens_dev, V, counts=None, accumulate=False):
    if counts is None:
        counts = torch.full((V,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")  # garbage to overwrite
    vt.vt_token_histogram(tokens_dev, V, counts, accumulate=accumulate)
    torch.cuda.synchronize()
    return counts


def as_u32(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("n,V,seed,bad", [
    (1000, V_FULL, 0, True),           # one group: counts written directly
    (4099, V_FULL, 1, False),          # n % 4 != 0
    ((1 << 22) + 3, V_FULL, 2, True),  # 64 groups x 4 slabs, partial sums
    ((1 << 20) + 1, 100000, 3, False),  # last slab partial
    (300000, 1000, 4, True),           # one slab, many groups
    (5000, 1, 5, True),                # a one-token vocabulary
    (1 << 26, V_FULL, 6, False),       # the measured corpus size
])
def test_histogram_matches_algorithm_1(n, V, seed, bad):
    say(f"histogram n={n} V={V} seed={seed}")
    toks = token_stream(V, n, seed=seed)
    if bad:  # ids that are not in the vocabulary are skipped
        rng = np.random.default_rng(seed)
        idx = rng.choice(n, size=min(n, 97), replace=False)
        toks[idx] = rng.choice(np.array([-1, -7, V, V + 5, np.iinfo(np.int32).max, np.iinfo(np.int32).min]),
                               size=len(idx))
    want = keepset.count_tokens(toks, V)
    got = as_u32(gpu_counts(dev(toks), V))
    assert np.array_equal(got.astype(np.uint64), want)


def test_histogram_unaligned_tokens_and_accumulate():
    V = V_FULL
    toks = token_stream(V, 700001, seed=11)
    td = dev(toks)
    part1 = td[1:300002]  # 4-byte aligned, not 16: the scalar path
    part2 = td[300002:]
    assert part1.data_ptr() % 16 != 0
    c = gpu_counts(part1, V)
    c = gpu_counts(part2, V, counts=c, accumulate=True)
    want = keepset.count_tokens(toks[300002:], V, keepset.count_tokens(toks[1:300002], V))
    assert np.array_equal(as_u32(c).astype(np.uint64), want)


def test_histogram_empty_input():
    V = 5000
    c = gpu_counts(torch.empty(0, dtype=torch.int32, device="cuda"), V)
    assert not as_u32(c).any()
    prev = torch.arange(V, dtype=torch.int32, device="cuda")
    c = gpu_counts(torch.empty(0, dtype=torch.int32, device="cuda"), V, counts=prev.clone(), accumulate=True)
    assert torch.equal(c, prev)


def gpu_select(counts_u32, rule, **kw):
    V = len(counts_u32)
    c = dev(counts_u32.view(np.int32))
    keep = torch.full((V,), -9, dtype=torch.int32, device="cuda")
    f2t = torch.full((V,), -9, dtype=torch.int32, device="cuda")
    nk = torch.full((1,), -9, dtype=torch.int32, device="cuda")
    vt.vt_keep_select(c, rule, keep, f2t, nk, **kw)
    torch.cuda.synchronize()
    K = int(nk.item())
    return keep.cpu().numpy()[:K], f2t.cpu().numpy(), K


@functools.lru_cache(maxsize=1)
def counts_cases():
    V = V_FULL
    zipf = keepset.count_tokens(token_stream(V, 1 << 22, seed=21), V).astype(np.uint32)
    rng = np.random.default_rng(22)
    ties = rng.integers(0, 4, size=V).astype(np.uint32)               # heavy ties
    wide = rng.integers(0, 1 << 32, size=V, dtype=np.uint64).astype(np.uint32)  # every digit in play
    wide[rng.choice(V, 50, replace=False)] = wide[:50]                  # some equal large counts
    small = rng.integers(0, 9, size=1000).astype(np.uint32)
    ragged = rng.integers(0, 50, size=1001).astype(np.uint32)  # V % 4 != 0 with non-zero tail counts
    return {"zipf": zipf, "ties": ties, "wide": wide, "small": small, "zeros": np.zeros(777, np.uint32),
            "one": np.array([5], np.uint32), "ragged": ragged}


CASE_NAMES = ["zipf", "ties", "wide", "small", "zeros", "one", "ragged"]


@pytest.mark.parametrize("name", CASE_NAMES)
def test_select_top_k(name):
    c = counts_cases()[name]
    V = len(c)
    for k in sorted(k for k in {1, 2, 17, 32768, 65536, max(1, V // 3), V} if k <= V):
        say(f"top_k {name} k={k}")
        keep_w, f2t_w = keepset.top_k(c, k)
        keep, f2t, K = gpu_select(c, vt.VT_SELECT_TOP_K, k=k)
        assert K == k
        assert np.array_equal(keep, keep_w)
        assert np.array_equal(f2t, f2t_w)


@pytest.mark.parametrize("name", CASE_NAMES)
def test_select_top_p(name):
    c = counts_cases()[name]
    for p in (1e-9, 0.1, 0.5, 0.9, 0.99, 0.999999, 1.0):
        say(f"top_p {name} p={p}")
        keep_w, f2t_w = keepset.top_p(c, p)
        keep, f2t, K = gpu_select(c, vt.VT_SELECT_TOP_P, p=p)
        assert K == len(keep_w)
        assert np.array_equal(keep, keep_w)
        assert np.array_equal(f2t, f2t_w)


@pytest.mark.parametrize("name", CASE_NAMES)
def test_select_min_frequency(name):
    c = counts_cases()[name]
    for f in (0, 1, 2, 3, 100, int(c.max()), int(c.max()) + 1 if c.max() < 0xFFFFFFFF else 0xFFFFFFFF):
        say(f"min_freq {name} f={f}")
        keep_w, f2t_w = keepset.min_frequency(c, f)
        keep, f2t, K = gpu_select(c, vt.VT_SELECT_MIN_FREQ, min_count=f)
        assert K == len(keep_w)
        assert np.array_equal(keep, keep_w)
        assert np.array_equal(f2t, f2t_w)


def test_trim_head_rows_and_out_of_range_ids():
    rng = np.random.default_rng(31)
    V, H = 3000, 520
    W = bf16_round(rng.standard_normal((V, H), dtype=np.float32))
    keep = np.sort(rng.choice(V, 1001, replace=False)).astype(np.int32)
    keep[[5, 500]] = [-1, V]  # not rows of W: zero rows
    out = torch.full((len(keep), H), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    vt.vt_trim_head(dev_bf16(W), dev(keep), out)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    ok = (keep >= 0) & (keep < V)
    assert np.array_equal(got[ok], keepset.trim_head(W, keep[ok]))
    assert not got[~ok].any()


def _k_tiled(trimmed: np.ndarray) -> np.ndarray:
    """The K-tiled layout of vt_trim_head_tiled, written as a reshape: [ceil(k/256)][H/32][256][32],
    rows past k zero."""
    k, H = trimmed.shape
    nb = -(-k // 256)
    x = np.zeros((nb * 256, H), trimmed.dtype)
    x[:k] = trimmed
    return x.reshape(nb, 256, H // 32, 32).transpose(0, 2, 1, 3).reshape(-1)


@pytest.mark.parametrize("k,rank_order", [(1001, False), (256, False), (700, True)])
def test_trim_head_tiled_layout(k, rank_order):
    rng = np.random.default_rng(37 + k)
    V, H = 3000, 96  # three 32-column K steps; k = 1001 and 700 leave a ragged last row block
    W = bf16_round(rng.standard_normal((V, H), dtype=np.float32))
    keep = rng.choice(V, k, replace=False).astype(np.int32)
    if not rank_order:
        keep = np.sort(keep)
    keep[[3, k - 1]] = [-1, V]  # not rows of W: zero rows
    want_rows = np.zeros((k, H), np.uint16)
    ok = (keep >= 0) & (keep < V)
    want_rows[ok] = keepset.trim_head(W, keep[ok])
    say(f"tiled W^Trim: V={V} H={H} k={k} rank order {rank_order}")
    out = torch.full((vt.lib().vt_trim_head_tiled_bytes(k, H) // 2,), 7, dtype=torch.int16,
                     device="cuda").view(torch.bfloat16)
    vt.vt_trim_head_tiled(dev_bf16(W), dev(keep), tiled=out)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, _k_tiled(want_rows))


def test_trim_head_tiled_without_keep_ids():
    rng = np.random.default_rng(43)
    V, H, k = 600, 64, 300
    W = bf16_round(rng.standard_normal((V, H), dtype=np.float32))
    got = vt.vt_trim_head_tiled(dev_bf16(W), None, k=k)
    torch.cuda.synchronize()
    assert np.array_equal(got.view(torch.int16).cpu().numpy().view(np.uint16), _k_tiled(W[:k]))


def test_stream_to_trimmed_head_end_to_end():
    """Counter -> Top-K -> W^Trim on the GPU; the trimmed head scored without keep_ids gives the
    same logits as the full head gathered through keep_ids (Eq. 1), bit for bit."""
    V, H, k = V_FULL, 3072, 32768
    toks = token_stream(V, 1 << 24, seed=41)
    counts = gpu_counts(dev(toks), V)
    keep = torch.empty(V, dtype=torch.int32, device="cuda")
    f2t = torch.empty(V, dtype=torch.int32, device="cuda")
    nk = torch.empty(1, dtype=torch.int32, device="cuda")
    vt.vt_keep_select(counts, vt.VT_SELECT_TOP_K, keep, f2t, nk, k=k)
    torch.cuda.synchronize()
    assert int(nk.item()) == k
    keep_w, f2t_w = keepset.top_k(keepset.count_tokens(toks, V), k)
    assert np.array_equal(keep[:k].cpu().numpy(), keep_w)
    assert np.array_equal(f2t.cpu().numpy(), f2t_w)
    from workloads.gen import lm_head_weights
    W = lm_head_weights(V, H)
    Wd = dev_bf16(W)
    trimmed = torch.empty(k, H, dtype=torch.bfloat16, device="cuda")
    vt.vt_trim_head(Wd, keep[:k].contiguous(), trimmed)
    torch.cuda.synchronize()
    sample = np.random.default_rng(42).choice(k, 2048, replace=False)
    got = trimmed.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got[sample], W[keep_w[sample]])
    hid = dev_bf16(bf16_round(np.random.default_rng(43).standard_normal((6, H), dtype=np.float32)))
    a = torch.empty(6, k, dtype=torch.float32, device="cuda")
    b = torch.empty(6, k, dtype=torch.float32, device="cuda")
    vt.vt_lmhead_trimmed(hid, trimmed, None, a)
    vt.vt_lmhead_trimmed(hid, Wd, keep[:k].contiguous(), b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)

"""Seeded synthetic inputs with the shapes and value distributions of the five workloads.

Everything here is input construction only.  Random draws the method itself makes are
supplied as arrays of uniform variates, so the GPU path and the CPU oracle consume the
same numbers and make the same draws.

Streams (numpy SeedSequence entropy = [key..., stream]):
  0  vocabulary permutation -> Zipf ranks          (keyed by V)
  1  LM-head weights W ~ N(0, 0.02) -> bf16        (keyed by H)
  2  hidden states ~ N(0, 1) -> bf16               (keyed by model id, per sequence)
  3  target-logit noise ~ N(0, 2)                  (keyed by model id, per sequence)
  4  u_draft, 5 u_accept, 6 u_final                (counter-based, keyed by config id)
  7  toy target table, 8 toy context-free unigram  (keyed by config id)
  9  calibration token stream (Zipf ranks)          (keyed by V and a stream seed)

Per-sequence streams make sequence b's inputs independent of the batch size B.

Uniforms are u = (k + 1) * 2**-24 with k a 24-bit integer, so every u is exact in fp32 and
lies in (0, 1].  k comes from the SplitMix64 output function (Steele, Lea and Flood, 2014)
applied to a Weyl counter, one counter value per (sequence, column).
"""
from __future__ import annotations

import dataclasses
import functools
import json
import os
from typing import Optional

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_MIX1 = np.uint64(0xBF58476D1CE4E5B9)
_MIX2 = np.uint64(0x94D049BB133111EB)
_COL_STRIDE = np.uint64(1 << 16)


@dataclasses.dataclass(frozen=True)
class Config:
    """One workload shape.  R = draft rows per sequence handed to the verifier (R >= gamma)."""

    cfg_id: int
    name: str
    B: int
    gamma: int
    V: int
    Vt: int
    H: int  # 0: no LM head (the toy)
    target_dtype: str  # "f32" or "bf16"
    T: float
    trimmed: bool  # a keep_ids map is passed (Vt < V, or an explicit identity map)
    model_id: int  # seeds hidden states and target noise; equal ids share them
    R: int

    @property
    def M(self) -> int:
        return self.B * self.R

    def scaled(self, **kw) -> "Config":
        """Same recipe at another size (parity cases the oracle finishes in seconds)."""
        c = dataclasses.replace(self, **kw)
        if "R" not in kw and "gamma" in kw and self.H > 0:
            c = dataclasses.replace(c, R=c.gamma + 1)
        return c


CONFIGS = {
    1: Config(1, "toy verify: B=1 gamma=4 V=18 fp32, q = 0.5 p + 0.5 q0", 1, 4, 18, 18, 0, "f32", 1.0, False, 1, 4),
    2: Config(2, "full drafter LM head + verify: B=1 gamma=5 H=3072 V=Vt=128256 fp32 target T=1",
              1, 5, 128256, 128256, 3072, "f32", 1.0, False, 2, 6),
    3: Config(3, "VocabTrim head: B=1 gamma=5 H=3072 V=128256 Vt=32768 fp32 target T=1",
              1, 5, 128256, 32768, 3072, "f32", 1.0, True, 2, 6),
    4: Config(4, "batched verification: B=64 gamma=7 H=3072 V=128256 Vt=32768 bf16 target T=0.7",
              64, 7, 128256, 32768, 3072, "bf16", 0.7, True, 4, 8),
    5: Config(5, "large drafter: B=256 gamma=8 H=4096 V=128256 Vt=65536 bf16 target T=0.8",
              256, 8, 128256, 65536, 4096, "bf16", 0.8, True, 5, 9),
}


def _rng(*entropy: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(entropy))))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even.  Inputs must be finite."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact bf16 -> fp32 widening (input construction for the aligned variant)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def counter_uniforms(cfg_id: int, stream: int, rows: int, cols: int, row0: int = 0) -> np.ndarray:
    """float32 [rows, cols] uniforms in (0, 1]; entry (b, j) depends only on (cfg_id, stream, b, j)."""
    seed = np.random.SeedSequence([cfg_id, stream]).generate_state(1, np.uint64)[0]
    b = np.arange(row0, row0 + rows, dtype=np.uint64)[:, None]
    j = np.arange(cols, dtype=np.uint64)[None, :]
    with np.errstate(over="ignore"):
        z = seed + (b * _COL_STRIDE + j + np.uint64(1)) * _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _MIX1
        z = (z ^ (z >> np.uint64(27))) * _MIX2
        z = z ^ (z >> np.uint64(31))
    k = z >> np.uint64(40)
    return ((k + np.uint64(1)).astype(np.float64) * 2.0 ** -24).astype(np.float32)


@functools.lru_cache(maxsize=4)
def zipf_ranking(V: int):
    """(ids in rank order, rank of each id in 1..V) from a seeded permutation of the vocabulary."""
    perm = _rng(V, 0).permutation(V).astype(np.int32)
    rank = np.empty(V, dtype=np.int64)
    rank[perm] = np.arange(1, V + 1)
    perm.setflags(write=False)
    rank.setflags(write=False)
    return perm, rank


@functools.lru_cache(maxsize=3)
def lm_head_weights(V: int, H: int) -> np.ndarray:
    """bf16 bits [V, H], W ~ N(0, 0.02) (0.02 read as the standard deviation)."""
    rng = _rng(H, 1)
    out = np.empty((V, H), dtype=np.uint16)
    step = 8192
    for r0 in range(0, V, step):
        r1 = min(V, r0 + step)
        out[r0:r1] = bf16_round(rng.standard_normal((r1 - r0, H), dtype=np.float32) * np.float32(0.02))
    out.setflags(write=False)
    return out


def hidden_states(cfg: Config, b0: int, B: int) -> np.ndarray:
    """bf16 bits [B*R, H], rows b*R + i; N(0, 1) per sequence."""
    out = np.empty((B * cfg.R, cfg.H), dtype=np.uint16)
    for k in range(B):
        rng = _rng(cfg.model_id, 2, b0 + k)
        out[k * cfg.R:(k + 1) * cfg.R] = bf16_round(rng.standard_normal((cfg.R, cfg.H), dtype=np.float32))
    return out


def target_logits(cfg: Config, b0: int, B: int) -> np.ndarray:
    """[B, gamma+1, V]: -1.1 ln rank(id) + N(0, 2) noise (2 read as the standard deviation).

    fp32 values for target_dtype "f32", bf16 bit patterns (uint16) for "bf16".
    """
    _, rank = zipf_ranking(cfg.V)
    bias = -1.1 * np.log(rank.astype(np.float64))
    shape = (cfg.gamma + 1, cfg.V)
    if cfg.target_dtype == "f32":
        out = np.empty((B,) + shape, dtype=np.float32)
    else:
        out = np.empty((B,) + shape, dtype=np.uint16)
    for k in range(B):
        noise = _rng(cfg.model_id, 3, b0 + k).standard_normal(shape)
        v = (bias[None, :] + 2.0 * noise).astype(np.float32)
        out[k] = v if cfg.target_dtype == "f32" else bf16_round(v)
    return out


@functools.lru_cache(maxsize=2)
def _zipf_rank_cdf(V: int, s: float) -> np.ndarray:
    w = np.arange(1, V + 1, dtype=np.float64) ** -s
    c = np.cumsum(w)
    return c / c[-1]


def token_stream(V: int, n: int, seed: int = 0, s: float = 1.1, chunk: int = 1 << 22) -> np.ndarray:
    """int32 [n] token ids of a synthetic calibration corpus: ranks drawn from a Zipf(s) law over
    1..V (P(rank r) proportional to r**-s), mapped to ids through the same seeded permutation
    that ranks the target logits, so frequent ids here are the ids the target favours."""
    perm, _ = zipf_ranking(V)
    cdf = _zipf_rank_cdf(V, s)
    rng = _rng(V, 9, seed)
    out = np.empty(n, dtype=np.int32)
    for i in range(0, n, chunk):
        u = rng.random(min(chunk, n - i))
        r = np.minimum(np.searchsorted(cdf, u, side="right"), V - 1)
        out[i:i + len(u)] = perm[r]
    return out


@dataclasses.dataclass
class ToyTables:
    """Order-1 toy: rows are contexts (row 0 = start-of-sequence, never emitted), columns tokens."""

    target_logits: np.ndarray  # f32 [V+1, V], N(0, 1)
    draft_logits: np.ndarray  # f32 [V+1, V], ln(w p + (1-w) q0)
    w: float


def toy_tables(cfg: Config = CONFIGS[1], w: float = 0.5) -> ToyTables:
    """Toy target and draft tables (the models of the toy workload).

    The target at each context is softmax of N(0,1) logits; the draft mixes that target with a
    context-free unigram q0 = softmax(N(0,1)), as the toy build of the rule does with its
    bigram/unigram pair.  The mixture is formed in float64 and handed over as fp32 log-weights.
    """
    V = cfg.V
    tl = _rng(cfg.cfg_id, 7).standard_normal((V + 1, V)).astype(np.float32)
    q0l = _rng(cfg.cfg_id, 8).standard_normal(V)
    t64 = tl.astype(np.float64)
    p = np.exp(t64 - t64.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    q0 = np.exp(q0l - q0l.max())
    q0 /= q0.sum()
    q = w * p + (1.0 - w) * q0[None, :]
    return ToyTables(target_logits=tl, draft_logits=np.log(q).astype(np.float32), w=w)


ARTICLE_TOY_FIXTURE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tests", "golden",
                                   "rr_toy.json")


@functools.lru_cache(maxsize=1)
def article_toy_counts():
    """The rejection-rule article's toy models, as counts ("A target and a draft small enough to
    print in full"): the vocabulary is the sorted set of the corpus's characters (18); the target is
    an order-1 bigram model with one pseudo-count per (context, token) pair plus one count per
    transition of the corpus, read from a start context before its first character (row 0 of the
    table; row r + 1 is the context "previous token = r"); the unigram q0 has one pseudo-count per
    token plus its occurrences.  Returns (vocabulary string, bigram counts [V+1, V], unigram counts [V])."""
    with open(ARTICLE_TOY_FIXTURE) as f:
        corpus = json.load(f)["corpus"]
    vocab = "".join(sorted(set(corpus)))
    index = {c: i for i, c in enumerate(vocab)}
    V = len(vocab)
    bigram = np.ones((V + 1, V), dtype=np.int64)
    ctx = 0
    for ch in corpus:
        bigram[ctx, index[ch]] += 1
        ctx = index[ch] + 1
    unigram = np.ones(V, dtype=np.int64)
    for ch in corpus:
        unigram[index[ch]] += 1
    return vocab, bigram, unigram


def article_toy(w: float) -> ToyTables:
    """The article's target p (normalised bigram counts) and draft q_w = w p + (1 - w) q0 (q0 the
    normalised unigram counts), formed in float64 and handed over as fp32 log-weights (T = 1)."""
    _, bigram, unigram = article_toy_counts()
    p = bigram / bigram.sum(axis=1, keepdims=True)
    q0 = unigram / unigram.sum()
    q = w * p + (1.0 - w) * q0[None, :]
    return ToyTables(target_logits=np.log(p).astype(np.float32), draft_logits=np.log(q).astype(np.float32), w=w)


@dataclasses.dataclass
class Workload:
    cfg: Config
    b0: int
    B: int
    T: np.float32
    hidden: Optional[np.ndarray] = None  # bf16 bits [B*R, H]
    weight: Optional[np.ndarray] = None  # bf16 bits [V, H], the full head
    keep_ids: Optional[np.ndarray] = None  # int32 [Vt]; None for the full head
    full_to_trim: Optional[np.ndarray] = None  # int32 [V], -1 off the kept set
    target: Optional[np.ndarray] = None  # [B, gamma+1, V] f32 or bf16 bits
    draft_logits: Optional[np.ndarray] = None  # f32 [B*R, Vt]; only for the aligned variant
    toy: Optional[ToyTables] = None
    u_draft: Optional[np.ndarray] = None  # f32 [B, R]
    u_acc: Optional[np.ndarray] = None  # f32 [B, gamma]
    u_fin: Optional[np.ndarray] = None  # f32 [B]


def keep_set(cfg: Config, order: str = "id"):
    """keep_ids = the Vt best-ranked ids and the inverse map (or None, None).

    order "id": the kept ids in ascending id order (the storage order of a trimmed head built
    by a sorted row gather); "rank": in rank order, best first.
    """
    if not cfg.trimmed:
        return None, None
    perm, _ = zipf_ranking(cfg.V)
    keep = np.ascontiguousarray(perm[: cfg.Vt], dtype=np.int32)
    if order == "id":
        keep = np.sort(keep)
    elif order != "rank":
        raise ValueError(order)
    inv = np.full(cfg.V, -1, dtype=np.int32)
    inv[keep] = np.arange(cfg.Vt, dtype=np.int32)
    return keep, inv


def following_head(cfg: Config, b0: int, B: int, noise: float):
    """A drafter that follows the target, for parity cases that reach long accepted runs.

    Hidden row (b, i) is 16 e_0 + 32 e_j with a seeded column j = j(b, i) >= 1, and column 0 of
    the head holds bf16(z(x) / 16), z(x) = -1.1 ln rank(x) the Zipf bias of the target recipe;
    the other columns are the usual N(0, 0.02) head.  The LM head then gives exactly (up to one
    fp32 rounding) 16 W[x, 0] + 32 W[x, j], and target row (b, i) is that value over all V ids
    plus N(0, noise) (row gamma takes a fresh column when there is no draft row gamma).  No
    product is formed here beyond the two scalings that define the rows.
    Returns (hidden bf16 bits [B*R, H], weight bf16 bits [V, H], target [B, gamma+1, V]).
    """
    V, H, R, g = cfg.V, cfg.H, cfg.R, cfg.gamma
    w = lm_head_weights(V, H).copy()
    _, rank = zipf_ranking(V)
    w[:, 0] = bf16_round((-1.1 * np.log(rank.astype(np.float64)) / 16.0).astype(np.float32))
    w0 = bf16_bits_to_f32(w[:, 0]).astype(np.float64)
    hidden = np.zeros((B * R, H), dtype=np.uint16)
    one = bf16_round(np.array([16.0, 32.0], dtype=np.float32))
    if cfg.target_dtype == "f32":
        target = np.empty((B, g + 1, V), dtype=np.float32)
    else:
        target = np.empty((B, g + 1, V), dtype=np.uint16)
    for k in range(B):
        rng = _rng(cfg.model_id, 7, b0 + k)
        cols = rng.integers(1, H, size=max(R, g + 1) + 1)
        hidden[k * R:(k + 1) * R, 0] = one[0]
        for i in range(R):
            hidden[k * R + i, cols[i]] = one[1]
        for i in range(g + 1):
            col = cols[i] if i < R else cols[-1]
            v = 16.0 * w0 + 32.0 * bf16_bits_to_f32(w[:, col]).astype(np.float64)
            v = (v + noise * rng.standard_normal(V)).astype(np.float32)
            target[k, i] = v if cfg.target_dtype == "f32" else bf16_round(v)
    w.setflags(write=False)
    return hidden, w, target


def make_workload(cfg: Config, B: Optional[int] = None, b0: int = 0, aligned: bool = False,
                  keep_order: str = "id", follow: float = 0.0) -> Workload:
    """Inputs for sequences b0 .. b0+B-1 of a config.

    aligned=True replaces the LM head by draft logits equal to the target logits gathered at
    keep_ids (same temperature): q is then p restricted to the kept set and renormalised.
    keep_order: storage order of the kept ids ("id" ascending, or "rank").
    follow > 0: the drafter follows the target (following_head, target noise N(0, follow)).
    """
    B = cfg.B if B is None else B
    wl = Workload(cfg=cfg, b0=b0, B=B, T=np.float32(cfg.T))
    wl.u_draft = counter_uniforms(cfg.cfg_id, 4, B, cfg.R, b0)
    wl.u_acc = counter_uniforms(cfg.cfg_id, 5, B, cfg.gamma, b0)
    wl.u_fin = counter_uniforms(cfg.cfg_id, 6, B, 1, b0)[:, 0].copy()
    if cfg.H == 0:
        wl.toy = toy_tables(cfg)
        return wl
    wl.keep_ids, wl.full_to_trim = keep_set(cfg, keep_order)
    if follow > 0:
        wl.hidden, wl.weight, wl.target = following_head(cfg, b0, B, follow)
        return wl
    wl.target = target_logits(cfg, b0, B)
    if aligned:
        t32 = wl.target if cfg.target_dtype == "f32" else bf16_bits_to_f32(wl.target)
        cols = wl.keep_ids if wl.keep_ids is not None else np.arange(cfg.V)
        d = np.ascontiguousarray(t32[:, : cfg.R, :][:, :, cols], dtype=np.float32)
        wl.draft_logits = d.reshape(B * cfg.R, cfg.Vt)
    else:
        wl.weight = lm_head_weights(cfg.V, cfg.H)
        wl.hidden = hidden_states(cfg, b0, B)
    return wl

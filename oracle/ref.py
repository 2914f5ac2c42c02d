"""Float64 CPU oracle (test infrastructure only; see the package docstring for who may use it).

Each function restates one step of the path from the pages, in float64, with no blocking,
fusion or reordering beyond what the definition states.  Readings taken where the pages leave
a step open are marked READING and listed with the design notes.

Pages: [VT] VocabTrim (arXiv 2506.22694v2); [GL] glossary "Speculative decoding";
[RR] "A rejection rule keeps speculative decoding's output exact".
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------- decoding of stored inputs

def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> float64, exactly: a bf16 is the top 16 bits of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def as_f64(x, dtype: str) -> np.ndarray:
    """Logit storage -> float64: "f32" values widen exactly, "bf16" bit patterns decode exactly."""
    if dtype == "bf16":
        return bf16_to_f64(x)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------- [VT] §3 Eq. 1: trimmed LM head

def lm_head(hidden_bits, weight_bits, keep_ids=None) -> np.ndarray:
    """Draft logits over the trimmed vocabulary.

    [VT] §3, Eq. 1: the trimmed head W^Trim is W restricted to the kept rows Top-K(c, k), in
    that order; the drafter's logits are the hidden state times W^Trim transposed.  keep_ids=None
    is the untrimmed head (all rows, in id order).
    hidden_bits: bf16 [M, H]; weight_bits: bf16 [V_rows, H]; returns float64 [M, Vt].
    """
    h = bf16_to_f64(hidden_bits)
    rows = weight_bits if keep_ids is None else np.asarray(weight_bits)[np.asarray(keep_ids)]
    w = bf16_to_f64(rows)
    return h @ w.T


# ---------------------------------------------------------------- temperature softmax ([GL] conditions)

def softmax_temp(logits, T: float):
    """Per row: lse = log sum_j exp(l_j / T) and probabilities exp(l_j / T - lse).

    [GL] "Distributional exactness has conditions": temperature must be applied to the very
    distributions the correction uses, so p and q are both softmax(logits / T).
    Returns (lse float64 [rows], probs float64 [rows, n]).
    """
    x = np.asarray(logits, dtype=np.float64) / np.float64(T)
    m = x.max(axis=-1, keepdims=True)
    s = np.exp(x - m).sum(axis=-1, keepdims=True)
    lse = m + np.log(s)
    return lse[..., 0], np.exp(x - lse)


# ---------------------------------------------------------------- inverse-CDF draw ([RR] sampler)

def draw(w, u: float):
    """Inverse-CDF draw from non-negative weights w with one uniform u in (0, 1].

    [RR] "A target and a draft small enough to print in full", the categorical sampler: walk the
    tokens in order, accumulating mass, and return the first token whose running total reaches
    the uniform; fall back to the last token if rounding leaves none.
    READING: weights need not be normalised: the uniform is scaled by Z, the last entry of the
    same running total, and the comparison is u*Z <= C[i].  The fallback returns the last index
    with positive weight, so a zero-weight token is never returned.
    Returns (index, margin): margin is the distance from u to the nearest interior CDF boundary
    C[i]/Z (0 < C[i] < Z) on either side of the drawn token; draws whose margin is tiny are
    decided by rounding and are the only ones allowed to differ from an fp32 implementation.
    """
    w = np.asarray(w, dtype=np.float64)
    C = np.cumsum(w)
    Z = C[-1]
    t = np.float64(u) * Z
    hit = np.nonzero(t <= C)[0]
    if hit.size:
        idx = int(hit[0])
    else:
        idx = int(np.nonzero(w > 0)[0][-1])
    margin = np.inf
    for k in (idx - 1, idx):
        if 0 <= k < w.size and 0.0 < C[k] < Z:
            margin = min(margin, abs(np.float64(u) - C[k] / Z))
    return idx, float(margin)


def draft_draws(probs, u):
    """One draft token per row: z[m] = draw(q[m, :], u[m]) over the trimmed ids in keep_ids order.

    [VT] Appendix C.1, Algorithm 2: the trimmed drafter samples in its own (trimmed) index space.
    Returns (ids int64 [rows], margins float64 [rows]).
    """
    probs = np.asarray(probs, dtype=np.float64)
    ids = np.empty(probs.shape[0], dtype=np.int64)
    margins = np.empty(probs.shape[0], dtype=np.float64)
    for r in range(probs.shape[0]):
        ids[r], margins[r] = draw(probs[r], float(u[r]))
    return ids, margins


# ---------------------------------------------------------------- modified rejection sampling

def verify_sequence(p_rows, q_rows, draft_ids, keep_ids, u_acc, u_fin, gamma: int, correction="residual"):
    """Verify one sequence's block of gamma drafts.

    p_rows: float64 [gamma+1, V] target probabilities at positions 0..gamma (full-id order).
    q_rows: float64 [R >= gamma, Vt] draft probabilities (trimmed-id order, keep_ids order).
    draft_ids: [R] trimmed ids drafted at each position; the first gamma are verified.
    keep_ids: [Vt] trimmed id -> full id, or None when the draft head is untrimmed.

    Steps ([GL] "Why a rejection needs a special draw"; [RR] "What the accept/reject rule has to
    balance" and "Extending the rule from one token to a drafted run"):
      1. map each drafted trimmed id to its full id through keep_ids ([VT] Appendix C.1,
         Algorithm 2, the token index mapper T_{d->t});
      2. left to right, accept draft i iff u_acc[i] <= min(1, p_i(y_i) / q_i(x_i))
         (READING: "<=" as in the article's code); stop at the first rejection, n = its index,
         else n = gamma;
      3. on a rejection at n draw the final token from max(0, p_n - q_n) over the full
         vocabulary, with q_n = 0 off the kept set ([VT] §3: the trimmed drafter puts no mass
         there; [GL]: vocabulary filtering must be reflected in q); if every draft was accepted
         draw a bonus token from p_gamma;
      READING: a residual that sums to <= 0 falls back to p_n (cannot happen in exact
         arithmetic after a rejection).
    correction="naive" is the negative control of [GL]: redraw from the unadjusted p_n.

    Returns (tokens int64 [gamma+1] padded with -1, n, ratios of the tests performed,
    final-draw margin).  A test whose |u_acc - ratio| is tiny is decided by rounding.
    """
    p_rows = np.asarray(p_rows, dtype=np.float64)
    q_rows = np.asarray(q_rows, dtype=np.float64)
    V = p_rows.shape[1]
    full = (lambda x: int(x)) if keep_ids is None else (lambda x: int(keep_ids[x]))
    n = gamma
    ratios = []
    for i in range(gamma):
        x = int(draft_ids[i])
        y = full(x)
        ratio = min(1.0, p_rows[i, y] / q_rows[i, x])
        ratios.append(ratio)
        if not float(u_acc[i]) <= ratio:
            n = i
            break
    if n == gamma:
        w = p_rows[gamma]
    elif correction == "naive":
        w = p_rows[n]
    else:
        q_full = np.zeros(V)
        if keep_ids is None:
            q_full[:] = q_rows[n]
        else:
            q_full[np.asarray(keep_ids)] = q_rows[n]
        w = np.maximum(p_rows[n] - q_full, 0.0)
        if not w.sum() > 0.0:
            w = p_rows[n]
    final, fmargin = draw(w, float(u_fin))
    tokens = np.full(gamma + 1, -1, dtype=np.int64)
    for i in range(n):
        tokens[i] = full(draft_ids[i])
    tokens[n] = final
    return tokens, n, ratios, fmargin


def verify(target_logits, target_T, draft_logits, draft_T, draft_ids, keep_ids, u_acc, u_fin,
           gamma: int, correction="residual"):
    """Batched verification: B independent sequences, each as in verify_sequence.

    target_logits float64 [B, gamma+1, V]; draft_logits float64 [B, R, Vt]; draft_ids [B, R].
    Returns dict(tokens [B, gamma+1], n [B], accept_ratios (list of lists), final_margin [B],
    target_lse [B, gamma+1], draft_lse [B, R]).
    """
    B = target_logits.shape[0]
    t_lse, p = softmax_temp(target_logits, target_T)
    d_lse, q = softmax_temp(draft_logits, draft_T)
    tokens = np.empty((B, gamma + 1), dtype=np.int64)
    n = np.empty(B, dtype=np.int64)
    acc_m, fin_m = [], np.empty(B)
    for b in range(B):
        tokens[b], n[b], m, fin_m[b] = verify_sequence(p[b], q[b], draft_ids[b], keep_ids,
                                                       u_acc[b], u_fin[b], gamma, correction)
        acc_m.append(m)
    return dict(tokens=tokens, n=n, accept_ratios=acc_m, final_margin=fin_m,
                target_lse=t_lse, draft_lse=d_lse)


# ---------------------------------------------------------------- whole blocks

def block(hidden_bits, weight_bits, keep_ids, draft_logits, target, target_dtype, T, u_draft, u_acc,
          u_fin, gamma: int, R: int):
    """One speculative block for B sequences whose rows do not depend on the drafted ids.

    Draft logits come from lm_head (or are given directly when draft_logits is not None).
    [VT] Appendix C.1, Algorithm 2 (drafting through the trimmed head, then verification),
    with the verification rule of [GL]/[RR] (see verify_sequence).
    Returns a dict with every intermediate the GPU path also produces.
    """
    if draft_logits is None:
        draft_logits = lm_head(hidden_bits, weight_bits, keep_ids)
    d = np.asarray(draft_logits, dtype=np.float64)
    d_lse, q = softmax_temp(d, T)
    ids, dmargins = draft_draws(q, np.asarray(u_draft).reshape(-1))
    t = as_f64(target, target_dtype)
    B = t.shape[0]
    out = verify(t, T, d.reshape(B, R, -1), T, ids.reshape(B, R), keep_ids, u_acc, u_fin, gamma)
    out.update(draft_logits=d, draft_probs=q, draft_lse_flat=d_lse, draft_ids=ids.reshape(B, R),
               draft_margins=dmargins.reshape(B, R))
    return out


def toy_block(target_table, draft_table, T, gamma: int, u_draft, u_acc, u_fin, correction="residual"):
    """One block of the order-1 toy for B sequences, each starting from the start context (row 0).

    [RR] "Extending the rule from one token to a drafted run": draft token i is drawn from
    q(. | previous token), the target is evaluated at gamma+1 positions along the draft, then
    the block is verified.  Table row r is the context "previous token = r-1" (row 0: start).
    Returns dict(tokens [B, gamma+1], n [B], draft_ids [B, gamma], margins).
    """
    tt = np.asarray(target_table, dtype=np.float64)
    dt = np.asarray(draft_table, dtype=np.float64)
    _, P = softmax_temp(tt, T)
    _, Q = softmax_temp(dt, T)
    B = np.asarray(u_fin).shape[0]
    tokens = np.empty((B, gamma + 1), dtype=np.int64)
    n = np.empty(B, dtype=np.int64)
    ids = np.empty((B, gamma), dtype=np.int64)
    dmarg = np.empty((B, gamma))
    acc_m, fin_m = [], np.empty(B)
    for b in range(B):
        ctx = [0]
        for i in range(gamma):
            ids[b, i], dmarg[b, i] = draw(Q[ctx[-1]], float(u_draft[b, i]))
            ctx.append(int(ids[b, i]) + 1)
        tokens[b], n[b], m, fin_m[b] = verify_sequence(P[ctx], Q[ctx[:gamma]], ids[b], None, u_acc[b],
                                                       u_fin[b], gamma, correction)
        acc_m.append(m)
    return dict(tokens=tokens, n=n, draft_ids=ids, draft_margins=dmarg, accept_ratios=acc_m,
                final_margin=fin_m)


def toy_generate(target_table, draft_table, target_T: float, draft_T: float, gamma: int, n_tokens: int, u,
                 band: float = 0.0):
    """Chained blocks of the order-1 toy until each sequence has n_tokens tokens.

    [RR] "Extending the rule from one token to a drafted run", the generation loop: every block
    starts from the last token emitted so far (the start context for the first block), drafts
    gamma tokens autoregressively from q, verifies them against p at the gamma+1 positions along
    the draft, and appends the accepted drafts plus the corrected or bonus token; [VT] Appendix
    C.1, Algorithm 2 has the same loop around the trimmed drafter.  Table row r is the context
    "previous token = r-1" (row 0: start).  A trimmed draft is a draft table with -inf logits off
    the kept set.
    u: float32 [B, n_tokens, 2*gamma+1]; block j of sequence b reads u[b, j]: slots 0..gamma-1 for
    the drafts, gamma..2*gamma-1 for the accept tests, 2*gamma for the final draw (a block emits at
    least one token, so n_tokens blocks always suffice).
    Returns dict: tokens int64 [B, n_tokens]; per sequence blocks, tests (accept tests performed:
    n+1 after a rejection at n, gamma when all pass), accepted (sum of n), emitted (tokens of all
    blocks, including any past n_tokens in the last one); tie_block: index of the first block
    holding a decision within `band` of its uniform (n_tokens if none) and tie_token: the number
    of tokens emitted before that block.
    """
    _, P = softmax_temp(np.asarray(target_table, dtype=np.float64), target_T)
    _, Q = softmax_temp(np.asarray(draft_table, dtype=np.float64), draft_T)
    u = np.asarray(u, dtype=np.float32)
    B = u.shape[0]
    tokens = np.full((B, n_tokens), -1, dtype=np.int64)
    stats = {k: np.zeros(B, dtype=np.int64) for k in ("blocks", "tests", "accepted", "emitted")}
    tie_block = np.full(B, n_tokens, dtype=np.int64)
    tie_token = np.full(B, n_tokens, dtype=np.int64)
    for b in range(B):
        out, ctx, j = [], 0, 0
        while len(out) < n_tokens:
            ub = u[b, j]
            rows, ids, near = [ctx], [], False
            for i in range(gamma):
                x, m = draw(Q[rows[-1]], float(ub[i]))
                near |= m < band
                ids.append(x)
                rows.append(x + 1)
            toks, n, ratios, fm = verify_sequence(P[rows], Q[rows[:gamma]], ids, None, ub[gamma:2 * gamma],
                                                  ub[2 * gamma], gamma)
            near |= fm < band or any(abs(float(ub[gamma + i]) - r) < band for i, r in enumerate(ratios))
            if near and tie_block[b] == n_tokens:
                tie_block[b], tie_token[b] = j, len(out)
            out.extend(int(t) for t in toks[: n + 1])
            stats["tests"][b] += n + 1 if n < gamma else gamma
            stats["accepted"][b] += n
            stats["emitted"][b] += n + 1
            ctx = int(toks[n]) + 1
            j += 1
        stats["blocks"][b] = j
        tokens[b] = out[:n_tokens]
    return dict(tokens=tokens, tie_block=tie_block, tie_token=tie_token, **stats)


# ---------------------------------------------------------------- greedy verification

def argmax_lowest(row) -> int:
    """Index of the largest entry, the lowest such index on ties."""
    row = np.asarray(row, dtype=np.float64)
    return int(np.flatnonzero(row == row.max())[0])


def greedy_verify(target_logits, draft_ids, keep_ids, gamma: int):
    """Greedy verification of B sequences ([VT] §4: the target is decoded greedily, so a draft
    token is accepted only if it equals the target's most likely token; [VT] Appendix C.1,
    Algorithm 2: on the first mismatch the target's own token is appended and the block ends).
    READING: ties go to the lowest id; after gamma accepted drafts the target's most likely token
    at position gamma is appended (the bonus of the sampling rule, in its greedy limit).
    target_logits [B, gamma+1, V] (any temperature: the argmax does not depend on it);
    draft_ids [B, R] trimmed ids; keep_ids [Vt] or None.
    Returns (tokens int64 [B, gamma+1] padded with -1, n int64 [B])."""
    t = np.asarray(target_logits, dtype=np.float64)
    B = t.shape[0]
    tokens = np.full((B, gamma + 1), -1, dtype=np.int64)
    n = np.empty(B, dtype=np.int64)
    for b in range(B):
        k = gamma
        for i in range(gamma):
            x = int(draft_ids[b, i])
            y = x if keep_ids is None else int(keep_ids[x])
            if y != argmax_lowest(t[b, i]):
                k = i
                break
            tokens[b, i] = y
        tokens[b, k] = argmax_lowest(t[b, k])
        n[b] = k
    return tokens, n

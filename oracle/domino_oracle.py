"""Plain, slow, obviously-correct CPU oracle of the Domino draft-head hot path.

TEST INFRASTRUCTURE.  Nothing on the product path imports, calls or links this
module: only the test suite, the smoke check and the benchmark's CPU-baseline
leg do.  It shares no code, header, table or helper with the HIP library.

Every value is computed in float64 with numpy; bf16 inputs are widened
exactly.  Each function writes out the plain definition the pages give, in
the pages' order, with one library primitive (a matrix product) per step and
no blocking, fusion or reordering.

Pages cited (by title and section):
  [notes]     "完全开源的语言模型学习记录--推理加速Domino" (gsyq.cn news article)
  [explainer] the yhxrc.cn article on the Domino paper (Traditional Chinese,
              sections 一 … 七 and a Q&A)
  [abstract]  "Домино: отделение каузального моделирования от
              авторегрессивного формирования черновика …" (chatpaper.ai;
              Russian abstract with the English original)
  [chapter]   "大三本科生一作，交出7.92倍加速的投机解码新答卷！DeepSeek和阶跃星辰双双引用"
              (ai-engineering-6yk.pages.dev, Ch01.1513)

Readings of points the pages leave open (each is also listed with its reason
in the design notes):
  * GRU cell: PyTorch ``GRUCell`` convention, gate rows ordered r|z|n, reset
    gate applied to (W_hn g + b_hn), new state (1-z)*n + z*g.
  * GRU input: the frozen input-embedding row of the token, no scaling.
  * GRU starts from a zero state; its first input is x_t; position i uses the
    state after reading x_t, y_0 … y_{i-1}.  All K positions are drafted.
  * W1 input is [h_i ; g_i] (hidden state first).
  * Residual L_i = L_i^base + ΔL_i with no scale.
  * Biases are present in the GRU, W1 and W2; the LM head has none.
  * Sampler: greedy argmax at T = 0, Gumbel-max argmax(L/T + G) at T > 0 with
    G from a Philox4x32-10 counter generator (counter = (v>>2, i, b, offset),
    key = (seed lo32, seed hi32), word = output[v & 3],
    U = ((word >> 9) + 1/2) * 2^-23, G = -ln(-ln U)).
  * The token decision is taken on the score rounded to float32, and ties
    go to the lowest vocabulary index.  The contract compares free-running
    tokens exactly except at near-ties (top-2 margin below 2e-2); rounding a
    score of magnitude below ~100 to float32 moves it by under 1e-5, so the
    rounding can change a decision only where the margin is far inside that
    band, where any token within 2e-2 of the top is correct.  Deciding on the
    rounded score fixes which of several exactly equal float32 values wins.
  * Acceptance length: the bare length of the longest matching prefix.
  * Verification of a sampled draft (the pages report T = 1 decoding, verified
    in parallel by the target model, without the rule): standard speculative
    sampling (Leviathan, Kalman, Matias, ICML 2023; Chen et al. 2023).
    Position i is accepted when U_i * p_d(y_i) < p_t(y_i); at the first
    rejection the next token is drawn from max(0, p_t - p_d) (renormalised),
    after a fully accepted block from the target's distribution one past it.
    U_i is the Philox word of entry 0 at counter (0, i, b, offset) mapped as
    for the Gumbel noise; the resampling noise uses offset + 1.

Pins (``tests/test_oracle_pins.py``), each against something other than the
function itself:
  as_f64, base_logits      hand-worked product, one-hot rows, torch linear on
                           bf16-widened data
  sigmoid, silu            values at 0, 1 and the tails worked with math
  gru_cell                 torch GRUCell over several steps, zero-weight closed
                           form, scalar hand case
  correction_logits        torch linear/silu composition, concatenation order
  philox4x32_10            rocRAND's header-only engine built with g++
  philox_words             counter layout, uniformity and serial-pair chi^2
  gumbel_noise             uniform-map endpoints, chi^2 of Gumbel-max draws
                           against the tempered softmax
  sampling_scores          chi^2 at T = 1 and 0.5, T -> 0+ equals greedy
  pick_token, top2_margin  hand cases with ties
  draft_block              brute-force enumeration of every token sequence on
                           a micro head, an independent teacher-forced chain,
                           residual invariants
  base_draft               hand case, equality with draft_block at zero W2
  curriculum_*, cross_entropy, position_weights
                           torch cross_entropy, closed form log V, limits at
                           lambda = 0 / 1, hand case, autograd gradients
  correction_backward, gru_backward
                           torch autograd of the same compositions
  accept_len               all 6561 pairs at V = 3, K = 4; geometric closed form
  uniform01                the uniform behind the Gumbel noise of entry 0
  softmax                  two-entry closed form 1 / (1 + e^{a/T}), torch
                           softmax at T = 0.5, 0.8, 1.5
  verify_sampled           first emission distributed as the target (chi^2),
                           acceptance rate sum min(p_t, p_d), residual support,
                           equal distributions, zero target mass (the expected
                           probabilities written out independently)
``tests/test_oracle_mutations.py`` plants a mistake in each of these and
checks that the pins reject it.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "as_f64",
    "base_logits",
    "sigmoid",
    "silu",
    "gru_cell",
    "correction_logits",
    "philox4x32_10",
    "philox_words",
    "gumbel_noise",
    "sampling_scores",
    "pick_token",
    "draft_block",
    "base_draft",
    "curriculum_lambda",
    "position_weights",
    "cross_entropy",
    "curriculum_loss",
    "correction_backward",
    "gru_backward",
    "accept_len",
    "top2_margin",
    "uniform01",
    "softmax",
    "verify_sampled",
]

_MASK32 = np.uint64(0xFFFFFFFF)


def as_f64(x) -> np.ndarray:
    """Widen an input to float64: uint16 arrays are bf16 bit patterns (exact widening)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def base_logits(hidden: np.ndarray, lm_head: np.ndarray) -> np.ndarray:
    """L^base = h W_lm^T for every block position at once.

    [notes] §二.1(1): the backbone emits hidden states for every position of
    the block in one forward, and the frozen target LM head turns them into
    base logits; [explainer] §三 (second paragraph) says the same.
    hidden [..., d], lm_head [V, d] -> [..., V].
    """
    return as_f64(hidden) @ as_f64(lm_head).T


def sigmoid(x):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    """SiLU(x) = x * sigmoid(x) ([explainer] §四, the correction head's activation)."""
    return x * sigmoid(x)


def gru_cell(x, g, w_ih, w_hh, b_ih, b_hh):
    """One GRU update g' = GRU(x, g) in the PyTorch GRUCell convention.

    [notes] §二.1(2) item 1 and [explainer] §四: a GRU with hidden size 1024
    reads the embeddings of the already-sampled tokens one position at a time
    and keeps a running summary state.  The pages name only "GRU"; the gate
    equations below are the standard cell (rows r|z|n):
        a = W_ih x + b_ih,  c = W_hh g + b_hh
        r = σ(a_r + c_r),   z = σ(a_z + c_z),   n = tanh(a_n + r ⊙ c_n)
        g' = (1 - z) ⊙ n + z ⊙ g
    x [..., d_in], g [..., H].
    """
    H = g.shape[-1]
    a = x @ w_ih.T + b_ih
    c = g @ w_hh.T + b_hh
    r = sigmoid(a[..., 0:H] + c[..., 0:H])
    z = sigmoid(a[..., H:2 * H] + c[..., H:2 * H])
    n = np.tanh(a[..., 2 * H:3 * H] + r * c[..., 2 * H:3 * H])
    return (1.0 - z) * n + z * g


def correction_logits(h_i, g, w1, b1, w2, b2):
    """ΔL_i = W2 SiLU(W1 [h_i ; g] + b1) + b2.

    [notes] §二.1(2) item 2 and [explainer] §四 (low-rank correction head):
    concatenate the base hidden state with the causal (GRU) state, project to
    the rank-256 bottleneck with W1, apply SiLU, project to the vocabulary
    with W2.  h_i [..., d], g [..., H] -> [..., V].
    """
    z = np.concatenate([h_i, g], axis=-1)
    u = silu(z @ w1.T + b1)
    return u @ w2.T + b2


# ---------------------------------------------------------------------------
# Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
# as 1, 2, 3", SC'11).  The pages do not name a sampler; the Gumbel noise of
# the T > 0 sampler is drawn from this counter-based generator.
# ---------------------------------------------------------------------------
_PHILOX_M0 = np.uint64(0xD2511F53)
_PHILOX_M1 = np.uint64(0xCD9E8D57)
_PHILOX_W0 = np.uint64(0x9E3779B9)
_PHILOX_W1 = np.uint64(0xBB67AE85)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Ten Philox-4x32 rounds on counter (c0..c3) with key (k0, k1).

    Each round multiplies c0 and c2 by the two round multipliers into 64-bit
    products and forms the new counter (hi1^c1^k0, lo1, hi0^c3^k1, lo0); the
    key is advanced by the two Weyl constants between rounds.  Arguments are
    array-likes of 32-bit values; returns four uint64 arrays holding 32-bit words.
    """
    c0, c1, c2, c3, k0, k1 = (np.asarray(v, dtype=np.uint64) & _MASK32
                              for v in (c0, c1, c2, c3, k0, k1))
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + _PHILOX_W0) & _MASK32
            k1 = (k1 + _PHILOX_W1) & _MASK32
        p0 = _PHILOX_M0 * c0
        p1 = _PHILOX_M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def philox_words(seed: int, offset: int, b, i, v) -> np.ndarray:
    """The 32-bit random word for vocabulary entry v of position i of block b.

    Counter = (v >> 2, i, b, offset), key = (seed low 32 bits, seed high 32
    bits); the word is output lane v & 3.  Arguments broadcast.
    """
    v = np.asarray(v, dtype=np.uint64)
    b = np.asarray(b, dtype=np.uint64)
    i = np.asarray(i, dtype=np.uint64)
    off = np.asarray(offset, dtype=np.uint64)
    seed = int(seed)
    k0 = np.uint64(seed & 0xFFFFFFFF)
    k1 = np.uint64((seed >> 32) & 0xFFFFFFFF)
    shape = np.broadcast_shapes(v.shape, b.shape, i.shape, off.shape)
    c0 = np.broadcast_to(v >> np.uint64(2), shape)
    out = philox4x32_10(c0, np.broadcast_to(i, shape), np.broadcast_to(b, shape),
                        np.broadcast_to(off, shape), k0, k1)
    lane = np.broadcast_to(v & np.uint64(3), shape)
    word = np.choose(lane.astype(np.int64), out)
    return word.astype(np.uint32)


def gumbel_noise(seed: int, offset: int, b, i, v) -> np.ndarray:
    """G = -ln(-ln U) with U = ((word >> 9) + 1/2) * 2^-23, strictly inside (0, 1)."""
    w = philox_words(seed, offset, b, i, v).astype(np.float64)
    u = (np.floor(w / 512.0) + 0.5) * 2.0 ** -23
    return -np.log(-np.log(u))


def sampling_scores(logits, temperature: float, seed: int, offset: int, b: int, i: int):
    """Scores whose argmax is the drafted token.

    T = 0: the logits themselves (greedy decoding).  T > 0: Gumbel-max,
    L / T + G, which draws from softmax(L / T).  The pages report greedy
    (T = 0) and sampled (T = 1) decoding ([notes] §三.2(1); [explainer] §六)
    without naming the sampler.
    """
    if temperature < 0:
        raise ValueError("temperature must be >= 0")
    if temperature == 0.0:
        return np.asarray(logits, dtype=np.float64)
    V = logits.shape[-1]
    return logits / temperature + gumbel_noise(seed, offset, b, i, np.arange(V))


def pick_token(scores) -> int:
    """First index of the maximum, decided on the float32-rounded score."""
    s32 = np.asarray(scores, dtype=np.float64).astype(np.float32)
    return int(np.argmax(s32))


def draft_block(head: dict, hidden, x_t, teacher=None, temperature: float = 0.0,
                seed: int = 0, offset: int = 0, base=None, batch_index=None):
    """One draft block per batch row, position by position.

    [notes] §二.1 and [explainer] §三–§四, in their order:
      1. base logits for all K positions from the frozen LM head (one pass);
      2. for i = 0 … K-1: the GRU reads the embedding of the previous token
         (x_t for i = 0, then y_{i-1}; in teacher-forced mode teacher[b, i-1]),
         starting from a zero state;
      3. ΔL_i = W2 SiLU(W1 [h_i ; g_i] + b1) + b2 and L_i = L_i^base + ΔL_i;
      4. the token y_i is picked from L_i.
    Teacher forcing follows [notes] §二.2(1) / [explainer] §五 (the causal
    encoder is fed the reference tokens instead of the sampled ones).

    head: dict with lm_head, embed, w_ih, w_hh, b_ih, b_hh, w1, b1, w2, b2
    (float64 or bf16 bits).  hidden [B, K, d]; x_t [B]; teacher [B, K] or None.
    batch_index [B] (optional): the block index b that keys the sampler's
    random stream for each row (default 0 … B-1), so that a subset of a
    larger batch can be recomputed.
    Returns dict(tokens [B, K] int32, logits [B, K, V], states [B, K, H],
    scores [B, K, V], base [B, K, V]).
    """
    f = {k: as_f64(v) for k, v in head.items()}
    hidden = as_f64(hidden)
    x_t = np.asarray(x_t)
    B, K, _ = hidden.shape
    V = f["lm_head"].shape[0]
    H = f["w_hh"].shape[1]
    if base is None:
        base = base_logits(hidden, f["lm_head"])
    base = np.asarray(base, dtype=np.float64)
    tokens = np.zeros((B, K), dtype=np.int32)
    logits = np.zeros((B, K, V))
    states = np.zeros((B, K, H))
    scores = np.zeros((B, K, V))
    rows = np.arange(B) if batch_index is None else np.asarray(batch_index)
    for b in range(B):
        g = np.zeros(H)
        prev = int(x_t[b])
        for i in range(K):
            g = gru_cell(f["embed"][prev], g, f["w_ih"], f["w_hh"], f["b_ih"], f["b_hh"])
            states[b, i] = g
            dl = correction_logits(hidden[b, i], g, f["w1"], f["b1"], f["w2"], f["b2"])
            logits[b, i] = base[b, i] + dl
            scores[b, i] = sampling_scores(logits[b, i], temperature, seed, offset, int(rows[b]), i)
            tokens[b, i] = pick_token(scores[b, i])
            prev = int(teacher[b, i]) if teacher is not None else int(tokens[b, i])
    return {"tokens": tokens, "logits": logits, "states": states, "scores": scores,
            "base": base}


def base_draft(base, temperature: float = 0.0, seed: int = 0, offset: int = 0) -> np.ndarray:
    """Head-off drafting: every position's token from its base logits alone.

    The configuration the pages measure the head against: the parallel
    backbone drafts the block from L^base by itself ([notes] §二.1(1); the head
    ablation of [notes] §三 and [explainer] §六).  Without the correction
    L_i = L_i^base, so each position is picked on its own, with the same
    sampler as the draft loop.  base [B, K, V]; returns tokens [B, K] int32.
    """
    base = np.asarray(base, dtype=np.float64)
    B, K, _ = base.shape
    tokens = np.zeros((B, K), dtype=np.int32)
    for b in range(B):
        for i in range(K):
            tokens[b, i] = pick_token(sampling_scores(base[b, i], temperature, seed, offset, b, i))
    return tokens


def curriculum_lambda(step: int, total_steps: int) -> float:
    """λ_t of the base-anchored curriculum: 1 at the first training step,
    falling linearly to 0 at total_steps and staying there ([notes] §二.2(2))."""
    if total_steps <= 0:
        return 0.0
    return max(0.0, 1.0 - step / total_steps)


def position_weights(K: int, gamma: float) -> np.ndarray:
    """w_i = gamma^i: the per-position weights that decay exponentially along
    the block, so the early positions, whose acceptance gates the whole block,
    count most ([notes] §二.2(2)).  gamma in (0, 1]; the pages give no value."""
    return np.power(float(gamma), np.arange(K, dtype=np.float64))


def cross_entropy(logits, target: int) -> float:
    """-log softmax(logits)[target] = logsumexp(logits) - logits[target]."""
    x = np.asarray(logits, dtype=np.float64)
    m = x.max()
    return float(m + np.log(np.exp(x - m).sum()) - x[target])


def curriculum_loss(base, final, targets, lam: float, gamma: float):
    """The base-anchored curriculum loss ([notes] §二.2(2)):

        loss = (1 - λ) L_final + λ L_base,

    with L_x the cross-entropy of logits x against the reference token at
    each drafted position, weighted by w_i = gamma^i, averaged over positions
    with those weights (Σ_i w_i CE_i / Σ_i w_i) and then over blocks.  The
    final logits are the teacher-forced ones (the GRU reads the reference
    tokens, [notes] §二.2(1)), so targets[b, i] is both the label of position
    i and the GRU input of position i + 1.

    base, final [B, K, V]; targets [B, K].  Returns dict(loss, ce_base [B, K],
    ce_final [B, K], grad_base, grad_final): the gradients of loss with
    respect to base and final, [B, K, V] each.
    """
    base = np.asarray(base, dtype=np.float64)
    final = np.asarray(final, dtype=np.float64)
    B, K, V = base.shape
    w = position_weights(K, gamma)
    wsum = w.sum()
    ce_b = np.zeros((B, K))
    ce_f = np.zeros((B, K))
    g_b = np.zeros((B, K, V))
    g_f = np.zeros((B, K, V))
    loss = 0.0
    for b in range(B):
        for i in range(K):
            y = int(targets[b, i])
            ce_b[b, i] = cross_entropy(base[b, i], y)
            ce_f[b, i] = cross_entropy(final[b, i], y)
            loss += w[i] * ((1.0 - lam) * ce_f[b, i] + lam * ce_b[b, i])
            # d CE / d logits = softmax(logits) - onehot(y)
            for grad, x, coef in ((g_f, final[b, i], (1.0 - lam)), (g_b, base[b, i], lam)):
                p = np.exp(x - x.max())
                p /= p.sum()
                p[y] -= 1.0
                grad[b, i] = coef * w[i] / (wsum * B) * p
    return {"loss": loss / (wsum * B), "ce_base": ce_b, "ce_final": ce_f, "grad_base": g_b, "grad_final": g_f}


def correction_backward(head: dict, hidden, states, grad_final):
    """Gradients of a loss through the low-rank correction head, given the
    loss's gradient G with respect to the final logits of every position.

    The head computes z_i = W1 [h_i ; g_i] + b1, u_i = SiLU(z_i) and
    L_i = L_i^base + W2 u_i + b2 ([notes] §二.1(2) items 2-3); the base logits
    come from the frozen LM head and carry no parameters of the head.  By the
    chain rule, summing over every block b and position i:
        dW2 = Σ G_i u_iᵀ,  db2 = Σ G_i,  du_i = W2ᵀ G_i,
        dz_i = du_i ⊙ SiLU'(z_i),  SiLU'(z) = σ(z) (1 + z (1 - σ(z))),
        dW1 = Σ dz_i [h_i ; g_i]ᵀ,  db1 = Σ dz_i,  dg_i = W1[:, d:]ᵀ dz_i
    (dg_i is what the GRU's own backward through time starts from).
    hidden [B, K, d]; states [B, K, H] (the teacher-forced GRU states);
    grad_final [B, K, V].  Returns dict(dw2 [V, r], db2 [V], dw1 [r, d + H],
    db1 [r], dg [B, K, H]).
    """
    f = {k: as_f64(v) for k, v in head.items() if k in ("w1", "b1", "w2", "b2")}
    h = as_f64(hidden)
    g = np.asarray(states, dtype=np.float64)
    G = np.asarray(grad_final, dtype=np.float64)
    B, K, d = h.shape
    x = np.concatenate([h, g], axis=-1).reshape(B * K, -1)  # [h_i ; g_i] per row
    z = x @ f["w1"].T + f["b1"]
    sz = sigmoid(z)
    u = z * sz
    Gr = G.reshape(B * K, -1)
    du = Gr @ f["w2"]
    dz = du * sz * (1.0 + z * (1.0 - sz))
    return {"dw2": Gr.T @ u, "db2": Gr.sum(axis=0), "dw1": dz.T @ x, "db1": dz.sum(axis=0),
            "dg": (dz @ f["w1"][:, d:]).reshape(B, K, -1)}


def gru_backward(head: dict, x_t, teacher, states, dg):
    """Backward through time of the teacher-forced GRU causal encoder.

    Forward ([notes] §二.1(2) item 1, teacher forcing §二.2(1)): g_{-1} = 0,
    g_i = GRU(E[tok_i], g_{i-1}) with tok_0 = x_t and tok_i = teacher[i-1].
    Given dg[b, i], a loss's gradient with respect to g_i from outside the
    recurrence (the correction head's state gradient), the chain rule through
    g_i = (1 - z) n + z g_{i-1}, n = tanh(a_n + r (c_n)), r = σ(a_r + c_r),
    z = σ(a_z + c_z), a = W_ih e + b_ih, c = W_hh g_{i-1} + b_hh, from the last
    position back to the first, carrying the gradient of g_{i-1}.
    states [B, K, H] are the forward states g_i.  Returns dict(dw_ih [3H, d],
    dw_hh [3H, H], db_ih [3H], db_hh [3H]); the embedding table is frozen.
    """
    f = {k: as_f64(v) for k, v in head.items() if k in ("embed", "w_ih", "w_hh", "b_ih", "b_hh")}
    g_all = np.asarray(states, dtype=np.float64)
    dg = np.asarray(dg, dtype=np.float64)
    B, K, H = g_all.shape
    out = {"dw_ih": np.zeros_like(f["w_ih"]), "dw_hh": np.zeros_like(f["w_hh"]),
           "db_ih": np.zeros(3 * H), "db_hh": np.zeros(3 * H)}
    for b in range(B):
        carry = np.zeros(H)  # gradient reaching g_i from position i + 1
        for i in range(K - 1, -1, -1):
            tok = int(x_t[b]) if i == 0 else int(teacher[b, i - 1])
            e = f["embed"][tok]
            g_prev = g_all[b, i - 1] if i > 0 else np.zeros(H)
            a = f["w_ih"] @ e + f["b_ih"]
            c = f["w_hh"] @ g_prev + f["b_hh"]
            r = sigmoid(a[:H] + c[:H])
            z = sigmoid(a[H:2 * H] + c[H:2 * H])
            n = np.tanh(a[2 * H:] + r * c[2 * H:])
            d_g = dg[b, i] + carry
            d_n = d_g * (1.0 - z)
            d_z = d_g * (g_prev - n)
            d_pn = d_n * (1.0 - n * n)
            d_r = d_pn * c[2 * H:]
            d_pr = d_r * r * (1.0 - r)
            d_pz = d_z * z * (1.0 - z)
            da = np.concatenate([d_pr, d_pz, d_pn])
            dc = np.concatenate([d_pr, d_pz, d_pn * r])
            out["dw_ih"] += np.outer(da, e)
            out["db_ih"] += da
            out["dw_hh"] += np.outer(dc, g_prev)
            out["db_hh"] += dc
            carry = d_g * z + f["w_hh"].T @ dc
    return out


def accept_len(draft, target) -> np.ndarray:
    """τ per row: how many leading draft tokens equal the target's.

    [notes] §一.1 item 1: the acceptance length is the number of draft tokens
    one verification accepts in a row.  Returns the bare prefix length 0 … K.
    """
    draft = np.asarray(draft)
    target = np.asarray(target)
    out = np.zeros(draft.shape[0], dtype=np.int32)
    for b in range(draft.shape[0]):
        n = 0
        while n < draft.shape[1] and draft[b, n] == target[b, n]:
            n += 1
        out[b] = n
    return out


def top2_margin(scores) -> np.ndarray:
    """Gap between the largest and second-largest score along the last axis."""
    s = np.sort(np.asarray(scores, dtype=np.float64), axis=-1)
    if s.shape[-1] < 2:
        return np.full(s.shape[:-1], np.inf)
    return s[..., -1] - s[..., -2]


# ---------------------------------------------------------------------------
# Verification of a sampled draft (speculative sampling).  The pages report
# sampled decoding at T = 1 ([notes] §三.2(1): "采样解码（T=1）") and say that
# the target model verifies the drafted block in parallel ([abstract],
# English original, first sentence) without giving the acceptance rule; the
# rule below is the published one (Leviathan, Kalman, Matias, "Fast Inference
# from Transformers via Speculative Decoding", ICML 2023, Algorithm 1; Chen et
# al., "Accelerating Large Language Model Decoding with Speculative
# Sampling", 2023), which leaves the target's distribution unchanged.
# ---------------------------------------------------------------------------
def uniform01(seed: int, offset: int, b, i) -> np.ndarray:
    """U in (0, 1) for position i of block b: the Philox word of entry 0 at
    counter (0, i, b, offset), mapped as U = ((word >> 9) + 1/2) * 2^-23."""
    w = philox_words(seed, offset, b, i, 0).astype(np.float64)
    return (np.floor(w / 512.0) + 0.5) * 2.0 ** -23


def softmax(logits, temperature: float) -> np.ndarray:
    """softmax(L / T) along the last axis, in float64."""
    x = as_f64(logits) / temperature
    x = x - x.max(axis=-1, keepdims=True)
    e = np.exp(x)
    return e / e.sum(axis=-1, keepdims=True)


def verify_sampled(target_logits, draft_logits, draft, temperature: float, seed: int, offset: int):
    """Accepted prefix length and the next token of each drafted block.

    target_logits [B, K + 1, V]: the target model's logits at the K drafted
    positions and one past them; draft_logits [B, K, V]: the logits the draft
    tokens draft [B, K] were sampled from; both distributions are
    softmax(logits / T).  For i = 0 … K-1, position i is accepted when
    U_i p_d(y_i) < p_t(y_i), i.e. with probability min(1, p_t(y_i) / p_d(y_i));
    the first rejected position n ends the block and the next token is drawn
    from max(0, p_t - p_d) at n; if all K are accepted, n = K and the next
    token is drawn from p_t at position K.  Draws use Gumbel-max with noise
    G(b, n, v) at offset + 1: scores log max(0, p_t - p_d) + G (log 0 = -inf)
    or L_t / T + G.  Returns (accept [B] int32, next_token [B] int32, scores),
    scores [B, V] being the scores of each block's draw.
    """
    if not temperature > 0:
        raise ValueError("verification of a sampled draft needs T > 0")
    tl = as_f64(target_logits)
    dl = as_f64(draft_logits)
    draft = np.asarray(draft)
    B, K = draft.shape
    V = tl.shape[-1]
    accept = np.zeros(B, dtype=np.int32)
    nxt = np.zeros(B, dtype=np.int32)
    scores = np.zeros((B, V))
    for b in range(B):
        n = K
        for i in range(K):
            pt = softmax(tl[b, i], temperature)
            pd = softmax(dl[b, i], temperature)
            y = int(draft[b, i])
            if not (uniform01(seed, offset, b, i) * pd[y] < pt[y]):
                n = i
                break
        accept[b] = n
        g = gumbel_noise(seed, offset + 1, b, n, np.arange(V))
        if n < K:
            q = softmax(tl[b, n], temperature) - softmax(dl[b, n], temperature)
            with np.errstate(divide="ignore"):
                s = np.where(q > 0, np.log(np.where(q > 0, q, 1.0)), -np.inf) + g
        else:
            s = tl[b, K] / temperature + g
        scores[b] = s
        nxt[b] = pick_token(s)
    return accept, nxt, scores

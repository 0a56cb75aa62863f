"""Pins of the CPU oracle against things other than itself.

Each test fixes one part of the oracle with a closed form, a hand-worked
case, brute force on tiny inputs, an invariant, an independent library
routine (torch, rocRAND's header-only Philox engine) or a statistical law, so
that a dropped term, a wrong sign or index, or a transposed operand anywhere
in the oracle fails at least one of them.
"""
import itertools
import json
import math
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import oracle as O
import domino_synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _head(rng, d, H, r, V, scale=0.5):
    return {
        "lm_head": rng.normal(0, scale, (V, d)),
        "embed": rng.normal(0, scale, (V, d)),
        "w_ih": rng.normal(0, scale, (3 * H, d)),
        "w_hh": rng.normal(0, scale, (3 * H, H)),
        "b_ih": rng.normal(0, scale, (3 * H,)),
        "b_hh": rng.normal(0, scale, (3 * H,)),
        "w1": rng.normal(0, scale, (r, d + H)),
        "b1": rng.normal(0, scale, (r,)),
        "w2": rng.normal(0, scale, (V, r)),
        "b2": rng.normal(0, scale, (V,)),
    }


# ----------------------------------------------------------------- base logits
def test_base_logits_hand_example():
    h = np.array([[1.0, 2.0, 3.0]])
    w = np.array([[1.0, 0.0, -1.0], [2.0, 1.0, 0.0], [0.5, 0.5, 0.5]])
    # worked by hand: 1-3 = -2; 2+2 = 4; 0.5+1+1.5 = 3
    np.testing.assert_array_equal(O.base_logits(h, w), [[-2.0, 4.0, 3.0]])


def test_base_logits_one_hot_rows_select_components():
    rng = np.random.default_rng(3)
    d, V = 9, 20
    h = rng.normal(size=(2, 4, d))
    pick = rng.integers(0, d, size=V)
    w = np.zeros((V, d))
    w[np.arange(V), pick] = 1.0
    np.testing.assert_array_equal(O.base_logits(h, w), h[..., pick])


def test_base_logits_vs_torch_linear_and_bf16_widening():
    rng = np.random.default_rng(4)
    h = S.f32_to_bf16_bits(rng.normal(size=(2, 3, 64)).astype(np.float32))
    w = S.f32_to_bf16_bits(rng.normal(size=(50, 64)).astype(np.float32))
    th = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).double()
    tw = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).double()
    ref = torch.nn.functional.linear(th, tw).numpy()
    np.testing.assert_allclose(O.base_logits(h, w), ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------------------- GRU
def test_gru_matches_torch_grucell_over_steps():
    rng = np.random.default_rng(5)
    d, H = 7, 5
    cell = torch.nn.GRUCell(d, H).double()
    with torch.no_grad():
        for p in cell.parameters():
            p.copy_(torch.from_numpy(rng.normal(0, 0.7, p.shape)))
    xs = rng.normal(size=(6, 3, d))
    g = np.zeros((3, H))
    tg = torch.zeros(3, H, dtype=torch.float64)
    for x in xs:
        g = O.gru_cell(x, g, cell.weight_ih.detach().numpy(), cell.weight_hh.detach().numpy(),
                       cell.bias_ih.detach().numpy(), cell.bias_hh.detach().numpy())
        with torch.no_grad():
            tg = cell(torch.from_numpy(x), tg)
        np.testing.assert_allclose(g, tg.numpy(), rtol=0, atol=1e-13)


def test_gru_zero_weights_closed_form():
    # With W_ih = W_hh = 0 the gates are constants:
    #   z = σ(b_iz + b_hz), n = tanh(b_in + r b_hn), r = σ(b_ir + b_hr)
    # and from a zero state g_t = n (1 - z^(t+1)).
    rng = np.random.default_rng(6)
    d, H = 4, 6
    b_ih, b_hh = rng.normal(size=3 * H), rng.normal(size=3 * H)
    zero_ih, zero_hh = np.zeros((3 * H, d)), np.zeros((3 * H, H))
    r = 1 / (1 + np.exp(-(b_ih[:H] + b_hh[:H])))
    z = 1 / (1 + np.exp(-(b_ih[H:2 * H] + b_hh[H:2 * H])))
    n = np.tanh(b_ih[2 * H:] + r * b_hh[2 * H:])
    g = np.zeros(H)
    for t in range(5):
        g = O.gru_cell(rng.normal(size=d), g, zero_ih, zero_hh, b_ih, b_hh)
        np.testing.assert_allclose(g, n * (1 - z ** (t + 1)), rtol=0, atol=1e-14)


def test_gru_scalar_hand_case():
    # d = H = 1, worked with the math module: rows are (r, z, n).
    wi, wh = np.array([[0.5], [-1.0], [2.0]]), np.array([[1.5], [0.25], [-0.75]])
    bi, bh = np.array([0.1, 0.2, -0.3]), np.array([-0.2, 0.05, 0.4])
    x, g = 0.8, 0.3
    sig = lambda v: 1 / (1 + math.exp(-v))
    r = sig(0.5 * x + 0.1 + 1.5 * g - 0.2)
    z = sig(-1.0 * x + 0.2 + 0.25 * g + 0.05)
    n = math.tanh(2.0 * x - 0.3 + r * (-0.75 * g + 0.4))
    want = (1 - z) * n + z * g
    got = O.gru_cell(np.array([x]), np.array([g]), wi, wh, bi, bh)
    assert abs(got[0] - want) < 1e-15


# ------------------------------------------------------------------ correction
def test_correction_vs_torch_modules():
    rng = np.random.default_rng(7)
    d, H, r, V = 6, 4, 3, 11
    h, g = rng.normal(size=(2, d)), rng.normal(size=(2, H))
    w1, b1 = rng.normal(size=(r, d + H)), rng.normal(size=r)
    w2, b2 = rng.normal(size=(V, r)), rng.normal(size=V)
    t = lambda a: torch.from_numpy(a)
    ref = torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(torch.cat([t(h), t(g)], -1), t(w1), t(b1))),
        t(w2), t(b2)).numpy()
    np.testing.assert_allclose(O.correction_logits(h, g, w1, b1, w2, b2), ref, rtol=0, atol=1e-12)


def test_correction_concat_order_hidden_first():
    rng = np.random.default_rng(8)
    d, H, r, V = 5, 3, 2, 7
    w1, b1 = rng.normal(size=(r, d + H)), rng.normal(size=r)
    w2, b2 = rng.normal(size=(V, r)), rng.normal(size=V)
    w1_g_only = w1.copy()
    w1_g_only[:, :d] = 0.0  # only the GRU-state columns remain
    g = rng.normal(size=H)
    a = O.correction_logits(rng.normal(size=d), g, w1_g_only, b1, w2, b2)
    b = O.correction_logits(rng.normal(size=d), g, w1_g_only, b1, w2, b2)
    np.testing.assert_array_equal(a, b)  # the hidden state cannot reach the output
    c = O.correction_logits(rng.normal(size=d), rng.normal(size=H), w1_g_only, b1, w2, b2)
    assert np.abs(a - c).max() > 1e-3


def test_silu_values():
    assert O.silu(np.array(0.0)) == 0.0
    assert abs(O.silu(np.array(1.0)) - 1 / (1 + math.exp(-1))) < 1e-15
    assert abs(O.silu(np.array(-40.0))) < 1e-15
    assert abs(O.silu(np.array(40.0)) - 40.0) < 1e-12


def test_residual_invariants_in_draft_block():
    rng = np.random.default_rng(9)
    d, H, r, V, K, B = 8, 4, 3, 13, 5, 2
    head = _head(rng, d, H, r, V)
    hidden = rng.normal(size=(B, K, d))
    x_t = rng.integers(0, V, size=B)
    # W2 = 0, b2 = 0: the final logits are exactly the base logits.
    h0 = dict(head, w2=np.zeros((V, r)), b2=np.zeros(V))
    out = O.draft_block(h0, hidden, x_t)
    np.testing.assert_array_equal(out["logits"], O.base_logits(hidden, head["lm_head"]))
    # W_lm = 0: the final logits are exactly the correction.
    h1 = dict(head, lm_head=np.zeros((V, d)))
    out1 = O.draft_block(h1, hidden, x_t)
    teach = out1["tokens"]
    for b in range(B):
        g = np.zeros(H)
        prev = x_t[b]
        for i in range(K):
            g = O.gru_cell(head["embed"][prev], g, head["w_ih"], head["w_hh"], head["b_ih"], head["b_hh"])
            dl = O.correction_logits(hidden[b, i], g, head["w1"], head["b1"], head["w2"], head["b2"])
            np.testing.assert_array_equal(out1["logits"][b, i], 0.0 + dl)
            prev = teach[b, i]
    # ΔL is linear in (W2, b2): doubling both doubles L - L^base.
    h2 = dict(head, w2=2 * head["w2"], b2=2 * head["b2"])
    tf = rng.integers(0, V, size=(B, K))
    o1 = O.draft_block(head, hidden, x_t, teacher=tf)
    o2 = O.draft_block(h2, hidden, x_t, teacher=tf)
    np.testing.assert_allclose(o2["logits"] - o2["base"], 2 * (o1["logits"] - o1["base"]), atol=1e-12)


def test_base_draft_hand_case():
    # greedy: each position's largest base logit; a tie goes to the lower index
    base = np.array([[[0.1, 2.0, -1.0, 2.0, 0.3],
                      [5.0, -5.0, 4.9, 0.0, 1.0],
                      [-3.0, -2.0, -1.0, -0.5, -0.75]]])
    np.testing.assert_array_equal(O.base_draft(base), [[1, 0, 3]])


def test_base_draft_is_draft_block_without_correction():
    # head off (W2 = 0, b2 = 0) the draft loop drafts from the base logits alone,
    # greedy and sampled (the same noise stream keyed by block and position)
    rng = np.random.default_rng(17)
    d, H, r, V, K, B = 6, 4, 3, 29, 4, 3
    head = dict(_head(rng, d, H, r, V, scale=1.0), w2=np.zeros((V, r)), b2=np.zeros(V))
    hidden = rng.normal(size=(B, K, d))
    x_t = rng.integers(0, V, size=B)
    base = O.base_logits(hidden, head["lm_head"])
    for T, seed, offset in ((0.0, 0, 0), (0.7, 5, 3), (1.0, 2**40 + 7, 11)):
        want = O.draft_block(head, hidden, x_t, temperature=T, seed=seed, offset=offset)["tokens"]
        np.testing.assert_array_equal(O.base_draft(base, T, seed, offset), want)


# ------------------------------------------------------- curriculum loss
def test_curriculum_lambda_anneals_linearly():
    assert O.curriculum_lambda(0, 1000) == 1.0
    assert O.curriculum_lambda(250, 1000) == 0.75
    assert O.curriculum_lambda(1000, 1000) == 0.0
    assert O.curriculum_lambda(5000, 1000) == 0.0


def test_cross_entropy_matches_torch_and_closed_form():
    rng = np.random.default_rng(21)
    x = rng.normal(0, 3, size=(6, 37))
    y = rng.integers(0, 37, 6)
    want = torch.nn.functional.cross_entropy(torch.from_numpy(x), torch.from_numpy(y), reduction="none").numpy()
    got = np.array([O.cross_entropy(x[j], y[j]) for j in range(6)])
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    assert abs(O.cross_entropy(np.full(1000, 4.25), 17) - math.log(1000)) < 1e-12  # uniform: log V


def test_curriculum_loss_limits_match_torch_mean_cross_entropy():
    # gamma = 1 (equal weights): lambda = 0 is the mean CE of the final logits
    # over every (block, position), lambda = 1 that of the base logits
    rng = np.random.default_rng(22)
    B, K, V = 3, 5, 41
    base, final = rng.normal(0, 2, (B, K, V)), rng.normal(0, 2, (B, K, V))
    y = rng.integers(0, V, (B, K))
    ce = lambda L: torch.nn.functional.cross_entropy(torch.from_numpy(L.reshape(-1, V)),  # noqa: E731
                                                     torch.from_numpy(y.reshape(-1))).item()
    assert abs(O.curriculum_loss(base, final, y, 0.0, 1.0)["loss"] - ce(final)) < 1e-12
    assert abs(O.curriculum_loss(base, final, y, 1.0, 1.0)["loss"] - ce(base)) < 1e-12


def test_curriculum_loss_position_weights_hand_case():
    # one block of two positions, V = 2, gamma = 1/2, lambda = 1/4:
    # weights 1, 1/2 (sum 3/2); CE of [0, 0] against 0 is ln 2, CE of [ln 3, 0]
    # against 1 is ln 4
    base = np.array([[[0.0, 0.0], [math.log(3.0), 0.0]]])
    final = np.array([[[math.log(3.0), 0.0], [0.0, 0.0]]])
    y = np.array([[0, 1]])
    out = O.curriculum_loss(base, final, y, 0.25, 0.5)
    ce_base = [math.log(2.0), math.log(4.0)]
    ce_final = [math.log(4.0 / 3.0), math.log(2.0)]
    want = (1.0 * (0.75 * ce_final[0] + 0.25 * ce_base[0]) + 0.5 * (0.75 * ce_final[1] + 0.25 * ce_base[1])) / 1.5
    assert abs(out["loss"] - want) < 1e-12
    np.testing.assert_allclose(out["ce_base"][0], ce_base, rtol=1e-12)
    np.testing.assert_allclose(out["ce_final"][0], ce_final, rtol=1e-12)


def test_curriculum_loss_gradients_match_autograd():
    rng = np.random.default_rng(23)
    B, K, V, lam, gamma = 2, 4, 19, 0.3, 0.7
    base, final = rng.normal(0, 2, (B, K, V)), rng.normal(0, 2, (B, K, V))
    y = rng.integers(0, V, (B, K))
    out = O.curriculum_loss(base, final, y, lam, gamma)
    tb = torch.tensor(base, requires_grad=True)
    tf = torch.tensor(final, requires_grad=True)
    w = torch.tensor([gamma ** i for i in range(K)], dtype=torch.float64)
    ty = torch.from_numpy(y)
    ce_b = torch.nn.functional.cross_entropy(tb.permute(0, 2, 1), ty, reduction="none")  # [B, K]
    ce_f = torch.nn.functional.cross_entropy(tf.permute(0, 2, 1), ty, reduction="none")
    loss = (((1 - lam) * ce_f + lam * ce_b) * w).sum() / (w.sum() * B)
    loss.backward()
    assert abs(out["loss"] - loss.item()) < 1e-12
    np.testing.assert_allclose(out["grad_base"], tb.grad.numpy(), atol=1e-14)
    np.testing.assert_allclose(out["grad_final"], tf.grad.numpy(), atol=1e-14)
    np.testing.assert_allclose(out["grad_final"].sum(-1), 0.0, atol=1e-14)  # softmax - onehot sums to 0


def test_correction_backward_matches_autograd():
    rng = np.random.default_rng(24)
    B, K, d, H, r, V = 2, 3, 8, 4, 5, 11
    head = _head(rng, d, H, r, V, scale=0.7)
    hidden = rng.normal(size=(B, K, d))
    states = rng.normal(0, 0.5, size=(B, K, H))
    G = rng.normal(size=(B, K, V))
    out = O.correction_backward(head, hidden, states, G)
    t = {k: torch.tensor(head[k], requires_grad=True) for k in ("w1", "b1", "w2", "b2")}
    tg = torch.tensor(states, requires_grad=True)
    x = torch.cat([torch.from_numpy(hidden), tg], -1)
    dl = torch.nn.functional.linear(torch.nn.functional.silu(torch.nn.functional.linear(x, t["w1"], t["b1"])),
                                    t["w2"], t["b2"])
    (dl * torch.from_numpy(G)).sum().backward()
    for name, key in (("dw2", "w2"), ("db2", "b2"), ("dw1", "w1"), ("db1", "b1")):
        np.testing.assert_allclose(out[name], t[key].grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out["dg"], tg.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_gru_backward_matches_autograd():
    # the teacher-forced GRU chain in torch (GRUCell), loss = Σ <dg_i, g_i>
    rng = np.random.default_rng(25)
    B, K, d, H, r, V = 2, 4, 6, 5, 3, 9
    head = _head(rng, d, H, r, V, scale=0.6)
    x_t = rng.integers(0, V, size=B)
    teacher = rng.integers(0, V, size=(B, K))
    dg = rng.normal(size=(B, K, H))
    cell = torch.nn.GRUCell(d, H).double()
    with torch.no_grad():
        cell.weight_ih.copy_(torch.from_numpy(head["w_ih"])); cell.weight_hh.copy_(torch.from_numpy(head["w_hh"]))
        cell.bias_ih.copy_(torch.from_numpy(head["b_ih"])); cell.bias_hh.copy_(torch.from_numpy(head["b_hh"]))
    emb = torch.from_numpy(head["embed"])
    loss = 0.0
    states = np.zeros((B, K, H))
    for b in range(B):
        g = torch.zeros(1, H, dtype=torch.float64)
        for i in range(K):
            tok = int(x_t[b]) if i == 0 else int(teacher[b, i - 1])
            g = cell(emb[tok:tok + 1], g)
            states[b, i] = g.detach().numpy()[0]
            loss = loss + (g[0] * torch.from_numpy(dg[b, i])).sum()
    loss.backward()
    out = O.gru_backward(head, x_t, teacher, states, dg)
    for name, t in (("dw_ih", cell.weight_ih), ("dw_hh", cell.weight_hh), ("db_ih", cell.bias_ih),
                    ("db_hh", cell.bias_hh)):
        np.testing.assert_allclose(out[name], t.grad.numpy(), rtol=1e-10, atol=1e-12)


# ------------------------------------------------------------- loop wiring
def _torch_chain_logits(head, hidden_b, x_t, seq):
    """Independent re-derivation with torch modules: logits of every position when
    the GRU reads x_t, seq[0], ..., seq[K-2] (position i sees x_t and seq[:i])."""
    t = {k: torch.from_numpy(np.asarray(v, dtype=np.float64)) for k, v in head.items()}
    d = hidden_b.shape[-1]
    H = t["w_hh"].shape[1]
    cell = torch.nn.GRUCell(d, H).double()
    with torch.no_grad():
        cell.weight_ih.copy_(t["w_ih"]); cell.weight_hh.copy_(t["w_hh"])
        cell.bias_ih.copy_(t["b_ih"]); cell.bias_hh.copy_(t["b_hh"])
        emb = torch.nn.Embedding.from_pretrained(t["embed"])
        inputs = [int(x_t)] + [int(s) for s in seq[:-1]]
        g = torch.zeros(1, H, dtype=torch.float64)
        hb = torch.from_numpy(hidden_b)
        rows = []
        for i, tok in enumerate(inputs):
            g = cell(emb(torch.tensor([tok])), g)
            z = torch.cat([hb[i:i + 1], g], -1)
            u = torch.nn.functional.silu(z @ t["w1"].T + t["b1"])
            rows.append((hb[i] @ t["lm_head"].T + (u @ t["w2"].T + t["b2"])[0]).numpy())
    return np.stack(rows)


def test_greedy_loop_brute_force_enumeration():
    rng = np.random.default_rng(11)
    d, H, r, V, K = 3, 2, 2, 5, 4
    found_nontrivial = False
    for trial in range(4):
        head = _head(rng, d, H, r, V, scale=1.5)
        hidden = rng.normal(size=(1, K, d))
        x_t = np.array([rng.integers(0, V)])
        consistent = []
        for seq in itertools.product(range(V), repeat=K):
            L = _torch_chain_logits(head, hidden[0], x_t[0], seq)
            if all(int(np.argmax(L[i].astype(np.float32))) == seq[i] for i in range(K)):
                consistent.append(seq)
        assert len(consistent) == 1
        out = O.draft_block(head, hidden, x_t)
        assert tuple(out["tokens"][0]) == consistent[0]
        np.testing.assert_allclose(out["logits"][0], _torch_chain_logits(head, hidden[0], x_t[0], consistent[0]),
                                   atol=1e-12)
        # the chain really depends on the fed-back tokens in at least one trial
        alt = _torch_chain_logits(head, hidden[0], x_t[0], tuple((s + 1) % V for s in consistent[0]))
        found_nontrivial |= np.abs(alt[1:] - out["logits"][0][1:]).max() > 1e-6
    assert found_nontrivial


def test_teacher_forcing_feeds_teacher_tokens():
    rng = np.random.default_rng(12)
    d, H, r, V, K = 4, 3, 2, 9, 6
    head = _head(rng, d, H, r, V, scale=1.0)
    hidden = rng.normal(size=(2, K, d))
    x_t = rng.integers(0, V, size=2)
    teacher = rng.integers(0, V, size=(2, K))
    out = O.draft_block(head, hidden, x_t, teacher=teacher)
    for b in range(2):
        np.testing.assert_allclose(out["logits"][b], _torch_chain_logits(head, hidden[b], x_t[b], teacher[b]),
                                   atol=1e-12)
        assert all(out["tokens"][b, i] == np.argmax(out["logits"][b, i].astype(np.float32)) for i in range(K))


# --------------------------------------------------------------------- Philox
_ROCRAND_SRC = r"""
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cstdlib>
int main(int argc, char** argv) {
  // stdin: lines "seed subsequence offset"; prints the four words of next4()
  unsigned long long seed, sub, off;
  while (std::scanf("%llu %llu %llu", &seed, &sub, &off) == 3) {
    rocrand_device::philox4x32_10_engine e(seed, sub, off);
    uint4 r = e.next4();
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
"""


def _rocrand_words(cases):
    if shutil.which("g++") is None or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("g++ or the rocRAND headers are not available")
    with tempfile.TemporaryDirectory() as td:
        src, exe = os.path.join(td, "p.cpp"), os.path.join(td, "p")
        open(src, "w").write(_ROCRAND_SRC)
        subprocess.run(["g++", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", src, "-o", exe],
                       check=True, capture_output=True)
        inp = "".join(f"{s} {sub} {off}\n" for s, sub, off in cases)
        res = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True)
    return np.array([[int(x) for x in line.split()] for line in res.stdout.strip().splitlines()],
                    dtype=np.uint64)


def test_philox_matches_rocrand_engine():
    # rocRAND's engine(seed, subsequence, offset) starts from key = (seed lo, seed hi)
    # and counter = (offset/4 lo, offset/4 hi, subsequence lo, subsequence hi); its
    # first next4() is the Philox4x32-10 block of that counter.
    cases, ctrs2 = [], []
    # keep c1 < 2^30 so that 4 * (c0 | c1 << 32) stays below 2^64
    rng = np.random.default_rng(14)
    for _ in range(200):
        seed = int(rng.integers(0, 2 ** 62)) * 4 + int(rng.integers(0, 4))
        c = [int(rng.integers(0, 2 ** 32)), int(rng.integers(0, 2 ** 30)),
             int(rng.integers(0, 2 ** 32)), int(rng.integers(0, 2 ** 32))]
        cases.append((seed, c[2] | (c[3] << 32), 4 * (c[0] | (c[1] << 32))))
        ctrs2.append(c)
    ref = _rocrand_words(cases)
    c = np.array(ctrs2, dtype=np.uint64)
    seeds = np.array([s for s, _, _ in cases], dtype=np.uint64)
    got = O.philox4x32_10(c[:, 0], c[:, 1], c[:, 2], c[:, 3], seeds & np.uint64(0xFFFFFFFF),
                          seeds >> np.uint64(32))
    np.testing.assert_array_equal(np.stack(got, axis=1), ref)


def test_philox_words_counter_layout():
    seed, off = 0x1234_5678_9ABC_DEF0, 7
    v = np.arange(0, 64)
    w = O.philox_words(seed, off, 3, 5, v)
    blocks = O.philox4x32_10(v[::4] >> 2, 5, 3, off, seed & 0xFFFFFFFF, seed >> 32)
    np.testing.assert_array_equal(w.reshape(-1, 4), np.stack(blocks, axis=1).astype(np.uint32))


def test_philox_uniformity_and_independence():
    w = O.philox_words(0, 0, np.arange(4)[:, None, None], np.arange(16)[None, :, None],
                       np.arange(16384)[None, None, :]).reshape(-1).astype(np.int64)
    n = w.size  # 2^20 words
    counts = np.bincount(w >> 24, minlength=256)
    chi2 = ((counts - n / 256) ** 2 / (n / 256)).sum()
    assert chi2 < 255 + 6 * math.sqrt(2 * 255)
    bits = ((w[:, None] >> np.arange(32)) & 1).mean(0)
    assert np.abs(bits - 0.5).max() < 5 / math.sqrt(n)
    # serial pairs: consecutive words' top nibbles
    pairs = np.bincount(((w[:-1] >> 28) << 4) | (w[1:] >> 28), minlength=256)
    chi2p = ((pairs - (n - 1) / 256) ** 2 / ((n - 1) / 256)).sum()
    assert chi2p < 255 + 6 * math.sqrt(2 * 255)


def test_uniform_map_endpoints():
    # U = ((w >> 9) + 1/2) 2^-23 lies strictly inside (0, 1) and is exact in float32
    lo = (0 + 0.5) * 2.0 ** -23
    hi = ((2 ** 32 - 1 >> 9) + 0.5) * 2.0 ** -23
    assert 0 < lo and hi < 1 and np.float32(lo) == lo and np.float32(hi) == hi
    g = O.gumbel_noise(0, 0, 0, 0, np.arange(1 << 16))
    assert np.isfinite(g).all()
    assert g.min() >= -math.log(-math.log(lo)) - 1e-12 and g.max() <= -math.log(-math.log(hi)) + 1e-12


def test_verify_uniform_is_the_gumbel_uniform_of_entry_zero():
    # the acceptance uniform U_i is the uniform behind the Gumbel noise of
    # vocabulary entry 0 at the same counter: -ln(-ln U_i) equals that noise
    for seed, off in ((0, 0), (0xDEAD_BEEF_0123, 9), (2 ** 64 - 1, 2 ** 32 - 1)):
        b, i = np.arange(5)[:, None], np.arange(7)[None, :]
        u = O.uniform01(seed, off, b, i)
        assert ((u > 0) & (u < 1)).all()
        np.testing.assert_array_equal(-np.log(-np.log(u)), O.gumbel_noise(seed, off, b, i, 0))
        # and it is not the uniform of another entry of the same word
        assert not np.array_equal(-np.log(-np.log(u)), O.gumbel_noise(seed, off, b, i, 1))


def test_gumbel_max_matches_softmax_chi2():
    L = np.array([0.3, -1.2, 2.0, 0.0, 1.1, -0.4, 0.9, 1.6])
    for T in (1.0, 0.5):
        N = 200_000
        offs = np.arange(N)
        s = L[None, :] / T + O.gumbel_noise(42, offs[:, None], 0, 0, np.arange(8)[None, :])
        y = np.argmax(s.astype(np.float32), axis=1)
        counts = np.bincount(y, minlength=8)
        p = np.exp(L / T - (L / T).max())
        p /= p.sum()
        chi2 = ((counts - N * p) ** 2 / (N * p)).sum()
        assert chi2 < 24.3  # chi2(7) upper 0.1% point
        # the same offsets at another (b, i) give a different stream
        s2 = L[None, :] / T + O.gumbel_noise(42, offs[:1000, None], 1, 3, np.arange(8)[None, :])
        assert (np.argmax(s2, 1) != y[:1000]).any()


def test_small_temperature_is_greedy():
    rng = np.random.default_rng(15)
    L = rng.normal(size=(20, 300))
    for row in range(20):
        s = O.sampling_scores(L[row], 1e-6, 9, 0, 0, row)
        if O.top2_margin(L[row]) > 1e-4:
            assert O.pick_token(s) == int(np.argmax(L[row]))
    np.testing.assert_array_equal(O.sampling_scores(L[0], 0.0, 1, 0, 0, 0), L[0])
    with pytest.raises(ValueError):
        O.sampling_scores(L[0], -1.0, 1, 0, 0, 0)


def test_pick_token_ties_take_lowest_index():
    assert O.pick_token(np.array([1.0, 3.0, 3.0, 2.0])) == 1
    assert O.pick_token(np.zeros(10)) == 0
    # values equal only after float32 rounding tie as well
    assert O.pick_token(np.array([1.0, 1.0 + 1e-12])) == 0


def test_top2_margin():
    np.testing.assert_allclose(O.top2_margin(np.array([[1.0, 5.0, 4.5], [2.0, 2.0, 0.0]])), [0.5, 0.0])


# ---------------------------------------------------------- acceptance length
def test_accept_len_brute_force_all_pairs():
    V, K = 3, 4
    seqs = np.array(list(itertools.product(range(V), repeat=K)))
    draft = np.repeat(seqs, len(seqs), axis=0)
    target = np.tile(seqs, (len(seqs), 1))
    got = O.accept_len(draft, target)
    mism = draft != target
    want = np.where(mism.any(1), mism.argmax(1), K)
    np.testing.assert_array_equal(got, want)
    assert got.max() == K and got.min() == 0


def test_accept_len_geometric_closed_form():
    # Each position matches independently with p = 0.9 + 0.1/V, so
    # E[τ] = Σ_{k=1..16} p^k.
    V, K, N = 50, 16, 100_000
    draft = S.make_tokens((N, K), V, seed=3)
    target = S.make_targets(draft, V, p=0.9, seed=1)
    acc = O.accept_len(draft, target)
    p = 0.9 + 0.1 / V
    mean = sum(p ** k for k in range(1, K + 1))
    pk = np.array([p ** k * (1 - p) for k in range(K)] + [p ** K])
    var = (pk * np.arange(K + 1) ** 2).sum() - mean ** 2
    assert abs(acc.mean() - mean) < 5 * math.sqrt(var / N)
    freq = np.bincount(acc, minlength=K + 1) / N
    assert np.abs(freq - pk).max() < 0.005


# -------------------------------------------------------------- page constants
def test_head_parameter_count_matches_pages():
    g = json.load(open(os.path.join(GOLDEN, "page_constants.json")))
    w = S.get_workload("qwen3_8b_b1_greedy")
    assert (w.block, w.gru_hidden, w.rank) == (g["block"], g["gru_hidden"], g["rank"])
    no_bias = S.head_param_count(w, biases=False)
    with_bias = S.head_param_count(w, biases=True)
    # GRU 3H(d+H) = 15,728,640; W1 r(d+H) = 1,310,720; W2 V r = 38,895,616
    assert no_bias == 15_728_640 + 1_310_720 + 38_895_616 == 55_934_976
    assert round(no_bias / 1e6) == g["head_params_millions"]
    assert round(with_bias / 1e6) == g["head_params_millions"]
    # a GRU whose input were the GRU width instead of d would miss the pages' figure
    alt = 3 * 1024 * 1024 * 2 + 256 * (4096 + 1024) + 151936 * 256
    assert round(alt / 1e6) != g["head_params_millions"]


# ---------------------------------------------------------------------------
# Verification of a sampled draft (speculative sampling).  The defining
# property of the rule (Leviathan et al. 2023, Theorem 1; Chen et al. 2023):
# the token emitted at the first drafted position is distributed exactly as
# the target's p_t, whatever p_d is, and the draft token survives with
# probability sum_x min(p_t(x), p_d(x)).  Both are checked by sampling the
# draft token from p_d with an independent generator and running the oracle
# once per trial (its own Philox stream decides acceptance and resampling).
# ---------------------------------------------------------------------------
def _tempered_probs(logits, T):
    """softmax(L / T) written out independently of the oracle: exp(L / T - max) normalised."""
    x = np.asarray(logits, dtype=np.float64) / T
    e = np.exp(x - x.max())
    return e / e.sum()


def test_softmax_two_entry_closed_form():
    # logits [0, a] at temperature T: p_0 = 1 / (1 + e^{a/T}), p_1 = 1 - p_0
    for a in (-2.0, 0.3, 1.7):
        for T in (0.25, 0.5, 1.0, 1.5, 4.0):
            p = O.softmax(np.array([0.0, a]), T)
            p0 = 1.0 / (1.0 + math.exp(a / T))
            assert abs(p[0] - p0) < 1e-15 and abs(p[1] - (1.0 - p0)) < 1e-15, (a, T, p)


def test_softmax_matches_torch_at_several_temperatures():
    rng = np.random.default_rng(17)
    L = rng.normal(0, 2, (3, 4, 37))
    for T in (0.5, 0.8, 1.5):
        want = torch.softmax(torch.from_numpy(L) / T, dim=-1).numpy()
        np.testing.assert_allclose(O.softmax(L, T), want, rtol=1e-12, atol=1e-15)
    # bf16 bit patterns are widened before the division
    bits = S.f32_to_bf16_bits(rng.normal(0, 1, 64).astype(np.float32))
    want = torch.softmax(torch.from_numpy(bits.astype(np.int32) << 16).view(torch.float32).double() / 0.7, dim=-1)
    np.testing.assert_allclose(O.softmax(bits, 0.7), want.numpy(), rtol=1e-12, atol=1e-15)


def _verify_trials(t_logits, d_logits, T, n, seed0=1000):
    rng = np.random.default_rng(7)
    pd = _tempered_probs(d_logits, T)
    V = pd.size
    emitted = np.zeros(V)
    accepted = 0
    residual = np.zeros(V)
    tl = np.stack([t_logits, np.zeros(V)])[None]  # position 1 (the bonus) is never the first emission
    for k in range(n):
        y = int(rng.choice(V, p=pd))
        acc, nxt, _ = O.verify_sampled(tl, d_logits[None, None], np.array([[y]]), T, seed0 + k, 3)
        if acc[0] == 1:
            accepted += 1
            emitted[y] += 1
        else:
            emitted[nxt[0]] += 1
            residual[nxt[0]] += 1
    return emitted / n, accepted / n, residual


def test_verify_first_emission_follows_target_and_acceptance_rate():
    t = np.array([1.2, -0.3, 0.4, 0.0, -1.1])
    d = np.array([-0.2, 0.9, 0.4, -0.7, 0.5])
    T, n = 0.8, 6000
    emp, acc, _ = _verify_trials(t, d, T, n)
    pt, pd = _tempered_probs(t, T), _tempered_probs(d, T)
    sd = np.sqrt(pt * (1 - pt) / n)
    assert np.all(np.abs(emp - pt) < 5 * sd + 1e-9), (emp, pt)
    p_acc = np.minimum(pt, pd).sum()
    assert abs(acc - p_acc) < 5 * np.sqrt(p_acc * (1 - p_acc) / n), (acc, p_acc)


def test_verify_residual_draw_is_positive_part():
    t = np.array([2.0, 0.0, 0.0, -1.0])
    d = np.array([0.0, 1.5, 0.0, 0.5])
    T, n = 1.0, 4000
    _, _, res = _verify_trials(t, d, T, n)
    q = np.maximum(_tempered_probs(t, T) - _tempered_probs(d, T), 0.0)
    q /= q.sum()
    m = res.sum()
    assert m > 500
    sd = np.sqrt(q * (1 - q) / m)
    assert np.all(np.abs(res / m - q) < 5 * sd + 1e-9), (res / m, q)
    assert res[q == 0].sum() == 0  # entries where p_t <= p_d are never drawn


def test_verify_equal_distributions_accept_every_position():
    rng = np.random.default_rng(3)
    B, K, V = 3, 6, 11
    d = rng.normal(0, 1, (B, K, V))
    t = np.concatenate([d, rng.normal(0, 1, (B, 1, V))], axis=1)
    y = rng.integers(0, V, (B, K))
    for seed in range(40):
        acc, nxt, scores = O.verify_sampled(t, d, y, 1.3, seed, 9)
        assert np.all(acc == K)
        # the bonus draw is Gumbel-max over the target's last distribution
        g = O.gumbel_noise(seed, 10, np.arange(B)[:, None], K, np.arange(V)[None, :])
        assert np.array_equal(nxt, np.argmax(t[:, K] / 1.3 + g, axis=-1))


def test_verify_zero_target_mass_always_rejects():
    rng = np.random.default_rng(4)
    B, K, V = 2, 5, 9
    d = rng.normal(0, 1, (B, K, V))
    t = np.concatenate([d + rng.normal(0, 0.1, (B, K, V)), rng.normal(0, 1, (B, 1, V))], axis=1)
    y = rng.integers(0, V, (B, K))
    j = 2
    t[np.arange(B), j, y[:, j]] = -1e4  # p_t(y_j) underflows to 0
    for seed in range(30):
        acc, nxt, _ = O.verify_sampled(t, d, y, 1.0, seed, 0)
        assert np.all(acc <= j)
        assert np.all((acc < j) | (nxt != y[:, j]))


def test_verify_needs_positive_temperature():
    with pytest.raises(ValueError):
        O.verify_sampled(np.zeros((1, 2, 3)), np.zeros((1, 1, 3)), np.zeros((1, 1), dtype=int), 0.0, 0, 0)

"""Backward through the correction head on the GPU against the oracle: the
gradients of W2, b2, W1, b1 and of the GRU states from a given gradient on
the final logits, on the stress head (float32) and at Qwen3-8B shapes (bf16,
one and two blocks); repeatability; and the curriculum loss's logit gradient
fed through it."""
import numpy as np
import pytest
import torch

import domino_synth as S
import oracle as O
from _helpers import device_head, head_f64, log, workload_arrays

pytestmark = pytest.mark.gpu

REL_TOL = 1e-4  # float32 sums over up to 151936 terms (du) or 2048 rows, against float64


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import draft_block_causal_amd as D

    D.load_library()
    return torch.device("cuda:0")


def _compare(got, want, name):
    scale = float(np.abs(want).max()) or 1.0
    err = float(np.abs(got - want).max()) / scale
    assert err <= REL_TOL, f"{name}: max error {err:.2e} of the largest magnitude"
    return err


def _run(dev, w, batch, seed):
    import draft_block_causal_amd as D

    head_np, inp = workload_arrays(w, batch)
    f = head_f64(w)
    head = device_head(w, dev)
    rng = np.random.default_rng(seed)
    states = rng.normal(0.0, 0.3, size=(batch, w.block, w.gru_hidden)).astype(np.float32)
    G = (rng.normal(0.0, 1e-3, size=(batch, w.block, w.vocab))).astype(np.float32)
    hidden = S.to_torch(inp["hidden"], dev)
    out = D.domino_correction_backward(head, hidden, torch.from_numpy(states).to(dev), torch.from_numpy(G).to(dev))
    torch.cuda.synchronize()
    want = O.correction_backward(f, inp["hidden"], states, G)
    errs = {k: _compare(out["d_" + k[1:] if k != "dg" else "d_states"].cpu().numpy(), want[k], k)
            for k in ("dw2", "db2", "dw1", "db1", "dg")}
    log(f"backward {w.name} B={batch}: " + ", ".join(f"{k} {e:.1e}" for k, e in errs.items()))
    return out


@pytest.mark.parametrize("name,batch", [("tiny_stress_b4", 4), ("qwen3_8b_b1_greedy", 1), ("qwen3_8b_b1_greedy", 2),
                                        ("qwen3_8b_b1_greedy", 9), ("qwen3_8b_b1_greedy", 20),
                                        ("qwen3_8b_b1_greedy", 32)])
def test_backward_matches_oracle(dev, name, batch):
    # from 128 rows dW1 runs on the matrix cores: 9 blocks in one K slice (K
    # padded 144 -> 160 rows), 20 in two, 32 in four
    _run(dev, S.get_workload(name), batch, seed=batch + 3)


@pytest.mark.parametrize("batch", [3, 27])
def test_backward_small_bf16_head(dev, batch):
    # 15 rows (partial row tiles of z and dg) and 135 rows (dW1 on the matrix
    # cores with every tile partial) of a small bf16 head (d = 96, H = 64,
    # r = 32, V = 777)
    w = S.Workload(name="small_bf16", batch=3, block=5, d=96, vocab=777, gru_hidden=64, rank=32, dtype="bf16",
                   tied=False, temperature=0.0, init="fanin")
    _run(dev, w, batch, seed=17 + batch)


def test_backward_repeatable_bf16(dev):
    w = S.get_workload("qwen3_8b_b1_greedy")
    a = _run(dev, w, 2, seed=19)
    b = _run(dev, w, 2, seed=19)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_backward_repeatable(dev):
    w = S.get_workload("tiny_stress_b4")
    a = _run(dev, w, 4, seed=9)
    b = _run(dev, w, 4, seed=9)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_loss_gradient_through_the_head(dev):
    # teacher-forced forward, curriculum loss with its logit gradient, backward
    # through the head: against the oracle's same chain
    import draft_block_causal_amd as D

    w = S.get_workload("tiny_stress_b4")
    head_np, inp = workload_arrays(w)
    f = head_f64(w)
    head = device_head(w, dev)
    gold = S.make_tokens((w.batch, w.block), w.vocab, seed=41)
    hidden = S.to_torch(inp["hidden"], dev)
    base = D.domino_base_logits(head, hidden)
    final = torch.empty_like(base)
    states = torch.empty((w.batch, w.block, w.gru_hidden), device=dev)
    D.domino_draft_block(head, hidden, base, S.to_torch(inp["x_t"], dev), teacher=S.to_torch(gold, dev),
                         logits=final, gru_states=states)
    gf = torch.empty_like(final)
    D.domino_curriculum_loss(base, final, S.to_torch(gold, dev), 0.3, 0.9, grad_final=gf)
    out = D.domino_correction_backward(head, hidden, states, gf)
    torch.cuda.synchronize()
    ref = O.draft_block(f, O.as_f64(inp["hidden"]), inp["x_t"], teacher=gold)
    g = O.curriculum_loss(ref["base"], ref["logits"], gold, 0.3, 0.9)["grad_final"]
    want = O.correction_backward(f, inp["hidden"], ref["states"], g)
    for k, key in (("dw2", "d_w2"), ("db2", "d_b2"), ("dw1", "d_w1"), ("db1", "d_b1"), ("dg", "d_states")):
        got = out[key].cpu().numpy()
        err = float(np.abs(got - want[k]).max()) / (float(np.abs(want[k]).max()) or 1.0)
        log(f"training chain {k}: relative error {err:.1e}")
        assert err <= 1e-3, k

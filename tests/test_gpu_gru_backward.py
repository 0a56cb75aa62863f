"""Backward through time of the teacher-forced GRU on the GPU against the
oracle: the gradients of W_ih, W_hh, b_ih and b_hh from given state
gradients, on the stress head (float32) and at Qwen3-8B shapes (bf16, one and
two blocks); repeatability; and the whole training backward (loss gradient ->
correction head -> GRU) against the oracle's chain."""
import numpy as np
import pytest
import torch

import domino_synth as S
import oracle as O
from _helpers import device_head, head_f64, log, workload_arrays

pytestmark = pytest.mark.gpu

REL_TOL = 1e-4


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import draft_block_causal_amd as D

    D.load_library()
    return torch.device("cuda:0")


def _rel(got, want):
    return float(np.abs(got - want).max()) / (float(np.abs(want).max()) or 1.0)


def _forward_states(D, w, head, inp, gold, dev):
    hidden = S.to_torch(inp["hidden"], dev)
    base = D.domino_base_logits(head, hidden)
    final = torch.empty_like(base)
    states = torch.empty((hidden.shape[0], w.block, w.gru_hidden), device=dev)
    D.domino_draft_block(head, hidden, base, S.to_torch(inp["x_t"], dev), teacher=S.to_torch(gold, dev),
                         logits=final, gru_states=states)
    return hidden, base, final, states


def _run(dev, w, batch, seed):
    import draft_block_causal_amd as D

    head_np, inp = workload_arrays(w, batch)
    f = head_f64(w)
    head = device_head(w, dev)
    gold = S.make_tokens((batch, w.block), w.vocab, seed=seed)
    _, _, _, states = _forward_states(D, w, head, inp, gold, dev)
    dg = np.random.default_rng(seed).normal(0.0, 1e-2, size=(batch, w.block, w.gru_hidden)).astype(np.float32)
    out = D.domino_gru_backward(head, S.to_torch(inp["x_t"], dev), S.to_torch(gold, dev), states,
                                torch.from_numpy(dg).to(dev))
    torch.cuda.synchronize()
    want = O.gru_backward(f, inp["x_t"], gold, states.cpu().numpy(), dg)
    errs = {k: _rel(out["d_" + k[1:]].cpu().numpy(), want[k]) for k in ("dw_ih", "dw_hh", "db_ih", "db_hh")}
    log(f"gru backward {w.name} B={batch}: " + ", ".join(f"{k} {e:.1e}" for k, e in errs.items()))
    for k, e in errs.items():
        assert e <= REL_TOL, (k, e)
    return out


@pytest.mark.parametrize("name,batch", [("tiny_stress_b4", 4), ("qwen3_8b_b1_greedy", 1), ("qwen3_8b_b1_greedy", 2),
                                        ("qwen3_8b_b1_greedy", 9), ("qwen3_8b_b1_greedy", 20)])
def test_gru_backward_matches_oracle(dev, name, batch):
    # (from 128 rows the bf16 weight gradients run on the matrix cores; 9
    # blocks: 144 rows, padded to 160 along the GEMMs' K)
    _run(dev, S.get_workload(name), batch, seed=batch + 50)


def _small_bf16():
    # every matrix-core tile of the weight gradients partial: 3H = 192, d = 96, H = 64
    return S.Workload(name="small_bf16", batch=3, block=5, d=96, vocab=777, gru_hidden=64, rank=32, dtype="bf16",
                      tied=False, temperature=0.0, init="fanin")


@pytest.mark.parametrize("batch", [3, 27, 40])
def test_gru_backward_small_bf16_head(dev, batch):
    # 15 rows (float32 outer products); 135 and 200 rows on the matrix cores
    # (K padded to 160 / 224: the last 64-row tile holds 7 / 8 rows)
    _run(dev, _small_bf16(), batch, seed=batch + 80)


def test_gru_backward_repeatable_bf16(dev):
    w = S.get_workload("qwen3_8b_b1_greedy")
    a = _run(dev, w, 9, seed=62)
    b = _run(dev, w, 9, seed=62)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_gru_backward_repeatable(dev):
    w = S.get_workload("tiny_stress_b4")
    a = _run(dev, w, 4, seed=61)
    b = _run(dev, w, 4, seed=61)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_training_backward_chain(dev):
    # curriculum loss gradient -> correction head -> GRU through time, against
    # the oracle's chain on its own teacher-forced forward
    import draft_block_causal_amd as D

    w = S.get_workload("tiny_stress_b4")
    head_np, inp = workload_arrays(w)
    f = head_f64(w)
    head = device_head(w, dev)
    gold = S.make_tokens((w.batch, w.block), w.vocab, seed=71)
    hidden, base, final, states = _forward_states(D, w, head, inp, gold, dev)
    gf = torch.empty_like(final)
    D.domino_curriculum_loss(base, final, S.to_torch(gold, dev), 0.4, 0.85, grad_final=gf)
    cb = D.domino_correction_backward(head, hidden, states, gf)
    gb = D.domino_gru_backward(head, S.to_torch(inp["x_t"], dev), S.to_torch(gold, dev), states, cb["d_states"])
    torch.cuda.synchronize()
    ref = O.draft_block(f, O.as_f64(inp["hidden"]), inp["x_t"], teacher=gold)
    g = O.curriculum_loss(ref["base"], ref["logits"], gold, 0.4, 0.85)["grad_final"]
    dst = O.correction_backward(f, inp["hidden"], ref["states"], g)["dg"]
    want = O.gru_backward(f, inp["x_t"], gold, ref["states"], dst)
    for k in ("dw_ih", "dw_hh", "db_ih", "db_hh"):
        e = _rel(gb["d_" + k[1:]].cpu().numpy(), want[k])
        log(f"training backward chain {k}: relative error {e:.1e}")
        assert e <= 1e-3, k

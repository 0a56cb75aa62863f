"""The base-anchored curriculum loss on the GPU against the oracle: the loss,
the per-position cross-entropies and the logit gradients, at the Qwen3
vocabulary and ragged ones; in-place gradients; repeatability; and the whole
teacher-forced training forward (base logits, teacher-forced draft block,
loss) on the stress head."""
import numpy as np
import pytest
import torch

import domino_synth as S
import oracle as O
from _helpers import device_head, head_f64, log, workload_arrays

pytestmark = pytest.mark.gpu

CE_TOL = 1e-4    # float32 log-sum-exp over up to 151936 entries of values ~ 1: ~1e-6 relative
GRAD_RTOL = 1e-4


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import draft_block_causal_amd as D

    D.load_library()
    return torch.device("cuda:0")


def _inputs(B, K, V, seed):
    rng = np.random.default_rng(seed)
    base = rng.normal(0.0, 1.3, size=(B, K, V)).astype(np.float32)
    final = (base + rng.normal(0.0, 0.3, size=(B, K, V))).astype(np.float32)
    y = rng.integers(0, V, size=(B, K)).astype(np.int32)
    return base, final, y


@pytest.mark.parametrize("B,K,V,lam,gamma", [
    (1, 16, 151936, 1.0, 0.8),     # Qwen3 vocabulary, start of the curriculum
    (4, 16, 151936, 0.35, 0.9),    # mid-curriculum, several blocks
    (3, 5, 777, 0.0, 1.0),         # end of the curriculum, equal weights, ragged vocabulary
    (2, 7, 4099, 0.5, 0.5),        # ragged
    (64, 16, 4096, 0.25, 0.95),    # many rows
    (1, 1, 1, 0.5, 1.0),           # a one-entry vocabulary: every cross-entropy is 0
])
def test_loss_matches_oracle(dev, B, K, V, lam, gamma):
    import draft_block_causal_amd as D

    base, final, y = _inputs(B, K, V, seed=B * 7 + K)
    tb, tf, ty = (torch.from_numpy(a).to(dev) for a in (base, final, y))
    ce_b = torch.empty((B, K), device=dev)
    ce_f = torch.empty((B, K), device=dev)
    g_b = torch.empty_like(tb)
    g_f = torch.empty_like(tf)
    loss = D.domino_curriculum_loss(tb, tf, ty, lam, gamma, ce_base=ce_b, ce_final=ce_f, grad_base=g_b,
                                    grad_final=g_f)
    torch.cuda.synchronize()
    want = O.curriculum_loss(base, final, y, lam, gamma)
    err = abs(loss.item() - want["loss"])
    log(f"loss B={B} K={K} V={V} lam={lam} gamma={gamma}: {loss.item():.6f} vs {want['loss']:.6f} (err {err:.1e})")
    assert err <= CE_TOL
    np.testing.assert_allclose(ce_b.cpu().numpy(), want["ce_base"], atol=CE_TOL)
    np.testing.assert_allclose(ce_f.cpu().numpy(), want["ce_final"], atol=CE_TOL)
    for got, ref in ((g_b, want["grad_base"]), (g_f, want["grad_final"])):
        scale = max(np.abs(ref).max(), 1e-30)
        np.testing.assert_allclose(got.cpu().numpy(), ref, rtol=GRAD_RTOL, atol=1e-6 * scale)


def test_gradient_in_place_and_repeatable(dev):
    import draft_block_causal_amd as D

    base, final, y = _inputs(2, 16, 151936, seed=5)
    tb, tf, ty = (torch.from_numpy(a).to(dev) for a in (base, final, y))
    g_b, g_f = torch.empty_like(tb), torch.empty_like(tf)
    l1 = D.domino_curriculum_loss(tb, tf, ty, 0.4, 0.85, grad_base=g_b, grad_final=g_f).clone()
    l2 = D.domino_curriculum_loss(tb, tf, ty, 0.4, 0.85).clone()
    ib, if_ = tb.clone(), tf.clone()
    l3 = D.domino_curriculum_loss(ib, if_, ty, 0.4, 0.85, grad_base=ib, grad_final=if_)
    torch.cuda.synchronize()
    assert torch.equal(l1, l2) and torch.equal(l1, l3)
    assert torch.equal(ib, g_b) and torch.equal(if_, g_f)


def test_empty_batch_is_noop(dev):
    import draft_block_causal_amd as D

    z = torch.zeros((0, 16, 10), device=dev)
    loss = torch.full((1,), 7.0, device=dev)
    D.domino_curriculum_loss(z, z, torch.zeros((0, 16), dtype=torch.int32, device=dev), 0.5, 0.9, loss=loss)
    torch.cuda.synchronize()
    assert loss.item() == 7.0


def test_teacher_forced_training_forward(dev):
    # base logits, the teacher-forced draft block (the GRU reads the reference
    # tokens) and the curriculum loss, against the oracle's same chain
    import draft_block_causal_amd as D

    w = S.get_workload("tiny_stress_b4")
    head_np, inp = workload_arrays(w)
    f = head_f64(w)
    head = device_head(w, dev)
    gold = S.make_tokens((w.batch, w.block), w.vocab, seed=31)
    hidden = S.to_torch(inp["hidden"], dev)
    base = D.domino_base_logits(head, hidden)
    final = torch.empty_like(base)
    D.domino_draft_block(head, hidden, base, S.to_torch(inp["x_t"], dev), teacher=S.to_torch(gold, dev),
                         logits=final)
    loss = D.domino_curriculum_loss(base, final, S.to_torch(gold, dev), 0.3, 0.9)
    torch.cuda.synchronize()
    ref = O.draft_block(f, O.as_f64(inp["hidden"]), inp["x_t"], teacher=gold)
    want = O.curriculum_loss(ref["base"], ref["logits"], gold, 0.3, 0.9)
    err = abs(loss.item() - want["loss"])
    log(f"teacher-forced training forward ({w.name}): loss {loss.item():.6f} vs {want['loss']:.6f} (err {err:.1e})")
    assert err <= 1e-3

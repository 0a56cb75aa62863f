"""Base-only (head-off) drafting on the GPU against the oracle: greedy tokens
bit-exact (both sides decide on the same float32 logits); sampled tokens
identical except where the oracle's top-2 score margin is within the few-ulp
difference of the two Gumbel transforms (the GPU token must then score within
that tolerance of the maximum).  Also: a head whose correction is zero drafts
the same tokens through domino_draft_block."""
import numpy as np
import pytest
import torch

import domino_synth as S
import oracle as O
from _helpers import device_head, log, workload_arrays

pytestmark = pytest.mark.gpu

SCORE_TOL = 1e-3  # Gumbel noise: hardware log2 against libm, a few ulps of values up to ~17


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import draft_block_causal_amd as D

    D.load_library()
    return torch.device("cuda:0")


def _logits(B, K, V, seed, ties=False):
    rng = np.random.default_rng(seed)
    L = rng.normal(0.0, 1.3, size=(B, K, V)).astype(np.float32)
    if ties:  # the row maximum repeated at a later index: the lower index must win
        for b in range(B):
            for i in range(K):
                j = int(np.argmax(L[b, i]))
                L[b, i, (j + 1 + (V - 1) // 2) % V] = L[b, i, j]
    return L


def _check(L, tok, T, seed, offset):
    B, K, _ = L.shape
    want = O.base_draft(L.astype(np.float64), T, seed, offset)
    if T == 0.0:
        np.testing.assert_array_equal(tok, want)
        return 0
    near = 0
    for b in range(B):
        for i in range(K):
            if tok[b, i] == want[b, i]:
                continue
            s = O.sampling_scores(L[b, i].astype(np.float64), T, seed, offset, b, i).astype(np.float32)
            assert s.max() - s[tok[b, i]] <= SCORE_TOL, (b, i, tok[b, i], want[b, i])
            near += 1
    assert near <= max(1, B * K // 64)
    return near


@pytest.mark.parametrize("B,K,V,T,ties", [
    (1, 16, 151936, 0.0, True),    # Qwen3 vocabulary, one block, planted ties
    (4, 16, 151936, 1.0, False),   # sampled, several blocks
    (3, 5, 777, 0.0, True),        # ragged vocabulary (V % 4 != 0), short block
    (2, 7, 4099, 0.37, False),     # ragged, low temperature
    (128, 16, 4096, 0.0, False),   # many rows
    (1, 1, 1, 0.0, False),         # a one-entry vocabulary
])
def test_base_draft_matches_oracle(dev, B, K, V, T, ties):
    import draft_block_causal_amd as D

    L = _logits(B, K, V, seed=B * 31 + K, ties=ties)
    tok = D.domino_base_draft(torch.from_numpy(L).to(dev), T, seed=3, offset=5)
    torch.cuda.synchronize()
    tok = tok.cpu().numpy()
    near = _check(L, tok, T, 3, 5)
    log(f"base_draft B={B} K={K} V={V} T={T}: {near} near-tie differences")


def test_base_draft_empty_batch_is_noop(dev):
    import draft_block_causal_amd as D

    tok = D.domino_base_draft(torch.zeros((0, 16, 10), device=dev))
    assert tok.shape == (0, 16)


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_head_without_correction_drafts_base_tokens(dev, T):
    # W2 = 0 and b2 = 0: the draft loop's logits are the base logits, so it picks
    # what base-only drafting picks (same sampler stream)
    import draft_block_causal_amd as D

    w = S.get_workload("tiny_stress_b4")
    head_np, inp = workload_arrays(w)
    h = device_head(w, dev)
    tens = dict(h.tensors)
    tens["w2"] = torch.zeros_like(tens["w2"])
    tens["b2"] = torch.zeros_like(tens["b2"])
    head0 = D.Head(tens, block=w.block)
    hidden = S.to_torch(inp["hidden"], dev)
    base = D.domino_base_logits(head0, hidden)
    t_loop = D.domino_draft_block(head0, hidden, base, S.to_torch(inp["x_t"], dev), temperature=T, seed=4, offset=2)
    t_base = D.domino_base_draft(base, T, seed=4, offset=2)
    torch.cuda.synchronize()
    assert torch.equal(t_loop.cpu(), t_base.cpu())

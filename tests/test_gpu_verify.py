"""Sampled-draft verification (speculative sampling) on the GPU against the
oracle: accepted lengths bit-exact and next tokens identical, except where
the oracle's float64 decision is within rounding of flipping (then the GPU's
choice must be one the oracle rates as tied)."""
import numpy as np
import pytest
import torch

import domino_synth as S
import oracle as O
from _helpers import log

pytestmark = pytest.mark.gpu

ACCEPT_REL_TOL = 1e-4   # |U p_d - p_t| / p_t below this: the accept test may go either way
SCORE_TOL = 2e-3        # draw scores this close to the maximum count as tied


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _decision_margin(t, d, y, T, seed, offset, b, i):
    pt = O.softmax(t[b, i], T)[y[b, i]]
    pd = O.softmax(d[b, i], T)[y[b, i]]
    u = float(O.uniform01(seed, offset, b, i))
    return abs(u * pd - pt) / max(pt, 1e-300)


def _compare(t, d, y, T, seed, offset, acc_g, nxt_g):
    acc_o, nxt_o, scores = O.verify_sampled(t, d, y, T, seed, offset)
    B, K = y.shape
    flips = 0
    for b in range(B):
        if acc_g[b] != acc_o[b]:
            i = min(acc_g[b], acc_o[b])
            m = _decision_margin(t, d, y, T, seed, offset, b, i)
            assert m < ACCEPT_REL_TOL, f"block {b}: accept {acc_g[b]} vs oracle {acc_o[b]} (margin {m:.2e})"
            flips += 1
            continue
        if nxt_g[b] != nxt_o[b]:
            s32 = scores[b].astype(np.float32).astype(np.float64)
            top = s32.max()
            assert top - s32[nxt_g[b]] <= SCORE_TOL * max(1.0, abs(top)), \
                f"block {b}: next {nxt_g[b]} vs oracle {nxt_o[b]} (scores {s32[nxt_g[b]]} vs {top})"
            flips += 1
    return acc_o, flips


def _run(dev, B, K, V, spread, T, seed, offset):
    import draft_block_causal_amd as D
    t, d, y = S.make_verify_inputs(B, K, V, spread, seed=seed + 11)
    tt, dd, yy = (torch.from_numpy(a).to(dev) for a in (t, d, y))
    acc, nxt = D.domino_verify_sampled(tt, dd, yy, T, seed=seed, offset=offset)
    torch.cuda.synchronize()
    acc_g, nxt_g = acc.cpu().numpy(), nxt.cpu().numpy()
    assert np.all((acc_g >= 0) & (acc_g <= K)) and np.all((nxt_g >= 0) & (nxt_g < V))
    acc_o, flips = _compare(t, d, y, T, seed, offset, acc_g, nxt_g)
    log(f"verify B={B} K={K} V={V} spread={spread} T={T}: mean accept {acc_o.mean():.2f}, "
        f"{flips} near-tie differences")
    assert flips <= max(1, B // 16)
    return acc_g, nxt_g


@pytest.mark.parametrize("B,K,V,spread,T", [
    (1, 16, 151936, 0.05, 1.0),   # Qwen3 vocabulary, one block
    (32, 16, 151936, 0.2, 1.0),   # the T = 1 batch of 32 blocks (mean accepted length ~9.5)
    (3, 5, 777, 0.5, 0.7),        # small ragged vocabulary, low acceptance
    (7, 1, 4099, 0.2, 1.5),       # a single drafted position
    (5, 16, 2048, 0.0, 1.0),      # identical distributions: every position accepted
])
def test_verify_matches_oracle(dev, B, K, V, spread, T):
    acc_g, _ = _run(dev, B, K, V, spread, T, seed=B * 1000 + K, offset=40)
    if spread == 0.0:
        assert np.all(acc_g == K)


def test_verify_replays_identically(dev):
    a1 = _run(dev, 4, 16, 10007, 0.2, 1.0, seed=5, offset=8)
    a2 = _run(dev, 4, 16, 10007, 0.2, 1.0, seed=5, offset=8)
    assert all(np.array_equal(x, y) for x, y in zip(a1, a2))


def test_verify_empty_batch_is_noop(dev):
    import draft_block_causal_amd as D
    z = torch.zeros((0, 4, 10), dtype=torch.float32, device=dev)
    acc, nxt = D.domino_verify_sampled(torch.zeros((0, 5, 10), device=dev), z,
                                       torch.zeros((0, 4), dtype=torch.int32, device=dev), 1.0)
    assert acc.numel() == 0 and nxt.numel() == 0

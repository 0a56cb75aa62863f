"""domino_draft_block_noalloc on the GPU, through the C ABI: its scratch is the
library's fixed device array, and its outputs must equal those of
domino_draft_block (with a workspace) on the same inputs, bit for bit (same
kernels, same order of operations).  Two calls in a row, the second on a
smaller input, check that a call does not depend on what the previous one
left in the shared array."""
import numpy as np
import pytest
import torch

import domino_synth as S
from _helpers import device_head, log, workload_arrays

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import draft_block_causal_amd as D

    D.load_library()
    return torch.device("cuda:0")


def _both(D, head, w, inp, batch, dev, temperature, seed):
    hidden = S.to_torch(np.ascontiguousarray(inp["hidden"][:batch]), dev)
    x_t = S.to_torch(np.ascontiguousarray(inp["x_t"][:batch]), dev)
    base = D.domino_base_logits(head, hidden)
    outs = []
    for noalloc in (True, False):
        tok = torch.empty((batch, w.block), dtype=torch.int32, device=dev)
        lg = torch.empty((batch, w.block, w.vocab), dtype=torch.float32, device=dev)
        st = torch.empty((batch, w.block, w.gru_hidden), dtype=torch.float32, device=dev)
        if noalloc:
            D.domino_draft_block_noalloc(head, hidden, base, x_t, tok, temperature=temperature, seed=seed,
                                         logits=lg, gru_states=st)
        else:
            D.domino_draft_block(head, hidden, base, x_t, temperature=temperature, seed=seed, tokens=tok,
                                 logits=lg, gru_states=st)
        torch.cuda.synchronize()
        outs.append([x.cpu().numpy() for x in (tok, lg, st)])
    return outs


def _check(outs, w, label):
    (tn, ln, sn), (tw, lw, sw) = outs
    assert tn.min() >= 0 and tn.max() < w.vocab, f"{label}: no-alloc tokens out of range (a loop gave up?)"
    np.testing.assert_array_equal(tn, tw)
    np.testing.assert_array_equal(ln, lw)
    np.testing.assert_array_equal(sn, sw)
    log(f"{label}: no-alloc outputs equal the workspace call's ({tn.size} tokens)")


def test_noalloc_equals_workspace_call_twice_shrinking(dev, monkeypatch):
    import draft_block_causal_amd as D

    monkeypatch.delenv("DOMINO_LOOP", raising=False)
    w = S.get_workload("qwen3_8b_b32_t1")
    _, inp = workload_arrays(w, 32)
    head = device_head(w, dev)
    # 1: 32 blocks sampled (per-position kernels; the largest input the array takes)
    _check(_both(D, head, w, inp, 32, dev, 1.0, 11), w, "32 blocks, T = 1")
    # 2: a smaller input right after: 8 blocks greedy
    _check(_both(D, head, w, inp, 8, dev, 0.0, 0), w, "8 blocks, greedy")
    # 3 and 4: the single-block loop (GRU input table), two blocks then one
    D.domino_prepare_gru_table(head)
    try:
        _check(_both(D, head, w, inp, 2, dev, 1.0, 5), w, "2 blocks, table, T = 1")
        _check(_both(D, head, w, inp, 1, dev, 0.0, 0), w, "1 block, table, greedy")
    finally:
        head.set_gru_input_table(None)


def test_noalloc_refuses_more_than_its_array(dev):
    import draft_block_causal_amd as D

    w = S.get_workload("qwen3_8b_b128_accept").with_(batch=64)
    _, inp = workload_arrays(w, 64)
    head = device_head(w, dev)
    hidden = S.to_torch(inp["hidden"], dev)
    base = torch.empty((64, w.block, w.vocab), dtype=torch.float32, device=dev)
    tok = torch.empty((64, w.block), dtype=torch.int32, device=dev)
    with pytest.raises(D.DominoError) as ex:
        D.domino_draft_block_noalloc(head, hidden, base, S.to_torch(inp["x_t"], dev), tok)
    assert ex.value.status == -8

"""The draft call's completion status, through the C ABI on the GPU.

The single-block schedule's workgroups wait on one another with bounded
waits.  domino_draft_status reports whether every block's loop completed.
A give-up is forced from the host (DOMINO_DEBUG_SPIN_LIMIT=0 makes every wait
give up at its first check, so every workgroup leaves the loop at once and
the kernel ends normally); the call must then report status 1 and -1 tokens,
and the next normal call on the same workspace must report 0 again.
"""
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


def _draft(D, head, inp, batch, ws, dev, temperature=0.0):
    hidden = S.to_torch(np.ascontiguousarray(inp["hidden"][:batch]), dev)
    x_t = S.to_torch(np.ascontiguousarray(inp["x_t"][:batch]), dev)
    base = D.domino_base_logits(head, hidden)
    tok = D.domino_draft_block(head, hidden, base, x_t, temperature=temperature, seed=3, workspace=ws)
    st = D.domino_draft_status(head, batch, ws)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), int(st.cpu().numpy()[0])


@pytest.mark.parametrize("batch", [1, 2, 8, 20])
def test_on_chip_loop_give_up_is_reported(dev, batch, monkeypatch):
    # one block: the single-block loop; two: it once per block; 8 and 20: the
    # several-block loop (20 blocks: two launches)
    import draft_block_causal_amd as D

    monkeypatch.setenv("DOMINO_LOOP", "blocks" if batch > 2 else "default")
    w = S.get_workload("qwen3_8b_b32_t1").with_(batch=batch, temperature=0.0)
    _, inp = workload_arrays(w, batch)
    head = device_head(w, dev)
    D.domino_prepare_gru_table(head)
    try:
        ws = torch.empty(D.domino_workspace_size(head, batch), dtype=torch.uint8, device=dev)
        tok, st = _draft(D, head, inp, batch, ws, dev)
        log(f"B={batch}: normal call status {st}")
        assert st == 0 and tok.min() >= 0 and tok.max() < w.vocab
        monkeypatch.setenv("DOMINO_DEBUG_SPIN_LIMIT", "0")
        tok_f, st_f = _draft(D, head, inp, batch, ws, dev)
        log(f"B={batch}: forced give-up status {st_f}, tokens {np.unique(tok_f).tolist()}")
        assert st_f == 1
        assert (tok_f == -1).all()
        monkeypatch.delenv("DOMINO_DEBUG_SPIN_LIMIT")
        tok2, st2 = _draft(D, head, inp, batch, ws, dev)
        assert st2 == 0
        np.testing.assert_array_equal(tok2, tok)
    finally:
        head.set_gru_input_table(None)


def test_per_position_schedule_status_is_zero(dev, monkeypatch):
    # the per-position kernels never wait on one another; the status word is
    # cleared by the call and stays 0, even after a forced give-up elsewhere
    import draft_block_causal_amd as D

    monkeypatch.delenv("DOMINO_LOOP", raising=False)
    w = S.get_workload("qwen3_8b_b32_t1").with_(batch=8)
    _, inp = workload_arrays(w, 8)
    head = device_head(w, dev)
    ws = torch.empty(D.domino_workspace_size(head, 8), dtype=torch.uint8, device=dev)
    ws.fill_(0xFF)  # a stale non-zero status word from earlier use
    tok, st = _draft(D, head, inp, 8, ws, dev, temperature=1.0)
    assert st == 0 and tok.min() >= 0

"""A draft call recorded in a HIP graph (through torch's graph capture) and
replayed: every replay gives the tokens of the eager call, with eager calls
and synchronisations between the replays, for each schedule the library
picks (three kernels per position, the several-block loop, the single-block
loop that forms the base logits itself).  No call inside records a memset or
allocates.
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


def _small_bf16(batch):
    return S.Workload(name="small", batch=batch, block=3, d=96, vocab=777, gru_hidden=64, rank=32, dtype="bf16",
                      tied=False, temperature=1.0, init="fanin", philox_seed=5)


CASES = {
    # more than 16 blocks: gates, u and W2 kernels per position
    "per_position_kernels": lambda: _small_bf16(17),
    # 2 .. 16 blocks at the GRU width and rank the on-chip loops take
    "several_block_loop": lambda: S.get_workload("qwen3_4b_b8_tied").with_(batch=4, temperature=1.0,
                                                                            philox_seed=3),
    # one block, base logits formed inside the loop
    "single_block_loop": lambda: S.get_workload("qwen3_4b_b8_tied").with_(batch=1),
}


@pytest.mark.parametrize("case", list(CASES))
def test_graph_replays_match_eager(dev, case, monkeypatch):
    import draft_block_causal_amd as D

    monkeypatch.delenv("DOMINO_LOOP", raising=False)
    w = CASES[case]()
    log(f"graph capture: {case} B={w.batch} d={w.d} V={w.vocab}")
    _, inp = workload_arrays(w)
    head = device_head(w, dev)
    D.domino_prepare_gru_table(head)
    hidden = S.to_torch(np.ascontiguousarray(inp["hidden"]), dev)
    x_t = S.to_torch(np.ascontiguousarray(inp["x_t"]), dev)
    fused = case == "single_block_loop"
    base = None if fused else torch.empty((w.batch, w.block, w.vocab), dtype=torch.float32, device=dev)
    ws = torch.empty(D.domino_workspace_size(head, w.batch), dtype=torch.uint8, device=dev)
    tok = torch.empty((w.batch, w.block), dtype=torch.int32, device=dev)

    def call():
        if not fused:
            D.domino_base_logits(head, hidden, base)
        D.domino_draft_block(head, hidden, base, x_t, temperature=w.temperature, seed=w.philox_seed, tokens=tok,
                             workspace=ws)

    call()
    torch.cuda.synchronize()
    ref = tok.clone()
    assert int(ref.min()) >= 0 and int(ref.max()) < w.vocab
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for r in range(3):
        tok.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(tok, ref), f"replay {r} differs from the eager call"
        assert int(D.domino_draft_status(head, w.batch, ws).item()) == 0
        call()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(tok, ref)

"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Every input is seeded and synthetic (domino_synth).  Rules:
  * base logits, teacher-forced logits: max-abs error <= 2e-2;
  * GRU states: max-abs error <= 1e-3;
  * free-running tokens: identical to the oracle re-run teacher-forced on the
    GPU's own tokens, except where that oracle's top-2 margin is below 2e-2
    (the GPU token must then score within 2e-2 of the maximum);
  * accept lengths and Philox words: bit-exact.
Diagnostic bounds (5e-3 on logits, 1e-4 on states) sit beside the contract.
Every block of every workload is replayed, the full-size ones in chunks.
"""
import numpy as np
import pytest
import torch

import domino_synth as S
import oracle as O
from _helpers import (LOGIT_DIAG_TOL, LOGIT_TOL, STATE_DIAG_TOL, STATE_TOL, check_replay, device_head,
                      head_f64, log, workload_arrays)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import draft_block_causal_amd as D

    D.load_library()
    return torch.device("cuda:0")


def _t(a, dev):
    return S.to_torch(np.ascontiguousarray(a), dev)


def _gpu_block(D, head, hidden_t, base, x_t, teacher_t, w, dev):
    B, K, V, H = hidden_t.shape[0], w.block, w.vocab, w.gru_hidden
    logits = torch.empty((B, K, V), dtype=torch.float32, device=dev)
    states = torch.empty((B, K, H), dtype=torch.float32, device=dev)
    tok = D.domino_draft_block(head, hidden_t, base, x_t, teacher=teacher_t, temperature=w.temperature,
                               seed=w.philox_seed, offset=0, logits=logits, gru_states=states)
    return tok, logits, states


def _sampled_checks(w, f, inp, teacher, base_gpu, logits_tf, states_tf, n=4096, seed=123):
    """Oracle values at random (b, i, v) for every block, one definition at a time."""
    rng = np.random.default_rng(seed)
    B, K, V = inp["hidden"].shape[0], w.block, w.vocab
    hid = O.as_f64(inp["hidden"])
    bs, is_, vs = rng.integers(0, B, n), rng.integers(0, K, n), rng.integers(0, V, n)
    base_o = np.einsum("nk,nk->n", hid[bs, is_], f["lm_head"][vs])
    err = np.abs(base_gpu[bs, is_, vs] - base_o).max()
    assert err <= LOGIT_TOL, f"sampled base logits err {err}"
    # teacher-forced GRU states for every block, batched over blocks
    g = np.zeros((B, w.gru_hidden))
    prev = inp["x_t"].astype(np.int64)
    states = np.zeros((B, K, w.gru_hidden))
    for i in range(K):
        g = O.gru_cell(f["embed"][prev], g, f["w_ih"], f["w_hh"], f["b_ih"], f["b_hh"])
        states[:, i] = g
        prev = teacher[:, i].astype(np.int64)
    serr = np.abs(states_tf - states).max()
    assert serr <= STATE_TOL, f"teacher-forced GRU states err {serr}"
    uniq = np.unique(vs)
    dl = O.correction_logits(hid, states, f["w1"], f["b1"], f["w2"][uniq], f["b2"][uniq])
    col = np.searchsorted(uniq, vs)
    L = base_o + dl[bs, is_, col]
    lerr = np.abs(logits_tf[bs, is_, vs] - L).max()
    assert lerr <= LOGIT_TOL, f"sampled teacher-forced logits err {lerr}"
    return err, serr, lerr


def _parity(w, dev, check_blocks=None, sampled=False, table=False, chunk=16, fused=False):
    import draft_block_causal_amd as D

    log(f"{w.name}: generating inputs")
    head_np, inp = workload_arrays(w)
    f = head_f64(w)
    head = device_head(w, dev)
    if table:
        D.domino_prepare_gru_table(head)
    try:
        return _parity_run(D, w, dev, head, head_np, inp, f, check_blocks, sampled, chunk, fused)
    finally:
        head.set_gru_input_table(None)


def _parity_run(D, w, dev, head, head_np, inp, f, check_blocks, sampled, chunk, fused=False):
    """GPU base logits, a teacher-forced and a free-running draft of every block;
    the oracle re-runs the blocks in `check_blocks` (default: all of them) in
    chunks of `chunk` blocks: base logits, teacher-forced logits and GRU states,
    and the free-running tokens by the replay rule.  `fused`: the draft calls
    get no base logits and form them themselves (the drafted logits then check
    those).  Returns the free-running tokens (numpy) and the device tensor that
    holds them."""
    B, K, V = inp["hidden"].shape[0], w.block, w.vocab
    hidden_t = _t(inp["hidden"], dev)
    x_t = _t(inp["x_t"], dev)
    teacher = S.make_tokens((B, K), V, seed=7)
    teacher_t = _t(teacher, dev)
    log(f"{w.name}: GPU base logits + teacher-forced + free-running")
    base = D.domino_base_logits(head, hidden_t)
    draft_base = None if fused else base
    tok_tf, log_tf, st_tf = _gpu_block(D, head, hidden_t, draft_base, x_t, teacher_t, w, dev)
    tok_fr_t, log_fr, st_fr = _gpu_block(D, head, hidden_t, draft_base, x_t, None, w, dev)
    torch.cuda.synchronize()
    base_g = base.cpu().numpy()
    tok_tf, log_tf, st_tf = tok_tf.cpu().numpy(), log_tf.cpu().numpy(), st_tf.cpu().numpy()
    tok_fr, log_fr, st_fr = tok_fr_t.cpu().numpy(), log_fr.cpu().numpy(), st_fr.cpu().numpy()
    assert tok_fr.min() >= 0 and tok_fr.max() < V
    assert tok_tf.min() >= 0 and tok_tf.max() < V

    sel_all = np.arange(B) if check_blocks is None else np.asarray(check_blocks)
    errs = dict(base=0.0, tf=0.0, st=0.0, fr=0.0, fst=0.0)
    ties_tf = ties_fr = npos = 0
    for c0 in range(0, len(sel_all), chunk):
        sel = sel_all[c0:c0 + chunk]
        log(f"{w.name}: oracle on blocks {sel[0]}..{sel[-1]} ({len(sel)})")
        hid = O.as_f64(inp["hidden"][sel])
        base_o = O.base_logits(hid, f["lm_head"])
        errs["base"] = max(errs["base"], float(np.abs(base_g[sel] - base_o).max()))
        o_tf = O.draft_block(f, hid, inp["x_t"][sel], teacher=teacher[sel], temperature=w.temperature,
                             seed=w.philox_seed, base=base_o, batch_index=sel)
        errs["tf"] = max(errs["tf"], float(np.abs(log_tf[sel] - o_tf["logits"]).max()))
        errs["st"] = max(errs["st"], float(np.abs(st_tf[sel] - o_tf["states"]).max()))
        t, _ = check_replay(tok_tf[sel], o_tf, block_ids=sel)
        ties_tf += t
        del o_tf
        o_fr = O.draft_block(f, hid, inp["x_t"][sel], teacher=tok_fr[sel], temperature=w.temperature,
                             seed=w.philox_seed, base=base_o, batch_index=sel)
        errs["fr"] = max(errs["fr"], float(np.abs(log_fr[sel] - o_fr["logits"]).max()))
        errs["fst"] = max(errs["fst"], float(np.abs(st_fr[sel] - o_fr["states"]).max()))
        t, n = check_replay(tok_fr[sel], o_fr, block_ids=sel)
        ties_fr += t
        npos += n
        del o_fr, base_o
        # contract bounds first (they name the failure), then the diagnostic ones
        assert errs["base"] <= LOGIT_TOL, f"base logits err {errs['base']}"
        assert errs["tf"] <= LOGIT_TOL, f"teacher-forced logits err {errs['tf']}"
        assert errs["st"] <= STATE_TOL, f"teacher-forced GRU state err {errs['st']}"
        assert errs["fr"] <= LOGIT_TOL, f"free-running replay logits err {errs['fr']}"
        assert errs["fst"] <= STATE_TOL, f"free-running replay GRU state err {errs['fst']}"
        for k in ("base", "tf", "fr"):
            assert errs[k] <= LOGIT_DIAG_TOL, f"{k} logits err {errs[k]} above the diagnostic bound"
        for k in ("st", "fst"):
            assert errs[k] <= STATE_DIAG_TOL, f"{k} GRU state err {errs[k]} above the diagnostic bound"
    log(f"{w.name}: {len(sel_all)} blocks: base {errs['base']:.2e}  tf-logits {errs['tf']:.2e}  "
        f"states {errs['st']:.2e}  fr-logits {errs['fr']:.2e}  fr-states {errs['fst']:.2e}  "
        f"near-ties tf {ties_tf}/{npos} fr {ties_fr}/{npos}")
    if sampled:
        e = _sampled_checks(w, f, inp, teacher, base_g, log_tf, st_tf)
        log(f"{w.name}: sampled over all blocks: base {e[0]:.2e} states {e[1]:.2e} logits {e[2]:.2e}")
    return tok_fr, tok_fr_t


# ----------------------------------------------------------------- workloads
def test_tiny_f32_b1(dev):
    _parity(S.get_workload("tiny_f32_b1"), dev)


# "default" lets the library choose (for the tiny heads: one workgroup per
# block runs the whole loop); the others force a schedule
LOOP_MODES = ["default", "persistent", "multi"]


@pytest.mark.parametrize("mode", LOOP_MODES)
def test_tiny_stress_b4_greedy(dev, mode, monkeypatch):
    monkeypatch.setenv("DOMINO_LOOP", mode)
    _parity(S.get_workload("tiny_stress_b4"), dev)


@pytest.mark.parametrize("mode", LOOP_MODES)
def test_tiny_stress_b4_sampled(dev, mode, monkeypatch):
    monkeypatch.setenv("DOMINO_LOOP", mode)
    _parity(S.get_workload("tiny_stress_b4").with_(temperature=1.0, philox_seed=0x1234_5678_9ABC), dev)


@pytest.mark.parametrize("mode", LOOP_MODES)
def test_qwen3_8b_b1_greedy(dev, mode, monkeypatch):
    monkeypatch.setenv("DOMINO_LOOP", mode)
    _parity(S.get_workload("qwen3_8b_b1_greedy"), dev)


@pytest.mark.parametrize("mode", LOOP_MODES)
def test_qwen3_8b_b32_t1(dev, mode, monkeypatch):
    monkeypatch.setenv("DOMINO_LOOP", mode)
    _parity(S.get_workload("qwen3_8b_b32_t1"), dev, sampled=True)


@pytest.mark.parametrize("temperature", [0.0, 1.0])
def test_qwen3_8b_b1_gru_table(dev, temperature):
    # single block: the on-chip-weight loop, fed by the GRU input table
    _parity(S.get_workload("qwen3_8b_b1_greedy").with_(temperature=temperature, philox_seed=5), dev, table=True)


def test_qwen3_4b_b1_tied_gru_table(dev):
    _parity(S.get_workload("qwen3_4b_b8_tied").with_(batch=1), dev, table=True)


@pytest.mark.parametrize("name,kw", [
    ("qwen3_8b_b1_greedy", dict(temperature=0.0)),
    ("qwen3_8b_b1_greedy", dict(temperature=1.0, philox_seed=9)),
    ("qwen3_4b_b8_tied", dict(batch=1)),
    # a ragged last vocabulary tile and a short block
    ("qwen3_8b_b1_greedy", dict(vocab=150001, block=7, temperature=1.0, philox_seed=3)),
])
def test_draft_forms_base_logits(dev, name, kw):
    # no base logits passed: the single-block loop streams the LM head itself
    _parity(S.get_workload(name).with_(**kw), dev, table=True, fused=True)


def test_draft_forms_base_logits_refuses_other_shapes(dev):
    import draft_block_causal_amd as D

    w = S.get_workload("tiny_stress_b4")
    head_np, inp = workload_arrays(w)
    head = device_head(w, dev)
    hidden_t = _t(inp["hidden"], dev)
    with pytest.raises(D.DominoError) as e:
        D.domino_draft_block(head, hidden_t, None, _t(inp["x_t"], dev))
    assert e.value.status == -8


@pytest.mark.parametrize("case", ["qwen3_8b_b32_t1", "qwen3_4b_b8_tied", "tiny_stress_b4", "small_b17", "small_b65"])
def test_batched_gru_table(dev, case, monkeypatch):
    # several blocks with the GRU input table: the three-kernel schedule reads
    # T[token] instead of forming W_ih e
    monkeypatch.delenv("DOMINO_LOOP", raising=False)
    if case.startswith("small"):
        w = _small("bf16", batch=int(case[7:]), vocab=777, block=3, d=96, gru_hidden=64)
        _parity(w, dev, table=True)
    elif case == "tiny_stress_b4":
        _parity(S.get_workload(case).with_(temperature=1.0, philox_seed=7), dev, table=True)
    else:
        _parity(S.get_workload(case), dev, sampled=True, table=True)


@pytest.mark.parametrize("batch,temperature", [(2, 1.0), (3, 0.0)])
@pytest.mark.parametrize("mode", ["default", "perblock"])
def test_qwen3_8b_few_blocks_gru_table(dev, batch, temperature, mode, monkeypatch):
    # two or three Qwen3-8B blocks with the GRU input table: by default the
    # several-block loop; forced, the single-block loop once per block (two
    # blocks; three take the per-position kernels), its sampler keyed by each
    # block's own index
    if mode == "default":
        monkeypatch.delenv("DOMINO_LOOP", raising=False)
    else:
        monkeypatch.setenv("DOMINO_LOOP", mode)
    w = S.get_workload("qwen3_8b_b1_greedy").with_(batch=batch, temperature=temperature, philox_seed=9)
    _parity(w, dev, table=True)


def test_gru_table_matches_oracle(dev):
    import draft_block_causal_amd as D

    for name in ("tiny_stress_b4", "qwen3_8b_b1_greedy"):
        w = S.get_workload(name)
        workload_arrays(w)
        f = head_f64(w)
        head = device_head(w, dev)
        try:
            table = D.domino_prepare_gru_table(head).cpu().numpy()
        finally:
            head.set_gru_input_table(None)
        rows = np.random.default_rng(3).integers(0, w.vocab, 256)
        want = f["embed"][rows] @ f["w_ih"].T + f["b_ih"]
        err = np.abs(table[rows] - want).max()
        log(f"{name}: GRU input table max err {err:.2e}")
        assert err <= 1e-4


def test_qwen3_4b_b8_tied(dev):
    _parity(S.get_workload("qwen3_4b_b8_tied"), dev, sampled=True)


def _bn_head(batch, **kw):
    # GRU width 1024 and rank 256 (what the several-block on-chip loop takes),
    # a small ragged vocabulary and fan-in scaled weights, so the recurrence
    # moves the logits by O(1)
    base = dict(name=f"bn_b{batch}", batch=batch, block=16, d=256, vocab=20011, gru_hidden=1024, rank=256,
                dtype="bf16", tied=False, temperature=0.0, init="fanin")
    base.update(kw)
    return S.Workload(**base)


@pytest.mark.parametrize("batch,temperature,mode", [
    (3, 0.0, "default"), (5, 1.0, "default"), (8, 0.0, "default"), (16, 0.6, "default"), (17, 1.0, "blocks"),
    (2, 0.0, "blocks"), (2, 1.3, "blocks"),
])
def test_several_block_loop(dev, batch, temperature, mode, monkeypatch):
    """The several-block on-chip loop (GRU input table): partial and full
    8-block passes, a call split into two launches (17 blocks), two blocks when
    forced, greedy and sampled, logits and states written."""
    if mode == "default":
        monkeypatch.delenv("DOMINO_LOOP", raising=False)
    else:
        monkeypatch.setenv("DOMINO_LOOP", mode)
    _parity(_bn_head(batch, temperature=temperature, philox_seed=21 + batch), dev, table=True)


@pytest.mark.parametrize("batch,temperature", [(8, 0.0), (13, 1.0), (32, 1.0)])
def test_several_block_loop_tokens_only(dev, batch, temperature, monkeypatch):
    """The same loop without the logits and states outputs (the serving path):
    every block's tokens by the replay rule against the oracle."""
    import draft_block_causal_amd as D

    monkeypatch.setenv("DOMINO_LOOP", "blocks")
    w = _bn_head(batch, temperature=temperature, philox_seed=5)
    head_np, inp = workload_arrays(w)
    f = head_f64(w)
    head = device_head(w, dev)
    D.domino_prepare_gru_table(head)
    try:
        hidden_t = _t(inp["hidden"], dev)
        base = D.domino_base_logits(head, hidden_t)
        tok = D.domino_draft_block(head, hidden_t, base, _t(inp["x_t"], dev), temperature=w.temperature,
                                   seed=w.philox_seed).cpu().numpy()
    finally:
        head.set_gru_input_table(None)
    assert tok.min() >= 0 and tok.max() < w.vocab
    hid = O.as_f64(inp["hidden"])
    rep = O.draft_block(f, hid, inp["x_t"], teacher=tok, temperature=w.temperature, seed=w.philox_seed)
    ties, n = check_replay(tok, rep)
    log(f"{w.name}: tokens-only replay, near-ties {ties}/{n}")


def test_qwen3_8b_b128_accept(dev):
    """The 128-block workload as one composition, as the benchmark runs it (GRU
    input table): the GPU drafts every block (each replayed against the
    oracle), the targets are derived from that draft
    (each position kept with probability 0.9, else a uniform token), and
    domino_accept_len scores the GPU's own draft tensor, bit-exact against the
    oracle on the same arrays."""
    import draft_block_causal_amd as D

    w = S.get_workload("qwen3_8b_b128_accept")
    tok_np, tok_dev = _parity(w, dev, sampled=True, table=True)
    target = S.make_targets(tok_np, w.vocab, p=0.9, seed=1)
    acc = D.domino_accept_len(tok_dev, _t(target, dev)).cpu().numpy()
    want = O.accept_len(tok_np, target)
    np.testing.assert_array_equal(acc, want)
    log(f"{w.name}: accept lengths mean {acc.mean():.2f} (geometric expectation "
        f"{sum((0.9 + 0.1 / w.vocab) ** k for k in range(1, w.block + 1)):.2f}), "
        f"{int((acc == w.block).sum())} full blocks")


# ---------------------------------------------------------------- edge cases
def _small(dtype="bf16", **kw):
    base = dict(name="small", batch=3, block=5, d=64, vocab=1000, gru_hidden=32, rank=32, dtype=dtype,
                tied=False, temperature=0.0, init="fanin")
    base.update(kw)
    return S.Workload(**base)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_vocab_and_block(dev, dtype):
    # V = 1000 is not a multiple of the 16-row tile; K = 5 is odd
    _parity(_small(dtype), dev)


@pytest.mark.parametrize("batch", [16, 17, 33, 65])
@pytest.mark.parametrize("mode", LOOP_MODES)
def test_batch_tile_boundaries(dev, batch, mode, monkeypatch):
    monkeypatch.setenv("DOMINO_LOOP", mode if batch <= 32 else "multi")
    _parity(_small("bf16", batch=batch, vocab=777, block=3, d=96, gru_hidden=64), dev)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_w_hh_units_partial_gate_tile(dev, dtype, monkeypatch):
    # 65 blocks on the three-kernel schedule: the W2 launch forms W_hh g in
    # units of 64 gate rows x 32 batch rows; with H = 32 the 96 gate rows end
    # inside the second unit, and the last batch group holds one block
    monkeypatch.setenv("DOMINO_LOOP", "multi")
    _parity(_small(dtype, batch=65, vocab=777, block=3, d=96, gru_hidden=32), dev)


def test_lm_head_more_tiles_than_lds(dev):
    """Base logits when a workgroup finishes more 16-row tiles than it can hold.

    The LM-head kernel keeps each workgroup's output tiles in LDS until its
    last tile; at d = 1024 (bf16) there is room for 111 of them.  With
    V = 460000 (28750 tiles over 256 workgroups, 113 each) the last tiles of
    every workgroup are stored directly.  Every column of those tiles and
    10000 random others are checked against the oracle.
    """
    import draft_block_causal_amd as D

    w = S.Workload("lm_head_460k_d1024", 1, 16, 1024, 460000, 32, 32, "bf16", True, 0.0)
    log(f"{w.name}: generating inputs")
    head_np, inp = workload_arrays(w)
    head = device_head(w, dev)
    base = D.domino_base_logits(head, _t(inp["hidden"], dev))
    torch.cuda.synchronize()
    got = base.cpu().numpy()[0]
    ntiles = (w.vocab + 15) // 16
    tail = np.arange(ntiles - 2 * 256, ntiles)  # the last tiles of every workgroup
    cols = np.concatenate([(tail[:, None] * 16 + np.arange(16)).ravel(),
                           np.random.default_rng(5).integers(0, w.vocab, 10000)])
    cols = np.unique(cols[cols < w.vocab])
    ref = O.base_logits(O.as_f64(inp["hidden"][0]), O.as_f64(head_np["lm_head"][cols]))
    err = np.abs(got[:, cols] - ref).max()
    log(f"{w.name}: {cols.size} columns, max err {err:.2e}")
    assert err <= LOGIT_TOL, f"base logits err {err}"


@pytest.mark.parametrize("batch,vocab,d", [(2, 60001, 1024), (2, 460000, 1024), (2, 20011, 4096)])
def test_lm_head_row_slices_sharing_w(dev, batch, vocab, d):
    """Base logits for 2 blocks (32 rows) through the row-streaming kernel,
    whose two 16-row slices take the same W ranges on one XCD: ragged
    vocabularies, and at V = 460000 more tiles per workgroup than LDS holds
    (the rest are stored directly).  Every row of the last 600 columns and
    3000 random columns are checked against the oracle."""
    import draft_block_causal_amd as D

    w = S.Workload(f"lm_head_rows_b{batch}_v{vocab}", batch, 16, d, vocab, 32, 32, "bf16", True, 0.0)
    log(f"{w.name}: generating inputs")
    head_np, inp = workload_arrays(w)
    head = device_head(w, dev)
    base = D.domino_base_logits(head, _t(inp["hidden"], dev))
    torch.cuda.synchronize()
    got = base.cpu().numpy().reshape(batch * 16, vocab)
    cols = np.unique(np.concatenate([np.arange(vocab - 600, vocab),
                                     np.random.default_rng(batch).integers(0, vocab, 3000)]))
    hid = O.as_f64(inp["hidden"]).reshape(batch * 16, -1)
    ref = O.base_logits(hid, O.as_f64(head_np["lm_head"][cols]))
    err = np.abs(got[:, cols] - ref).max()
    log(f"{w.name}: {cols.size} columns x {batch * 16} rows, max err {err:.2e}")
    assert err <= LOGIT_TOL, f"base logits err {err}"


@pytest.mark.parametrize("batch,vocab,d", [(3, 20001, 256), (13, 65531, 256), (19, 5003, 256), (5, 20001, 4096),
                                           (19, 9001, 4096)])
def test_lm_head_tile_shapes(dev, batch, vocab, d):
    """Base logits through both shapes of the many-row matrix-core kernel.

    48 rows (one partial M tile) and 208 rows (two) take 128 x 256 tiles, 304
    rows take 256 x 256 tiles; every vocabulary is larger than the row-streaming
    kernel takes and ends in a partial tile.  At d = 4096 the 128-row tiles run
    with 8 waves (80 rows here).  All rows of the last 600 columns and 3000
    random columns are checked against the oracle.
    """
    import draft_block_causal_amd as D

    w = S.Workload(f"lm_head_b{batch}_v{vocab}_d{d}", batch, 16, d, vocab, 32, 32, "bf16", False, 0.0)
    log(f"{w.name}: generating inputs")
    head_np, inp = workload_arrays(w)
    head = device_head(w, dev)
    base = D.domino_base_logits(head, _t(inp["hidden"], dev))
    torch.cuda.synchronize()
    got = base.cpu().numpy().reshape(batch * 16, vocab)
    cols = np.unique(np.concatenate([np.arange(vocab - 600, vocab),
                                     np.random.default_rng(batch).integers(0, vocab, 3000)]))
    hid = O.as_f64(inp["hidden"]).reshape(batch * 16, -1)
    ref = O.base_logits(hid, O.as_f64(head_np["lm_head"][cols]))
    err = np.abs(got[:, cols] - ref).max()
    log(f"{w.name}: {cols.size} columns x {batch * 16} rows, max err {err:.2e}")
    assert err <= LOGIT_TOL, f"base logits err {err}"


@pytest.mark.parametrize("name,batch", [("qwen3_8b_b1_greedy", 8), ("qwen3_4b_b8_tied", 8), ("qwen3_8b_b1_greedy", 16)])
def test_lm_head_narrow_last_round(dev, name, batch):
    """128 or 256 rows against the full Qwen3 vocabulary: 594 tiles of M x 256
    on 256 compute units leave a last round of 82, which runs as 163 tiles of
    M x 128 in a second launch (8 waves at d = 4096, 4 at d = 2560), checked
    against the oracle at every fifth column past the full rounds (all
    rows), the 300 columns on either side of that boundary, and 4000 random
    columns."""
    import draft_block_causal_amd as D

    w = S.get_workload(name).with_(batch=batch)
    head_np, inp = workload_arrays(w)
    head = device_head(w, dev)
    base = D.domino_base_logits(head, _t(inp["hidden"], dev))
    torch.cuda.synchronize()
    V = w.vocab
    got = base.cpu().numpy().reshape(batch * w.block, V)
    n_full = (((V + 255) // 256) // 256) * 256 * 256  # columns of the full rounds on 256 CUs
    cols = np.unique(np.concatenate([np.arange(n_full, V, 5), np.arange(n_full - 300, n_full + 300),
                                     np.arange(V - 300, V), np.random.default_rng(5).integers(0, V, 4000)]))
    hid = O.as_f64(inp["hidden"]).reshape(batch * w.block, -1)
    ref = O.base_logits(hid, O.as_f64(head_np["lm_head"][cols]))
    err = np.abs(got[:, cols] - ref).max()
    log(f"{name} x {batch} blocks: {cols.size} columns x {batch * w.block} rows, max err {err:.2e}")
    assert err <= LOGIT_DIAG_TOL, f"base logits err {err}"


def test_sampled_small_temperature_and_ties(dev):
    _parity(_small("bf16", temperature=0.37, philox_seed=99), dev)


def test_all_equal_logits_pick_lowest_index(dev):
    import draft_block_causal_amd as D

    w = _small("bf16", batch=2)
    head_np, inp = S.make_workload(w)
    head_np = dict(head_np)
    for k in ("lm_head", "w2", "b2"):
        head_np[k] = np.zeros_like(head_np[k])
    t = {k: _t(v, dev) for k, v in head_np.items()}
    head = D.Head(t, block=w.block)
    hidden = _t(inp["hidden"], dev)
    base = D.domino_base_logits(head, hidden)
    tok = D.domino_draft_block(head, hidden, base, _t(inp["x_t"], dev))
    assert (tok.cpu().numpy() == 0).all()


def test_empty_batch_is_noop(dev):
    import draft_block_causal_amd as D

    w = _small("bf16")
    head_np, inp = S.make_workload(w, batch=0)
    head = D.Head({k: _t(v, dev) for k, v in head_np.items()}, block=w.block)
    hidden = _t(inp["hidden"], dev)
    base = D.domino_base_logits(head, hidden)
    tok = D.domino_draft_block(head, hidden, base, _t(inp["x_t"], dev))
    assert tok.shape == (0, w.block)
    acc = D.domino_accept_len(torch.zeros((0, 16), dtype=torch.int32, device=dev),
                              torch.zeros((0, 16), dtype=torch.int32, device=dev))
    assert acc.shape == (0,)


def test_teacher_last_position_is_unused(dev):
    import draft_block_causal_amd as D

    w = _small("bf16")
    head_np, inp = S.make_workload(w)
    head = D.Head({k: _t(v, dev) for k, v in head_np.items()}, block=w.block)
    hidden = _t(inp["hidden"], dev)
    base = D.domino_base_logits(head, hidden)
    teacher = S.make_tokens((w.batch, w.block), w.vocab, seed=3)
    outs = []
    for last in (0, w.vocab - 1):
        teacher[:, -1] = last
        lg = torch.empty((w.batch, w.block, w.vocab), device=dev)
        tok = D.domino_draft_block(head, hidden, base, _t(inp["x_t"], dev), teacher=_t(teacher, dev), logits=lg)
        outs.append((tok.cpu().numpy(), lg.cpu().numpy()))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])


def test_determinism_qwen3_8b_b1(dev):
    import draft_block_causal_amd as D

    w = S.get_workload("qwen3_8b_b1_greedy")
    _, inp = workload_arrays(w)
    head = device_head(w, dev)
    hidden, x_t = _t(inp["hidden"], dev), _t(inp["x_t"], dev)
    runs = []
    for _ in range(2):
        base = D.domino_base_logits(head, hidden)
        lg = torch.empty((1, w.block, w.vocab), device=dev)
        st = torch.empty((1, w.block, w.gru_hidden), device=dev)
        tok = D.domino_draft_block(head, hidden, base, x_t, logits=lg, gru_states=st)
        runs.append([x.cpu().numpy() for x in (base, tok, lg, st)])
    for a, b in zip(*runs):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("batch,table", [(2, True), (32, True), (32, False)])
def test_determinism_batched_schedules(dev, batch, table, monkeypatch):
    # the per-block single-block loop (2 blocks, GRU input table) and the
    # per-position kernels (32 blocks, sampled): two calls give the same bits
    import draft_block_causal_amd as D

    monkeypatch.delenv("DOMINO_LOOP", raising=False)
    w = S.get_workload("qwen3_8b_b32_t1").with_(batch=batch)
    _, inp = workload_arrays(w)
    head = device_head(w, dev)
    if table:
        D.domino_prepare_gru_table(head)
    try:
        hidden, x_t = _t(inp["hidden"], dev), _t(inp["x_t"], dev)
        runs = []
        for _ in range(2):
            base = D.domino_base_logits(head, hidden)
            lg = torch.empty((batch, w.block, w.vocab), device=dev)
            st = torch.empty((batch, w.block, w.gru_hidden), device=dev)
            tok = D.domino_draft_block(head, hidden, base, x_t, temperature=1.0, seed=3, logits=lg, gru_states=st)
            runs.append([x.cpu().numpy() for x in (base, tok, lg, st)])
        for a, b in zip(*runs):
            np.testing.assert_array_equal(a, b)
    finally:
        head.set_gru_input_table(None)


# --------------------------------------------------------------- bit-exact
@pytest.mark.parametrize("seed,offset,b,pos,v0,n", [
    (0, 0, 0, 0, 0, 4096),
    (0x0123_4567_89AB_CDEF, 7, 31, 15, 151000, 936),
    (2 ** 64 - 1, 2 ** 32 - 1, 127, 63, 3, 1001),
])
def test_philox_words_bit_exact(dev, seed, offset, b, pos, v0, n):
    import draft_block_causal_amd as D

    got = D.domino_debug_philox(seed, offset, b, pos, v0, n, device=dev).cpu().numpy().view(np.uint32)
    want = O.philox_words(seed, offset, b, pos, np.arange(v0, v0 + n))
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("nbytes", [0, 16, 4096 * 3 + 16, 10 << 20, (64 << 20) + 48])
def test_read_stream_xor(dev, nbytes):
    # the read-bandwidth calibration kernel reads every byte once: its XOR of
    # the 32-bit words matches the host's (ragged ranges included)
    import draft_block_causal_amd as D

    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(dev)
    sink = D.domino_debug_read_stream(buf)
    want = int(np.bitwise_xor.reduce(host)) if nbytes else 0
    assert int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))) == want


def test_accept_len_bit_exact_edges(dev):
    import draft_block_causal_amd as D

    rng = np.random.default_rng(5)
    for B, K in [(1, 1), (7, 16), (128, 16), (300, 33)]:
        draft = rng.integers(0, 5, size=(B, K)).astype(np.int32)
        target = np.where(rng.random((B, K)) < 0.8, draft, rng.integers(0, 5, size=(B, K))).astype(np.int32)
        target[0] = draft[0]  # a full match
        if B > 1:
            target[1, 0] = draft[1, 0] + 1  # an immediate mismatch
        got = D.domino_accept_len(_t(draft, dev), _t(target, dev)).cpu().numpy()
        np.testing.assert_array_equal(got, O.accept_len(draft, target))

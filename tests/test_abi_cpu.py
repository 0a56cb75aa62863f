"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
its host-side validation returns the documented status codes (no GPU call is
made for rejected arguments; accepted arguments fail cleanly without a GPU)."""
import ctypes
import os
import re

import pytest
import torch

import draft_block_causal_amd as D
from draft_block_causal_amd._lib import DominoHeadStruct

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "domino.h")

OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_ARG, E_WS, E_HIP, E_UNSUP = 0, -1, -2, -3, -4, -5, -6, -7, -8


@pytest.fixture(scope="module")
def lib():
    return D.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(domino_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(names) == sorted(D.EXPORTED)


def test_version_and_status_strings(lib):
    assert lib.domino_version() >= 100
    for code in range(-8, 1):
        assert lib.domino_status_string(code)
    assert lib.domino_status_string(-99) == b"unknown status"


def fake_head(**kw):
    base = 0x10000
    f = dict(d=256, vocab=4096, gru_hidden=128, rank=32, block=16, dtype=1)
    f.update({k: v for k, v in kw.items() if k in f})
    ptrs = {k: base * (i + 1) for i, k in enumerate(
        ["lm_head", "embed", "w_ih", "w_hh", "b_ih", "b_hh", "w1", "b1", "w2", "b2"])}
    ptrs.update({k: v for k, v in kw.items() if k in ptrs})
    return DominoHeadStruct(f["d"], f["vocab"], f["gru_hidden"], f["rank"], f["block"], f["dtype"],
                            *[ptrs[k] for k in ["lm_head", "embed", "w_ih", "w_hh", "b_ih", "b_hh", "w1", "b1",
                                                "w2", "b2"]], kw.get("gru_input_table"))


@pytest.mark.parametrize("kw,code", [
    ({}, OK),
    ({"dtype": 0}, OK),
    ({"dtype": 7}, E_DTYPE),
    ({"d": 0}, E_SHAPE),
    ({"d": 100}, E_SHAPE),
    ({"gru_hidden": 48}, E_SHAPE),
    ({"rank": 20}, E_SHAPE),
    ({"block": 0}, E_SHAPE),
    ({"block": 65}, E_SHAPE),
    ({"vocab": 0}, E_SHAPE),
    ({"lm_head": 0}, E_NULL),
    ({"w2": 0}, E_NULL),
    ({"b_ih": 0, "b_hh": 0, "b1": 0, "b2": 0}, OK),
    ({"w1": 0x10008}, E_ALIGN),
    ({"d": 4096}, OK),
    ({"d": 4128}, E_UNSUP),
    ({"d": 4096, "dtype": 0}, E_UNSUP),
    ({"d": 2048, "dtype": 0}, OK),
    ({"gru_input_table": 0x900000}, OK),
    ({"gru_input_table": 0x900004}, E_ALIGN),
    ({"vocab": 1 << 24}, E_UNSUP),
])
def test_check_head(lib, kw, code):
    h = fake_head(**kw)
    assert lib.domino_check_head(ctypes.byref(h)) == code
    assert lib.domino_check_head(None) == E_NULL


def test_gru_table_size_and_prepare_validation(lib):
    h = fake_head(d=4096, vocab=151936, gru_hidden=1024, rank=256)
    sz = ctypes.c_size_t(0)
    assert lib.domino_gru_table_size(ctypes.byref(h), ctypes.byref(sz)) == OK
    assert sz.value == 151936 * 3 * 1024 * 4
    assert lib.domino_gru_table_size(ctypes.byref(h), None) == E_NULL
    assert lib.domino_prepare_gru_table(ctypes.byref(h), None, None) == E_NULL
    assert lib.domino_prepare_gru_table(ctypes.byref(h), 0x900004, None) == E_ALIGN
    bad = fake_head(d=100)
    assert lib.domino_prepare_gru_table(ctypes.byref(bad), 0x900000, None) == E_SHAPE


def test_workspace_size(lib):
    h = fake_head(d=4096, vocab=151936, gru_hidden=1024, rank=256)
    sz = ctypes.c_size_t(0)
    assert lib.domino_workspace_size(ctypes.byref(h), 1, ctypes.byref(sz)) == OK
    one = sz.value
    assert one > 0 and one % 256 == 0
    assert lib.domino_workspace_size(ctypes.byref(h), 128, ctypes.byref(sz)) == OK
    assert sz.value > one
    assert lib.domino_workspace_size(ctypes.byref(h), -1, ctypes.byref(sz)) == E_SHAPE
    assert lib.domino_workspace_size(ctypes.byref(h), 129, ctypes.byref(sz)) == E_UNSUP
    assert lib.domino_workspace_size(ctypes.byref(h), 1, None) == E_NULL


def _draft(lib, h, batch=1, hidden=0x20000, base=0x30000, x_t=0x40000, teacher=None, temp=0.0, tokens=0x50000,
           logits=None, states=None, ws=0x100000, ws_bytes=1 << 30):
    return lib.domino_draft_block(ctypes.byref(h), batch, hidden, base, x_t, teacher, temp, 0, 0, tokens, logits,
                                  states, ws, ws_bytes, None)


def test_draft_block_validation(lib):
    h = fake_head()
    assert _draft(lib, h, batch=-1) == E_SHAPE
    assert _draft(lib, h, batch=129) == E_UNSUP
    assert _draft(lib, h, temp=-1.0) == E_ARG
    assert _draft(lib, h, temp=float("nan")) == E_ARG
    assert _draft(lib, h, temp=float("inf")) == E_ARG
    assert _draft(lib, h, hidden=None) == E_NULL
    assert _draft(lib, h, x_t=None) == E_NULL
    assert _draft(lib, h, tokens=None) == E_NULL
    assert _draft(lib, h, hidden=0x20004) == E_ALIGN
    assert _draft(lib, h, logits=0x60008) == E_ALIGN
    assert _draft(lib, h, ws=None) == E_WS
    assert _draft(lib, h, ws=0x100010) == E_WS
    assert _draft(lib, h, ws_bytes=1024) == E_WS
    assert _draft(lib, h, batch=0) == OK  # empty batch: nothing to do, no GPU needed
    bad = fake_head(d=100)
    assert _draft(lib, bad) == E_SHAPE


def test_draft_block_without_base_logits_validation(lib):
    # base_logits == NULL asks the single-block loop to form the base logits:
    # one block of a bf16 head with its GRU input table, d 2560 or 4096,
    # H 1024, r 256, K <= 16; anything else is refused before any GPU call
    q8 = dict(d=4096, vocab=151936, gru_hidden=1024, rank=256, gru_input_table=0x900000)
    assert _draft(lib, fake_head(**q8), base=None, batch=2) == E_UNSUP
    assert _draft(lib, fake_head(**dict(q8, gru_input_table=None)), base=None) == E_UNSUP
    assert _draft(lib, fake_head(**dict(q8, d=2048)), base=None) == E_UNSUP
    assert _draft(lib, fake_head(**dict(q8, block=17)), base=None) == E_UNSUP
    assert _draft(lib, fake_head(**dict(q8, rank=128)), base=None) == E_UNSUP
    assert _draft(lib, fake_head(**dict(q8, dtype=0, d=2048)), base=None) == E_UNSUP
    assert _draft(lib, fake_head(**q8), base=None, batch=0) == OK
    assert _draft(lib, fake_head(**q8), base=None, hidden=None) == E_NULL
    if not torch.cuda.is_available():
        assert _draft(lib, fake_head(**q8), base=None) == E_HIP
        assert _draft(lib, fake_head(**dict(q8, d=2560)), base=None) == E_HIP


def test_draft_status_validation(lib):
    h = fake_head()
    sz = ctypes.c_size_t(0)
    assert lib.domino_workspace_size(ctypes.byref(h), 2, ctypes.byref(sz)) == OK
    ws = 0x100000

    def st(batch=2, w=ws, nbytes=sz.value, out=0x2000, head=h):
        return lib.domino_draft_status(ctypes.byref(head), batch, w, nbytes, out, None)

    assert st(batch=0) == E_SHAPE
    assert st(batch=129) == E_UNSUP
    assert st(out=None) == E_NULL
    assert st(out=0x2002) == E_ALIGN
    assert st(w=None) == E_WS
    assert st(w=ws + 16) == E_WS
    assert st(nbytes=sz.value - 1) == E_WS
    assert st(head=fake_head(d=100)) == E_SHAPE


def test_draft_block_noalloc_validation(lib):
    # the same argument checks as domino_draft_block, and a call whose scratch
    # would exceed the library's fixed 16 MiB array is refused on the host
    q8 = fake_head(d=4096, vocab=151936, gru_hidden=1024, rank=256)

    def na(h, batch=1, hidden=0x20000, base=0x30000, x_t=0x40000, temp=0.0, tokens=0x50000):
        return lib.domino_draft_block_noalloc(ctypes.byref(h), batch, hidden, base, x_t, None, temp, 0, 0, tokens,
                                              None, None, None)

    assert na(q8, batch=-1) == E_SHAPE
    assert na(q8, batch=129) == E_UNSUP
    assert na(q8, temp=-1.0) == E_ARG
    assert na(q8, hidden=None) == E_NULL
    assert na(q8, tokens=0x50004) == E_ALIGN
    assert na(q8, batch=0) == OK
    sz = ctypes.c_size_t(0)
    assert lib.domino_workspace_size(ctypes.byref(q8), 64, ctypes.byref(sz)) == OK and sz.value > 16 << 20
    assert na(q8, batch=64) == E_UNSUP
    assert na(q8, batch=128) == E_UNSUP
    assert lib.domino_workspace_size(ctypes.byref(q8), 32, ctypes.byref(sz)) == OK and sz.value <= 16 << 20


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the behaviour without a GPU")
def test_valid_call_without_gpu_reports_hip_error(lib):
    h = fake_head()
    assert _draft(lib, h) == E_HIP
    assert lib.domino_base_logits(ctypes.byref(h), 1, 0x20000, 0x30000, None) == E_HIP
    assert lib.domino_accept_len(4, 16, 0x1000, 0x2000, 0x3000, None) == E_HIP
    assert lib.domino_draft_block_noalloc(ctypes.byref(h), 1, 0x20000, 0x30000, 0x40000, None, 0.0, 0, 0, 0x50000,
                                          None, None, None) == E_HIP


def test_read_stream_validation(lib):
    assert lib.domino_debug_read_stream(0x10000, 64, None, None) == E_NULL
    assert lib.domino_debug_read_stream(None, 64, 0x2000, None) == E_NULL
    assert lib.domino_debug_read_stream(0x10008, 64, 0x2000, None) == E_ALIGN
    assert lib.domino_debug_read_stream(0x10000, 64, 0x2002, None) == E_ALIGN
    assert lib.domino_debug_read_stream(0x10000, 72, 0x2000, None) == E_SHAPE
    assert lib.domino_debug_read_stream(0x10000, (1 << 40) + 16, 0x2000, None) == E_SHAPE


def test_base_logits_and_accept_validation(lib):
    h = fake_head()
    assert lib.domino_base_logits(ctypes.byref(h), -1, 0x20000, 0x30000, None) == E_SHAPE
    assert lib.domino_base_logits(ctypes.byref(h), 1, None, 0x30000, None) == E_NULL
    assert lib.domino_base_logits(ctypes.byref(h), 1, 0x20002, 0x30000, None) == E_ALIGN
    assert lib.domino_base_logits(ctypes.byref(h), 0, None, None, None) == OK
    assert lib.domino_accept_len(-1, 16, 0x1000, 0x2000, 0x3000, None) == E_SHAPE
    assert lib.domino_accept_len(4, 0, 0x1000, 0x2000, 0x3000, None) == E_SHAPE
    assert lib.domino_accept_len(4, 16, None, 0x2000, 0x3000, None) == E_NULL
    assert lib.domino_accept_len(0, 16, None, None, None, None) == OK
    assert lib.domino_debug_philox(0, 0, 0, 0, 0, -1, 0x1000, None) == E_SHAPE
    assert lib.domino_debug_philox(0, 0, 0, 0, 0, 0, None, None) == OK
    assert lib.domino_debug_philox(0, 0, 0, 0, 0, 5, None, None) == E_NULL


def test_binding_rejects_bad_tensors():
    t = {"lm_head": torch.zeros(64, 32), "embed": torch.zeros(64, 32), "w_ih": torch.zeros(96, 32),
         "w_hh": torch.zeros(96, 32), "b_ih": torch.zeros(96), "b_hh": torch.zeros(96),
         "w1": torch.zeros(32, 64), "b1": torch.zeros(32), "w2": torch.zeros(64, 32), "b2": torch.zeros(64)}
    h = D.Head(t, block=4)
    assert (h.vocab, h.d, h.gru_hidden, h.rank) == (64, 32, 32, 32)
    bad = dict(t, w2=torch.zeros(64, 31))
    with pytest.raises(ValueError):
        D.Head(bad)
    with pytest.raises(TypeError):
        D.Head(dict(t, w1=t["w1"].double()))


def test_verify_validation_and_workspace(lib):
    ws = lib.domino_verify_workspace_size(2, 16, 151936)
    assert ws > 0 and ws % 256 == 0
    assert lib.domino_verify_workspace_size(0, 16, 100) == 0
    assert lib.domino_verify_workspace_size(1, 256, 100) == 0
    assert lib.domino_verify_workspace_size(1, 16, 1 << 24) == 0
    args = dict(B=2, K=16, V=151936, t=0x10000, d=0x20000, y=0x30000, T=1.0, a=0x40000, n=0x50000,
                w=0x100000, wb=ws)

    def call(**kw):
        a = {**args, **kw}
        return lib.domino_verify_sampled(a["B"], a["K"], a["V"], a["t"], a["d"], a["y"], a["T"], 7, 3,
                                         a["a"], a["n"], a["w"], a["wb"], None)

    assert call() == E_HIP  # valid arguments, no GPU here
    assert call(B=-1) == E_SHAPE
    assert call(K=0) == E_SHAPE
    assert call(K=256) == E_SHAPE
    assert call(V=0) == E_SHAPE
    assert call(T=0.0) == E_ARG
    assert call(T=-1.0) == E_ARG
    assert call(T=float("inf")) == E_ARG
    assert call(T=float("nan")) == E_ARG
    assert call(t=None) == E_NULL
    assert call(n=None) == E_NULL
    assert call(d=0x20002) == E_ALIGN
    assert call(w=None) == E_WS
    assert call(w=0x100010) == E_WS
    assert call(wb=ws - 1) == E_WS
    assert call(B=0, t=None, d=None, y=None, a=None, n=None, w=None, wb=0) == OK


def test_base_draft_validation_and_workspace(lib):
    ws = lib.domino_base_draft_workspace_size(3, 16)
    assert ws >= 3 * 16 * 8 and ws % 256 == 0
    assert lib.domino_base_draft_workspace_size(0, 16) == 0
    assert lib.domino_base_draft_workspace_size(1, 1025) == 0
    args = dict(B=3, K=16, V=151936, L=0x10000, T=0.0, y=0x30000, w=0x100000, wb=ws)

    def call(**kw):
        a = {**args, **kw}
        return lib.domino_base_draft(a["B"], a["K"], a["V"], a["L"], a["T"], 7, 3, a["y"], a["w"], a["wb"], None)

    assert call() == E_HIP  # valid arguments, no GPU here
    assert call(T=1.0) == E_HIP
    assert call(B=-1) == E_SHAPE
    assert call(K=0) == E_SHAPE
    assert call(V=0) == E_SHAPE
    assert call(V=1 << 24) == E_SHAPE
    assert call(T=-0.5) == E_ARG
    assert call(T=float("nan")) == E_ARG
    assert call(T=float("inf")) == E_ARG
    assert call(L=None) == E_NULL
    assert call(y=None) == E_NULL
    assert call(L=0x10002) == E_ALIGN
    assert call(w=None) == E_WS
    assert call(w=0x100010) == E_WS
    assert call(wb=ws - 1) == E_WS
    assert call(B=0, L=None, y=None, w=None, wb=0) == OK


def test_curriculum_loss_validation_and_workspace(lib):
    ws = lib.domino_curriculum_loss_workspace_size(2, 16, 151936)
    assert ws > 0 and ws % 256 == 0
    assert lib.domino_curriculum_loss_workspace_size(0, 16, 100) == 0
    assert lib.domino_curriculum_loss_workspace_size(1, 1025, 100) == 0
    assert lib.domino_curriculum_loss_workspace_size(1, 16, 1 << 24) == 0
    args = dict(B=2, K=16, V=151936, b=0x10000, f=0x20000, y=0x30000, lam=0.5, g=0.8, loss=0x40000, cb=None,
                cf=None, gb=None, gf=None, w=0x100000, wb=ws)

    def call(**kw):
        a = {**args, **kw}
        return lib.domino_curriculum_loss(a["B"], a["K"], a["V"], a["b"], a["f"], a["y"], a["lam"], a["g"],
                                          a["loss"], a["cb"], a["cf"], a["gb"], a["gf"], a["w"], a["wb"], None)

    assert call() == E_HIP  # valid arguments, no GPU here
    assert call(cb=0x50000, cf=0x60000, gb=0x70000, gf=0x20000) == E_HIP  # gradient over its own logits
    assert call(B=-1) == E_SHAPE
    assert call(K=0) == E_SHAPE
    assert call(K=1025) == E_SHAPE
    assert call(V=0) == E_SHAPE
    assert call(lam=-0.1) == E_ARG
    assert call(lam=1.5) == E_ARG
    assert call(lam=float("nan")) == E_ARG
    assert call(g=0.0) == E_ARG
    assert call(g=1.01) == E_ARG
    assert call(g=float("inf")) == E_ARG
    assert call(b=None) == E_NULL
    assert call(f=None) == E_NULL
    assert call(y=None) == E_NULL
    assert call(loss=None) == E_NULL
    assert call(f=0x20002) == E_ALIGN
    assert call(gb=0x70001) == E_ALIGN
    assert call(w=None) == E_WS
    assert call(w=0x100010) == E_WS
    assert call(wb=ws - 1) == E_WS
    assert call(B=0, b=None, f=None, y=None, loss=None, w=None, wb=0) == OK


def test_correction_backward_validation(lib):
    h = fake_head(d=4096, vocab=151936, gru_hidden=1024, rank=256)
    sz = ctypes.c_size_t(0)
    assert lib.domino_correction_backward_workspace_size(ctypes.byref(h), 2, ctypes.byref(sz)) == OK
    ws = sz.value
    assert ws > 0 and ws % 256 == 0
    assert lib.domino_correction_backward_workspace_size(ctypes.byref(h), 129, ctypes.byref(sz)) == E_UNSUP
    assert lib.domino_correction_backward_workspace_size(ctypes.byref(h), 1, None) == E_NULL
    big_rank = fake_head(d=4096, vocab=151936, gru_hidden=1024, rank=544)
    assert lib.domino_correction_backward_workspace_size(ctypes.byref(big_rank), 1, ctypes.byref(sz)) == E_UNSUP
    args = dict(B=2, x=0x20000, g=0x30000, G=0x40000, dw2=0x50000, db2=0x60000, dw1=0x70000, db1=0x80000,
                ds=0x90000, w=0x100000, wb=ws)

    def call(head=h, **kw):
        a = {**args, **kw}
        return lib.domino_correction_backward(ctypes.byref(head), a["B"], a["x"], a["g"], a["G"], a["dw2"], a["db2"],
                                              a["dw1"], a["db1"], a["ds"], a["w"], a["wb"], None)

    assert call() == E_HIP  # valid arguments, no GPU here
    assert call(db2=None, db1=None, ds=None) == E_HIP
    assert call(B=-1) == E_SHAPE
    assert call(B=129) == E_UNSUP
    assert call(x=None) == E_NULL
    assert call(g=None) == E_NULL
    assert call(G=None) == E_NULL
    assert call(dw2=None) == E_NULL
    assert call(dw1=None) == E_NULL
    assert call(x=0x20008) == E_ALIGN
    assert call(G=0x40002) == E_ALIGN
    assert call(w=None) == E_WS
    assert call(wb=ws - 1) == E_WS
    assert call(B=0, x=None, g=None, G=None, dw2=None, dw1=None, w=None, wb=0) == OK


def test_gru_backward_validation(lib):
    h = fake_head(d=4096, vocab=151936, gru_hidden=1024, rank=256)
    sz = ctypes.c_size_t(0)
    assert lib.domino_gru_backward_workspace_size(ctypes.byref(h), 2, ctypes.byref(sz)) == OK
    ws = sz.value
    assert ws > 0 and ws % 256 == 0
    assert lib.domino_gru_backward_workspace_size(ctypes.byref(h), 129, ctypes.byref(sz)) == E_UNSUP
    assert lib.domino_gru_backward_workspace_size(ctypes.byref(h), 1, None) == E_NULL
    args = dict(B=2, x=0x20000, t=0x30000, g=0x40000, dg=0x50000, wi=0x60000, wh=0x70000, bi=0x80000, bh=0x90000,
                w=0x100000, wb=ws)

    def call(**kw):
        a = {**args, **kw}
        return lib.domino_gru_backward(ctypes.byref(h), a["B"], a["x"], a["t"], a["g"], a["dg"], a["wi"], a["wh"],
                                       a["bi"], a["bh"], a["w"], a["wb"], None)

    assert call() == E_HIP  # valid arguments, no GPU here
    assert call(bi=None, bh=None) == E_HIP
    assert call(B=-1) == E_SHAPE
    assert call(B=129) == E_UNSUP
    for k in ("x", "t", "g", "dg", "wi", "wh"):
        assert call(**{k: None}) == E_NULL, k
    assert call(g=0x40002) == E_ALIGN
    assert call(w=None) == E_WS
    assert call(wb=ws - 1) == E_WS
    assert call(B=0, x=None, t=None, g=None, dg=None, wi=None, wh=None, w=None, wb=0) == OK

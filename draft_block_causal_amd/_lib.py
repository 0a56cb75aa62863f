"""ctypes binding of libdomino.so.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, then their pointers and the current HIP stream are handed to the
C ABI declared in include/domino.h.  Every step of the path runs in the HIP
library; there is no other implementation behind these functions, and they
raise if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdomino.so")

DOMINO_F32 = 0
DOMINO_BF16 = 1
READ_STREAM_SINK = 2048  # entries of domino_debug_read_stream's sink

_STATUS = {
    0: "DOMINO_OK",
    -1: "DOMINO_ERR_NULL",
    -2: "DOMINO_ERR_SHAPE",
    -3: "DOMINO_ERR_DTYPE",
    -4: "DOMINO_ERR_ALIGN",
    -5: "DOMINO_ERR_ARG",
    -6: "DOMINO_ERR_WORKSPACE",
    -7: "DOMINO_ERR_HIP",
    -8: "DOMINO_ERR_UNSUPPORTED",
}

EXPORTED = [
    "domino_version",
    "domino_status_string",
    "domino_check_head",
    "domino_gru_table_size",
    "domino_prepare_gru_table",
    "domino_workspace_size",
    "domino_base_logits",
    "domino_draft_block",
    "domino_draft_status",
    "domino_draft_block_noalloc",
    "domino_accept_len",
    "domino_verify_sampled",
    "domino_verify_workspace_size",
    "domino_base_draft",
    "domino_base_draft_workspace_size",
    "domino_curriculum_loss",
    "domino_curriculum_loss_workspace_size",
    "domino_correction_backward",
    "domino_correction_backward_workspace_size",
    "domino_gru_backward",
    "domino_gru_backward_workspace_size",
    "domino_debug_read_stream",
    "domino_debug_philox",
]


class DominoError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)} ({text})")
        self.status = status


class DominoHeadStruct(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int32),
        ("vocab", ctypes.c_int32),
        ("gru_hidden", ctypes.c_int32),
        ("rank", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("lm_head", ctypes.c_void_p),
        ("embed", ctypes.c_void_p),
        ("w_ih", ctypes.c_void_p),
        ("w_hh", ctypes.c_void_p),
        ("b_ih", ctypes.c_void_p),
        ("b_hh", ctypes.c_void_p),
        ("w1", ctypes.c_void_p),
        ("b1", ctypes.c_void_p),
        ("w2", ctypes.c_void_p),
        ("b2", ctypes.c_void_p),
        ("gru_input_table", ctypes.c_void_p),
    ]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdomino.so (built in-tree by draft_block_causal_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m draft_block_causal_amd.build` "
                           "(the Domino engine has no other implementation)")
    lib = ctypes.CDLL(path)
    P, I32, U32, U64, SZ, F = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64,
                               ctypes.c_size_t, ctypes.c_float)
    HP = ctypes.POINTER(DominoHeadStruct)
    sig = {
        "domino_version": (ctypes.c_int, []),
        "domino_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "domino_check_head": (ctypes.c_int, [HP]),
        "domino_gru_table_size": (ctypes.c_int, [HP, ctypes.POINTER(SZ)]),
        "domino_prepare_gru_table": (ctypes.c_int, [HP, P, P]),
        "domino_workspace_size": (ctypes.c_int, [HP, I32, ctypes.POINTER(SZ)]),
        "domino_base_logits": (ctypes.c_int, [HP, I32, P, P, P]),
        "domino_draft_block": (ctypes.c_int, [HP, I32, P, P, P, P, F, U64, U32, P, P, P, P, SZ, P]),
        "domino_draft_status": (ctypes.c_int, [HP, I32, P, SZ, P, P]),
        "domino_draft_block_noalloc": (ctypes.c_int, [HP, I32, P, P, P, P, F, U64, U32, P, P, P, P]),
        "domino_accept_len": (ctypes.c_int, [I32, I32, P, P, P, P]),
        "domino_verify_sampled": (ctypes.c_int, [I32, I32, I32, P, P, P, F, U64, U32, P, P, P, SZ, P]),
        "domino_verify_workspace_size": (SZ, [I32, I32, I32]),
        "domino_base_draft": (ctypes.c_int, [I32, I32, I32, P, F, U64, U32, P, P, SZ, P]),
        "domino_base_draft_workspace_size": (SZ, [I32, I32]),
        "domino_curriculum_loss": (ctypes.c_int, [I32, I32, I32, P, P, P, F, F, P, P, P, P, P, P, SZ, P]),
        "domino_curriculum_loss_workspace_size": (SZ, [I32, I32, I32]),
        "domino_correction_backward": (ctypes.c_int, [HP, I32, P, P, P, P, P, P, P, P, P, SZ, P]),
        "domino_correction_backward_workspace_size": (ctypes.c_int, [HP, I32, ctypes.POINTER(SZ)]),
        "domino_gru_backward": (ctypes.c_int, [HP, I32, P, P, P, P, P, P, P, P, P, SZ, P]),
        "domino_gru_backward_workspace_size": (ctypes.c_int, [HP, I32, ctypes.POINTER(SZ)]),
        "domino_debug_read_stream": (ctypes.c_int, [P, SZ, P, P]),
        "domino_debug_philox": (ctypes.c_int, [U64, U32, I32, I32, I32, I32, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        text = load_library().domino_status_string(status).decode()
        raise DominoError(fn, status, text)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_ptr(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _need(t: torch.Tensor, name: str, dtype, shape, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


class Head:
    """A Domino head whose parameters are device tensors (the caller owns them)."""

    NAMES = ("lm_head", "embed", "w_ih", "w_hh", "b_ih", "b_hh", "w1", "b1", "w2", "b2")

    def __init__(self, tensors: dict, block: int = 16, gru_input_table: Optional[torch.Tensor] = None):
        lm = tensors["lm_head"]
        self.dtype = lm.dtype
        if self.dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("head tensors must be float32 or bfloat16")
        self.device = lm.device
        self.vocab, self.d = lm.shape
        self.gru_hidden = tensors["w_hh"].shape[1]
        self.rank = tensors["w1"].shape[0]
        self.block = int(block)
        V, d, H, r = self.vocab, self.d, self.gru_hidden, self.rank
        shapes = {"lm_head": (V, d), "embed": (V, d), "w_ih": (3 * H, d), "w_hh": (3 * H, H),
                  "b_ih": (3 * H,), "b_hh": (3 * H,), "w1": (r, d + H), "b1": (r,), "w2": (V, r), "b2": (V,)}
        self.tensors = {}
        for k in self.NAMES:
            t = tensors.get(k)
            if t is None and k in ("b_ih", "b_hh", "b1", "b2"):
                self.tensors[k] = None
                continue
            _need(t, k, self.dtype, shapes[k], self.device)
            self.tensors[k] = t
        self.table = None
        self.struct = DominoHeadStruct(
            d, V, H, r, self.block, DOMINO_BF16 if self.dtype == torch.bfloat16 else DOMINO_F32,
            *[_ptr(self.tensors[k]) for k in self.NAMES], None)
        if gru_input_table is not None:
            self.set_gru_input_table(gru_input_table)

    def set_gru_input_table(self, table: Optional[torch.Tensor]) -> None:
        """Attach (or detach, with None) the [V, 3H] float32 GRU input table."""
        if table is not None:
            _need(table, "gru_input_table", torch.float32, (self.vocab, 3 * self.gru_hidden), self.device)
        self.table = table
        self.struct.gru_input_table = _ptr(table)

    @property
    def ref(self):
        return ctypes.byref(self.struct)


def domino_version() -> int:
    return load_library().domino_version()


def domino_check_head(head: Head) -> None:
    _check("domino_check_head", load_library().domino_check_head(head.ref))


def domino_workspace_size(head: Head, batch: int) -> int:
    out = ctypes.c_size_t(0)
    _check("domino_workspace_size", load_library().domino_workspace_size(head.ref, int(batch), ctypes.byref(out)))
    return out.value


def domino_gru_table_size(head: Head) -> int:
    out = ctypes.c_size_t(0)
    _check("domino_gru_table_size", load_library().domino_gru_table_size(head.ref, ctypes.byref(out)))
    return out.value


def domino_prepare_gru_table(head: Head, table: Optional[torch.Tensor] = None, attach: bool = True,
                             stream=None) -> torch.Tensor:
    """Compute T = W_ih E^T + b_ih ([V, 3H] float32) on the device; by default attach it to the head."""
    if table is None:
        table = torch.empty((head.vocab, 3 * head.gru_hidden), dtype=torch.float32, device=head.device)
    _need(table, "table", torch.float32, (head.vocab, 3 * head.gru_hidden), head.device)
    _check("domino_prepare_gru_table", load_library().domino_prepare_gru_table(
        head.ref, _ptr(table), _stream_ptr(stream)))
    if attach:
        head.set_gru_input_table(table)
    return table


def domino_base_logits(head: Head, hidden: torch.Tensor, base_logits: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    B = hidden.shape[0]
    _need(hidden, "hidden", head.dtype, (B, head.block, head.d), head.device)
    if base_logits is None:
        base_logits = torch.empty((B, head.block, head.vocab), dtype=torch.float32, device=head.device)
    _need(base_logits, "base_logits", torch.float32, (B, head.block, head.vocab), head.device)
    _check("domino_base_logits", load_library().domino_base_logits(
        head.ref, B, _ptr(hidden), _ptr(base_logits), _stream_ptr(stream)))
    return base_logits


def domino_draft_block(head: Head, hidden: torch.Tensor, base_logits: Optional[torch.Tensor], x_t: torch.Tensor,
                       teacher: Optional[torch.Tensor] = None, temperature: float = 0.0, seed: int = 0,
                       offset: int = 0, tokens: Optional[torch.Tensor] = None,
                       logits: Optional[torch.Tensor] = None, gru_states: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """base_logits=None: the call forms the base logits itself (one block of a
    bf16 head with its GRU input table; other shapes raise DominoError with
    DOMINO_ERR_UNSUPPORTED)."""
    B, K, dev = hidden.shape[0], head.block, head.device
    _need(hidden, "hidden", head.dtype, (B, K, head.d), dev)
    if base_logits is not None:
        _need(base_logits, "base_logits", torch.float32, (B, K, head.vocab), dev)
    _need(x_t, "x_t", torch.int32, (B,), dev)
    if teacher is not None:
        _need(teacher, "teacher", torch.int32, (B, K), dev)
    if tokens is None:
        tokens = torch.empty((B, K), dtype=torch.int32, device=dev)
    _need(tokens, "tokens", torch.int32, (B, K), dev)
    if logits is not None:
        _need(logits, "logits", torch.float32, (B, K, head.vocab), dev)
    if gru_states is not None:
        _need(gru_states, "gru_states", torch.float32, (B, K, head.gru_hidden), dev)
    need = domino_workspace_size(head, B)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 device tensor")
    _check("domino_draft_block", load_library().domino_draft_block(
        head.ref, B, _ptr(hidden), _ptr(base_logits), _ptr(x_t), _ptr(teacher), float(temperature),
        int(seed) & 0xFFFFFFFFFFFFFFFF, int(offset) & 0xFFFFFFFF, _ptr(tokens), _ptr(logits), _ptr(gru_states),
        _ptr(workspace), workspace.numel(), _stream_ptr(stream)))
    return tokens


def domino_draft_block_noalloc(head: Head, hidden: torch.Tensor, base_logits: Optional[torch.Tensor],
                               x_t: torch.Tensor, tokens: torch.Tensor, teacher: Optional[torch.Tensor] = None,
                               temperature: float = 0.0, seed: int = 0, offset: int = 0,
                               logits: Optional[torch.Tensor] = None, gru_states: Optional[torch.Tensor] = None,
                               stream=None) -> torch.Tensor:
    """domino_draft_block over the library's fixed scratch array: no workspace,
    and nothing is allocated (the caller passes every output, tokens included)."""
    B, K, dev = hidden.shape[0], head.block, head.device
    _need(hidden, "hidden", head.dtype, (B, K, head.d), dev)
    if base_logits is not None:
        _need(base_logits, "base_logits", torch.float32, (B, K, head.vocab), dev)
    _need(x_t, "x_t", torch.int32, (B,), dev)
    _need(tokens, "tokens", torch.int32, (B, K), dev)
    if teacher is not None:
        _need(teacher, "teacher", torch.int32, (B, K), dev)
    if logits is not None:
        _need(logits, "logits", torch.float32, (B, K, head.vocab), dev)
    if gru_states is not None:
        _need(gru_states, "gru_states", torch.float32, (B, K, head.gru_hidden), dev)
    _check("domino_draft_block_noalloc", load_library().domino_draft_block_noalloc(
        head.ref, B, _ptr(hidden), _ptr(base_logits), _ptr(x_t), _ptr(teacher), float(temperature),
        int(seed) & 0xFFFFFFFFFFFFFFFF, int(offset) & 0xFFFFFFFF, _ptr(tokens), _ptr(logits), _ptr(gru_states),
        _stream_ptr(stream)))
    return tokens


def domino_draft_status(head: Head, batch: int, workspace: torch.Tensor, status: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """The status word of the last draft call on `workspace` (a one-element int32
    device tensor): 0 = every block's loop completed, 1 = a loop gave up."""
    if status is None:
        status = torch.empty((1,), dtype=torch.int32, device=head.device)
    _need(status, "status", torch.int32, (1,), head.device)
    if workspace.dtype != torch.uint8 or workspace.device != head.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 device tensor")
    _check("domino_draft_status", load_library().domino_draft_status(
        head.ref, int(batch), _ptr(workspace), workspace.numel(), _ptr(status), _stream_ptr(stream)))
    return status


def domino_accept_len(draft: torch.Tensor, target: torch.Tensor, accept: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    B, K = draft.shape
    _need(draft, "draft", torch.int32, (B, K), draft.device)
    _need(target, "target", torch.int32, (B, K), draft.device)
    if accept is None:
        accept = torch.empty((B,), dtype=torch.int32, device=draft.device)
    _need(accept, "accept", torch.int32, (B,), draft.device)
    _check("domino_accept_len", load_library().domino_accept_len(
        B, K, _ptr(draft), _ptr(target), _ptr(accept), _stream_ptr(stream)))
    return accept


def domino_verify_workspace_size(batch: int, block: int, vocab: int) -> int:
    return int(load_library().domino_verify_workspace_size(int(batch), int(block), int(vocab)))


def domino_verify_sampled(target_logits: torch.Tensor, draft_logits: torch.Tensor, draft: torch.Tensor,
                          temperature: float, seed: int = 0, offset: int = 0,
                          accept: Optional[torch.Tensor] = None, next_token: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, stream=None):
    """Speculative-sampling verification; returns (accept [B], next_token [B]) int32."""
    B, K = draft.shape
    V = draft_logits.shape[-1]
    dev = draft.device
    _need(target_logits, "target_logits", torch.float32, (B, K + 1, V), dev)
    _need(draft_logits, "draft_logits", torch.float32, (B, K, V), dev)
    _need(draft, "draft", torch.int32, (B, K), dev)
    if accept is None:
        accept = torch.empty((B,), dtype=torch.int32, device=dev)
    if next_token is None:
        next_token = torch.empty((B,), dtype=torch.int32, device=dev)
    _need(accept, "accept", torch.int32, (B,), dev)
    _need(next_token, "next_token", torch.int32, (B,), dev)
    need = domino_verify_workspace_size(B, K, V) if B > 0 else 0
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 device tensor")
    _check("domino_verify_sampled", load_library().domino_verify_sampled(
        B, K, V, _ptr(target_logits), _ptr(draft_logits), _ptr(draft), float(temperature),
        int(seed) & 0xFFFFFFFFFFFFFFFF, int(offset) & 0xFFFFFFFF, _ptr(accept), _ptr(next_token),
        _ptr(workspace), workspace.numel(), _stream_ptr(stream)))
    return accept, next_token


def domino_base_draft_workspace_size(batch: int, block: int) -> int:
    return int(load_library().domino_base_draft_workspace_size(batch, block))


def domino_base_draft(base_logits: torch.Tensor, temperature: float = 0.0, seed: int = 0, offset: int = 0,
                      tokens: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """Base-only (head-off) drafting: each position's token from its base logits alone."""
    if base_logits.dim() != 3:
        raise ValueError("base_logits must be [batch, block, vocab]")
    B, K, V = base_logits.shape
    dev = base_logits.device
    _need(base_logits, "base_logits", torch.float32, (B, K, V), dev)
    if tokens is None:
        tokens = torch.empty((B, K), dtype=torch.int32, device=dev)
    _need(tokens, "tokens", torch.int32, (B, K), dev)
    need = domino_base_draft_workspace_size(B, K) if B > 0 else 0
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check("domino_base_draft", load_library().domino_base_draft(
        B, K, V, _ptr(base_logits), float(temperature), int(seed), int(offset), _ptr(tokens), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream_ptr(stream)))
    return tokens


def domino_curriculum_loss(base_logits: torch.Tensor, final_logits: torch.Tensor, targets: torch.Tensor,
                           lam: float, gamma: float, loss: Optional[torch.Tensor] = None,
                           ce_base: Optional[torch.Tensor] = None, ce_final: Optional[torch.Tensor] = None,
                           grad_base: Optional[torch.Tensor] = None, grad_final: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The base-anchored curriculum loss (a one-element device tensor); the optional
    per-position cross-entropies and logit gradients are written when given."""
    if base_logits.dim() != 3:
        raise ValueError("base_logits must be [batch, block, vocab]")
    B, K, V = base_logits.shape
    dev = base_logits.device
    _need(base_logits, "base_logits", torch.float32, (B, K, V), dev)
    _need(final_logits, "final_logits", torch.float32, (B, K, V), dev)
    _need(targets, "targets", torch.int32, (B, K), dev)
    if loss is None:
        loss = torch.zeros((1,), dtype=torch.float32, device=dev)
    _need(loss, "loss", torch.float32, (1,), dev)
    for t, name in ((ce_base, "ce_base"), (ce_final, "ce_final")):
        if t is not None:
            _need(t, name, torch.float32, (B, K), dev)
    for t, name in ((grad_base, "grad_base"), (grad_final, "grad_final")):
        if t is not None:
            _need(t, name, torch.float32, (B, K, V), dev)
    need = int(load_library().domino_curriculum_loss_workspace_size(B, K, V)) if B > 0 else 0
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check("domino_curriculum_loss", load_library().domino_curriculum_loss(
        B, K, V, _ptr(base_logits), _ptr(final_logits), _ptr(targets), float(lam), float(gamma), _ptr(loss),
        _ptr(ce_base), _ptr(ce_final), _ptr(grad_base), _ptr(grad_final), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream_ptr(stream)))
    return loss


def domino_correction_backward(head: Head, hidden: torch.Tensor, gru_states: torch.Tensor,
                               grad_final: torch.Tensor, d_b: bool = True, d_states: bool = True, stream=None):
    """Gradients of W2, b2, W1, b1 (and of the GRU states) from the loss's gradient on
    the final logits; returns dict(d_w2, d_b2, d_w1, d_b1, d_states) of float32 tensors."""
    B = hidden.shape[0]
    K, V, d, H, r, dev = head.block, head.vocab, head.d, head.gru_hidden, head.rank, head.device
    _need(hidden, "hidden", head.dtype, (B, K, d), dev)
    _need(gru_states, "gru_states", torch.float32, (B, K, H), dev)
    _need(grad_final, "grad_final", torch.float32, (B, K, V), dev)
    f = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)  # noqa: E731
    out = {"d_w2": f(V, r), "d_b2": f(V) if d_b else None, "d_w1": f(r, d + H), "d_b1": f(r) if d_b else None,
           "d_states": f(B, K, H) if d_states else None}
    sz = ctypes.c_size_t(0)
    _check("domino_correction_backward_workspace_size",
           load_library().domino_correction_backward_workspace_size(head.ref, B, ctypes.byref(sz)))
    ws = torch.empty(max(int(sz.value), 1), dtype=torch.uint8, device=dev)
    _check("domino_correction_backward", load_library().domino_correction_backward(
        head.ref, B, _ptr(hidden), _ptr(gru_states), _ptr(grad_final), _ptr(out["d_w2"]), _ptr(out["d_b2"]),
        _ptr(out["d_w1"]), _ptr(out["d_b1"]), _ptr(out["d_states"]), _ptr(ws), ws.numel(), _stream_ptr(stream)))
    return out


def domino_gru_backward(head: Head, x_t: torch.Tensor, teacher: torch.Tensor, gru_states: torch.Tensor,
                        d_states: torch.Tensor, d_b: bool = True, stream=None):
    """Gradients of W_ih, W_hh (and b_ih, b_hh) of the teacher-forced GRU from the state
    gradients; returns dict(d_w_ih, d_w_hh, d_b_ih, d_b_hh) of float32 tensors."""
    B = x_t.shape[0]
    K, d, H, dev = head.block, head.d, head.gru_hidden, head.device
    _need(x_t, "x_t", torch.int32, (B,), dev)
    _need(teacher, "teacher", torch.int32, (B, K), dev)
    _need(gru_states, "gru_states", torch.float32, (B, K, H), dev)
    _need(d_states, "d_states", torch.float32, (B, K, H), dev)
    f = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)  # noqa: E731
    out = {"d_w_ih": f(3 * H, d), "d_w_hh": f(3 * H, H), "d_b_ih": f(3 * H) if d_b else None,
           "d_b_hh": f(3 * H) if d_b else None}
    sz = ctypes.c_size_t(0)
    _check("domino_gru_backward_workspace_size",
           load_library().domino_gru_backward_workspace_size(head.ref, B, ctypes.byref(sz)))
    ws = torch.empty(max(int(sz.value), 1), dtype=torch.uint8, device=dev)
    _check("domino_gru_backward", load_library().domino_gru_backward(
        head.ref, B, _ptr(x_t), _ptr(teacher), _ptr(gru_states), _ptr(d_states), _ptr(out["d_w_ih"]),
        _ptr(out["d_w_hh"]), _ptr(out["d_b_ih"]), _ptr(out["d_b_hh"]), _ptr(ws), ws.numel(), _stream_ptr(stream)))
    return out


def domino_debug_read_stream(buf: torch.Tensor, sink: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One plain streaming read of `buf` (a contiguous device tensor whose byte
    size is a multiple of 16); returns sink, 2048 int32 (device) whose XOR is
    the XOR of the buffer's 32-bit words."""
    if not isinstance(buf, torch.Tensor) or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    if sink is None:
        sink = torch.empty((READ_STREAM_SINK,), dtype=torch.int32, device=buf.device)
    _need(sink, "sink", torch.int32, (READ_STREAM_SINK,), buf.device)
    _check("domino_debug_read_stream", load_library().domino_debug_read_stream(
        _ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream_ptr(stream)))
    return sink


def domino_debug_philox(seed: int, offset: int, b: int, pos: int, v0: int, n: int,
                        out: Optional[torch.Tensor] = None, device="cuda", stream=None) -> torch.Tensor:
    if out is None:
        out = torch.empty((n,), dtype=torch.int32, device=device)
    _need(out, "out", torch.int32, (n,), out.device)
    _check("domino_debug_philox", load_library().domino_debug_philox(
        int(seed) & 0xFFFFFFFFFFFFFFFF, int(offset) & 0xFFFFFFFF, b, pos, v0, n, _ptr(out), _stream_ptr(stream)))
    return out

"""Seeded synthetic inputs for the Domino draft-head path.

This module only draws random numbers and packs them into arrays. It holds
none of the method's arithmetic: both the HIP path (through the Python
binding) and the CPU oracle receive the same arrays from here.

Workloads stand in for the pages' datasets and trained checkpoints, which are
not available: the path's cost depends only on shapes, so weights and hidden
states are Gaussian draws with the shapes of the Qwen3 draft heads that the
pages describe (block 16, GRU hidden 1024, rank 256; page
"完全开源的语言模型学习记录--推理加速Domino", section 二.1(2) and 三.1).

Generation recipe (fixed so that every caller sees the same values):
  * every tensor has its own numpy PCG64 stream: tensor number t of the fixed
    order below draws from ``SeedSequence(seed, spawn_key=(t, chunk))`` for
    each consecutive chunk of 2^22 elements (chunks are filled in parallel;
    the values do not depend on the thread count);
  * float32 standard normals scaled by the tensor's standard deviation; bf16
    tensors are rounded to nearest-even from those float32 values and stored
    as raw ``uint16`` bit patterns;
  * order: lm_head, embed (skipped when tied), w_ih, w_hh, b_ih, b_hh, w1, b1,
    w2, b2, hidden, x_t (x_t uses ``default_rng(SeedSequence(seed,
    spawn_key=(11,)))``).
  * hidden states N(0, 1); x_t uniform on [0, V).
  * accept-length targets (``make_targets``): a separate generator seeded 1;
    each position copies the draft token with probability p (0.9), otherwise
    takes a uniform token on [0, V).
  * sampled-draft verification inputs (``make_verify_inputs``): one
    ``default_rng(seed)``; draft logits N(0, 2^2) [B, K, V]; target logits =
    draft logits + N(0, spread^2) at the K drafted positions and N(0, 2^2)
    one past them; each draft token is the draft row's largest logit with
    probability 0.8, otherwise a uniform token.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_CHUNK = 1 << 22
_THREADS = max(1, min(16, os.cpu_count() or 1))

__all__ = [
    "Workload",
    "WORKLOADS",
    "get_workload",
    "make_head",
    "make_block_inputs",
    "make_workload",
    "make_targets",
    "make_tokens",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "head_param_count",
    "to_torch",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int  # B: draft blocks per call
    block: int  # K: positions per block
    d: int  # hidden size of the backbone / LM head input
    vocab: int  # V
    gru_hidden: int  # H
    rank: int  # r
    dtype: str  # "f32" or "bf16" for weights and hidden states
    tied: bool  # embedding table is the LM head matrix
    temperature: float  # 0 = greedy
    init: str = "small"  # "small": every parameter N(0, 0.02); "fanin": N(0, 1/sqrt(fan_in))
    accept: bool = False  # the workload also scores the draft with accept_len
    seed: int = 0
    philox_seed: int = 0

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Workloads named by what they are.  The Qwen3 hidden sizes (4096 for 8B,
# 2560 for 4B) and vocabulary (151936) are the public model shapes; block 16,
# GRU hidden 1024 and rank 256 are the pages' head shapes.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32_b1", 1, 16, 256, 4096, 128, 32, "f32", False, 0.0),
        Workload("qwen3_8b_b1_greedy", 1, 16, 4096, 151936, 1024, 256, "bf16", False, 0.0),
        Workload("qwen3_8b_b32_t1", 32, 16, 4096, 151936, 1024, 256, "bf16", False, 1.0),
        Workload("qwen3_4b_b8_tied", 8, 16, 2560, 151936, 1024, 256, "bf16", True, 0.0),
        Workload("qwen3_8b_b128_accept", 128, 16, 4096, 151936, 1024, 256, "bf16", False, 0.0,
                 accept=True),
        # test-only: fan-in scaled weights make the GRU signal O(1) so that a
        # wrong recurrence moves the logits far beyond the tolerance.
        Workload("tiny_stress_b4", 4, 16, 256, 4096, 128, 32, "f32", False, 0.0, init="fanin"),
    ]
}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in = x.reshape(-1).view(np.uint32)
    flat_out = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_in.size, step):
        u = flat_in[s:s + step].astype(np.uint32)
        bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
        flat_out[s:s + step] = ((u + bias) >> 16).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(seed: int, tensor_id: int, shape, std: float, dtype: str) -> np.ndarray:
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)

    def fill(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tensor_id, c))))
        x = rng.standard_normal(size=hi - lo, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[lo:hi] = f32_to_bf16_bits(x) if dtype == "bf16" else x

    chunks = range((n + _CHUNK - 1) // _CHUNK)
    if len(chunks) > 1:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, chunks))
    else:
        for c in chunks:
            fill(c)
    return out.reshape(shape)


def _std(w: Workload, kind: str, fan_in: int) -> float:
    if w.init == "small":
        return 0.02
    if kind == "embed":
        return 1.0
    return 1.0 / math.sqrt(fan_in)


def make_head(w: Workload) -> dict:
    """Draw every head parameter; bf16 tensors come back as uint16 bits."""
    d, V, H, r, dt, sd = w.d, w.vocab, w.gru_hidden, w.rank, w.dtype, w.seed
    head = {}
    head["lm_head"] = _normal(sd, 0, (V, d), _std(w, "linear", d), dt)
    head["embed"] = head["lm_head"] if w.tied else _normal(sd, 1, (V, d), _std(w, "embed", d), dt)
    head["w_ih"] = _normal(sd, 2, (3 * H, d), _std(w, "linear", d), dt)
    head["w_hh"] = _normal(sd, 3, (3 * H, H), _std(w, "linear", H), dt)
    head["b_ih"] = _normal(sd, 4, (3 * H,), _std(w, "linear", d), dt)
    head["b_hh"] = _normal(sd, 5, (3 * H,), _std(w, "linear", H), dt)
    head["w1"] = _normal(sd, 6, (r, d + H), _std(w, "linear", d + H), dt)
    head["b1"] = _normal(sd, 7, (r,), _std(w, "linear", d + H), dt)
    head["w2"] = _normal(sd, 8, (V, r), _std(w, "linear", r), dt)
    head["b2"] = _normal(sd, 9, (V,), _std(w, "linear", r), dt)
    return head


def make_block_inputs(w: Workload, batch: int | None = None) -> dict:
    B = w.batch if batch is None else batch
    hidden = _normal(w.seed, 10, (B, w.block, w.d), 1.0, w.dtype)
    rng = np.random.default_rng(np.random.SeedSequence(w.seed, spawn_key=(11,)))
    x_t = rng.integers(0, w.vocab, size=(B,), dtype=np.int64).astype(np.int32)
    return {"hidden": hidden, "x_t": x_t}


def make_workload(w: Workload, batch: int | None = None):
    """Head parameters and one batch of block inputs."""
    return make_head(w), make_block_inputs(w, batch)


def make_tokens(shape, vocab: int, seed: int) -> np.ndarray:
    """Uniform token ids (teacher sequences, synthetic drafts)."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, vocab, size=shape, dtype=np.int64).astype(np.int32)


def make_targets(draft: np.ndarray, vocab: int, p: float = 0.9, seed: int = 1) -> np.ndarray:
    """Synthetic verification targets: copy the draft token w.p. ``p``, else a uniform token."""
    rng = np.random.default_rng(seed)
    keep = rng.random(size=draft.shape) < p
    other = rng.integers(0, vocab, size=draft.shape, dtype=np.int64).astype(np.int32)
    return np.where(keep, draft, other).astype(np.int32)


def make_verify_inputs(batch: int, block: int, vocab: int, spread: float, seed: int = 2):
    """(target_logits [B, K+1, V], draft_logits [B, K, V], draft [B, K]) for sampled-draft verification."""
    rng = np.random.default_rng(seed)
    d = (rng.standard_normal((batch, block, vocab), dtype=np.float32) * 2.0).astype(np.float32)
    t = np.empty((batch, block + 1, vocab), dtype=np.float32)
    t[:, :block] = d + rng.standard_normal((batch, block, vocab), dtype=np.float32) * np.float32(spread)
    t[:, block] = rng.standard_normal((batch, vocab), dtype=np.float32) * 2.0
    top = np.argmax(d, axis=-1)
    uni = rng.integers(0, vocab, size=(batch, block))
    y = np.where(rng.random((batch, block)) < 0.8, top, uni).astype(np.int32)
    return t, d, y


def to_torch(a: np.ndarray, device=None):
    """Host array -> torch tensor: uint16 arrays are bf16 bit patterns (reinterpreted, not converted)."""
    import torch

    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device) if device is not None else t


def head_param_count(w: Workload, biases: bool = True) -> int:
    """Number of trainable head parameters (GRU + W1 + W2), excluding the frozen LM head/embedding."""
    d, V, H, r = w.d, w.vocab, w.gru_hidden, w.rank
    n = 3 * H * d + 3 * H * H + r * (d + H) + V * r
    if biases:
        n += 3 * H + 3 * H + r + V
    return n

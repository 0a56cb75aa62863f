#!/usr/bin/env python3
"""Benchmark of the Domino draft-head hot path on one MI355X.

One step = one draft call on the Qwen3-8B-shaped head at B = 1: the frozen LM
head over the 16 positions (base logits) + the draft block (GRU + low-rank
correction + greedy pick, 16 serial positions).  Where the single-block loop
can form the base logits itself (one block of a bf16 head with its GRU input
table), the step is the one call domino_draft_block(base_logits=None);
otherwise, or with --unfused, domino_base_logits then domino_draft_block.
Inputs are resident in HBM before the timed region, which holds the steps
alone (no event records between them); a second pass with HIP events gives
the per-call breakdown.  domino_accept_len is timed on its
own, on targets derived from the run's draft.  The run checks its own output
(status word, token range, and block 0 against the oracle by the replay rule
in the CPU-baseline leg) and exits non-zero if a check fails.  Prints one JSON
line.

    python bench.py [--gpus 1] [--steps 200] [--warmup 10] [--workload qwen3_8b_b1_greedy]
    python bench.py --sweep 1,2,4,8,16,32,64,128 [--steps 30]   # concurrency sweep of one head
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "draft blocks/sec + ms/block (block 16, Qwen3-8B shapes) and % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak of MI355X
RIDGE_FLOP_PER_BYTE = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lmhead_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "draft_block_causal_amd", "csrc", f) for f in ("rowstream.hip", "common.h")]
# the tiled LM-head GEMM (256-row tiles, many blocks)
GEMM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lmhead_gemm_traffic.json")
GEMM_KERNEL_SOURCES = [os.path.join(ROOT, "draft_block_causal_amd", "csrc", f)
                       for f in ("gemm.hip", "common.h", "kernels.h")]
# the single-block loop that forms the base logits itself
FUSED_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "draft_b1_fused_traffic.json")
FUSED_KERNEL_SOURCES = [os.path.join(ROOT, "draft_block_causal_amd", "csrc", f)
                        for f in ("loop_b1.hip", "common.h", "xchg.h", "kernels.h")]


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for p in sources or KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def lmhead_algorithmic_bytes(B: int, K: int, d: int, V: int, elem: int) -> int:
    """Compulsory bytes of one LM-head launch: W_lm once, hidden in, fp32 base logits out."""
    return V * d * elem + B * K * d * elem + B * K * V * 4


def lmhead_flops(B: int, K: int, d: int, V: int) -> int:
    return 2 * B * K * d * V


def block_algorithmic_bytes(B: int, K: int, d: int, V: int, H: int, r: int, elem: int,
                            base_in_hbm: bool = True) -> int:
    """Compulsory HBM bytes of one draft call (base logits + draft block) over B
    blocks: every weight once (the LM head, W2, W_ih, W_hh, W1 and the biases;
    a tied embedding is the LM head), the gathered embedding rows, the hidden
    states in, the float32 base logits written and read back once (not when
    the call forms them on chip: base_in_hbm=False), x_t in and the tokens out.
    Re-reads of per-position weights across the 16 positions are a schedule's
    choice and are not counted."""
    weights = (V * d + V * r + 3 * H * d + 3 * H * H + r * (d + H)) * elem
    biases = (3 * H * 2 + r + V) * elem
    acts = B * K * d * elem * 2 + (2 * B * K * V * 4 if base_in_hbm else 0) + B * 4 + B * K * 4
    return weights + biases + acts


def block_flops(B: int, K: int, d: int, V: int, H: int, r: int) -> int:
    """Multiply-adds x 2 of one draft call: the LM head, W2, the GRU's two
    products and W1, for every block position."""
    M = B * K
    return 2 * M * (V * d + V * r + 3 * H * (d + H) + r * (d + H))


def block_floor_us(B: int, K: int, d: int, V: int, H: int, r: int, elem: int, base_in_hbm: bool = True) -> float:
    """Roofline floor of one draft call: the larger of its compulsory bytes at
    the HBM peak and its FLOPs at the dense bf16 matrix-core peak."""
    t_hbm = block_algorithmic_bytes(B, K, d, V, H, r, elem, base_in_hbm) / (HBM_PEAK_GBS * 1e9)
    t_mfma = block_flops(B, K, d, V, H, r) / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    return max(t_hbm, t_mfma) * 1e6


def measured_traffic(kernel_hash: str, path: str = TRAFFIC_FILE, workload=None):
    """HBM bytes per launch of a kernel (the LM head by default) from the committed
    rocprofv3 counter runs, if they were taken on the current kernel source (and,
    when `workload` is given, on that workload's shapes); else None."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_hash:
        return None
    if workload is not None and t.get("workload") != workload:
        return None
    return t.get("hbm_bytes_per_launch")


def replay_mismatches(O, f, hidden, x_t, gpu_tokens, w, tol: float = 2e-2):
    """Positions of one block where the GPU's free-running token breaks the
    replay rule: the oracle is run teacher-forced on the GPU's own tokens, and
    each GPU token must be the oracle's pick, or, where the oracle's top-2 score
    margin is below tol, score within tol of the top.  Returns a list of
    (position, gpu token, oracle token)."""
    rep = O.draft_block(f, hidden, x_t, teacher=gpu_tokens, temperature=w.temperature, seed=w.philox_seed)
    bad = []
    for i in range(gpu_tokens.shape[1]):
        s = rep["scores"][0, i]
        y, best = int(gpu_tokens[0, i]), O.pick_token(s)
        if y == best:
            continue
        if not (0 <= y < s.size and O.top2_margin(s) < tol and s[y] > s.max() - tol):
            bad.append((i, y, best))
    return bad


def cpu_baseline(w, head_np, inp, min_seconds: float = 10.0, gpu_tokens=None):
    """The CPU oracle, as it is, on a bounded sample of the same workload.  When
    the GPU's tokens of block 0 are given, they are also checked against the
    oracle by the replay rule (result in "gpu_block0_check")."""
    import oracle as O

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = os.cpu_count() or 1
    f = {k: O.as_f64(v) for k, v in head_np.items() if not (k == "embed" and w.tied)}
    if w.tied:
        f["embed"] = f["lm_head"]
    hid = O.as_f64(inp["hidden"][:1])
    n, t0 = 0, time.perf_counter()
    while True:
        base = O.base_logits(hid, f["lm_head"])
        out = O.draft_block(f, hid, inp["x_t"][:1], temperature=w.temperature, seed=w.philox_seed, base=base)
        n += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or n >= 1000:
            break
    res = {"value": n / el, "unit": "draft blocks/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{n} x one {w.name} block (B=1): float64 numpy base logits + 16-position loop, "
                     f"{el:.1f} s wall"}
    if gpu_tokens is not None:
        bad = replay_mismatches(O, f, hid, inp["x_t"][:1], gpu_tokens[:1], w)
        res["gpu_block0_check"] = {"rule": "replay (tokens equal except at top-2 margin < 2e-2)",
                                   "positions": int(gpu_tokens.shape[1]), "mismatches": bad,
                                   "equal_to_free_running_oracle": int((out["tokens"][0] == gpu_tokens[0]).sum())}
    return res


def sweep(args, w, batches) -> int:
    """Draft blocks/s of one head at several batch sizes (blocks per call): the
    concurrency axis of the pages' serving measurements. Each row times
    base logits + draft block on the first B blocks of one input set."""
    import torch

    import domino_synth as S
    import draft_block_causal_amd as D

    dev = torch.device("cuda:0")
    Bmax = max(batches)
    head_np, inp = S.make_workload(w, batch=Bmax)
    tensors = {k: S.to_torch(v, dev) for k, v in head_np.items() if not (k == "embed" and w.tied)}
    if w.tied:
        tensors["embed"] = tensors["lm_head"]
    head = D.Head(tensors, block=w.block)
    if not args.no_table:
        D.domino_prepare_gru_table(head)
    hidden_all = S.to_torch(inp["hidden"], dev)
    x_all = S.to_torch(inp["x_t"], dev)
    rows = []
    for B in batches:
        hidden, x_t = hidden_all[:B], x_all[:B]
        base = torch.empty((B, w.block, w.vocab), dtype=torch.float32, device=dev)
        tokens = torch.empty((B, w.block), dtype=torch.int32, device=dev)
        ws = torch.empty(D.domino_workspace_size(head, B), dtype=torch.uint8, device=dev)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        fused = forms_base_logits(w, B, not args.no_table) and not args.unfused

        def step(e=None):
            if e:
                e[0].record()
            if not fused:
                D.domino_base_logits(head, hidden, base)
            if e:
                e[1].record()
            D.domino_draft_block(head, hidden, None if fused else base, x_t, temperature=w.temperature,
                                 seed=w.philox_seed, tokens=tokens, workspace=ws)
            if e:
                e[2].record()

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        for i in range(args.steps):  # the breakdown, in a pass of its own
            step(ev[i])
        torch.cuda.synchronize()
        rows.append({"batch": B, "blocks_per_s": B / (ms * 1e-3), "ms_per_call": ms, "ms_per_block": ms / B,
                     "base_logits": "inside the draft call" if fused else "domino_base_logits",
                     "lm_head_ms": None if fused else float(np.mean([e[0].elapsed_time(e[1]) for e in ev])),
                     "draft_block_ms": float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))})
        print(f"sweep B={B}: {rows[-1]['blocks_per_s']:.1f} blocks/s, {ms:.4f} ms/call", file=sys.stderr, flush=True)
        st = int(D.domino_draft_status(head, B, ws).cpu().numpy()[0])
        if st != 0 or int(tokens.min()) < 0:
            print(f"bench.py: sweep B={B}: a loop gave up (status {st})", file=sys.stderr)
            return 3
        del base, tokens, ws
    print(json.dumps({"metric": "draft blocks/s vs blocks per call (concurrency sweep)", "unit": "draft blocks/s",
                      "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "dtype": w.dtype,
                      "data": "synthetic (seeded Gaussian weights and hidden states)",
                      "config": {"workload": w.name, "block": w.block, "d": w.d, "vocab": w.vocab,
                                 "gru_hidden": w.gru_hidden, "rank": w.rank, "temperature": w.temperature,
                                 "tied": w.tied, "gru_input_table": not args.no_table},
                      "sweep": rows}), flush=True)
    return 0


def library_gemm(args, w) -> int:
    """The workload's LM-head product C = h W_lm^T through torch's bf16 matmul
    (hipBLASLt), with float32 and bf16 outputs, timed with HIP events next to
    domino_base_logits on the same operands. A reference point only: the
    Domino path never calls it."""
    import torch

    import domino_synth as S
    import draft_block_causal_amd as D

    if w.dtype != "bf16":
        print("bench.py: --library-gemm needs a bf16 workload", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    head_np, inp = S.make_workload(w)
    lm = S.to_torch(head_np["lm_head"], dev).view(torch.bfloat16)
    hidden = S.to_torch(inp["hidden"], dev).view(torch.bfloat16)
    M, V, d = w.batch * w.block, w.vocab, w.d
    A = hidden.reshape(M, d)
    z = lambda *shape: torch.zeros(*shape, dtype=torch.bfloat16, device=dev)  # noqa: E731
    H, r = w.gru_hidden, w.rank
    head = D.Head({"lm_head": lm, "embed": lm, "w_ih": z(3 * H, d), "w_hh": z(3 * H, H), "w1": z(r, d + H),
                   "w2": z(V, r)}, block=w.block)
    base = torch.empty((w.batch, w.block, V), dtype=torch.float32, device=dev)
    out32 = torch.empty((M, V), dtype=torch.float32, device=dev)
    out16 = torch.empty((M, V), dtype=torch.bfloat16, device=dev)

    def timeit(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    flops = lmhead_flops(w.batch, w.block, d, V)
    rows = {"domino_base_logits (float32 out)": timeit(lambda: D.domino_base_logits(head, hidden, base)),
            "torch.matmul bf16 (bf16 out)": timeit(lambda: torch.matmul(A, lm.t(), out=out16))}
    try:
        rows["torch.mm bf16 (float32 out)"] = timeit(
            lambda: torch.mm(A, lm.t(), out_dtype=torch.float32, out=out32))
    except (TypeError, RuntimeError) as ex:  # older torch: no out_dtype
        print(f"bench.py: float32-output matmul unavailable: {ex}", file=sys.stderr)
    res = {name: {"ms": ms, "tflops": flops / (ms * 1e-3) / 1e12,
                  "mfma_frac": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS} for name, ms in rows.items()}
    print(json.dumps({"workload": w.name, "M": M, "N": V, "K": d, "steps": args.steps, "results": res}), flush=True)
    return 0


def next_rows(args, w) -> int:
    """Timings (HIP events, mean over --steps after --warmup) of the calls beyond
    the draft path, at the workload's shapes, with the HBM rate of each
    bandwidth-bound kernel group against the 8 TB/s peak:
      train_forward: base logits + teacher-forced draft block (final logits and
                     GRU states out) + curriculum loss with both logit gradients
                     written in place, then the backward through the correction head
                     and through time of the GRU (the whole head's gradients);
      verify:        sampled-draft verification on synthetic target / draft logits;
      head_off:      base logits + base-only drafting, beside base logits + draft block."""
    import torch

    import domino_synth as S
    import draft_block_causal_amd as D

    dev = torch.device("cuda:0")
    head_np, inp = S.make_workload(w)
    tensors = {k: S.to_torch(v, dev) for k, v in head_np.items() if not (k == "embed" and w.tied)}
    if w.tied:
        tensors["embed"] = tensors["lm_head"]
    head = D.Head(tensors, block=w.block)
    if not args.no_table:
        D.domino_prepare_gru_table(head)
    B, K, V = w.batch, w.block, w.vocab
    hidden = S.to_torch(inp["hidden"], dev)
    x_t = S.to_torch(inp["x_t"], dev)
    gold = S.to_torch(S.make_tokens((B, K), V, seed=31), dev)
    base = torch.empty((B, K, V), dtype=torch.float32, device=dev)
    final = torch.empty_like(base)
    tokens = torch.empty((B, K), dtype=torch.int32, device=dev)
    ws = torch.empty(D.domino_workspace_size(head, B), dtype=torch.uint8, device=dev)
    lws = torch.empty(max(1, int(D.load_library().domino_curriculum_loss_workspace_size(B, K, V))),
                      dtype=torch.uint8, device=dev)
    bws = torch.empty(max(1, D.domino_base_draft_workspace_size(B, K)), dtype=torch.uint8, device=dev)
    loss = torch.zeros((1,), dtype=torch.float32, device=dev)

    def timed(stages):
        """mean ms of each stage (list of callables run in order) over the timed steps"""
        n = len(stages)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(args.steps)]
        for _ in range(args.warmup):
            for f in stages:
                f()
        torch.cuda.synchronize()
        for e in ev:
            e[0].record()
            for j, f in enumerate(stages):
                f()
                e[j + 1].record()
        torch.cuda.synchronize()
        return [float(np.mean([e[j].elapsed_time(e[j + 1]) for e in ev])) for j in range(n)]

    lm = lambda: D.domino_base_logits(head, hidden, base)  # noqa: E731
    states = torch.empty((B, K, w.gru_hidden), dtype=torch.float32, device=dev)
    tf = lambda: D.domino_draft_block(head, hidden, base, x_t, teacher=gold, temperature=w.temperature,  # noqa: E731
                                      seed=w.philox_seed, tokens=tokens, logits=final, gru_states=states,
                                      workspace=ws)
    cl = lambda: D.domino_curriculum_loss(base, final, gold, 0.5, 0.9, loss=loss, grad_base=base,  # noqa: E731
                                          grad_final=final, workspace=lws)
    cbw = {}

    def bw():
        cbw["out"] = D.domino_correction_backward(head, hidden, states, final)

    gb = lambda: D.domino_gru_backward(head, x_t, gold, states, cbw["out"]["d_states"])  # noqa: E731
    t_lm, t_tf, t_cl, t_bw, t_gb = timed([lm, tf, cl, bw, gb])
    loss_bytes = 2 * B * K * V * 4 * 3  # pass 1 reads both tensors; the gradient pass reads and writes both
    out = {"train_forward": {"base_logits_ms": t_lm, "teacher_forced_draft_ms": t_tf, "curriculum_loss_ms": t_cl,
                             "correction_backward_ms": t_bw, "gru_backward_ms": t_gb,
                             "blocks_per_s": B / ((t_lm + t_tf + t_cl) * 1e-3),
                             "with_backward_blocks_per_s": B / ((t_lm + t_tf + t_cl + t_bw + t_gb) * 1e-3),
                             "loss_kernels_gb_s": loss_bytes / (t_cl * 1e-3) / 1e9,
                             "loss_kernels_hbm_frac": loss_bytes / (t_cl * 1e-3) / 1e9 / HBM_PEAK_GBS,
                             "loss_bytes": loss_bytes}}

    vt, vd, vy = S.make_verify_inputs(B, K, V, 0.2, seed=2)
    tt, dd, yy = (torch.from_numpy(a).to(dev) for a in (vt, vd, vy))
    acc = torch.empty((B,), dtype=torch.int32, device=dev)
    nxt = torch.empty((B,), dtype=torch.int32, device=dev)
    vws = torch.empty(max(1, D.domino_verify_workspace_size(B, K, V)), dtype=torch.uint8, device=dev)
    (t_v,) = timed([lambda: D.domino_verify_sampled(tt, dd, yy, 1.0, seed=0, offset=40, accept=acc, next_token=nxt,
                                                    workspace=vws)])
    v_bytes = B * (2 * K + 1) * V * 4  # the normaliser pass; the draw reads at most 2 B V more
    out["verify"] = {"ms": t_v, "blocks_per_s": B / (t_v * 1e-3), "gb_s": v_bytes / (t_v * 1e-3) / 1e9,
                     "hbm_frac": v_bytes / (t_v * 1e-3) / 1e9 / HBM_PEAK_GBS, "bytes": v_bytes}
    del tt, dd, yy, vws

    fr = lambda: D.domino_draft_block(head, hidden, base, x_t, temperature=w.temperature,  # noqa: E731
                                      seed=w.philox_seed, tokens=tokens, workspace=ws)
    bd = lambda: D.domino_base_draft(base, w.temperature, seed=w.philox_seed, tokens=tokens, workspace=bws)  # noqa: E731
    t_lm2, t_fr, t_bd = timed([lm, fr, bd])
    bd_bytes = B * K * V * 4
    out["head_off"] = {"base_logits_ms": t_lm2, "head_on_draft_ms": t_fr, "head_off_draft_ms": t_bd,
                       "head_on_blocks_per_s": B / ((t_lm2 + t_fr) * 1e-3),
                       "head_off_blocks_per_s": B / ((t_lm2 + t_bd) * 1e-3),
                       "base_draft_gb_s": bd_bytes / (t_bd * 1e-3) / 1e9}
    print(json.dumps({"workload": w.name, "batch": B, "block": K, "vocab": V, "steps": args.steps, **out}),
          flush=True)
    return 0


def read_calibration(args) -> int:
    """GB/s of one plain streaming read of 151936 x 4096 bf16 (the Qwen3-8B LM
    head's bytes), HIP events over --steps launches after --warmup; the XOR the
    kernel returns is checked against the host's."""
    import torch

    import draft_block_causal_amd as D

    nbytes = 151936 * 4096 * 2
    g = torch.Generator().manual_seed(5)
    host = torch.randint(-(1 << 31), (1 << 31) - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    buf = host.to("cuda:0")
    sink = torch.empty((2048,), dtype=torch.int32, device="cuda:0")
    for _ in range(args.warmup):
        D.domino_debug_read_stream(buf, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        D.domino_debug_read_stream(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    want = int(np.bitwise_xor.reduce(host.numpy().view(np.uint32)))
    got = int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)))
    print(json.dumps({"read_calibration_bytes": nbytes, "launches": args.steps, "ms": ms,
                      "gb_s": nbytes / (ms * 1e-3) / 1e9, "frac_of_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                      "xor_ok": got == want}), flush=True)
    return 0 if got == want else 3


def forms_base_logits(w, B: int, table: bool) -> bool:
    """Whether the draft call can form the base logits itself at these shapes
    (the library's own rule: one block of at most 16 positions of a bf16 head
    with its GRU input table, d 2560 or 4096, H 1024, r 256)."""
    return (B == 1 and w.dtype == "bf16" and table and w.block <= 16 and w.d in (2560, 4096)
            and w.gru_hidden == 1024 and w.rank == 256)


def cpu_only(args) -> int:
    """The CPU oracle alone on one block of the workload: with every host thread
    its BLAS uses, then limited to one thread."""
    import domino_synth as S

    w = S.get_workload(args.workload)
    head_np, inp = S.make_workload(w, batch=1)
    res = {"workload": w.name, "all_threads": cpu_baseline(w, head_np, inp)}
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover - threadpoolctl missing
        threadpool_limits = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            one = cpu_baseline(w, head_np, inp)
        one["cores"] = 1
        res["one_thread"] = one
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen3_8b_b1_greedy")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="instead of the benchmark, run a plain device-to-device copy of 1 GiB five times; its "
                         "FETCH_SIZE / WRITE_SIZE counters calibrate the HBM-traffic counters of the LM head")
    ap.add_argument("--read-calibration", action="store_true",
                    help="instead of the benchmark, time a plain streaming read (domino_debug_read_stream) of a "
                         "buffer the size of the Qwen3-8B LM head: the read bandwidth the HBM-bound kernels can reach")
    ap.add_argument("--sweep", default=None, metavar="B1,B2,...",
                    help="concurrency sweep: the workload's head at each batch size in the list (e.g. "
                         "1,2,4,8,16,32,64,128); prints one JSON line with a row per batch size instead of the "
                         "benchmark line")
    ap.add_argument("--library-gemm", action="store_true",
                    help="instead of the benchmark, time the LM-head product of the workload through torch's bf16 "
                         "matmul (hipBLASLt on ROCm) next to domino_base_logits, as a reference for the kernel")
    ap.add_argument("--next-rows", action="store_true",
                    help="instead of the benchmark, time the rows beyond the draft path at the workload's shapes: "
                         "the teacher-forced training forward with the curriculum loss and its logit gradients, "
                         "sampled-draft verification, and head-off drafting beside the full head")
    ap.add_argument("--cold", action="store_true",
                    help="write a 512 MB buffer between steps (outside the timed events) so that every step starts "
                         "with the weights evicted from the on-die cache; value is then the mean of the per-step "
                         "HIP-event times")
    ap.add_argument("--cpu-only", action="store_true",
                    help="time only the CPU oracle on one block of the workload, with all host threads and with one "
                         "(no GPU needed); prints one JSON line")
    ap.add_argument("--unfused", action="store_true",
                    help="time domino_base_logits + domino_draft_block even where the draft call can form the base "
                         "logits itself")
    ap.add_argument("--no-table", action="store_true",
                    help="do not build the per-head GRU input table (W_ih E^T + b_ih); the loop then multiplies "
                         "by W_ih at every position")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU only (--gpus {args.gpus} requested); "
              "the multi-GPU sharding of the path is a design, not an implementation.", file=sys.stderr)
        return 2

    if args.cpu_only:
        return cpu_only(args)

    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.read_calibration:
        return read_calibration(args)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": src.numel() * 4, "launches": 5}), flush=True)
        return 0
    import domino_synth as S
    import draft_block_causal_amd as D

    D.load_library()
    dev = torch.device("cuda:0")
    w = S.get_workload(args.workload)
    if args.sweep:
        return sweep(args, w, [int(x) for x in args.sweep.split(",") if x.strip()])
    if args.library_gemm:
        return library_gemm(args, w)
    if args.next_rows:
        return next_rows(args, w)
    head_np, inp = S.make_workload(w)
    B, K, V, d, H, r = w.batch, w.block, w.vocab, w.d, w.gru_hidden, w.rank
    tensors = {k: S.to_torch(v, dev) for k, v in head_np.items() if not (k == "embed" and w.tied)}
    if w.tied:
        tensors["embed"] = tensors["lm_head"]
    head = D.Head(tensors, block=K)
    hidden = S.to_torch(inp["hidden"], dev)
    x_t = S.to_torch(inp["x_t"], dev)
    base = torch.empty((B, K, V), dtype=torch.float32, device=dev)
    tokens = torch.empty((B, K), dtype=torch.int32, device=dev)
    accept = torch.empty((B,), dtype=torch.int32, device=dev)
    ws = torch.empty(D.domino_workspace_size(head, B), dtype=torch.uint8, device=dev)
    prepare_ms = None
    if not args.no_table:
        # one-time, per-head preparation (outside the timed region): T = W_ih E^T + b_ih
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        D.domino_prepare_gru_table(head)
        e1.record()
        torch.cuda.synchronize()
        prepare_ms = e0.elapsed_time(e1)
    torch.cuda.synchronize()

    fused = forms_base_logits(w, B, not args.no_table) and not args.unfused
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    ev_end = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if args.cold else None

    def step(i=None):
        """One draft call: base logits (A1) + the draft block (A2-A5); fused, the
        draft call forms the base logits itself."""
        if i is not None:
            ev[i][0].record()
        if not fused:
            D.domino_base_logits(head, hidden, base)
        if i is not None:
            ev[i][1].record()
        D.domino_draft_block(head, hidden, None if fused else base, x_t, temperature=w.temperature,
                             seed=w.philox_seed, tokens=tokens, workspace=ws)
        if i is not None:
            ev_end[i].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed region: the steps alone (an event record between launches costs
    # GPU time of its own); cold runs take the per-step event times instead
    t0 = time.perf_counter()
    if not args.cold:
        for _ in range(args.steps):
            step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # the per-call breakdown, in a pass of its own, with HIP events on the stream
    # the calls run on (torch's current stream)
    for i in range(args.steps):
        if flush is not None:
            flush.fill_(i & 255)
        step(i)
    torch.cuda.synchronize()
    step_ms = np.array([a.elapsed_time(e) for (a, _), e in zip(ev, ev_end)])
    ms_per_step = float(step_ms.mean()) if args.cold else (t1 - t0) * 1e3 / args.steps
    lm_all = np.array([a.elapsed_time(b) for a, b in ev])
    draft_all = np.array([b.elapsed_time(c) for (_, b), c in zip(ev, ev_end)])
    lm_ms, draft_ms = (None if fused else float(lm_all.mean())), float(draft_all.mean())

    # the run's own output: every loop completed and every token is a valid id
    status = int(D.domino_draft_status(head, B, ws).cpu().numpy()[0])
    tok_np = tokens.cpu().numpy()
    failures = []
    if status != 0:
        failures.append(f"draft status {status}: a loop gave up")
    if tok_np.min() < 0 or tok_np.max() >= V:
        failures.append(f"tokens outside [0, V): min {tok_np.min()}, max {tok_np.max()}")

    # acceptance length (A6), timed on its own, against targets derived from
    # this run's draft: each position keeps the drafted token with probability
    # 0.9, else a uniform token (seeded)
    target_np = S.make_targets(tok_np, V, p=0.9, seed=1)
    target = S.to_torch(target_np, dev)
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(args.warmup):
        D.domino_accept_len(tokens, target, accept)
    ea.record()
    for _ in range(args.steps):
        D.domino_accept_len(tokens, target, accept)
    eb.record()
    torch.cuda.synchronize()
    accept_ms = ea.elapsed_time(eb) / args.steps
    acc_np = accept.cpu().numpy()

    pct = lambda x: {"p10": float(np.percentile(x, 10)), "p50": float(np.percentile(x, 50)),  # noqa: E731
                     "p90": float(np.percentile(x, 90))}
    elem = 2 if w.dtype == "bf16" else 4
    alg = lmhead_algorithmic_bytes(B, K, d, V, elem)
    flops = lmhead_flops(B, K, d, V)
    M = B * K
    # the counter record of the kernel that forms the base logits, taken on this workload
    if M <= 32:
        traffic = measured_traffic(kernel_source_hash(), TRAFFIC_FILE, workload=w.name)
    elif w.dtype == "bf16" and M >= 256:
        traffic = measured_traffic(kernel_source_hash(GEMM_KERNEL_SOURCES), GEMM_TRAFFIC_FILE, workload=w.name)
    else:
        traffic = None
    if fused:
        # the dominant kernel is the loop that streams the LM head itself: the
        # whole call's compulsory bytes (no base logits in HBM) over the draft
        # call's event time (its short pre-launch included)
        alg = block_algorithmic_bytes(B, K, d, V, H, r, elem, base_in_hbm=False)
        achieved = alg / (draft_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS,
                "traffic": measured_traffic(kernel_source_hash(FUSED_KERNEL_SOURCES), FUSED_TRAFFIC_FILE,
                                            workload=w.name),
                "algorithmic_bytes": alg}
    elif flops / alg > RIDGE_FLOP_PER_BYTE:
        achieved = flops / (lm_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": traffic, "algorithmic_flops": flops}
    else:
        achieved = alg / (lm_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "algorithmic_bytes": alg}
    if fused:
        kname = ("draft_b1_kernel<8,10,8,%s,false,%d> (the LM head streamed into an on-chip base-logit table, "
                 "then the 16-position loop, one launch; the events also bracket the pre-loop launch)"
                 % ("true" if w.temperature > 0 else "false", d * 2 // 4 // 64))
    elif M <= 32:
        kname = "rowstream_gemm_kernel (LM head, K split over 8 waves, row-contiguous non-temporal loads)"
    elif w.dtype == "bf16":
        kname = ("gemm_bf16_tn_big_kernel<%d> (LM head, %dx256 tiles, LDS-DMA operand loads)"
                 % ((256, 256) if M >= 256 else (128, 128)))
    else:
        kname = "panel_gemm_kernel (LM head, f32)"
    floor_us = block_floor_us(B, K, d, V, H, r, elem, base_in_hbm=not fused)
    roof.update({"kernel": kname, "avg_launch_ms": draft_ms if fused else lm_ms,
                 # the whole draft call against its own roofline floor (compulsory
                 # bytes at 8 TB/s or FLOPs at the bf16 peak, whichever is larger)
                 "block_floor_us": floor_us, "block_frac": floor_us * 1e-3 / ms_per_step,
                 "block_algorithmic_bytes": block_algorithmic_bytes(B, K, d, V, H, r, elem, base_in_hbm=not fused),
                 "block_flops": block_flops(B, K, d, V, H, r)})

    result = {
        "metric": METRIC,
        "value": B / (ms_per_step * 1e-3),
        "unit": "draft blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_block": ms_per_step / B,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian weights and hidden states; no datasets or checkpoints)",
        "config": {"workload": w.name, "batch": B, "block": K, "d": d, "vocab": V, "gru_hidden": H,
                   "rank": w.rank, "temperature": w.temperature, "tied": w.tied, "parallelism": "none (1 GPU)",
                   "gru_input_table": not args.no_table,
                   "base_logits": "formed inside the draft call" if fused else "domino_base_logits, then the draft call"},
        "gru_table_prepare_ms": prepare_ms,
        "lm_head_ms": lm_ms,
        "draft_block_ms": draft_ms,
        "accept_len_ms": accept_ms,
        "accept_len_mean": float(acc_np.mean()),
        "draft_status": status,
        "step_ms_events": pct(step_ms),
        "lm_head_ms_events": None if fused else pct(lm_all),
        "draft_block_ms_events": pct(draft_all),
        "cold": bool(args.cold),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, head_np, inp, gpu_tokens=tok_np)
        result["cpu_baseline"] = cb
        if cb["gpu_block0_check"]["mismatches"]:
            failures.append(f"block 0 breaks the replay rule at {cb['gpu_block0_check']['mismatches']}")
    if failures:
        result["failures"] = failures
    print(json.dumps(result), flush=True)
    if failures:
        print("bench.py: the run's own output failed its checks: " + "; ".join(failures), file=sys.stderr)
        return 3
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""The benchmark's own arithmetic and contract on the CPU: the compulsory
bytes and FLOPs of the LM-head launch at the Qwen3 workloads (the counts the
roofline fractions are computed from), the traffic record's source check, and
the single-GPU refusal."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_lmhead_bytes_and_flops_at_qwen3_shapes():
    # Qwen3-8B head, one block of 16 positions: W_lm once (151936 x 4096 bf16),
    # 16 hidden rows in, 16 x V float32 base logits out
    assert bench.lmhead_algorithmic_bytes(1, 16, 4096, 151936, 2) == 1_254_514_688
    assert 151936 * 4096 * 2 == 1_244_659_712
    # 32 blocks: 2 * 512 * 151936 * 4096 FLOPs = 637.3 GFLOP, above the ridge
    flops = bench.lmhead_flops(32, 16, 4096, 151936)
    assert flops == 637_265_772_544
    assert flops / bench.lmhead_algorithmic_bytes(32, 16, 4096, 151936, 2) > bench.RIDGE_FLOP_PER_BYTE
    # one block stays far below it (HBM-bound)
    assert bench.lmhead_flops(1, 16, 4096, 151936) / 1_254_514_688 < bench.RIDGE_FLOP_PER_BYTE


def test_traffic_record_matches_current_source_or_is_ignored():
    got = bench.measured_traffic(bench.kernel_source_hash())
    assert got is None or abs(got / bench.lmhead_algorithmic_bytes(1, 16, 4096, 151936, 2) - 1.0) < 0.01
    assert bench.measured_traffic("0" * 64) is None
    # a record only counts for the workload it was taken on (the tiny float32
    # head has 16 rows too)
    assert bench.measured_traffic(bench.kernel_source_hash(), workload="qwen3_8b_b1_greedy") == got
    assert bench.measured_traffic(bench.kernel_source_hash(), workload="tiny_f32_b1") is None
    # the tiled GEMM at 32 blocks (512 rows): W_lm fetched about once, the
    # float32 output written with partial-line overhead; within 1.0 .. 1.3 x
    gemm = bench.measured_traffic(bench.kernel_source_hash(bench.GEMM_KERNEL_SOURCES), bench.GEMM_TRAFFIC_FILE,
                                  workload="qwen3_8b_b32_t1")
    alg32 = bench.lmhead_algorithmic_bytes(32, 16, 4096, 151936, 2)
    assert gemm is None or 1.0 <= gemm / alg32 < 1.3
    # the single-block loop that streams the LM head itself: within 10 % of
    # the call's compulsory bytes without base logits in HBM
    fused = bench.measured_traffic(bench.kernel_source_hash(bench.FUSED_KERNEL_SOURCES), bench.FUSED_TRAFFIC_FILE,
                                   workload="qwen3_8b_b1_greedy")
    alg = bench.block_algorithmic_bytes(1, 16, 4096, 151936, 1024, 256, 2, base_in_hbm=False)
    assert fused is None or abs(fused / alg - 1.0) < 0.1


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=300)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_cpu_only_mode_reports_both_thread_counts():
    import json

    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--cpu-only", "--workload", "tiny_f32_b1"],
                         capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-2000:]
    line = json.loads(res.stdout.strip().splitlines()[-1])
    assert line["all_threads"]["kind"] == "oracle" and line["all_threads"]["value"] > 0
    assert line["one_thread"]["cores"] == 1 and line["one_thread"]["value"] > 0


def test_whole_call_bytes_flops_and_floors_at_the_workloads():
    # compulsory bytes of one draft call: each weight once, gathered embedding
    # rows, hidden in, float32 base logits written and read, x_t in, tokens out
    q8 = dict(K=16, d=4096, V=151936, H=1024, r=256, elem=2)
    assert bench.block_algorithmic_bytes(1, **q8) == 1_376_556_356
    assert bench.block_algorithmic_bytes(32, **q8) == 1_987_566_976
    assert bench.block_algorithmic_bytes(128, **q8) == 3_879_728_896
    assert bench.block_algorithmic_bytes(8, 16, 2560, 151936, 1024, 256, 2) == 1_036_769_056
    # per block: LM head 19.915 G, W2 1.245 G, GRU 0.503 G, W1 0.042 G
    per_block = bench.block_flops(1, 16, 4096, 151936, 1024, 256)
    assert abs(per_block - (19.915e9 + 1.245e9 + 0.503e9 + 0.042e9)) < 0.01e9
    # floors: one Qwen3-8B block is HBM-bound (172.1 us), 32 and 128 blocks
    # are matrix-core-bound (277.8 and 1,111 us)
    assert abs(bench.block_floor_us(1, **q8) - 172.07) < 0.05
    assert abs(bench.block_floor_us(32, **q8) - 277.8) < 0.1
    assert abs(bench.block_floor_us(128, **q8) - 1111.1) < 0.5
    assert abs(bench.block_floor_us(8, 16, 2560, 151936, 1024, 256, 2) - 129.6) < 0.1
    # one block whose call forms the base logits on chip: 16 x V float32
    # written and read back no more (2 x 9,723,904 bytes less)
    assert bench.block_algorithmic_bytes(1, **q8, base_in_hbm=False) == 1_376_556_356 - 2 * 16 * 151936 * 4
    assert abs(bench.block_floor_us(1, **q8, base_in_hbm=False) - 169.64) < 0.05


def test_fused_step_rule_matches_the_library():
    import domino_synth as S

    q8 = S.get_workload("qwen3_8b_b1_greedy")
    assert bench.forms_base_logits(q8, 1, True)
    assert not bench.forms_base_logits(q8, 1, False)  # no GRU input table
    assert not bench.forms_base_logits(q8, 2, True)
    assert bench.forms_base_logits(S.get_workload("qwen3_4b_b8_tied"), 1, True)
    assert not bench.forms_base_logits(S.get_workload("tiny_f32_b1"), 1, True)

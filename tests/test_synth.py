"""The seeded input generator: bf16 rounding, determinism and shapes."""
import numpy as np
import torch

import domino_synth as S


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(size=100_000).astype(np.float32) * 7,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.0078125, 3.4e38, -1e-40], dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(S.f32_to_bf16_bits(x), ref)
    np.testing.assert_array_equal(S.bf16_bits_to_f32(ref), torch.from_numpy(ref.view(np.int16)).view(
        torch.bfloat16).float().numpy())


def test_workload_is_deterministic_and_shaped():
    w = S.get_workload("tiny_f32_b1")
    h1, i1 = S.make_workload(w)
    h2, i2 = S.make_workload(w)
    for k in h1:
        np.testing.assert_array_equal(h1[k], h2[k])
    assert h1["lm_head"].shape == (4096, 256) and h1["w1"].shape == (32, 256 + 128)
    assert i1["hidden"].shape == (1, 16, 256) and i1["x_t"].dtype == np.int32
    assert (0 <= i1["x_t"]).all() and (i1["x_t"] < 4096).all()
    assert abs(h1["w2"].std() - 0.02) < 0.002


def test_tied_workload_shares_the_table():
    w = S.get_workload("qwen3_4b_b8_tied").with_(vocab=64, d=64, gru_hidden=32, rank=32, batch=2)
    h, _ = S.make_workload(w)
    assert h["embed"] is h["lm_head"] and h["lm_head"].dtype == np.uint16


def test_targets_copy_rate():
    draft = S.make_tokens((2000, 16), 1000, seed=5)
    t = S.make_targets(draft, 1000, p=0.9, seed=1)
    rate = (t == draft).mean()
    assert abs(rate - (0.9 + 0.1 / 1000)) < 0.01

"""Plant plausible mistakes in a scratch copy of the oracle and check that the
pin suite rejects every one of them (the mistakes live only in a temporary
directory on the CPU; the real oracle is never modified)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = {
    "update_sign": ("return (1.0 - z) * n + z * g", "return z * n + (1.0 - z) * g"),
    "reset_before_matmul": ("n = np.tanh(a[..., 2 * H:3 * H] + r * c[..., 2 * H:3 * H])",
                            "n = np.tanh(a[..., 2 * H:3 * H] + c[..., 2 * H:3 * H])"),
    "gate_order": ("r = sigmoid(a[..., 0:H] + c[..., 0:H])\n    z = sigmoid(a[..., H:2 * H] + c[..., H:2 * H])",
                   "z = sigmoid(a[..., 0:H] + c[..., 0:H])\n    r = sigmoid(a[..., H:2 * H] + c[..., H:2 * H])"),
    "concat_order": ("z = np.concatenate([h_i, g], axis=-1)", "z = np.concatenate([g, h_i], axis=-1)"),
    "dropped_b2": ("return u @ w2.T + b2", "return u @ w2.T"),
    "feedback_off_by_one": ("else int(tokens[b, i])", "else int(tokens[b, max(i - 1, 0)])"),
    "philox_swapped_products": ("c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0",
                                "c0, c1, c2, c3 = hi0 ^ c1 ^ k0, lo1, hi1 ^ c3 ^ k1, lo0"),
    "philox_no_key_bump": ("k0 = (k0 + _PHILOX_W0) & _MASK32", "k0 = k0"),
    "gumbel_sign": ("return -np.log(-np.log(u))", "return np.log(-np.log(u))"),
    "silu_as_sigmoid": ("return x * sigmoid(x)", "return sigmoid(x)"),
    "accept_len_short": ("while n < draft.shape[1] and", "while n < draft.shape[1] - 1 and"),
    "philox_lane": ("lane = np.broadcast_to(v & np.uint64(3), shape)",
                    "lane = np.broadcast_to((v >> np.uint64(1)) & np.uint64(3), shape)"),
    "temperature_ignored": ("return logits / temperature + gumbel_noise", "return logits + gumbel_noise"),
    "softmax_ignores_temperature": ("x = as_f64(logits) / temperature", "x = as_f64(logits)"),
    "verify_uniform_wrong_lane": ("w = philox_words(seed, offset, b, i, 0).astype(np.float64)",
                                  "w = philox_words(seed, offset, b, i, 1).astype(np.float64)"),
    "verify_ratio_inverted": ("if not (uniform01(seed, offset, b, i) * pd[y] < pt[y]):",
                              "if not (uniform01(seed, offset, b, i) * pt[y] < pd[y]):"),
    "verify_residual_reversed": ("q = softmax(tl[b, n], temperature) - softmax(dl[b, n], temperature)",
                                 "q = softmax(dl[b, n], temperature) - softmax(tl[b, n], temperature)"),
    "verify_bonus_position": ("s = tl[b, K] / temperature + g", "s = tl[b, K - 1] / temperature + g"),
    "verify_shared_noise_stream": ("g = gumbel_noise(seed, offset + 1, b, n, np.arange(V))",
                                   "g = gumbel_noise(seed, offset, b, n, np.arange(V))"),
    "base_draft_position_keys_swapped": ("sampling_scores(base[b, i], temperature, seed, offset, b, i)",
                                         "sampling_scores(base[b, i], temperature, seed, offset, i, b)"),
    "curriculum_lambda_swapped": ("loss += w[i] * ((1.0 - lam) * ce_f[b, i] + lam * ce_b[b, i])",
                                  "loss += w[i] * (lam * ce_f[b, i] + (1.0 - lam) * ce_b[b, i])"),
    "position_weights_growing": ("return np.power(float(gamma), np.arange(K, dtype=np.float64))",
                                 "return np.power(float(gamma), -np.arange(K, dtype=np.float64))"),
    "gradient_without_onehot": ("p[y] -= 1.0", "p[y] -= 0.0"),
    "silu_derivative_wrong": ("dz = du * sz * (1.0 + z * (1.0 - sz))", "dz = du * sz * (1.0 - sz)"),
    "backward_state_columns": ("\"dg\": (dz @ f[\"w1\"][:, d:])", "\"dg\": (dz @ f[\"w1\"][:, :g.shape[-1]])"),
    "bptt_carry_without_recurrence": ("carry = d_g * z + f[\"w_hh\"].T @ dc", "carry = d_g * z"),
    "bptt_reset_gradient_position": ("dc = np.concatenate([d_pr, d_pz, d_pn * r])", "dc = np.concatenate([d_pr, d_pz, d_pn])"),
    "base_logits_transposed_operand": ("return as_f64(hidden) @ as_f64(lm_head).T",
                                       "return (as_f64(lm_head) @ as_f64(hidden).swapaxes(-1, -2)).swapaxes(-1, -2)[..., ::-1]"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_reject_planted_mistake(name, tmp_path):
    before, after = MUTATIONS[name]
    for sub in ("oracle", "domino_synth", "tests"):
        shutil.copytree(os.path.join(ROOT, sub), tmp_path / sub,
                        ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutations.py"))
    path = tmp_path / "oracle" / "domino_oracle.py"
    src = path.read_text()
    assert before in src, f"mutation site for {name} not found"
    path.write_text(src.replace(before, after))
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          "tests/test_oracle_pins.py"], cwd=tmp_path, capture_output=True, text=True,
                         timeout=600)
    assert res.returncode != 0, f"pins accepted the planted mistake {name}:\n{res.stdout[-2000:]}"

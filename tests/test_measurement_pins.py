"""Pins of the measurement arithmetic against the paper's printed worked example
(tests/golden/llama3_8b_flops_per_token.txt) and of the workload shapes."""

import os

import synthetic

GOLD = os.path.join(os.path.dirname(__file__), "golden", "llama3_8b_flops_per_token.txt")


def load_gold():
    out = {}
    for line in open(GOLD):
        line = line.split("#")[0].strip()
        if line:
            k, v = (s.strip() for s in line.split("="))
            out[k] = float(v)
    return out


def test_eq12_flops_per_token():
    g = load_gold()
    f = 6 * (g["N"] - g["N_emb"]) + 12 * g["L"] * g["H"] * g["d_h"] * g["S"]
    assert f == g["F_model_per_token"]


def test_eq13_mfu_round_trip():
    g = load_gold()
    rate = g["mfu_h32_route"] * g["peak_bf16_flops"] / g["F_model_per_token"]
    assert 37200 <= rate <= 37300           # the summary's "37.2K tokens/s/GPU"


def test_ffn_workload_shapes_reproduce_parameter_count():
    # hidden 4096, FFN 14336 (the FFN-step workload), 32 layers, 32 query and
    # 8 key/value heads of 128, vocabulary 128256 reproduce N and N_emb exactly.
    g = load_gold()
    spec = synthetic.WORKLOADS["ffn_step_8192x4096x14336"]["tensors"]
    D, F = spec["W2"][0], spec["W2"][1]
    vocab, layers, kv = 128256, 32, 8 * 128
    attn = 2 * D * D + 2 * D * kv
    per_layer = attn + 3 * D * F + 2 * D
    n = layers * per_layer + D + 2 * vocab * D
    assert vocab * D == g["N_emb"]
    assert n == g["N"]


def test_bench_refuses_more_than_one_gpu():
    """bench.py --gpus 2 exits with status 2 and a JSON error line before it
    touches a GPU."""
    import json
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert out.returncode == 2
    line = json.loads(out.stdout.strip().splitlines()[-1])
    assert line["gpus_requested"] == 2 and "--gpus must be 1" in line["error"]

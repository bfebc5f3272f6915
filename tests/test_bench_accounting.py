"""The benchmark's byte accounting, which every reported bandwidth and
roofline share divides by, against closed forms of the cost model (Go under
the hood 20.3.2: a step reads every weight once and each row's K/V once),
worked out here from the shapes by hand; and the one-GPU contract of the
command line."""
import subprocess
import sys
import os

import numpy as np

import bench
from continuous_batching_decode_forward_amd import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_8b_layer_weight_bytes_closed_form():
    # one 8B-shaped layer: QKV 6144 x 4096, O 4096 x 4096, gate and up
    # 14336 x 4096, down 4096 x 14336, two norm gains of 4096; LM head
    # 128256 x 4096 and the final gain; all bf16
    layer = 6144 * 4096 + 4096 * 4096 + 3 * 14336 * 4096 + 2 * 4096
    total = 2 * (layer + 128256 * 4096 + 4096)
    ctx = np.array([0])
    # W + one embedding row + 1 cached position read + 1 appended (4 KB
    # each for 8 KV heads x 128 dims x K and V in bf16) + the fp32 logits
    want = total + 4096 * 2 + 2 * 4096 + 128256 * 4
    assert bench.step_bytes(configs.LLAMA8B_1L, ctx, 1) == want
    assert total == 1_486_905_344


def test_class_bytes_sum_to_the_step_bytes():
    shape = configs.LLAMA8B_1L
    ctx = np.array([511, 4095, 1000, 7])
    cb = bench.class_bytes(shape, ctx, len(ctx))
    assert cb["qkv"] == 2 * 6144 * 4096 and cb["o"] == 2 * 4096 * 4096
    assert cb["gateup"] == 2 * 2 * 14336 * 4096 and cb["down"] == 2 * 4096 * 14336
    assert cb["attn"] == sum((c + 2) * 4096 for c in ctx)
    assert cb["lm_head"] == 128256 * 4096 * 2 + 4 * 4096 * 2 + 4 * 128256 * 4
    # the step adds the norm gains and embedding rows, and the LM head's
    # activation rows are counted only by its class
    rest = 2 * (2 * 4096 + 4096) + len(ctx) * 4096 * 2 - len(ctx) * 4096 * 2
    assert sum(cb.values()) + rest == bench.step_bytes(shape, ctx, len(ctx))


def test_kv_bytes_scale_with_layers_and_format():
    assert bench.kv_bytes_per_pos(configs.LLAMA8B) == 131072
    assert bench.kv_bytes_per_pos(configs.QWEN2B) == 114688
    assert bench.kv_bytes_per_pos(configs.LLAMA8B, elem=1) == 65536


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr

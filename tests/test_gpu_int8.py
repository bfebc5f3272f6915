"""GPU parity with int8 weights (every projection and the LM head as int8
codes with one float32 scale per matrix row, read as q * scale; the
embedding and the norm gains bf16), against the oracle's int8 model on the
same codes and scales.

Checks:
  * the tiny 2-layer decoder end to end (prefill chunks, then greedy
    decode): logits within the stated tolerance, greedy ids on decidable
    rows; chunks of 100 rows put more than 64 rows through the streaming
    GEMM (two row groups), 8-row chunks one;
  * one 8B-shaped layer + LM head at B = 1, 8, 64 (one row group) and
    B = 96, 200 (two and four row groups): sampled rows' logits against the
    oracle, every row's attention, greedy ids equal to the argmax of the
    GPU's own logits on every row."""
import numpy as np
import pytest
import torch

import oracle as O
from continuous_batching_decode_forward_amd import configs, synth

from gpu_util import weights_to
import test_gpu_8b
import test_gpu_tiny

pytestmark = pytest.mark.gpu

ATTN_TOL = 2.0 ** -12


@pytest.fixture(scope="module")
def tiny8w():
    w = synth.make_weights_int8(configs.TINY, seed=0)
    return w, O.Model(configs.TINY, w), weights_to(w, "cuda")


@pytest.mark.parametrize("bs,chunk", [(16, 8), (32, 100), (8, 40)])
def test_tiny_int8_weights_prefill_then_decode(tiny8w, bs, chunk):
    cfg = configs.TINY
    # first step: bs - 1 + 1 + min(chunk, 120) + min(chunk, 70) rows (at most 202)
    prompts = [synth.uniform_ints(bs, f"p{i}", L, 0, cfg.vocab - 1)
               for i, L in enumerate([bs - 1, 1, 120, 70])]
    res = test_gpu_tiny.run_schedule(tiny8w, prompts, 6, chunk=chunk, bs=bs, nb=80, seed=bs)
    test_gpu_tiny.check(res)
    worst = max(r[2] for r in res)
    print(f"tiny int8 weights bs={bs} chunk={chunk}: {len(res)} steps, max abs logit error "
          f"{worst:.2e}")


@pytest.fixture(scope="module")
def big8w():
    shape = configs.LLAMA8B_1L
    wg = synth.make_weights_int8(shape, seed=0, device="cuda")
    wc = {k: ([t.cpu() for t in v] if isinstance(v, list) else v.cpu()) for k, v in wg.items()}
    return wg, O.Model(shape, wc)


@pytest.mark.parametrize("Bn,rows", [(1, [0]), (8, [0, 7]), (64, [0, 33, 63]), (96, [0, 70, 95]),
                                     (200, [0, 130, 199])])
def test_8b_layer_int8_weights_decode_step(big8w, Bn, rows):
    wg, om = big8w
    ok, mx, res, g_tk, r_tk, own, all_tk, att = test_gpu_8b.decode_step(
        (wg, om), Bn, seed=200 + Bn, sample_rows=rows, om=om)
    print(f"8b int8 weights B={Bn}: max abs logit error {mx:.4f}, decidable rows "
          f"{int(res.sum())}/{len(rows)}, attention of all {Bn} rows: largest error {att.max():.2e}")
    assert ok, f"max abs logit error {mx:.3g}"
    assert att.max() <= ATTN_TOL
    assert np.array_equal(g_tk[res], r_tk[res])
    assert np.array_equal(own, all_tk)


def test_tiny_int8_weights_with_an_e4m3_cache():
    """Both storage formats at once: int8 weights and an 8-bit KV cache, on
    the tiny decoder end to end, against the oracle run with both."""
    from continuous_batching_decode_forward_amd import binding as B
    cfg = configs.TINY
    w = synth.make_weights_int8(cfg, seed=2)
    kv = dict(kv_dtype=B.CBD_KV_FP8_E4M3, k_scale=0.05, v_scale=0.03)
    om = O.Model(cfg, w, kv_fp8=True, k_scale=kv["k_scale"], v_scale=kv["v_scale"])
    bs, chunk = 16, 40
    prompts = [synth.uniform_ints(5, f"p{i}", L, 0, cfg.vocab - 1)
               for i, L in enumerate([bs - 1, 1, 90, 37])]
    res = test_gpu_tiny.run_schedule((w, om, weights_to(w, "cuda")), prompts, 6, chunk=chunk,
                                     bs=bs, nb=80, seed=7, kv=kv)
    test_gpu_tiny.check(res)
    print(f"tiny int8 weights + e4m3 cache: {len(res)} steps, max abs logit error "
          f"{max(r[2] for r in res):.2e}")

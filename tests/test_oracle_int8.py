"""Pins of the oracle's int8-weight model (codes q with one float32 scale
per matrix row, read as q * scale; the follow-up "int8 weights" of the
RWKV-Runner Albatross article's roadmap).

Each pin reduces to something the bf16 model or plain arithmetic fixes:
  * with power-of-two row scales, q * scale is exactly a bf16 value, so the
    int8 linear equals the bf16 linear over those dequantised weights bit
    for bit (scaling by a power of two commutes with every rounding);
  * a whole paged step of the int8 model equals the bf16 model's over the
    dequantised weights, byte for byte, with different scales in every row
    of every matrix (a scale applied per column, or taken from the wrong
    matrix, fails it);
  * K = 1 closed form; the batched step equals serial decoding."""
import numpy as np
import pytest
import torch

import oracle as O
from continuous_batching_decode_forward_amd import configs, synth


def pow2_scales(n, seed):
    rng = np.random.default_rng(seed)
    return (2.0 ** -rng.integers(5, 12, n)).astype(np.float32)


def dequant_bf16(q, s):
    """bf16 bits of q * s (exact for power-of-two s and |q| <= 127)."""
    v = (q.astype(np.float64) * s.astype(np.float64)[:, None]).astype(np.float32)
    bits = v.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "not exactly a bf16 value"
    return (bits >> 16).astype(np.uint16)


def test_int8_linear_equals_bf16_linear_on_exact_dequantised_weights():
    rng = np.random.default_rng(0)
    N, K = 37, 300  # not square: a row/column mix-up changes the shape
    q = rng.integers(-127, 128, (N, K)).astype(np.int8)
    s = pow2_scales(N, 1)
    x = rng.standard_normal(K)
    y8 = O.linear_i8(x, q, s)
    y16 = O.linear(x, dequant_bf16(q, s))
    assert np.array_equal(y8, y16)
    # scales belong to rows: scaling one row scales only that output
    s2 = s.copy()
    s2[5] *= 2
    y8b = O.linear_i8(x, q, s2)
    assert y8b[5] == 2 * y8[5] and np.array_equal(np.delete(y8b, 5), np.delete(y8, 5))


def test_int8_linear_k1_closed_form():
    q = np.array([[-127], [0], [1], [127]], np.int8)
    s = np.array([0.5, 3.0, 0.1, 2.0 ** -20], np.float32)
    y = O.linear_i8(np.array([1.5]), q, s)
    assert np.array_equal(y, [float(np.float32(0.5)) * -127 * 1.5, 0.0, float(np.float32(0.1)) * 1.5,
                              2.0 ** -20 * 127 * 1.5])


def test_generated_codes_and_scales():
    q = synth.int8_codes(0, "t", (64, 1024))
    assert q.dtype == torch.int8 and int(q.abs().max()) <= 127
    assert 35 < float(q.float().std()) < 46
    s = synth.row_scales(0, "t", 4096, 0.02)
    assert float(s.min()) >= 0.02 / 40 * 0.75 and float(s.max()) < 0.02 / 40 * 1.25
    assert torch.equal(q, synth.int8_codes(0, "t", (64, 1024)))  # seeded


def _int8_weights_pow2(shape, seed):
    """int8 weights whose row scales are powers of two, and the bf16 weight
    set of their exact dequantised values."""
    w8 = synth.make_weights_int8(shape, seed)
    w16 = dict(w8)
    rng = np.random.default_rng(seed)
    for k, sk in O.SCALES.items():
        if k == "lm_head":
            s = pow2_scales(shape.vocab, rng.integers(1 << 30))
            w8[sk] = torch.from_numpy(s)
            w16[k] = torch.from_numpy(dequant_bf16(w8[k].numpy(), s).view(np.int16)).view(torch.bfloat16)
        else:
            w8[sk], w16[k] = [], []
            for q in w8[k]:
                s = pow2_scales(q.shape[0], rng.integers(1 << 30))
                w8[sk].append(torch.from_numpy(s))
                w16[k].append(torch.from_numpy(dequant_bf16(q.numpy(), s).view(np.int16))
                              .view(torch.bfloat16))
    for sk in O.SCALES.values():
        w16.pop(sk, None)
    return w8, w16


def test_int8_step_equals_bf16_step_on_exact_dequantised_weights():
    shape = configs.TINY
    w8, w16 = _int8_weights_pow2(shape, 3)
    m8, m16 = O.Model(shape, w8), O.Model(shape, w16)
    assert m8.w_int8 and not m16.w_int8
    bs, nb = 4, 32
    tables = np.arange(nb, dtype=np.int32).reshape(4, 8)
    ctx, nn = [0, 0, 0, 0], [5, 9, 1, 14]
    toks = synth.uniform_ints(3, "tok", sum(nn), 0, shape.vocab - 1)
    out = []
    for m in (m8, m16):
        pool = m.paged_pool(nb, bs)
        lg, tk = O.paged_step(m, pool, tables, ctx, nn, toks, [1, 1, 1, 1])
        out.append((lg, tk, pool))
    assert np.array_equal(out[0][0], out[1][0])
    assert np.array_equal(out[0][1], out[1][1])
    assert np.array_equal(out[0][2], out[1][2])  # the appended K/V too


def test_int8_batched_step_equals_serial():
    shape = configs.TINY
    w8 = synth.make_weights_int8(shape, 5)
    m = O.Model(shape, w8)
    prompts = [synth.uniform_ints(5, f"p{i}", n, 0, shape.vocab - 1) for i, n in enumerate([3, 7, 12])]
    # serial: each sequence alone, token by token
    serial = []
    for p in prompts:
        kv = m.dense_kv(16)
        serial.append(O.serial_forward(m, kv, p, 0))
    # batched: one paged step with every prompt as a chunk
    bs = 4
    tables = np.arange(12, dtype=np.int32).reshape(3, 4)
    pool = m.paged_pool(12, bs)
    lg, _ = O.paged_step(m, pool, tables, [0, 0, 0], [len(p) for p in prompts],
                         np.concatenate(prompts), [1, 1, 1])
    for i in range(3):
        assert np.array_equal(lg[i], serial[i])

"""Pins for the oracle's FP8 (OCP E4M3) KV cache: the code conversions
against PyTorch's float8_e4m3fn (an independent implementation of the same
format), exhaustively over codes and over every midpoint between
neighbouring values, plus the stated saturation; and the fp8 step itself:
batched equals serial byte for byte, the appended codes are the rounded
rotated keys and values, and attention over the cache equals dense attention
over the decoded values (the "Continuous Batching" practice article, section
6: quantise the KV cache to FP8)."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from continuous_batching_decode_forward_amd import configs, synth

CFG = configs.TINY


def torch_decode(codes):
    t = torch.as_tensor(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.float().numpy().astype(np.float64)


def torch_encode(x):
    return torch.as_tensor(np.asarray(x, np.float64)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_decode_of_every_code_matches_torch():
    ref = torch_decode(np.arange(256))
    got = np.array([O.e4m3_to_float(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2  # 0x7f and 0xff
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7e] == 448.0 and got[0x01] == 2.0 ** -9


def test_encode_matches_torch_on_codes_midpoints_and_their_neighbours():
    # binary32 inputs (torch rounds through binary32; on those the exact
    # nearest-code rule and torch's must agree bit for bit)
    vals = np.array([O.e4m3_to_float(c) for c in range(0x7f)], np.float32)
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)  # exact
    xs = np.concatenate([vals, mids, np.nextafter(mids, np.float32(0)),
                         np.nextafter(mids, np.float32(1e9))])
    xs = np.concatenate([xs, -xs, np.linspace(-448, 448, 20001).astype(np.float32)])
    got = np.array([O.float_to_e4m3(float(x)) for x in xs], np.uint8)
    ref = torch_encode(xs.astype(np.float64))
    # negative zero: both give the sign bit with a zero magnitude
    assert np.array_equal(got, ref)
    # round to nearest, ties to the even code; from a double, the exact
    # nearest (a value one double ulp below a midpoint goes down)
    assert O.float_to_e4m3(1.0 + 1 / 16) == O.float_to_e4m3(1.0)
    assert O.float_to_e4m3(1.0 + 3 / 16) == O.float_to_e4m3(1.25)
    below = np.nextafter(1.0 + 3 / 16, 0.0)
    assert O.float_to_e4m3(below) == O.float_to_e4m3(1.125)


def test_encode_saturates_and_roundtrips():
    for x in (448.0, 449.0, 464.0, 465.0, 1e4, 1e300):
        assert O.float_to_e4m3(x) == 0x7E and O.float_to_e4m3(-x) == 0xFE
    assert O.float_to_e4m3(float("nan")) == 0x7F
    for c in list(range(0x7F)) + list(range(0x80, 0xFF)):
        assert O.float_to_e4m3(O.e4m3_to_float(c)) == (c if c != 0x80 else 0x80)
    rng = np.random.default_rng(1)
    xs = np.sort(rng.standard_normal(4000) * 3)
    dq = np.array([O.e4m3_to_float(O.float_to_e4m3(x)) for x in xs])
    assert np.all(np.diff(dq) >= 0)  # monotone
    # within half a spacing: 2^-4 relative for normals, 2^-10 absolute below
    assert np.all(np.abs(dq - xs) <= np.maximum(np.abs(xs) * 2.0 ** -4, 2.0 ** -10) * 1.0000001)


def fp8_model(seed, k_scale=1.0, v_scale=1.0, layers=2):
    cfg = CFG.with_layers(layers)
    return cfg, synth.make_weights(cfg, seed), dict(kv_fp8=True, k_scale=k_scale, v_scale=v_scale)


def test_fp8_batched_step_equals_serial_byte_for_byte():
    cfg, w, kw = fp8_model(0, k_scale=0.5, v_scale=2.0)
    m = O.Model(cfg, w, **kw)
    prompts = [synth.uniform_ints(3, f"p{i}", n, 0, cfg.vocab - 1) for i, n in enumerate((9, 4, 13))]
    perm = synth.permutation(3, "blocks", 48)
    tables = np.stack([perm[i * 16:(i + 1) * 16] for i in range(3)]).astype(np.int32)
    pool = m.paged_pool(48, 4)
    nn = [len(p) for p in prompts]
    lg, g = O.paged_step(m, pool, tables, [0, 0, 0], nn, np.concatenate(prompts), [1, 1, 1])
    toks = [int(t) for t in g]
    lg2, _ = O.paged_step(m, pool, tables, nn, [1, 1, 1], toks, [1, 1, 1])
    for i, p in enumerate(prompts):
        kv = m.dense_kv(32)
        ser = O.serial_forward(m, kv, p, 0, last_only=False)
        assert np.array_equal(ser[-1], lg[i])
        assert np.array_equal(O.serial_forward(m, kv, [toks[i]], len(p)), lg2[i])
    assert pool.dtype == np.uint8 and pool.any()


def test_fp8_appends_are_the_rounded_rotated_keys_and_values():
    cfg, w, kw = fp8_model(5, k_scale=0.25, v_scale=4.0, layers=1)
    w["w_gate"] = [torch.zeros_like(t) for t in w["w_gate"]]
    m = O.Model(cfg, w, **kw)
    kv = m.dense_kv(4)
    toks = [11, 2222]
    lg = O.serial_forward(m, kv, toks, 0, last_only=False)
    hq, hkv, hd = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    wqkv = O.bf16_to_f64(w["w_qkv"][0]).reshape(-1, cfg.d_model)
    x = O.bf16_to_f64(w["embed"][toks[1]])
    qkv = wqkv @ O.rmsnorm(x, w["attn_norm"][0], cfg.rms_eps)
    k1 = np.concatenate([O.rope(qkv[(hq + i) * hd:(hq + i + 1) * hd], 1, cfg.rope_base)
                         for i in range(hkv)])
    v1 = qkv[(hq + hkv) * hd:]
    assert np.array_equal(kv[0, 0, 1].reshape(-1), torch_encode(k1 / 0.25))
    assert np.array_equal(kv[0, 1, 1].reshape(-1), torch_encode(v1 / 4.0))
    # the layer's attention reads value = decode(code) * scale: dense
    # attention over the decoded cache (numpy) rebuilds the logits
    q = np.concatenate([O.rope(qkv[j * hd:(j + 1) * hd], 1, cfg.rope_base) for j in range(hq)])
    K = torch_decode(kv[0, 0, :2].reshape(-1)).reshape(2, hkv, hd) * 0.25
    V = torch_decode(kv[0, 1, :2].reshape(-1)).reshape(2, hkv, hd) * 4.0
    o = np.empty(hq * hd)
    for h in range(hq):
        g = h * hkv // hq
        s = K[:, g] @ q[h * hd:(h + 1) * hd] / math.sqrt(hd)
        p = np.exp(s - s.max())
        o[h * hd:(h + 1) * hd] = (p / p.sum()) @ V[:, g]
    assert np.allclose(O.attention_dense_fp8(q, kv[0, 0, :2], kv[0, 1, :2], hq, hkv, hd, 0.25, 4.0),
                       o, rtol=0, atol=1e-12)
    t = O.bf16_to_f64(w["w_o"][0]).reshape(cfg.d_model, hq * hd) @ o
    hf = O.rmsnorm(x + t, w["final_norm"], cfg.rms_eps)
    # the LM head takes its input rounded to bf16
    lm = O.bf16_to_f64(w["lm_head"]).reshape(cfg.vocab, cfg.d_model) @ O.bf16_to_f64(O.bf16_round(hf))
    assert np.allclose(lg[1], lm, rtol=0, atol=1e-9)

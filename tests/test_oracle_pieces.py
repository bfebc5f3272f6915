"""Pins for the oracle's building blocks, against things other than itself:
exact special cases, closed forms, invariants, brute force and library
routines (numpy float64 products and softmax, numpy's Philox generator)."""
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from continuous_batching_decode_forward_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits via torch (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------- bf16

def test_bf16_round_trip_and_halfway_cases():
    # values exactly representable in bf16 survive
    for v in (0.0, 1.0, -2.5, 0.0078125, 1.5, 2.0 ** 100):
        assert O.bf16_to_float(O.f64_to_bf16(v)) == v
    one = 1.0
    ulp = 2.0 ** -7                      # bf16 spacing just above 1
    # exactly halfway between 1 and 1+ulp -> even (1.0)
    assert O.bf16_to_float(O.f64_to_bf16(one + ulp / 2)) == 1.0
    # halfway between 1+ulp and 1+2ulp -> even (1+2ulp)
    assert O.bf16_to_float(O.f64_to_bf16(one + 1.5 * ulp)) == one + 2 * ulp
    # a hair above halfway rounds up, a hair below rounds down
    assert O.bf16_to_float(O.f64_to_bf16(one + ulp / 2 + 1e-12)) == one + ulp
    assert O.bf16_to_float(O.f64_to_bf16(one + ulp / 2 - 1e-12)) == 1.0
    assert O.bf16_to_float(O.f64_to_bf16(-(one + 1.5 * ulp))) == -(one + 2 * ulp)
    assert math.isinf(O.bf16_to_float(O.f64_to_bf16(1e39)))


def test_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(20000).astype(np.float32) * \
        np.float32(10.0) ** rng.integers(-20, 20, 20000).astype(np.float32)
    ref = bf16_bits(x)
    got = np.array([O.f64_to_bf16(float(v)) for v in x], np.uint16)
    assert np.array_equal(ref, got)


# ------------------------------------------------------------------ linear

def test_linear_matches_numpy_float64():
    rng = np.random.default_rng(2)
    K, N = 300, 37
    x = rng.standard_normal(K)
    W = bf16_bits(rng.standard_normal((N, K)).astype(np.float32))
    got = O.linear(x, W.reshape(N, K))
    ref = O.bf16_to_f64(W).reshape(N, K) @ x
    assert np.allclose(got, ref, rtol=0, atol=1e-12)
    # a transposed operand would not agree
    assert not np.allclose(got, (O.bf16_to_f64(W).reshape(N, K).T[:N, :N] @ x[:N]))


# ----------------------------------------------------------------- rmsnorm

def test_rmsnorm_unit_gain_gives_unit_mean_square():
    rng = np.random.default_rng(3)
    for d in (64, 256, 4096):
        x = rng.standard_normal(d) * 3.7
        g = bf16_bits(np.ones(d, np.float32))
        y = O.rmsnorm(x, g, 1e-5)
        # mean(y^2) = ms / (ms + eps) exactly
        ms = np.mean(x * x)
        assert abs(np.mean(y * y) - ms / (ms + 1e-5)) < 1e-12
        # direction kept: y is a positive multiple of x
        ratio = y / x
        assert np.allclose(ratio, ratio[0], rtol=1e-12) and ratio[0] > 0


def test_rmsnorm_gain_is_elementwise_and_eps_matters_for_tiny_inputs():
    rng = np.random.default_rng(4)
    d = 128
    x = rng.standard_normal(d)
    g1 = bf16_bits(np.ones(d, np.float32))
    g2 = bf16_bits(np.full(d, 2.0, np.float32))
    y1, y2 = O.rmsnorm(x, g1, 1e-5), O.rmsnorm(x, g2, 1e-5)
    assert np.array_equal(2.0 * y1, y2)          # doubling is exact
    gz = np.ones(d, np.float32)
    gz[5] = 0
    yz = O.rmsnorm(x, bf16_bits(gz), 1e-5)
    assert yz[5] == 0 and np.array_equal(np.delete(yz, 5), np.delete(y1, 5))
    # all-zero input: eps keeps it finite and the output is zero
    assert np.all(O.rmsnorm(np.zeros(d), g1, 1e-5) == 0)
    # a tiny input is damped by eps: y = x / sqrt(ms + eps)
    t = np.full(d, 1e-4)
    assert abs(O.rmsnorm(t, g1, 1e-5)[0] - 1e-4 / math.sqrt(1e-8 + 1e-5)) < 1e-15


# -------------------------------------------------------------------- rope

def test_rope_position_zero_is_identity_and_pairing():
    hd = 64
    rng = np.random.default_rng(5)
    v = rng.standard_normal(hd)
    assert np.array_equal(O.rope(v, 0, 10000.0), v)
    # element 0 turns by exactly `pos` radians against element hd/2; element
    # i turns by pos * base^(-2i/hd)
    for i in (0, 5, 31):
        e = np.zeros(hd)
        e[i] = 1.0
        ang = 7 * 10000.0 ** (-2 * i / hd)
        r = O.rope(e, 7, 10000.0)
        assert abs(r[i] - math.cos(ang)) < 1e-14 and abs(r[i + hd // 2] - math.sin(ang)) < 1e-14
        assert np.count_nonzero(r) == 2
    # the second half rotates the other way round: (0, 1) -> (-sin, cos)
    e = np.zeros(hd)
    e[hd // 2] = 1.0
    r = O.rope(e, 1, 10000.0)
    assert abs(r[0] + math.sin(1.0)) < 1e-14 and abs(r[hd // 2] - math.cos(1.0)) < 1e-14


def test_rope_preserves_pair_norms_and_relative_positions():
    hd = 128
    rng = np.random.default_rng(6)
    q = rng.standard_normal(hd)
    k = rng.standard_normal(hd)
    for pos in (1, 17, 3000):
        rq = O.rope(q, pos, 10000.0)
        n0 = q[:hd // 2] ** 2 + q[hd // 2:] ** 2
        n1 = rq[:hd // 2] ** 2 + rq[hd // 2:] ** 2
        assert np.allclose(n0, n1, rtol=1e-12, atol=0)
    # q(p+t).k(p'+t) = q(p).k(p') for any shift t
    def dot(p1, p2):
        return float(np.dot(O.rope(q, p1, 1e4), O.rope(k, p2, 1e4)))
    base = dot(10, 3)
    for t in (1, 50, 700):
        assert abs(dot(10 + t, 3 + t) - base) < 1e-9 * (1 + abs(base))
    assert abs(dot(11, 3) - base) > 1e-3          # it does depend on the offset


# --------------------------------------------------------------- attention

def brute_attention(q, K, V, hq, hkv, hd, group=None):
    """softmax(q k^T / sqrt(hd)) v per head in numpy float64; query head h
    reads KV head group(h), by default h // (hq // hkv)."""
    qf = np.asarray(q, np.float64).reshape(hq, hd)
    Kf = O.bf16_to_f64(K).reshape(-1, hkv, hd)
    Vf = O.bf16_to_f64(V).reshape(-1, hkv, hd)
    out = np.empty((hq, hd))
    for h in range(hq):
        g = group(h) if group else h // (hq // hkv)
        s = Kf[:, g, :] @ qf[h] / math.sqrt(hd)
        p = np.exp(s - s.max())
        p /= p.sum()
        out[h] = p @ Vf[:, g, :]
    return out


@pytest.mark.parametrize("n,hq,hkv,hd", [(1, 4, 2, 64), (7, 4, 2, 64), (33, 8, 2, 32),
                                         (130, 32, 8, 128)])
def test_attention_matches_dense_brute_force(n, hq, hkv, hd):
    rng = np.random.default_rng(n + hq)
    q = rng.standard_normal(hq * hd)
    K = bf16_bits(rng.standard_normal((n, hkv, hd)).astype(np.float32))
    V = bf16_bits(rng.standard_normal((n, hkv, hd)).astype(np.float32))
    got = O.attention_dense(q, K, V, hq, hkv, hd).reshape(hq, hd)
    ref = brute_attention(q, K, V, hq, hkv, hd)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)
    if n == 1:   # a single key: the output is that value vector
        for h in range(hq):
            assert np.array_equal(got[h], O.bf16_to_f64(V)[0, h // (hq // hkv)])
    # the wrong group mapping (h % hkv instead of h // G) disagrees
    if hkv > 1 and n > 1:
        wrong = brute_attention(q, K, V, hq, hkv, hd, group=lambda h: h % hkv)
        assert not np.allclose(got, wrong, atol=1e-6)


def test_attention_equal_keys_average_values():
    n, hq, hkv, hd = 9, 4, 2, 64
    rng = np.random.default_rng(11)
    q = rng.standard_normal(hq * hd)
    K = np.repeat(bf16_bits(rng.standard_normal((1, hkv, hd)).astype(np.float32)), n, 0)
    V = bf16_bits(rng.standard_normal((n, hkv, hd)).astype(np.float32))
    got = O.attention_dense(q, K, V, hq, hkv, hd).reshape(hq, hd)
    mean = O.bf16_to_f64(V).reshape(n, hkv, hd).mean(0)
    for h in range(hq):
        assert np.allclose(got[h], mean[h // 2], rtol=0, atol=1e-14)


# ------------------------------------------------------------------ argmax

def test_argmax_ties_go_to_lowest_id():
    x = np.zeros(1000, np.float32)
    x[[17, 400, 999]] = 3.0
    assert O.argmax_f32(x) == 17
    x[3] = np.nextafter(np.float32(3.0), np.float32(0))
    assert O.argmax_f32(x) == 17
    x[900] = np.nextafter(np.float32(3.0), np.float32(4))
    assert O.argmax_f32(x) == 900
    assert O.argmax_f32(np.full(10, -np.inf, np.float32)) == 0
    assert O.argmax_f64(np.array([1.0, 2.0, 2.0])) == 1


# ------------------------------------------------------------------ Philox

def test_philox_known_answer_vectors():
    with open(os.path.join(HERE, "golden", "philox4x64_10_kat.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            v = [int(t, 16) for t in line.split()]
            assert O.philox4x64_10(v[:4], v[4:6]) == v[6:10]


@pytest.mark.parametrize("ctr,key", [([1, 0, 0, 0], [0, 0]), ([5, 7, 0, 0], [123, 456]),
                                     ([2 ** 64 - 1, 3, 9, 0], [2 ** 63, 1])])
def test_philox_matches_numpy(ctr, key):
    # numpy's Philox advances its counter by one before producing a block
    prev = list(ctr)
    for i in range(4):
        if prev[i] > 0:
            prev[i] -= 1
            break
        prev[i] = 2 ** 64 - 1
    raw = np.random.Philox(counter=np.array(prev, np.uint64),
                          key=np.array(key, np.uint64)).random_raw(4)
    assert O.philox4x64_10(ctr, key) == [int(x) for x in raw]


def test_uniform24_is_uniform_and_keyed():
    us = np.array([O.uniform24(7, rid, st) for rid in range(40) for st in range(100)])
    assert us.min() >= 0 and us.max() < 1
    assert np.all(us * 2 ** 24 == np.floor(us * 2 ** 24))   # 24-bit grid
    hist, _ = np.histogram(us, bins=20, range=(0, 1))
    exp = len(us) / 20
    chi2 = ((hist - exp) ** 2 / exp).sum()
    assert chi2 < 60                                          # 19 dof
    assert O.uniform24(7, 1, 2) != O.uniform24(8, 1, 2)
    assert O.uniform24(7, 1, 2) != O.uniform24(7, 2, 1)


def test_synth_is_device_independent_and_sliceable():
    a = synth.normal_tensor(3, "w", (64, 33), 0.02)
    idx = torch.arange(64 * 33, dtype=torch.int64)[100:200]
    b = synth.normal_like(synth.tag_key(3, "w"), idx, 0.02)
    assert torch.equal(a.view(-1)[100:200], b)
    assert abs(float(a.float().std()) - 0.02) < 0.003

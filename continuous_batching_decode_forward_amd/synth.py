"""Seeded synthetic inputs for the tests, the smoke check and the benchmark.

This module holds none of the method's arithmetic. It only produces numbers:
weights, cached K/V contents, token ids, context lengths and block
permutations, from a seed. Both the GPU path and the CPU oracle receive what
it makes; neither side computes inputs for the other.

Values are a pure function of (seed, tag, element index): a 32-bit integer
hash (the "lowbias32" finaliser from C. Wellons' hash-prospector: xor-shift
16, multiply 0x7feb352d, xor-shift 15, multiply 0x846ca68b, xor-shift 16)
evaluated with int64 tensor ops, so the same bytes come out on the CPU and on
the GPU, and any slice can be regenerated on its own. A normal-looking value
is the Irwin-Hall sum of the hash's four bytes, centred and scaled to the
requested standard deviation (variance of the sum: 4 * (256^2 - 1) / 12),
then rounded to bf16 by torch (round to nearest even on both devices).
"""
from __future__ import annotations

import math
import zlib

import numpy as np
import torch

M32 = 0xFFFFFFFF
_IH4_STD = math.sqrt(4.0 * (256.0 ** 2 - 1.0) / 12.0)


def _hash32(x: torch.Tensor) -> torch.Tensor:
    """lowbias32 on uint32 values held in an int64 tensor (no overflow:
    every product is below 2^63)."""
    x = x & M32
    x = x ^ (x >> 16)
    x = (x * 0x7FEB352D) & M32
    x = x ^ (x >> 15)
    x = (x * 0x846CA68B) & M32
    x = x ^ (x >> 16)
    return x


def _hash32_int(v: int) -> int:
    v &= M32
    v ^= v >> 16
    v = (v * 0x7FEB352D) & M32
    v ^= v >> 15
    v = (v * 0x846CA68B) & M32
    v ^= v >> 16
    return v


def tag_key(seed: int, tag: str) -> int:
    """Stream key of a named tensor under a seed."""
    return _hash32_int(_hash32_int(seed & M32) ^ zlib.crc32(tag.encode()) ^ ((seed >> 32) & M32))


def hash_stream(key: int, idx: torch.Tensor) -> torch.Tensor:
    """uint32 hash of element indices (int64, up to 2^62) under a stream key."""
    lo = idx & M32
    hi = idx >> 32
    return _hash32(lo ^ _hash32(hi ^ key))


def normal_like(key: int, idx: torch.Tensor, std: float) -> torch.Tensor:
    """Approximately N(0, std^2) bf16 values (Irwin-Hall of 4 bytes)."""
    h = hash_stream(key, idx)
    s = (h & 255) + ((h >> 8) & 255) + ((h >> 16) & 255) + ((h >> 24) & 255) - 510
    scale = torch.tensor(np.float32(std / _IH4_STD), dtype=torch.float32, device=idx.device)
    return (s.to(torch.float32) * scale).to(torch.bfloat16)


def normal_tensor(seed: int, tag: str, shape, std: float, device="cpu",
                  chunk: int = 1 << 26) -> torch.Tensor:
    """A bf16 tensor of the given shape; element i (row-major) depends only on
    (seed, tag, i). Generated in chunks to bound temporaries."""
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=torch.bfloat16, device=device)
    key = tag_key(seed, tag)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        idx = torch.arange(s, e, dtype=torch.int64, device=device)
        out[s:e] = normal_like(key, idx, std)
    return out.view(*shape)


def uniform_ints(seed: int, tag: str, n: int, lo: int, hi: int) -> np.ndarray:
    """n integers uniform on [lo, hi] (inclusive), int32, CPU."""
    key = tag_key(seed, tag)
    h = hash_stream(key, torch.arange(n, dtype=torch.int64))
    return (lo + (h % (hi - lo + 1))).to(torch.int32).numpy()


def permutation(seed: int, tag: str, n: int) -> np.ndarray:
    """A seeded permutation of 0..n-1 (int32)."""
    rng = np.random.Generator(np.random.PCG64(tag_key(seed, tag)))
    return rng.permutation(n).astype(np.int32)


# ---------------------------------------------------------------- weights

def weight_shapes(cfg) -> dict:
    d, hq, hkv, hd, f, v = (cfg.d_model, cfg.n_heads, cfg.n_kv_heads,
                            cfg.head_dim, cfg.ffn_dim, cfg.vocab)
    return {
        "embed": (v, d),
        "final_norm": (d,),
        "lm_head": (v, d),
        "attn_norm": (d,),
        "w_qkv": ((hq + 2 * hkv) * hd, d),
        "w_o": (d, hq * hd),
        "ffn_norm": (d,),
        "w_gate": (f, d),
        "w_up": (f, d),
        "w_down": (d, f),
    }


PER_LAYER = ("attn_norm", "w_qkv", "w_o", "ffn_norm", "w_gate", "w_up", "w_down")


def make_weights(cfg, seed: int, device="cpu", std: float = 0.02) -> dict:
    """bf16 weights ~N(0, std^2) with RMSNorm gains 1.0. Per-layer entries are
    lists indexed by layer."""
    shapes = weight_shapes(cfg)
    w = {}
    for name in ("embed", "lm_head"):
        w[name] = normal_tensor(seed, name, shapes[name], std, device)
    w["final_norm"] = torch.ones(shapes["final_norm"], dtype=torch.bfloat16, device=device)
    for name in PER_LAYER:
        w[name] = []
        for layer in range(cfg.n_layers):
            if name.endswith("norm"):
                w[name].append(torch.ones(shapes[name], dtype=torch.bfloat16, device=device))
            else:
                w[name].append(normal_tensor(seed, f"{name}.{layer}", shapes[name], std, device))
    return w


def int8_codes(seed: int, tag: str, shape, device="cpu", chunk: int = 1 << 26) -> torch.Tensor:
    """int8 weight codes of the given shape, element i (row-major) depending
    only on (seed, tag, i): the Irwin-Hall sum of 4 hash bytes scaled to a
    standard deviation of about 40 in integer arithmetic, clamped to
    [-127, 127]."""
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=torch.int8, device=device)
    key = tag_key(seed, tag)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        h = hash_stream(key, torch.arange(s, e, dtype=torch.int64, device=device))
        t = (h & 255) + ((h >> 8) & 255) + ((h >> 16) & 255) + ((h >> 24) & 255) - 510
        out[s:e] = torch.clamp(torch.div(t * 35 + 64, 128, rounding_mode="floor"), -127, 127).to(torch.int8)
    return out.view(*shape)


def row_scales(seed: int, tag: str, n: int, std: float, device="cpu") -> torch.Tensor:
    """float32 per-row scales std / 40 * (0.75 + 0.5 u), u uniform on [0, 1)
    from the hash, so that codes of standard deviation 40 dequantise to
    about `std`, with rows of different scales."""
    h = hash_stream(tag_key(seed, tag), torch.arange(n, dtype=torch.int64, device=device))
    u = (h & 0xFFFF).to(torch.float32) / 65536.0
    return (np.float32(std / 40.0) * (0.75 + 0.5 * u)).to(torch.float32)


def make_weights_int8(cfg, seed: int, device="cpu", std: float = 0.02) -> dict:
    """Weight-only int8: every projection (QKV, O, gate, up, down per layer,
    and the LM head) as int8 codes [rows][cols] with one float32 scale per
    row (s_qkv ... s_down, lm_head_scale); the embedding (bf16 ~N(0, std^2))
    and the RMSNorm gains (1.0) as make_weights makes them."""
    shapes = weight_shapes(cfg)
    w = {"embed": normal_tensor(seed, "embed", shapes["embed"], std, device),
         "final_norm": torch.ones(shapes["final_norm"], dtype=torch.bfloat16, device=device),
         "lm_head": int8_codes(seed, "q.lm_head", shapes["lm_head"], device),
         "lm_head_scale": row_scales(seed, "s.lm_head", shapes["lm_head"][0], std, device)}
    for name in PER_LAYER:
        w[name] = []
        if not name.endswith("norm"):
            w["s" + name[1:]] = []
        for layer in range(cfg.n_layers):
            if name.endswith("norm"):
                w[name].append(torch.ones(shapes[name], dtype=torch.bfloat16, device=device))
            else:
                w[name].append(int8_codes(seed, f"q.{name}.{layer}", shapes[name], device))
                w["s" + name[1:]].append(row_scales(seed, f"s.{name}.{layer}", shapes[name][0],
                                                    std, device))
    return w


def weight_bytes(cfg, int8: bool = False) -> int:
    """Bytes of every weight read by one step (embedding rows excluded):
    bf16 throughout, or int8 projections with a float32 scale per row (the
    norm gains stay bf16)."""
    s = weight_shapes(cfg)
    if not int8:
        per_layer = sum(int(np.prod(s[k])) for k in PER_LAYER)
        return 2 * (cfg.n_layers * per_layer + int(np.prod(s["lm_head"])) + cfg.d_model)
    proj = [k for k in PER_LAYER if not k.endswith("norm")]
    per_layer = sum(int(np.prod(s[k])) + 4 * s[k][0] for k in proj) + 2 * 2 * cfg.d_model
    return cfg.n_layers * per_layer + int(np.prod(s["lm_head"])) + 4 * cfg.vocab + 2 * cfg.d_model


# ------------------------------------------------------ cached K/V contents

def kv_values(seed: int, layer: int, kind: int, block: torch.Tensor, kvh: torch.Tensor,
              off: torch.Tensor, dim: torch.Tensor, n_kv_heads: int, block_size: int,
              head_dim: int, std: float = 1.0) -> torch.Tensor:
    """Cached K (kind 0) or V (kind 1) values ~N(0, std^2), keyed by the
    physical location (layer, kind, block, kv head, offset in block, dim).
    Index tensors broadcast; the result takes their broadcast shape."""
    key = tag_key(seed, f"kv.{layer}.{kind}")
    idx = ((block.to(torch.int64) * n_kv_heads + kvh) * block_size + off) * head_dim + dim
    return normal_like(key, idx, std)


def kv_codes_fp8(seed: int, layer: int, kind: int, block: torch.Tensor, kvh: torch.Tensor,
                 off: torch.Tensor, dim: torch.Tensor, n_kv_heads: int, block_size: int,
                 head_dim: int) -> torch.Tensor:
    """Cached K or V of an 8-bit (E4M3) cache as raw codes (uint8), keyed by
    the physical location like kv_values: a random sign, an exponent field
    uniform on 0..9 (field 0: the subnormal codes, zero among them) and a
    random 3-bit mantissa -- magnitudes from 0 to 7.5, never the NaN codes.
    Each side decodes the codes by its own rules."""
    key = tag_key(seed, f"kv8.{layer}.{kind}")
    idx = ((block.to(torch.int64) * n_kv_heads + kvh) * block_size + off) * head_dim + dim
    h = hash_stream(key, idx)
    sign = (h >> 31) & 1
    expo = (h >> 8) % 10
    mant = h & 7
    return ((sign << 7) | (expo << 3) | mant).to(torch.uint8)


def logical_kv(seed: int, layer: int, kind: int, table: np.ndarray, n_pos: int,
               n_kv_heads: int, block_size: int, head_dim: int) -> torch.Tensor:
    """The cached K or V of one sequence as [n_pos][Hkv][hd] bf16 (CPU), for
    positions 0..n_pos-1 reached through its block table."""
    pos = torch.arange(n_pos, dtype=torch.int64)
    blk = torch.from_numpy(np.asarray(table, dtype=np.int64))[pos // block_size]
    return kv_values(seed, layer, kind, blk.view(-1, 1, 1),
                     torch.arange(n_kv_heads).view(1, -1, 1),
                     (pos % block_size).view(-1, 1, 1),
                     torch.arange(head_dim).view(1, 1, -1),
                     n_kv_heads, block_size, head_dim)

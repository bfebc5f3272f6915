"""Helpers shared by the GPU parity tests: engines over seeded weights,
synthetic KV pools laid out on both sides, and the logit comparison."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
from continuous_batching_decode_forward_amd import synth
from continuous_batching_decode_forward_amd.engine import Engine

# Logit tolerance (elementwise allclose form): |gpu - oracle| <= ATOL + RTOL*|oracle|.
ATOL, RTOL = 2e-2, 1e-2


def weights_to(weights: dict, device) -> dict:
    out = {}
    for k, v in weights.items():
        out[k] = [t.to(device) for t in v] if isinstance(v, list) else v.to(device)
    return out


def make_engine(shape, weights_gpu, *, block_size, num_blocks, max_blocks_per_seq, max_rows,
                max_seqs, max_position, max_slots=None, block_order=None):
    return Engine(shape, weights_gpu, block_size=block_size, num_blocks=num_blocks,
                  max_blocks_per_seq=max_blocks_per_seq, max_slots=max_slots or max_seqs,
                  max_rows=max_rows, max_seqs=max_seqs, max_position=max_position,
                  block_order=block_order)


def fill_pool(eng: Engine, seed: int, blocks: np.ndarray) -> None:
    """Write synthetic cached K/V (keyed by physical location) into the given
    blocks of every layer of the engine's pool, in the pool's layout."""
    s = eng.shape
    bs, hkv, hd = eng.block_size, s.n_kv_heads, s.head_dim
    dev = eng.kv_pool.device
    blocks = torch.as_tensor(np.asarray(blocks, np.int64), device=dev)
    for layer in range(s.n_layers):
        k, v = eng.kv_views(layer)
        for c0 in range(0, len(blocks), 4096):
            b = blocks[c0:c0 + 4096]
            kh = torch.arange(hkv, device=dev)
            off = torch.arange(bs, device=dev)
            dim = torch.arange(hd, device=dev)
            kv_k = synth.kv_values(seed, layer, 0, b.view(-1, 1, 1, 1), kh.view(1, -1, 1, 1),
                                   off.view(1, 1, -1, 1), dim.view(1, 1, 1, -1), hkv, bs, hd)
            k[b] = kv_k
            kv_v = synth.kv_values(seed, layer, 1, b.view(-1, 1, 1, 1), kh.view(1, -1, 1, 1),
                                   off.view(1, 1, 1, -1), dim.view(1, 1, -1, 1), hkv, bs, hd)
            v[b] = kv_v


def oracle_pool(shape, seed: int, tables: list, n_cached: list, block_size: int,
                n_new: list):
    """An oracle-layout pool holding the cached positions of the given
    sequences. Block ids are renumbered 0.. in table order (paging is pure
    addressing); returns (pool, compact tables)."""
    hkv, hd = shape.n_kv_heads, shape.head_dim
    need = [-(-(c + n) // block_size) for c, n in zip(n_cached, n_new)]
    total = sum(need)
    pool = np.zeros((shape.n_layers, 2, max(total, 1), block_size, hkv, hd), np.uint16)
    width = max(need)
    compact = np.full((len(tables), width), -1, np.int32)
    nxt = 0
    for i, (tab, c) in enumerate(zip(tables, n_cached)):
        ids = np.arange(nxt, nxt + need[i], dtype=np.int32)
        compact[i, :need[i]] = ids
        nxt += need[i]
        nb_cached = -(-c // block_size)
        if nb_cached == 0:
            continue
        phys = torch.as_tensor(np.asarray(tab[:nb_cached], np.int64))
        kh = torch.arange(hkv)
        off = torch.arange(block_size)
        dim = torch.arange(hd)
        for layer in range(shape.n_layers):
            for kind in (0, 1):
                vals = synth.kv_values(seed, layer, kind, phys.view(-1, 1, 1, 1),
                                       kh.view(1, 1, -1, 1), off.view(1, -1, 1, 1),
                                       dim.view(1, 1, 1, -1), hkv, block_size, hd)
                pool[layer, kind, ids[:nb_cached]] = O.as_u16(vals).reshape(
                    nb_cached, block_size, hkv, hd)
    return pool, compact


def compare_logits(gpu: np.ndarray, ref: np.ndarray):
    """Returns (ok, max_abs_err, per-row max abs err)."""
    err = np.abs(gpu.astype(np.float64) - ref)
    ok = np.all(err <= ATOL + RTOL * np.abs(ref))
    return bool(ok), float(err.max()), err.max(axis=-1)


def resolvable_rows(ref: np.ndarray, row_err: np.ndarray):
    """Rows whose oracle top-2 gap exceeds twice the observed error: there
    the greedy id is decided, elsewhere it is a near tie."""
    top2 = np.sort(ref, axis=-1)[:, -2:]
    gap = top2[:, 1] - top2[:, 0]
    return gap > 2.0 * np.maximum(row_err, 1e-6)

"""Helpers shared by the GPU parity tests: engines over seeded weights,
synthetic KV pools laid out on both sides, and the logit comparison."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
from continuous_batching_decode_forward_amd import synth
from continuous_batching_decode_forward_amd.binding import CBD_BUF_ATTN as B_CBD_BUF_ATTN
from continuous_batching_decode_forward_amd.binding import CBD_BUF_Q as B_CBD_BUF_Q
from continuous_batching_decode_forward_amd.engine import Engine

# Logit tolerance (elementwise allclose form): |gpu - oracle| <= ATOL + RTOL*|oracle|.
ATOL, RTOL = 2e-2, 1e-2


def weights_to(weights: dict, device) -> dict:
    out = {}
    for k, v in weights.items():
        out[k] = [t.to(device) for t in v] if isinstance(v, list) else v.to(device)
    return out


def make_engine(shape, weights_gpu, *, block_size, num_blocks, max_blocks_per_seq, max_rows,
                max_seqs, max_position, max_slots=None, block_order=None, **kv):
    """kv: the cache format (kv_dtype, k_scale, v_scale), bf16 by default."""
    return Engine(shape, weights_gpu, block_size=block_size, num_blocks=num_blocks,
                  max_blocks_per_seq=max_blocks_per_seq, max_slots=max_slots or max_seqs,
                  max_rows=max_rows, max_seqs=max_seqs, max_position=max_position,
                  block_order=block_order, **kv)


def _kv(seed, layer, kind, b, kh, off, dim, hkv, bs, hd, fp8):
    gen = synth.kv_codes_fp8 if fp8 else synth.kv_values
    return gen(seed, layer, kind, b, kh, off, dim, hkv, bs, hd)


def fill_pool(eng: Engine, seed: int, blocks: np.ndarray) -> None:
    """Write synthetic cached K/V (keyed by physical location) into the given
    blocks of every layer of the engine's pool, in the pool's layout: bf16
    values, or E4M3 codes for an 8-bit cache."""
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
            k[b] = _kv(seed, layer, 0, b.view(-1, 1, 1, 1), kh.view(1, -1, 1, 1),
                       off.view(1, 1, -1, 1), dim.view(1, 1, 1, -1), hkv, bs, hd, eng.kv_fp8)
            v[b] = _kv(seed, layer, 1, b.view(-1, 1, 1, 1), kh.view(1, -1, 1, 1),
                       off.view(1, 1, 1, -1), dim.view(1, 1, -1, 1), hkv, bs, hd, eng.kv_fp8)


def oracle_pool(shape, seed: int, tables: list, n_cached: list, block_size: int,
                n_new: list, kv_fp8: bool = False):
    """An oracle-layout pool holding the cached positions of the given
    sequences (bf16 bits, or E4M3 codes when kv_fp8). Block ids are
    renumbered 0.. in table order (paging is pure addressing); returns
    (pool, compact tables)."""
    hkv, hd = shape.n_kv_heads, shape.head_dim
    need = [-(-(c + n) // block_size) for c, n in zip(n_cached, n_new)]
    total = sum(need)
    pool = np.zeros((shape.n_layers, 2, max(total, 1), block_size, hkv, hd),
                    np.uint8 if kv_fp8 else np.uint16)
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
                vals = _kv(seed, layer, kind, phys.view(-1, 1, 1, 1), kh.view(1, 1, -1, 1),
                           off.view(1, -1, 1, 1), dim.view(1, 1, 1, -1), hkv, block_size, hd,
                           kv_fp8)
                vals = vals.numpy() if kv_fp8 else O.as_u16(vals)
                pool[layer, kind, ids[:nb_cached]] = vals.reshape(nb_cached, block_size, hkv, hd)
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


def stage_error(gpu: np.ndarray, ref: np.ndarray, slack=None) -> float:
    """max_i (|gpu_i - ref_i| - slack_i) / (|ref_i| + rms(ref)): relative for
    large elements, relative to the vector's scale for small ones."""
    g = np.asarray(gpu, np.float64).reshape(-1)
    o = np.asarray(ref, np.float64).reshape(-1)
    rms = float(np.sqrt(np.mean(o * o))) or 1.0
    d = np.abs(g - o)
    if slack is not None:
        d = np.maximum(d - slack.reshape(-1), 0.0)
    return float((d / (np.abs(o) + rms)).max())


def gather_kv(eng: Engine, layer: int, table, n_pos: int):
    """One sequence's first n_pos cached K and V positions of a layer, read
    from the engine's pool through its block table: two arrays
    [n_pos][Hkv][hd], uint16 bf16 bits (uint8 E4M3 codes for an 8-bit
    cache)."""
    s = eng.shape
    bs = eng.block_size
    nb = -(-n_pos // bs)
    k, v = eng.kv_views(layer)
    blocks = torch.as_tensor(np.asarray(table[:nb], np.int64), device=k.device)
    # K [blocks][Hkv][bs][hd] and V [blocks][Hkv][hd][bs] -> [positions][Hkv][hd]
    kk = k[blocks].permute(0, 2, 1, 3).reshape(nb * bs, s.n_kv_heads, s.head_dim)[:n_pos]
    vv = v[blocks].permute(0, 3, 1, 2).reshape(nb * bs, s.n_kv_heads, s.head_dim)[:n_pos]
    if eng.kv_fp8:
        return kk.contiguous().cpu().numpy(), vv.contiguous().cpu().numpy()
    return O.as_u16(kk.contiguous().cpu()), O.as_u16(vv.contiguous().cpu())


def attention_rows_vs_oracle(eng: Engine, tables, ctx, n_new, threads: int = 16):
    """Every row's attention output after a step (the last layer's, as the
    engine keeps it) against the oracle's dense attention over the same
    inputs: the row's rotated query as the device computed it and the K/V
    the device's pool holds for positions 0..pos (the cached prefix plus
    what the step appended), so the comparison isolates the attention
    kernels, the key schedule and the combine. Returns the per-row error
    measure (stage_error) as an array in row order."""
    from concurrent.futures import ThreadPoolExecutor
    s = eng.shape
    hq, hkv, hd = s.n_heads, s.n_kv_heads, s.head_dim
    R = int(sum(n_new))
    q = eng.debug_buffer(B_CBD_BUF_Q, R, hq * hd)
    att = eng.debug_buffer(B_CBD_BUF_ATTN, R, hq * hd)
    layer = s.n_layers - 1
    err = np.full(R, np.inf)

    def one(r, pos, K, V):
        if eng.kv_fp8:
            ref = O.attention_dense_fp8(q[r], K[:pos + 1], V[:pos + 1], hq, hkv, hd,
                                        eng.cfg.k_scale or 1.0, eng.cfg.v_scale or 1.0)
        else:
            ref = O.attention_dense(q[r], K[:pos + 1], V[:pos + 1], hq, hkv, hd)
        err[r] = stage_error(att[r], ref)

    pending = []
    r0 = 0
    with ThreadPoolExecutor(max_workers=threads) as ex:
        for i, (c, n) in enumerate(zip(ctx, n_new)):
            c, n = int(c), int(n)
            K, V = gather_kv(eng, layer, tables[i], c + n)
            for j in range(n):
                pending.append(ex.submit(one, r0 + j, c + j, K, V))
            r0 += n
            while len(pending) > 2 * threads:  # bound the K/V copies held on the host
                pending.pop(0).result()
        for f in pending:
            f.result()
    return err

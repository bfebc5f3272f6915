"""Host replay of the attention work schedule (no GPU).

The per-tile and block attention kernels, the prep kernel and the combine
decode their work with the integer arithmetic of csrc/attn_sched.h; the
checker library (csrc/check/attn_sched_check.cpp) runs that same code on the
host for a step's metadata and checks every bound the kernels rely on:
segments and items that load K/V have keys, block-table slices fit the LDS
table and the sequence's table row, partial slots stay below max_splits and
are written once, every key step is covered once, and the combine reads
exactly the slots that were written (selective batching over paged K/V, Go
under the hood 20.3.2).

The plans come from the reference composer on the same request streams the
GPU loop tests and the benchmark drive, so they are the plans those runs
execute (the composer's plans do not depend on token values unless a token
is the EOS id; the replay commits non-EOS tokens).
"""
import ctypes as C
import os
import random

import numpy as np
import pytest

from continuous_batching_decode_forward_amd import build as native_build
from continuous_batching_decode_forward_amd import configs, synth
from oracle.composer_ref import RESERVE, ComposerRef

from cb_streams import (Q_BS, Q_CHUNK, Q_MBPS, Q_POOL, Q_ROWS, Q_SEED, Q_SLOTS, Q_STEPS, QWEN,
                        qwen_loop_stream, request_stream)

WAVES_MI355X = 256 * 4 * 2  # resident per-tile attention waves: 256 CUs, 2 per SIMD

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(native_build.CHECK_LIB):
            native_build.build()
        _lib = C.CDLL(native_build.CHECK_LIB)
        I32P = C.POINTER(C.c_int32)
        _lib.cbd_check_attention_schedule.argtypes = [
            I32P, C.c_int32, C.c_int32, C.c_int32, C.c_int32, I32P, I32P, I32P, I32P,
            C.POINTER(C.c_int64), C.c_char_p, C.c_int32]
        _lib.cbd_check_attention_schedule.restype = C.c_int32
    return _lib


def check_step(shape, *, block_size, num_blocks, max_position, max_rows, max_slots, slots,
               tables, ctx, n_new, mbps, waves=WAVES_MI355X, kv_fp8=0):
    """Run the replay; returns (violations, first message, stats dict)."""
    i32 = lambda a: np.ascontiguousarray(np.asarray(a, np.int64).astype(np.int32))
    cfg = i32([shape.n_heads, shape.n_kv_heads, shape.head_dim, block_size, num_blocks,
               max_position, max_rows, max_slots, waves, kv_fp8])
    slots, ctx, n_new = i32(slots), i32(ctx), i32(n_new)
    tab = np.full((len(ctx), mbps), -1, np.int32)
    for i, t in enumerate(tables):
        t = list(t)[:mbps]
        tab[i, :len(t)] = t
    n_rows = int(n_new.sum())
    max_ctx = int((ctx + n_new).max())
    st = (C.c_int64 * 8)()
    msg = C.create_string_buffer(256)
    P = lambda a: a.ctypes.data_as(C.POINTER(C.c_int32))
    v = lib().cbd_check_attention_schedule(P(cfg), len(ctx), n_rows, max_ctx, mbps, P(slots),
                                           P(tab), P(ctx), P(n_new), st, msg, 256)
    names = ("segments", "pieces", "block_items", "waves", "block_grid", "max_table",
             "max_slot", "served")
    return v, msg.value.decode(), dict(zip(names, list(st)))


def composer_plans(slots, bs, pool, mbps, rows, chunk, reqs, n_steps, order, seed):
    """The reference composer's first n_steps plans on the request stream,
    committing seeded non-EOS tokens (EOS = 0)."""
    ref = ComposerRef(slots, bs, pool, rows, chunk, 0, RESERVE, block_order=list(order),
                      max_blocks_per_seq=mbps)
    for rid, prompt, mx in reqs:
        ref.submit(rid, prompt, mx)
    rng = np.random.default_rng(seed)
    plans = []
    for _ in range(n_steps):
        p = ref.plan()
        if p.n_rows == 0:
            break
        plans.append(p)
        n_out = sum(p.want_token)
        ref.commit([int(t) for t in rng.integers(1, 1000, n_out)])
    return plans


def check_plans(shape, plans, *, bs, pool, max_position, rows, slots, mbps, waves=WAVES_MI355X):
    seen = {"segments": 0, "block_items": 0, "max_table": 0, "max_slot": 0, "chunked": 0}
    for j, p in enumerate(plans):
        v, msg, st = check_step(shape, block_size=bs, num_blocks=pool, max_position=max_position,
                                max_rows=rows, max_slots=slots, slots=p.slots,
                                tables=p.block_tables, ctx=p.ctx_lens, n_new=p.n_new, mbps=mbps,
                                waves=waves)
        assert v == 0, f"plan {j}: {v} violations, first: {msg}"
        assert st["served"] == len(p.n_new), f"plan {j}: a sequence was refused"
        for k in ("segments", "block_items"):
            seen[k] += st[k]
        seen["max_table"] = max(seen["max_table"], st["max_table"])
        seen["max_slot"] = max(seen["max_slot"], st["max_slot"])
        seen["chunked"] += int(max(p.n_new) > 1)
    return seen


def test_the_2b_loop_plans_replay_cleanly():
    # The plans of the full-size 2B 28-layer loop test (and well past its
    # 48 steps): 512-token chunks on the block kernel next to short chunk
    # remainders and decode rows on the per-tile kernel.
    order = synth.permutation(Q_SEED, "blocks", Q_POOL).astype(np.int32)
    plans = composer_plans(Q_SLOTS, Q_BS, Q_POOL, Q_MBPS, Q_ROWS, Q_CHUNK, qwen_loop_stream(),
                           400, order, seed=1)
    assert len(plans) >= Q_STEPS
    for waves in (WAVES_MI355X, 512, 64):
        seen = check_plans(QWEN, plans, bs=Q_BS, pool=Q_POOL, max_position=Q_MBPS * Q_BS,
                           rows=Q_ROWS, slots=Q_SLOTS, mbps=Q_MBPS, waves=waves)
        assert seen["chunked"] > 10 and seen["block_items"] > 0 and seen["segments"] > 0
    print(f"2b loop: {len(plans)} plans replayed, {seen}")


@pytest.mark.parametrize("n_slots", [8, 32])
def test_the_2b_benchmark_loop_plans_replay_cleanly(n_slots):
    # bench.py's 2B continuous-batching workload: closed loop, 256 steps.
    pool, rows, bs = 16 * n_slots, 512 + n_slots, 32
    mbps = -(-(512 + 300) // bs)
    order = synth.permutation(0, "blocks", pool).astype(np.int32)
    reqs = request_stream(n_slots, 600, (16, 512), (2, 300), QWEN.vocab)
    plans = composer_plans(n_slots, bs, pool, mbps, rows, 512, reqs, 256, order, seed=2)
    assert len(plans) == 256
    check_plans(QWEN, plans, bs=bs, pool=pool, max_position=mbps * bs, rows=rows,
                slots=n_slots, mbps=mbps)


def test_the_tiny_figure_loop_plans_replay_cleanly():
    # The figure constants: 4 slots, 4-position blocks, 8-token chunks, 12 rows.
    order = synth.permutation(7, "blocks", 40).astype(np.int32)
    reqs = request_stream(7, 10, (5, 40), (2, 16), configs.TINY.vocab)
    plans = composer_plans(4, 4, 40, 16, 12, 8, reqs, 400, order, seed=3)
    check_plans(configs.TINY, plans, bs=4, pool=40, max_position=64, rows=12, slots=4, mbps=16)


def _decode_step(shape, ctx, bs, max_position, waves=WAVES_MI355X, chunk=None):
    n = len(ctx)
    need = [-(-(int(c) + 1) // bs) for c in ctx]
    nn = [1] * n
    ctx = [int(c) for c in ctx]
    if chunk is not None:  # (offset, rows) prefill chunk first
        o, r = chunk
        ctx = [o] + ctx
        nn = [r] + nn
        need = [-(-(o + r) // bs)] + need
    perm = synth.permutation(5, "blocks", int(sum(need)))
    tables, at = [], 0
    for k in need:
        tables.append(perm[at:at + k])
        at += k
    mbps = max(need)
    return check_step(shape, block_size=bs, num_blocks=int(sum(need)), max_position=max_position,
                      max_rows=sum(nn), max_slots=len(nn), slots=list(range(len(nn))),
                      tables=tables, ctx=ctx, n_new=nn, mbps=mbps, waves=waves)


@pytest.mark.parametrize("B", [1, 8, 32, 64, 400])
def test_the_8b_layer_decode_steps_replay_cleanly(B):
    ctx = synth.uniform_ints(0, "ctx", B, 512, 4096)
    v, msg, st = _decode_step(configs.LLAMA8B_1L, ctx, 32, 4097)
    assert v == 0, msg


def test_the_long_context_b256_step_replays_cleanly():
    ctx = synth.uniform_ints(0, "ctx", 256, 8192, 32768)
    v, msg, st = _decode_step(configs.LLAMA8B_1L_V64K, ctx, 32, 32769)
    assert v == 0, msg
    assert st["max_table"] <= 512


@pytest.mark.parametrize("offset", [0, 1536, 3584])
def test_the_8b_mixed_steps_replay_cleanly(offset):
    ctx = synth.uniform_ints(0, "ctx", 48, 1024, 8192)
    v, msg, st = _decode_step(configs.LLAMA8B, ctx, 32, 8200, chunk=(offset, 512))
    assert v == 0, msg
    assert st["block_items"] > 0


def test_random_step_mixes_replay_cleanly():
    # Every head grouping, block size and a spread of context lengths, chunk
    # lengths (on both kernels) and launch sizes.
    rnd = random.Random(11)
    for trial in range(250):
        G = rnd.choice([1, 2, 4, 8, 16])
        kvh = rnd.choice([1, 2, 8])
        hd = rnd.choice([64, 128])
        shape = configs.ModelShape("rand", 1, 256, G * kvh, kvh, hd, 256, 1024)
        bs = rnd.choice([4, 8, 16, 32, 64])
        max_position = rnd.choice([64, 100, 512, 4097, 9000, 33000])
        waves = rnd.choice([64, 256, WAVES_MI355X])
        n = rnd.randint(1, 40)
        ctx, nn = [], []
        for _ in range(n):
            k = min(rnd.choice([1, 1, 1, 2, 5, 17, 31, 32, 40, 200, 512]), max_position)
            ctx.append(rnd.randint(0, max_position - k))
            nn.append(k)
        need = [-(-(c + k) // bs) for c, k in zip(ctx, nn)]
        perm = list(range(sum(need)))
        rnd.shuffle(perm)
        tables, at = [], 0
        for k in need:
            tables.append(perm[at:at + k])
            at += k
        v, msg, st = check_step(shape, block_size=bs, num_blocks=sum(need),
                                max_position=max_position, max_rows=sum(nn), max_slots=n,
                                slots=list(range(n)), tables=tables, ctx=ctx, n_new=nn,
                                mbps=max(need), waves=waves, kv_fp8=trial % 3 == 0)
        assert v == 0, f"trial {trial}: {msg}"
        assert st["served"] == n


def test_the_replay_reports_a_block_id_outside_the_pool():
    # The replay is live: a table entry past the pool is named (on the device
    # the kernels replace it by block 0 and raise CBD_STATUS_BAD_BLOCK).
    shape = configs.LLAMA8B_1L
    v, msg, _ = check_step(shape, block_size=32, num_blocks=8, max_position=512, max_rows=2,
                           max_slots=2, slots=[0, 1], tables=[[0, 1, 2], [3, 9]],
                           ctx=[70, 40], n_new=[1, 1], mbps=3)
    assert v > 0 and "block id 9" in msg

"""Continuous batching end to end: the host composer (cbd_sched_*) attached
to the engine, driving steps on the GPU.

  * tiny 2-layer decoder on the scaled-down figure constants of Go under the
    hood 20.3.2 (4 slots, 4-position blocks, 8-token chunks, 12 rows per
    step), a stream of requests with admission under reservation: every step
    the GPU's logits are compared with the oracle's paged-batched step on the
    same plan, and the composer is fed the oracle's tokens (teacher forcing);
  * the native loop call (cbd_sched_step) against the same loop written out
    with plan / step / commit: identical plans and tokens, bit for bit;
  * the full 28-layer 2B-shaped decoder at 8 slots with the workload's
    constants (32-position blocks, 512-token chunks, 16 blocks per slot,
    prompts 16..512, answers 2..300): every plan equals the reference
    composer's on the same tokens, the device status stays clear, and the
    first four emissions of the shortest-prompt request match the oracle's
    serial decode of that request alone."""
import numpy as np
import pytest
import torch

import oracle as O
from continuous_batching_decode_forward_amd import binding as B
from continuous_batching_decode_forward_amd import configs, synth
from continuous_batching_decode_forward_amd.engine import ComposerLoop, Engine
from oracle.composer_ref import ComposerRef

from cb_streams import (Q_BS, Q_CHUNK, Q_MBPS, Q_POOL, Q_ROWS, Q_SEED, Q_SLOTS, Q_STEPS, QWEN,
                        qwen_loop_stream, request_stream)
from gpu_util import compare_logits, resolvable_rows, weights_to

pytestmark = pytest.mark.gpu


def plan_arrays(p):
    n = p.n_seqs
    mb = p.max_blocks_per_seq
    tab = np.ctypeslib.as_array(p.block_tables, shape=(n * mb,)).reshape(n, mb).copy() \
        if n else np.zeros((0, mb), np.int32)
    return dict(slots=list(p.slots[:n]), tables=tab, ctx=list(p.ctx_lens[:n]),
                n_new=list(p.n_new[:n]), tokens=list(p.tokens[:p.n_rows]),
                want=list(p.want_token[:n]), step_ids=list(p.step_ids[:n]),
                rids=list(p.request_ids[:n]))


def sched_cfg(slots, bs, pool, mbps, rows, chunk, eos=0):
    c = B.cbd_sched_config()
    c.max_slots, c.block_size, c.num_blocks = slots, bs, pool
    c.max_blocks_per_seq, c.max_rows, c.chunk_size = mbps, rows, chunk
    c.eos_id, c.policy = eos, B.CBD_ADMIT_RESERVE
    return c


TINY = configs.TINY
T_SLOTS, T_BS, T_POOL, T_MBPS, T_ROWS, T_CHUNK = 4, 4, 40, 16, 12, 8


@pytest.fixture(scope="module")
def tiny():
    w = synth.make_weights(TINY, seed=1)
    return w, O.Model(TINY, w), weights_to(w, "cuda")


def tiny_engine(wg, order):
    return Engine(TINY, wg, block_size=T_BS, num_blocks=T_POOL, max_blocks_per_seq=T_MBPS,
                  max_slots=T_SLOTS, max_rows=T_ROWS, max_seqs=T_SLOTS,
                  max_position=T_MBPS * T_BS, block_order=order)


def test_tiny_loop_teacher_forced_against_the_oracle(tiny):
    torch.cuda.set_device(0)
    _, om, wg = tiny
    order = synth.permutation(7, "blocks", T_POOL).astype(np.int32)
    eng = tiny_engine(wg, order)
    s = B.cbd_sched_create(sched_cfg(T_SLOTS, T_BS, T_POOL, T_MBPS, T_ROWS, T_CHUNK), eng.handle)
    reqs = request_stream(7, 10, (5, 40), (2, 16), TINY.vocab)
    for rid, prompt, mx in reqs:
        B.cbd_sched_submit(s, prompt, mx, None, rid)
    pool = om.paged_pool(T_POOL, T_BS)
    worst, n_steps, n_cmp, n_res, finished = 0.0, 0, 0, 0, []
    try:
        for _ in range(400):
            p = B.cbd_sched_plan(s)
            if p.n_rows == 0:
                assert not p.stalled
                break
            a = plan_arrays(p)
            ref_lg, ref_tok = O.paged_step(om, pool, a["tables"], a["ctx"], a["n_new"],
                                           a["tokens"], a["want"])
            meta = eng.upload_step(slots=a["slots"], block_tables=a["tables"],
                                   ctx_lens=a["ctx"], n_new=a["n_new"], tokens=a["tokens"],
                                   want_token=a["want"], step_ids=a["step_ids"])
            n_out = meta.n_out
            lg = torch.empty((max(n_out, 1), TINY.vocab), dtype=torch.float32, device="cuda")
            tk = torch.full((max(n_out, 1),), -1, dtype=torch.int32, device="cuda")
            eng.step_forward(meta, lg, tk)
            torch.cuda.synchronize()
            assert eng.status() == 0
            if n_out:
                g_lg, g_tk = lg[:n_out].cpu().numpy(), tk[:n_out].cpu().numpy()
                ok, mx, row_err = compare_logits(g_lg, ref_lg)
                assert ok, f"step {n_steps}: max abs logit error {mx:.3g}"
                res = resolvable_rows(ref_lg, row_err)
                assert np.array_equal(g_tk[res], ref_tok[res])
                worst = max(worst, mx)
                n_cmp += n_out
                n_res += int(res.sum())
            B.cbd_sched_commit(s, [int(t) for t in ref_tok[:n_out]])
            while (f := B.cbd_sched_pop_finished(s)) is not None:
                finished.append(f)
            n_steps += 1
        st = B.cbd_sched_stats_get(s)
        assert st.active == 0 and st.queued == 0
        assert sorted(f[0] for f in finished) == list(range(len(reqs)))
        assert B.cbd_blocks_available(eng.handle) == T_POOL
    finally:
        B.cbd_sched_destroy(s)
        eng.close()
    print(f"tiny loop: {n_steps} steps, {n_cmp} emitted rows compared "
          f"({n_res} decidable), max abs logit error {worst:.2e}")


def test_native_loop_step_equals_the_written_out_loop(tiny):
    torch.cuda.set_device(0)
    _, _, wg = tiny
    order = synth.permutation(9, "blocks", T_POOL).astype(np.int32)
    reqs = request_stream(9, 10, (5, 40), (2, 16), TINY.vocab)
    cfg = sched_cfg(T_SLOTS, T_BS, T_POOL, T_MBPS, T_ROWS, T_CHUNK)

    def native():
        eng = tiny_engine(wg, order)
        loop = ComposerLoop(eng, max_rows=T_ROWS, chunk_size=T_CHUNK, eos_id=0)
        for rid, prompt, mx in reqs:
            loop.submit(prompt, mx, None, rid)
        trace = []
        try:
            for _ in range(400):
                p = loop.step()
                if p.n_rows == 0:
                    break
                a = plan_arrays(p)
                trace.append((a, list(loop.last_tokens(p.n_out))))
            fin = loop.pop_finished()
            assert eng.status() == 0
        finally:
            loop.close()
            eng.close()
        return trace, fin

    def written_out():
        eng = tiny_engine(wg, order)
        s = B.cbd_sched_create(cfg, eng.handle)
        for rid, prompt, mx in reqs:
            B.cbd_sched_submit(s, prompt, mx, None, rid)
        trace, fin = [], []
        try:
            for _ in range(400):
                p = B.cbd_sched_plan(s)
                if p.n_rows == 0:
                    break
                a = plan_arrays(p)
                meta = eng.upload_step(slots=a["slots"], block_tables=a["tables"],
                                       ctx_lens=a["ctx"], n_new=a["n_new"], tokens=a["tokens"],
                                       want_token=a["want"], step_ids=a["step_ids"])
                tk = torch.full((max(p.n_out, 1),), -1, dtype=torch.int32, device="cuda")
                eng.step_forward(meta, None, tk)
                toks = [int(t) for t in tk[:p.n_out].cpu().numpy()]
                trace.append((a, toks))
                B.cbd_sched_commit(s, toks)
            while (f := B.cbd_sched_pop_finished(s)) is not None:
                fin.append(f)
            assert eng.status() == 0
        finally:
            B.cbd_sched_destroy(s)
            eng.close()
        return trace, fin

    t1, f1 = native()
    t2, f2 = written_out()
    assert len(t1) == len(t2)
    for (a, x), (b, y) in zip(t1, t2):
        for k in ("slots", "ctx", "n_new", "tokens", "want", "step_ids", "rids"):
            assert a[k] == b[k], k
        assert np.array_equal(a["tables"], b["tables"])
        assert x == y
    assert f1 == f2 and len(f1) == len(reqs)
    print(f"native loop: {len(t1)} steps identical to the written-out loop")


def test_2b_28layer_loop_full_size():
    torch.cuda.set_device(0)
    seed, n_steps, n_check = Q_SEED, Q_STEPS, 4
    wg = synth.make_weights(QWEN, seed=seed, device="cuda")
    order = synth.permutation(seed, "blocks", Q_POOL).astype(np.int32)
    eng = Engine(QWEN, wg, block_size=Q_BS, num_blocks=Q_POOL, max_blocks_per_seq=Q_MBPS,
                 max_slots=Q_SLOTS, max_rows=Q_ROWS, max_seqs=Q_SLOTS,
                 max_position=Q_MBPS * Q_BS, block_order=order)
    loop = ComposerLoop(eng, max_rows=Q_ROWS, chunk_size=Q_CHUNK, eos_id=0)
    # the engine's block free list starts as `order`; the reference composer
    # keeps its own copy of the same FIFO
    ref = ComposerRef(Q_SLOTS, Q_BS, Q_POOL, Q_ROWS, Q_CHUNK, 0, B.CBD_ADMIT_RESERVE,
                      block_order=list(order), max_blocks_per_seq=Q_MBPS)
    reqs = qwen_loop_stream()
    for rid, prompt, mx in reqs:
        loop.submit(prompt, mx, None, rid)
        ref.submit(rid, prompt, mx)
    target = 0  # the 16-token request: the oracle decodes it alone below
    got, got_toks = [], []
    lg = torch.empty((Q_SLOTS, QWEN.vocab), dtype=torch.float32, device="cuda")
    try:
        for step in range(n_steps):
            p = loop.step(logits_out=lg)
            q = ref.plan()
            a = plan_arrays(p)
            assert a["slots"] == q.slots and a["ctx"] == q.ctx_lens and a["n_new"] == q.n_new
            assert a["tokens"] == q.tokens and a["want"] == q.want_token
            assert a["rids"] == q.request_ids and a["step_ids"] == q.step_ids
            for i in range(p.n_seqs):
                k = len(q.block_tables[i])
                assert list(a["tables"][i, :k]) == q.block_tables[i]
            toks = [int(t) for t in loop.last_tokens(p.n_out)]
            ref.commit(toks)
            o = 0
            for i in range(p.n_seqs):
                if a["want"][i]:
                    if a["rids"][i] == target and len(got) < n_check:
                        got.append(lg[o].cpu().numpy().copy())
                        got_toks.append(toks[o])
                    o += 1
        assert eng.status() == 0
        st = loop.stats()
        assert st.free_blocks == len(ref.free_blocks)
    finally:
        loop.close()
        eng.close()
    assert len(got) == n_check, "the 16-token request did not emit enough tokens"
    # the oracle decodes the same request alone, fed the GPU's tokens
    wc = {k: ([t.cpu() for t in v] if isinstance(v, list) else v.cpu()) for k, v in wg.items()}
    model = O.Model(QWEN, wc)
    kv = model.dense_kv(16 + n_check)
    prompt = reqs[target][1]
    ref_lg = [O.serial_forward(model, kv, prompt, 0)]
    for j in range(n_check - 1):
        ref_lg.append(O.serial_forward(model, kv, [got_toks[j]], 16 + j))
    ok, mx, row_err = compare_logits(np.stack(got), np.stack(ref_lg))
    res = resolvable_rows(np.stack(ref_lg), row_err)
    ids = np.array([O.argmax_f32(r) for r in np.stack(ref_lg)])
    print(f"2b 28-layer loop: {n_steps} steps; request 0 (16-token prompt) "
          f"max abs logit error {mx:.2e} over {n_check} emissions, "
          f"{int(res.sum())} decidable")
    assert ok, f"max abs logit error {mx:.3g}"
    assert np.array_equal(np.array(got_toks)[res], ids[res])

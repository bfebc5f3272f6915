"""The step under HIP graph capture and replay (the CUDAGraph decode path the
RWKV-Runner Albatross article lists as a follow-up).

  * cbd_step_forward enqueues only kernel launches on the caller's stream (no
    allocation, no memset, no host synchronisation), so a caller can capture
    one step and replay it: replays with the program's own eager work and
    synchronisations between them give the eager step's logits and tokens
    bit for bit (the step is idempotent: the same metadata appends the same
    K/V at the same positions);
  * cbd_step_forward_graph records one graph per step shape and replays it
    for later steps of that shape, which read their new metadata through the
    same device pointers: eight decode steps with advancing contexts equal
    the eager steps bit for bit (greedy on the 8B layer, sampled on the tiny
    decoder), a second shape records a second graph, the first replays again;
  * the native composer loop with graph replay of its decode-only steps
    commits the same tokens as the eager loop."""
import numpy as np
import pytest
import torch

import bench
from continuous_batching_decode_forward_amd import configs, synth
from continuous_batching_decode_forward_amd.engine import Engine

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape,B,ctx_range", [(configs.LLAMA8B_1L, 64, (512, 4096)),
                                               (configs.TINY, 6, (5, 300))],
                         ids=["8b-layer-b64", "tiny-b6"])
def test_captured_step_replays_equal_the_eager_step(shape, B, ctx_range):
    torch.cuda.set_device(0)
    wg = synth.make_weights(shape, seed=2, device="cuda")
    wl = bench.build_workload(shape, B, 2, ctx_range=ctx_range, bs=32)
    eng = Engine(shape, wg, block_size=32, num_blocks=wl["total"], max_blocks_per_seq=wl["mbps"],
                 max_slots=B, max_rows=B, max_seqs=B, max_position=wl["max_position"])
    try:
        bench.fill_pool(eng, 2, wl["perm"])
        meta = eng.upload_step(slots=list(range(B)), block_tables=wl["tables"], ctx_lens=wl["ctx"],
                               n_new=[1] * B, tokens=wl["tokens"], want_token=[1] * B)
        s = torch.cuda.Stream()
        lg = torch.empty((B, shape.vocab), dtype=torch.float32, device="cuda")
        tk = torch.empty(B, dtype=torch.int32, device="cuda")
        with torch.cuda.stream(s):
            eng.step_forward(meta, lg, tk, s)  # eager (also sets up every kernel attribute)
        torch.cuda.synchronize()
        ref_lg, ref_tk = lg.clone(), tk.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            eng.step_forward(meta, lg, tk, s)
        torch.cuda.synchronize()
        for rep in range(4):
            lg.fill_(float("nan"))
            tk.fill_(-1)
            junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
            torch.cuda.synchronize()
            with torch.cuda.stream(s):
                g.replay()
            torch.cuda.synchronize()
            assert torch.equal(lg, ref_lg), f"replay {rep}: logits differ"
            assert torch.equal(tk, ref_tk), f"replay {rep}: tokens differ"
            assert float(junk) == float(junk)
        assert eng.status() == 0
    finally:
        eng.close()


# ------------------------------------------------- cbd_step_forward_graph

def _advance(eng, meta, wl, B, j, max_ctx, mode, step_ids=None):
    """Write decode step j's metadata (contexts advanced by j, fresh tokens)
    into meta's device buffer in place, so that the step's device pointers
    stay fixed."""
    tokens = synth.uniform_ints(100 + j, "tok", B, 0, eng.shape.vocab - 1)
    m2 = eng.upload_step(slots=list(range(B)), block_tables=wl["tables"][:B],
                         ctx_lens=wl["ctx"][:B] + j, n_new=[1] * B, tokens=tokens,
                         want_token=[1] * B, step_ids=step_ids, mode=mode, max_ctx=max_ctx)
    meta.buf.copy_(m2.buf)
    return meta


@pytest.mark.parametrize("shape,B,mode,fmt", [(configs.LLAMA8B_1L, 32, 0, None),
                                              (configs.TINY, 6, 1, None),
                                              (configs.LLAMA8B_1L, 32, 0, "int8-e4m3")],
                         ids=["8b-layer-b32-greedy", "tiny-b6-sampled", "8b-layer-b32-int8w-e4m3kv"])
def test_graph_entry_point_replays_equal_eager_steps(shape, B, mode, fmt):
    """Eight decode steps with advancing contexts and fresh tokens, once
    eagerly and once through cbd_step_forward_graph (one recording, seven
    replays reading the updated metadata), from the same pool contents and
    sampler state: logits and tokens equal bit for bit at every step. Then
    a second step shape records a second graph, and the first shape replays
    its cached graph again. Also with int8 weights over an E4M3 cache."""
    from continuous_batching_decode_forward_amd import binding as Bd
    torch.cuda.set_device(0)
    if fmt:
        wg = synth.make_weights_int8(shape, seed=3, device="cuda")
        kv = dict(kv_dtype=Bd.CBD_KV_FP8_E4M3, **bench.FP8_KV)
    else:
        wg = synth.make_weights(shape, seed=3, device="cuda")
        kv = {}
    wl = bench.build_workload(shape, B, 3, ctx_range=(40, 900), bs=32)
    n_steps = 8
    # room for the appended positions: each table gets blocks past its context
    need = [-(-(int(c) + n_steps) // 32) for c in wl["ctx"]]
    total = sum(need)
    perm = synth.permutation(3, "blocks", total)
    mbps = max(need) + 4
    # a rounded-up bound of ctx + 1, fixed over the steps
    max_ctx = min(int(wl["ctx"].max()) + n_steps + 100, mbps * 32)
    tables = np.full((B, mbps), -1, np.int32)
    o = 0
    for i in range(B):
        tables[i, :need[i]] = perm[o:o + need[i]]
        o += need[i]
    wl["tables"] = tables
    eng = Engine(shape, wg, block_size=32, num_blocks=total, max_blocks_per_seq=mbps,
                 max_slots=B, max_rows=B, max_seqs=B, max_position=mbps * 32, **kv)
    s = torch.cuda.Stream()
    try:
        bench.fill_pool(eng, 3, perm)
        sp = configs.SamplingParams(top_p=0.9, top_k=50, freq_penalty=0.5)
        slots = []
        if mode == Bd.CBD_MODE_SAMPLE:
            params = Bd.cbd_sampling.from_params(sp)
            slots = [Bd.cbd_slot_alloc(eng.handle, params, r) for r in range(B)]
            assert slots == list(range(B))
        counts0 = eng.slot_counts().clone()
        lg = torch.empty((B, shape.vocab), dtype=torch.float32, device="cuda")
        tk = torch.empty(B, dtype=torch.int32, device="cuda")
        step_ids = lambda j: [j] * B if mode == Bd.CBD_MODE_SAMPLE else None
        meta = eng.upload_step(slots=list(range(B)), block_tables=tables, ctx_lens=wl["ctx"],
                               n_new=[1] * B, tokens=wl["tokens"], want_token=[1] * B,
                               step_ids=step_ids(0), mode=mode, max_ctx=max_ctx)

        def run(graph):
            eng.slot_counts().copy_(counts0)
            out = []
            for j in range(n_steps):
                _advance(eng, meta, wl, B, j, max_ctx, mode, step_ids(j))
                lg.fill_(float("nan"))
                tk.fill_(-1)
                torch.cuda.synchronize()
                with torch.cuda.stream(s):
                    if graph:
                        eng.step_forward_graph(meta, lg, tk, s)
                    else:
                        eng.step_forward(meta, lg, tk, s)
                torch.cuda.synchronize()
                out.append((lg.clone(), tk.clone()))
                junk = torch.randn(1 << 18, device="cuda").sum()  # eager work between steps
                assert float(junk) == float(junk)
            return out

        eager = run(False)
        assert eng.graph_stats() == (0, 0, 0)
        replayed = run(True)
        assert eng.graph_stats() == (1, n_steps - 1, 1)
        for j, ((l0, t0), (l1, t1)) in enumerate(zip(eager, replayed)):
            assert torch.equal(t0, t1), f"step {j}: tokens differ"
            assert torch.equal(l0, l1), f"step {j}: logits differ"
        # a second shape (the first B - 1 sequences) records a second graph
        m_small = eng.upload_step(slots=list(range(B - 1)), block_tables=tables[:B - 1],
                                  ctx_lens=wl["ctx"][:B - 1], n_new=[1] * (B - 1),
                                  tokens=wl["tokens"][:B - 1], want_token=[1] * (B - 1),
                                  step_ids=step_ids(0)[:B - 1] if step_ids(0) else None,
                                  mode=mode, max_ctx=max_ctx)
        with torch.cuda.stream(s):
            eng.step_forward_graph(m_small, lg, tk, s)
            eng.step_forward_graph(meta, lg, tk, s)  # the first shape: a replay
        torch.cuda.synchronize()
        assert eng.graph_stats() == (2, n_steps, 2)
        # the null stream cannot record a graph: refused before anything runs
        with pytest.raises(Bd.CbdError):
            Bd.cbd_step_forward_graph(eng.handle, meta.step, lg.data_ptr(), tk.data_ptr(), None)
        assert eng.status() == 0
    finally:
        eng.close()


def test_composer_loop_with_graph_replay_equals_the_eager_loop():
    """The tiny decoder under the native composer loop (figure constants),
    decode-only steps with max_ctx rounded up to a multiple of 16: replayed
    from recorded graphs, the loop commits the same tokens at every step and
    finishes the same requests as the eager loop with the same rounding."""
    torch.cuda.set_device(0)
    from continuous_batching_decode_forward_amd.engine import ComposerLoop
    from cb_streams import request_stream
    shape = configs.TINY
    wg = synth.make_weights(shape, seed=1, device="cuda")
    slots, bs, pool, mbps, rows, chunk = 4, 4, 40, 16, 12, 8
    order = synth.permutation(9, "blocks", pool).astype(np.int32)
    reqs = request_stream(9, 10, (5, 40), (2, 16), shape.vocab)

    def loop_run(graph):
        eng = Engine(shape, wg, block_size=bs, num_blocks=pool, max_blocks_per_seq=mbps,
                     max_slots=slots, max_rows=rows, max_seqs=slots, max_position=mbps * bs,
                     block_order=order)
        loop = ComposerLoop(eng, max_rows=rows, chunk_size=chunk, eos_id=0, ctx_round=16,
                            graph_decode=graph)
        if not graph:  # the same side stream arrangement as the graph loop
            loop.stream = torch.cuda.Stream()
        for rid, prompt, mx in reqs:
            loop.submit(prompt, mx, None, rid)
        trace = []
        try:
            for _ in range(400):
                p = loop.step()
                if p.n_rows == 0:
                    break
                trace.append((p.n_prefill_rows, list(loop.last_tokens(p.n_out))))
            fin = sorted(loop.pop_finished())
            stats = eng.graph_stats()
            assert eng.status() == 0
        finally:
            loop.close()
            eng.close()
        return trace, fin, stats

    t0, f0, s0 = loop_run(False)
    t1, f1, s1 = loop_run(True)
    assert s0 == (0, 0, 0)
    decode_steps = sum(1 for n_pre, _ in t1 if n_pre == 0)
    assert s1[0] + s1[1] == decode_steps and s1[1] > s1[0] > 0
    print(f"composer loop: {len(t1)} steps, {decode_steps} decode-only: {s1[0]} graphs recorded, "
          f"{s1[1]} replays")
    assert t0 == t1
    assert f0 == f1 and len(f0) == len(reqs)


def test_graph_cache_keeps_the_16_most_recent_shapes():
    """Eighteen step shapes (1..6 sequences x three max_ctx bounds) through
    cbd_step_forward_graph, each equal to the eager step bit for bit; the
    cache then holds the 16 most recent, and the first shape, evicted, is
    recorded again (and still equal)."""
    from continuous_batching_decode_forward_amd import binding as Bd
    torch.cuda.set_device(0)
    shape, Bmax = configs.TINY, 6
    wg = synth.make_weights(shape, seed=4, device="cuda")
    wl = bench.build_workload(shape, Bmax, 4, ctx_range=(20, 200), bs=32)
    eng = Engine(shape, wg, block_size=32, num_blocks=wl["total"], max_blocks_per_seq=wl["mbps"],
                 max_slots=Bmax, max_rows=Bmax, max_seqs=Bmax, max_position=1024)
    s = torch.cuda.Stream()
    lg = torch.empty((Bmax, shape.vocab), dtype=torch.float32, device="cuda")
    tk = torch.empty(Bmax, dtype=torch.int32, device="cuda")
    try:
        bench.fill_pool(eng, 4, wl["perm"])
        metas = []
        for i in range(18):
            n = 1 + i % 6
            bound = int(wl["ctx"][:n].max()) + 1 + 64 * (i // 6)  # three distinct bounds
            metas.append(eng.upload_step(slots=list(range(n)), block_tables=wl["tables"][:n],
                                         ctx_lens=wl["ctx"][:n], n_new=[1] * n,
                                         tokens=wl["tokens"][:n], want_token=[1] * n,
                                         max_ctx=bound))

        def both(m):
            n = m.n_seqs
            with torch.cuda.stream(s):
                eng.step_forward(m, lg, tk, s)
            torch.cuda.synchronize()
            ref = (lg[:n].clone(), tk[:n].clone())
            lg.fill_(float("nan"))
            tk.fill_(-1)
            with torch.cuda.stream(s):
                eng.step_forward_graph(m, lg, tk, s)
            torch.cuda.synchronize()
            assert torch.equal(lg[:n], ref[0]) and torch.equal(tk[:n], ref[1])

        for m in metas:
            both(m)
        assert eng.graph_stats() == (18, 0, Bd.CBD_GRAPH_CACHE)
        both(metas[-1])                      # the most recent: replayed
        assert eng.graph_stats() == (18, 1, Bd.CBD_GRAPH_CACHE)
        both(metas[0])                       # evicted: recorded again
        assert eng.graph_stats() == (19, 1, Bd.CBD_GRAPH_CACHE)
        assert eng.status() == 0
    finally:
        eng.close()

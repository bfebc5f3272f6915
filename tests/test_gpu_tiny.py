"""GPU parity on the tiny 2-layer decoder (d_model 256, 4/2 heads, head_dim
64, FFN 688, vocab 4096; 4-position blocks over a shuffled 64-block pool):
prefill through the chunk path, then 20 greedy decode steps, every step
compared with the oracle's paged-batched step on the same metadata. Tokens
are teacher-forced with the oracle's, so one near tie cannot desynchronise
the rest."""
import numpy as np
import pytest
import torch

import oracle as O
from continuous_batching_decode_forward_amd import binding as B
from continuous_batching_decode_forward_amd import configs, synth

from gpu_util import (attention_rows_vs_oracle, compare_logits, fill_pool, make_engine,
                      oracle_pool, resolvable_rows, weights_to)

pytestmark = pytest.mark.gpu

CFG = configs.TINY


@pytest.fixture(scope="module")
def tiny():
    w = synth.make_weights(CFG, seed=0)
    return w, O.Model(CFG, w), weights_to(w, "cuda")


def run_schedule(tiny, prompts, n_decode, chunk, bs, nb, seed, order=None, kv=None, final=None,
                 cfg=CFG):
    """Drive both sides through the same steps; return per-step stats.
    kv: the engine's cache format (the oracle model in `tiny` must match);
    final(eng, pool, tables, ctx) runs after the last step; cfg: the shape
    the weights in `tiny` have."""
    w, om, wg = tiny
    n = len(prompts)
    perm = synth.permutation(seed, "blocks", nb)
    per = nb // n
    tables = np.stack([perm[i * per:(i + 1) * per] for i in range(n)]).astype(np.int32)
    eng = make_engine(cfg, wg, block_size=bs, num_blocks=nb, max_blocks_per_seq=per,
                      max_rows=256, max_seqs=8, max_position=per * bs, **(kv or {}))
    pool = om.paged_pool(nb, bs)
    ctx = [0] * n
    last = [None] * n
    order = list(range(n)) if order is None else order
    results = []
    for step in range(10_000):
        seqs, nn, toks, want = [], [], [], []
        budget = 10_000
        for i in order:      # prefill chunks first, then decode rows
            if ctx[i] < len(prompts[i]):
                k = min(chunk, len(prompts[i]) - ctx[i])
                seqs.append(i); nn.append(k); toks += list(prompts[i][ctx[i]:ctx[i] + k])
                want.append(int(ctx[i] + k == len(prompts[i])))
        for i in order:
            if ctx[i] >= len(prompts[i]) and last[i] is not None and \
                    ctx[i] < len(prompts[i]) + n_decode:
                seqs.append(i); nn.append(1); toks.append(last[i]); want.append(1)
        if not seqs:
            break
        ref_lg, ref_tok = O.paged_step(om, pool, tables[seqs], [ctx[i] for i in seqs], nn,
                                       toks, want)
        meta = eng.upload_step(slots=seqs, block_tables=tables[seqs],
                               ctx_lens=[ctx[i] for i in seqs], n_new=nn, tokens=toks,
                               want_token=want)
        n_out = meta.n_out
        lg = torch.empty((max(n_out, 1), cfg.vocab), dtype=torch.float32, device="cuda")
        tk = torch.full((max(n_out, 1),), -1, dtype=torch.int32, device="cuda")
        eng.step_forward(meta, lg, tk)
        torch.cuda.synchronize()
        assert eng.status() == 0
        g_lg, g_tk = lg[:n_out].cpu().numpy(), tk[:n_out].cpu().numpy()
        if n_out:
            ok, mx, row_err = compare_logits(g_lg, ref_lg)
            res = resolvable_rows(ref_lg, row_err)
            # the argmax of the GPU's own fp32 logits, lowest id on ties
            own = np.array([O.argmax_f32(r) for r in g_lg])
            results.append((step, ok, mx, int(res.sum()), int((g_tk != ref_tok)[res].sum()),
                            bool(np.array_equal(own, g_tk))))
        o = 0
        for i, k, wt in zip(seqs, nn, want):
            ctx[i] += k
            if wt:
                last[i] = int(ref_tok[o])  # teacher forcing with the oracle's token
                o += 1
    if final is not None:
        final(eng, pool, tables, ctx)
    eng.close()
    return results


def check(results):
    assert results
    for step, ok, mx, n_res, n_bad, own_ok in results:
        assert ok, f"step {step}: logits outside tolerance (max abs err {mx:.3g})"
        assert n_bad == 0, f"step {step}: {n_bad} resolvable greedy ids differ"
        assert own_ok, f"step {step}: the argmax kernel disagrees with argmax of its logits"


def prompts_for(seed, n=4, lo=5, hi=40):
    lens = synth.uniform_ints(seed, "ctx", n, lo, hi)
    return [synth.uniform_ints(seed, f"prompt.{i}", int(lens[i]), 0, CFG.vocab - 1)
            for i in range(n)]


def test_tiny_prefill_then_20_greedy_steps(tiny):
    res = run_schedule(tiny, prompts_for(0), 20, chunk=64, bs=4, nb=64, seed=0)
    assert len(res) == 21
    check(res)


@pytest.mark.parametrize("vocab", [16, 48, 528])
def test_tiny_small_vocabularies(vocab):
    """Vocabularies narrower than one LM-head workgroup (512 columns): the
    argmax partials of every wave tile, most of them past the vocabulary,
    fit their buffer, and the ids stay the lowest maximum."""
    from dataclasses import replace
    cfg = replace(CFG, vocab=vocab, name=f"tiny-v{vocab}")
    w = synth.make_weights(cfg, seed=4)
    prompts = [synth.uniform_ints(4, f"p{i}", L, 0, vocab - 1) for i, L in enumerate([9, 30, 1, 17])]
    res = run_schedule((w, O.Model(cfg, w), weights_to(w, "cuda")), prompts, 6, chunk=64, bs=4,
                       nb=64, seed=4, cfg=cfg)
    check(res)


def test_tiny_chunked_prefill_mixed_with_decode(tiny):
    """8-token chunks: later steps carry prefill chunks and decode rows
    together, and chunks start at offsets inside blocks."""
    res = run_schedule(tiny, prompts_for(1), 12, chunk=8, bs=4, nb=64, seed=1, order=[2, 0, 3, 1])
    check(res)


# chunk 7 keeps every sequence on the per-tile attention kernel; chunks of
# 32+ rows on 32- and 64-position blocks take the block kernel.
@pytest.mark.parametrize("bs,chunk", [(8, 7), (16, 7), (32, 7), (64, 7), (32, 40), (64, 64)])
def test_tiny_block_sizes_and_ragged_contexts(tiny, bs, chunk):
    # contexts around block boundaries: bs-1, bs, bs+1, and a single token
    prompts = [synth.uniform_ints(bs, f"p{i}", L, 0, CFG.vocab - 1)
               for i, L in enumerate([bs - 1, bs, bs + 1, 1])]
    res = run_schedule(tiny, prompts, 5, chunk=chunk, bs=bs, nb=64 if bs < 32 else 32, seed=bs)
    check(res)


@pytest.mark.parametrize("bs", [4, 8, 16, 32, 64])
def test_row_kernel_decode_matches_oracle_at_every_block_size(tiny, bs):
    """32 sequences x 2 KV heads = 64 (sequence, KV head) pairs, one decode
    row each over 5..120 cached positions through shuffled block tables:
    attention runs on the row kernel. Every row's attention output and
    logits against the oracle."""
    w, om, wg = tiny
    n = 32
    ctx = synth.uniform_ints(bs, "rowctx", n, 5, 120)
    need = [-(-(int(c) + 1) // bs) for c in ctx]
    total = int(sum(need))
    perm = synth.permutation(bs, "rowblocks", total)
    mbps = -(-121 // bs)
    tables = np.full((n, mbps), -1, np.int32)
    o = 0
    for i in range(n):
        tables[i, :need[i]] = perm[o:o + need[i]]
        o += need[i]
    tokens = synth.uniform_ints(bs, "rowtok", n, 0, CFG.vocab - 1)
    eng = make_engine(CFG, wg, block_size=bs, num_blocks=total, max_blocks_per_seq=mbps,
                      max_rows=n, max_seqs=n, max_position=mbps * bs)
    fill_pool(eng, bs, perm)
    meta = eng.upload_step(slots=list(range(n)), block_tables=tables, ctx_lens=ctx, n_new=[1] * n,
                           tokens=tokens, want_token=[1] * n)
    lg = torch.empty((n, CFG.vocab), dtype=torch.float32, device="cuda")
    tk = torch.empty(n, dtype=torch.int32, device="cuda")
    eng.step_forward(meta, lg, tk)
    torch.cuda.synchronize()
    assert eng.status() == 0
    att = attention_rows_vs_oracle(eng, tables, ctx, [1] * n)
    g_lg, g_tk = lg.cpu().numpy(), tk.cpu().numpy()
    eng.close()
    pool, compact = oracle_pool(CFG, bs, list(tables), [int(c) for c in ctx], bs, [1] * n)
    ref_lg, ref_tk = O.paged_step(om, pool, compact, [int(c) for c in ctx], [1] * n,
                                  [int(t) for t in tokens], [1] * n)
    ok, mx, row_err = compare_logits(g_lg, ref_lg)
    assert ok, f"max abs logit error {mx:.3g}"
    assert att.max() <= 2.0 ** -12, f"attention rows {np.nonzero(att > 2.0 ** -12)[0][:8].tolist()}"
    res = resolvable_rows(ref_lg, row_err)
    assert np.array_equal(g_tk[res], np.asarray(ref_tk)[res])


def test_row_kernel_refuses_a_sequence_that_is_not_one_decode_row(tiny):
    """A step with as many rows as sequences runs attention on the row kernel
    (32 sequences x 2 KV heads = 64 workgroups). If the device metadata does
    not give every sequence one row (here 2 + 0 for the first two), that
    sequence is refused with BAD_SHAPE and the step completes."""
    w, om, wg = tiny
    n = 32
    eng = make_engine(CFG, wg, block_size=4, num_blocks=2 * n, max_blocks_per_seq=4,
                      max_rows=2 * n, max_seqs=n, max_position=16)
    tk = torch.zeros(n, dtype=torch.int32, device="cuda")
    tables = [[2 * i, 2 * i + 1, -1, -1] for i in range(n)]
    n_new = [2, 0] + [1] * (n - 2)
    want = [1 if k > 0 else 0 for k in n_new]
    meta = eng.upload_step(slots=list(range(n)), block_tables=tables, ctx_lens=[3] * n,
                           n_new=n_new, tokens=[1] * n, want_token=want)
    eng.step_forward(meta, None, tk)
    assert eng.status() & B.CBD_STATUS_BAD_SHAPE
    # the same sequences as decode rows run cleanly
    meta = eng.upload_step(slots=list(range(n)), block_tables=tables, ctx_lens=[3] * n,
                           n_new=[1] * n, tokens=[1] * n, want_token=[1] * n)
    eng.step_forward(meta, None, tk)
    assert eng.status() == 0
    eng.close()


def test_device_refuses_bad_metadata_without_faulting(tiny):
    w, om, wg = tiny
    eng = make_engine(CFG, wg, block_size=4, num_blocks=16, max_blocks_per_seq=4, max_rows=16,
                      max_seqs=4, max_position=16)
    tk = torch.zeros(2, dtype=torch.int32, device="cuda")
    # block id 99 is outside the 16-block pool
    meta = eng.upload_step(slots=[0, 1], block_tables=[[0, 1, 2, 3], [99, 5, 6, 7]],
                           ctx_lens=[0, 0], n_new=[2, 2], tokens=[1, 2, 3, 4], want_token=[1, 1])
    eng.step_forward(meta, None, tk)
    assert eng.status() & B.CBD_STATUS_BAD_BLOCK
    # token outside the vocabulary
    meta = eng.upload_step(slots=[0], block_tables=[[0, 1, 2, 3]], ctx_lens=[0], n_new=[1],
                           tokens=[CFG.vocab + 5], want_token=[1])
    eng.step_forward(meta, None, tk)
    assert eng.status() & B.CBD_STATUS_BAD_TOKEN
    # ctx + n_new beyond the block table
    meta = eng.upload_step(slots=[0], block_tables=[[0, 1, 2, 3]], ctx_lens=[15], n_new=[2],
                           tokens=[1, 2], want_token=[1], max_ctx=16)
    eng.step_forward(meta, None, tk)
    assert eng.status() & B.CBD_STATUS_BAD_SHAPE
    # host-side checks
    with pytest.raises(B.CbdError):
        bad = eng.upload_step(slots=[0], block_tables=[[0, 1, 2, 3]], ctx_lens=[0], n_new=[1],
                              tokens=[1], want_token=[1], max_ctx=999)
        eng.step_forward(bad, None, tk)
    # a clean step still works afterwards
    meta = eng.upload_step(slots=[0], block_tables=[[0, 1, 2, 3]], ctx_lens=[0], n_new=[3],
                           tokens=[1, 2, 3], want_token=[1])
    eng.step_forward(meta, None, tk)
    assert eng.status() == 0
    eng.close()

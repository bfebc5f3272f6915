"""Prefill chunks longer than one key split, on 32-position blocks: the
attention items of such a chunk include (query tile, split) pairs with no
keys (the chunk's first rows end before its later splits begin), which the
kernel must skip without touching the pool. Small decoders (head_dim 64 and
128, two query heads per KV head), contexts up to 1024 positions (up to 8 key
splits); every step is compared with the oracle's paged-batched step on the
same metadata, tokens teacher-forced with the oracle's."""
import numpy as np
import pytest
import torch

import oracle as O
from continuous_batching_decode_forward_amd import configs, synth

from gpu_util import compare_logits, make_engine, resolvable_rows, weights_to

pytestmark = pytest.mark.gpu

SHAPES = [configs.TINY, configs.ModelShape("small-hd128", 2, 256, 2, 1, 128, 512, 1024)]
BS, NB, MBPS = 32, 64, 32


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: s.name)
def test_long_chunks_span_several_key_splits(shape):
    torch.cuda.set_device(0)
    w = synth.make_weights(shape, seed=11)
    om, wg = O.Model(shape, w), weights_to(w, "cuda")
    perm = synth.permutation(11, "blocks", NB).astype(np.int32)
    tables = np.stack([perm[i * 16:(i + 1) * 16] for i in range(3)]).astype(np.int32)
    tables = np.concatenate([tables, np.full((3, MBPS - 16), -1, np.int32)], axis=1)
    eng = make_engine(shape, wg, block_size=BS, num_blocks=NB, max_blocks_per_seq=MBPS,
                      max_rows=600, max_seqs=4, max_position=MBPS * BS)
    pool = om.paged_pool(NB, BS)
    prompts = [synth.uniform_ints(11, f"p{i}", n, 0, shape.vocab - 1).tolist()
               for i, n in enumerate((300, 40, 500))]
    # step plans: (seq, n_new) with the prompt cut into the given chunks,
    # then decode rows
    plans = [[(0, 300), (1, 40), (2, 250)], [(2, 250), (0, 1), (1, 1)],
             [(0, 1), (1, 1), (2, 1)], [(0, 1), (1, 1), (2, 1)]]
    ctx, last, worst, n_res = [0, 0, 0], [None] * 3, 0.0, 0
    try:
        for step, plan in enumerate(plans):
            seqs, nn, toks, want = [], [], [], []
            for i, k in plan:
                seqs.append(i)
                nn.append(k)
                if ctx[i] < len(prompts[i]):
                    toks += prompts[i][ctx[i]:ctx[i] + k]
                    want.append(int(ctx[i] + k == len(prompts[i])))
                else:
                    toks.append(last[i])
                    want.append(1)
            ref_lg, ref_tok = O.paged_step(om, pool, tables[seqs], [ctx[i] for i in seqs], nn,
                                           toks, want)
            meta = eng.upload_step(slots=seqs, block_tables=tables[seqs],
                                   ctx_lens=[ctx[i] for i in seqs], n_new=nn, tokens=toks,
                                   want_token=want)
            n_out = meta.n_out
            lg = torch.empty((max(n_out, 1), shape.vocab), dtype=torch.float32, device="cuda")
            tk = torch.full((max(n_out, 1),), -1, dtype=torch.int32, device="cuda")
            eng.step_forward(meta, lg, tk)
            torch.cuda.synchronize()
            assert eng.status() == 0
            g_lg, g_tk = lg[:n_out].cpu().numpy(), tk[:n_out].cpu().numpy()
            ok, mx, row_err = compare_logits(g_lg, ref_lg)
            assert ok, f"step {step}: max abs logit error {mx:.3g}"
            res = resolvable_rows(ref_lg, row_err)
            assert np.array_equal(g_tk[res], ref_tok[res])
            worst, n_res = max(worst, mx), n_res + int(res.sum())
            o = 0
            for i, k, wt in zip(seqs, nn, want):
                ctx[i] += k
                if wt:
                    last[i] = int(ref_tok[o])
                    o += 1
    finally:
        eng.close()
    print(f"{shape.name}: long chunks, max abs logit error {worst:.2e}, {n_res} decidable rows")


def test_8b_layer_512_row_chunk_at_offset_3584():
    """The last 512-token chunk of a 4096-token prompt on one 8B-shaped layer
    + LM head: the chunk at offset 3584 over a paged prefix of 3584 cached
    positions, emitting its last row (the request's first answer token),
    beside 4 decode rows with contexts 1024..4096. The chunk runs on the
    block attention kernel at its real shape (256-column items over 7 key
    splits) and the projections on the dense GEMM at 516 rows. Checks: every
    row's attention output against the oracle's dense attention over the
    same query and K/V (2^-12 of its scale), and the emitting rows' logits
    against the oracle's paged step over all 516 rows."""
    from continuous_batching_decode_forward_amd.engine import Engine

    from gpu_util import attention_rows_vs_oracle, fill_pool, oracle_pool

    torch.cuda.set_device(0)
    shape, seed, bs, off, chunk = configs.LLAMA8B_1L, 5, 32, 3584, 512
    wg = synth.make_weights(shape, seed=seed, device="cuda")
    dec_ctx = [int(c) for c in synth.uniform_ints(seed, "ctx", 4, 1024, 4096)]
    ctx = [off] + dec_ctx
    nn = [chunk] + [1] * len(dec_ctx)
    need = [-(-(c + n) // bs) for c, n in zip(ctx, nn)]
    perm = synth.permutation(seed, "blocks", int(sum(need)))
    mbps = max(need)
    tables = np.full((len(ctx), mbps), -1, np.int32)
    at = 0
    for i, k in enumerate(need):
        tables[i, :k] = perm[at:at + k]
        at += k
    cached = np.concatenate([tables[i, :-(-c // bs)] for i, c in enumerate(ctx)])
    prompt = synth.uniform_ints(seed, "prompt", off + chunk, 0, shape.vocab - 1)
    toks = [int(t) for t in prompt[off:]] + \
        [int(t) for t in synth.uniform_ints(seed, "dec", len(dec_ctx), 0, shape.vocab - 1)]
    want = [1] * len(ctx)
    eng = Engine(shape, wg, block_size=bs, num_blocks=len(perm), max_blocks_per_seq=mbps,
                 max_slots=len(ctx), max_rows=sum(nn), max_seqs=len(ctx),
                 max_position=mbps * bs)
    try:
        fill_pool(eng, seed, cached)
        meta = eng.upload_step(slots=list(range(len(ctx))), block_tables=tables, ctx_lens=ctx,
                               n_new=nn, tokens=toks, want_token=want)
        lg = torch.empty((len(ctx), shape.vocab), dtype=torch.float32, device="cuda")
        tk = torch.empty(len(ctx), dtype=torch.int32, device="cuda")
        eng.step_forward(meta, lg, tk)
        torch.cuda.synchronize()
        assert eng.status() == 0
        g_lg, g_tk = lg.cpu().numpy(), tk.cpu().numpy()
        att = attention_rows_vs_oracle(eng, tables, ctx, nn)
    finally:
        eng.close()
    print(f"512-row chunk at offset {off}: attention of all {len(att)} rows, largest error "
          f"{att.max():.2e}")
    assert att.max() <= 2.0 ** -12, f"attention rows {np.nonzero(att > 2.0 ** -12)[0][:8].tolist()}"
    assert np.array_equal(g_tk, np.argmax(g_lg, axis=1))
    wc = {k: ([t.cpu() for t in v] if isinstance(v, list) else v.cpu()) for k, v in wg.items()}
    del wg
    model = O.Model(shape, wc)
    pool, compact = oracle_pool(shape, seed, list(tables), ctx, bs, nn)
    ref_lg, ref_tok = O.paged_step(model, pool, compact, ctx, nn, toks, want)
    ok, mx, row_err = compare_logits(g_lg, ref_lg)
    res = resolvable_rows(ref_lg, row_err)
    print(f"512-row chunk at offset {off}: emitting rows' max abs logit error {mx:.2e}, "
          f"{int(res.sum())}/{len(ctx)} decidable")
    assert ok, f"max abs logit error {mx:.3g}"
    assert np.array_equal(g_tk[res], ref_tok[res])

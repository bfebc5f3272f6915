"""GPU parity on one 8B-shaped decoder layer + LM head (d_model 4096, 32/8
heads, head_dim 128, FFN 14336, vocab 128256): one greedy decode step over
B rows whose contexts (512..4096) are synthetic N(0,1) KV in 32-position
blocks reached through shuffled block tables. The full step runs at full
size on the GPU in the benchmark's launch configuration; the oracle checks a
sample of rows' logits one by one (on a compact copy of their blocks --
paging is addressing only, which the oracle's own tests pin), and every
row's attention output against its dense attention over the same query and
K/V (the attention schedule cuts pieces across sequence and tile
boundaries, so every row is checked, not a sample)."""
import numpy as np
import pytest
import torch

import oracle as O
from continuous_batching_decode_forward_amd import configs, synth

from gpu_util import (attention_rows_vs_oracle, compare_logits, fill_pool, make_engine,
                      oracle_pool, resolvable_rows)

# Attention output against the oracle's dense attention on identical inputs:
# fp32 online softmax and accumulation over at most 4097 keys; 2^-12 is 16
# times below a bf16 ulp, while a key step left out or counted twice moves a
# row's output by more than 2^-7 of its scale.
ATTN_TOL = 2.0 ** -12

pytestmark = pytest.mark.gpu

SHAPE = configs.LLAMA8B_1L


@pytest.fixture(scope="module")
def big():
    wg = synth.make_weights(SHAPE, seed=0, device="cuda")
    wc = {k: ([t.cpu() for t in v] if isinstance(v, list) else v.cpu()) for k, v in wg.items()}
    return wg, O.Model(SHAPE, wc)


def decode_step(big, B, seed, sample_rows, lo=512, hi=4096, ctx=None, kv=None, om=None):
    """kv: the engine's cache format, om: the oracle model of that format."""
    wg, om0 = big
    om = om or om0
    kv = kv or {}
    bs = 32
    if ctx is None:
        ctx = synth.uniform_ints(seed, "ctx", B, lo, hi)
    ctx = np.asarray(ctx, np.int32)
    need = [-(-(int(c) + 1) // bs) for c in ctx]
    total = sum(need)
    perm = synth.permutation(seed, "blocks", total)
    mbps = -(-(hi + 1) // bs)
    tables = np.full((B, mbps), -1, np.int32)
    o = 0
    for i in range(B):
        tables[i, :need[i]] = perm[o:o + need[i]]
        o += need[i]
    tokens = synth.uniform_ints(seed, "tok", B, 0, SHAPE.vocab - 1)
    eng = make_engine(SHAPE, wg, block_size=bs, num_blocks=total, max_blocks_per_seq=mbps,
                      max_rows=max(B, 16), max_seqs=max(B, 16), max_position=hi + 1, **kv)
    fill_pool(eng, seed, perm)
    meta = eng.upload_step(slots=list(range(B)), block_tables=tables, ctx_lens=ctx,
                           n_new=[1] * B, tokens=tokens, want_token=[1] * B)
    lg = torch.empty((B, SHAPE.vocab), dtype=torch.float32, device="cuda")
    tk = torch.empty(B, dtype=torch.int32, device="cuda")
    eng.step_forward(meta, lg, tk)
    torch.cuda.synchronize()
    assert eng.status() == 0
    g_lg, g_tk = lg.cpu().numpy(), tk.cpu().numpy()
    att_err = attention_rows_vs_oracle(eng, tables, ctx, [1] * B)
    eng.close()
    rows = list(sample_rows)
    pool, compact = oracle_pool(SHAPE, seed, [tables[i] for i in rows], [int(ctx[i]) for i in rows],
                                bs, [1] * len(rows), kv_fp8=om.kv_fp8)
    ref_lg, ref_tk = O.paged_step(om, pool, compact, [int(ctx[i]) for i in rows], [1] * len(rows),
                                  [int(tokens[i]) for i in rows], [1] * len(rows))
    ok, mx, row_err = compare_logits(g_lg[rows], ref_lg)
    res = resolvable_rows(ref_lg, row_err)
    own = np.array([O.argmax_f32(r) for r in g_lg])
    return ok, mx, res, g_tk[rows], ref_tk, own, g_tk, att_err


# One case per GEMM shape: 16-row fragments (1, 8, 16), 32 rows (24: a
# partly filled second fragment), 64 rows (40: partly filled; 64: the 8-wave
# LM head) and the dense path, whose tile height and K split depend on the
# row count: 96 (128-row tiles, down in 16 splits), 150 (192-row tiles, a
# partly filled tile), 300 (QKV in 5 splits, O on 128-row tiles), 400
# (256-row tiles, O in 4 splits, a partly filled second row group).
@pytest.mark.parametrize("B,rows", [(1, [0]), (8, [0, 3, 7]), (16, [0, 15]), (24, [0, 11, 23]),
                                    (40, [0, 39]), (64, [0, 17, 40, 63]), (96, [0, 65, 95]),
                                    (150, [0, 77, 149]), (300, [0, 299]), (400, [0, 211, 399])])
def test_8b_layer_decode_step_matches_oracle(big, B, rows):
    ok, mx, res, g_tk, r_tk, own, all_tk, att = decode_step(big, B, seed=B, sample_rows=rows)
    print(f"B={B}: max abs logit error {mx:.4f}, resolvable rows {int(res.sum())}/{len(rows)}, "
          f"attention of all {B} rows: largest error {att.max():.2e}")
    assert ok, f"max abs logit error {mx:.3g}"
    assert att.max() <= ATTN_TOL, f"attention rows {np.nonzero(att > ATTN_TOL)[0][:8].tolist()}"
    assert np.array_equal(g_tk[res], r_tk[res])
    # every row: the fused argmax equals the lowest-id argmax of the logits
    assert np.array_equal(own, all_tk)


@pytest.mark.parametrize("B,hi", [(8, 1023), (32, 1023), (32, 1024), (64, 1023)])
def test_8b_layer_decode_over_contexts_up_to_1k(big, B, hi):
    """Decode-only steps whose keys fit 1024, over 64 to 256 (sequence, KV
    head) pairs, run on the row kernel (a workgroup per pair, merged in
    LDS); one key more (hi 1024), or more pairs than CUs (B = 64), runs on
    the per-tile kernel and its combine. Every row's attention is checked."""
    rows = [0, B // 2, B - 1]
    ok, mx, res, g_tk, r_tk, own, all_tk, att = decode_step(big, B, seed=B + hi, sample_rows=rows,
                                                            lo=16, hi=hi)
    assert ok, f"max abs logit error {mx:.3g}"
    assert att.max() <= ATTN_TOL, f"attention rows {np.nonzero(att > ATTN_TOL)[0][:8].tolist()}"
    assert np.array_equal(g_tk[res], r_tk[res])
    assert np.array_equal(own, all_tk)


def test_8b_layer_short_contexts_and_block_edges(big):
    # contexts 31, 32, 33, 63, 64 around 32-position block edges
    ok, mx, res, g_tk, r_tk, own, all_tk, att = decode_step(big, 5, seed=77, sample_rows=range(5),
                                                            lo=31, hi=64, ctx=[31, 32, 33, 63, 64])
    assert ok, f"max abs logit error {mx:.3g}"
    assert att.max() <= ATTN_TOL
    assert np.array_equal(g_tk[res], r_tk[res])

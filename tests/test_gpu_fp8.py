"""GPU parity with an 8-bit KV cache (OCP FP8 E4M3 codes of value / scale,
one scale for keys and one for values, dequantised as code x scale when
read): the same steps as the bf16 tests, against the oracle run with the
same cache format.

Checks:
  * the tiny 2-layer decoder end to end (prefill chunks, then greedy decode,
    on 8-, 16-, 32- and 64-position blocks): logits within the stated
    tolerance of the oracle's paged step, greedy ids on decidable rows, and
    the pools the two sides wrote hold the same code, or the adjacent one,
    at every position (one rounding of an fp32 versus an fp64 value);
  * one 8B-shaped layer + LM head at B = 8 and 64 over cached codes: sampled
    rows' logits, and every row's attention against the oracle's dense
    attention over the same query and the codes the pool holds;
  * a 512-row chunk of that layer at offset 1024: every appended K (after
    RoPE) and V code is the E4M3 rounding of a value within the GPU's fp32
    error bound of the exact one divided by its scale (saturating at 448),
    every row's attention, and the emitting row's logits;
  * the long-context B = 256 step (contexts 8k..32k) over cached codes:
    every row's attention and the three shortest rows' logits."""
import numpy as np
import pytest
import torch

import bench
import oracle as O
from continuous_batching_decode_forward_amd import binding as B
from continuous_batching_decode_forward_amd import configs, synth
from continuous_batching_decode_forward_amd.engine import Engine

from gpu_util import (attention_rows_vs_oracle, compare_logits, fill_pool, oracle_pool,
                      resolvable_rows, weights_to)
import test_gpu_8b
import test_gpu_tiny

pytestmark = pytest.mark.gpu

# Attention on identical inputs (the codes decode exactly to bf16; the key
# scale is folded into the softmax scale, the value scale applied to the
# result): the bar of the bf16 tests.
ATTN_TOL = 2.0 ** -12

# E4M3 values in ascending order with +0 and -0 merged, for the distance of
# two codes in the value lattice.
_DEC = np.array([O.e4m3_to_float(c) for c in range(256)])
_FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
_LATTICE = np.unique(_DEC[_FINITE])


def lattice_rank(codes):
    return np.searchsorted(_LATTICE, _DEC[np.asarray(codes, np.int64)])


def e4m3_half_spacing(g):
    """Half the E4M3 spacing at |g| (the spacing above for a power of two);
    subnormals below 2^-6 are spaced 2^-9."""
    a = np.abs(g)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 2.0 ** (e - 4)


# ------------------------------------------------------------------ tiny

TINY_KV = dict(kv_dtype=B.CBD_KV_FP8_E4M3, k_scale=0.05, v_scale=0.03)


@pytest.fixture(scope="module")
def tiny8():
    cfg = configs.TINY
    w = synth.make_weights(cfg, seed=0)
    om = O.Model(cfg, w, kv_fp8=True, k_scale=TINY_KV["k_scale"], v_scale=TINY_KV["v_scale"])
    return w, om, weights_to(w, "cuda")


@pytest.mark.parametrize("bs,chunk", [(8, 7), (16, 8), (32, 40), (64, 64)])
def test_tiny_fp8_prefill_then_decode(tiny8, bs, chunk):
    cfg = configs.TINY
    prompts = [synth.uniform_ints(bs, f"p{i}", L, 0, cfg.vocab - 1)
               for i, L in enumerate([bs - 1, bs, bs + 1, 1, 3 * bs + 5])]
    cmp = {}

    def pools(eng, pool, tables, ctx):
        # every position the run wrote, on both sides; V is dimension-major
        # in the engine's pool, position-major in the oracle's
        for layer in range(cfg.n_layers):
            k, v = eng.kv_views(layer)
            gk = k.cpu().numpy().transpose(0, 2, 1, 3)      # [blk][bs][Hkv][hd]
            gv = v.cpu().numpy().transpose(0, 3, 1, 2)
            diff = far = total = 0
            for i, c in enumerate(ctx):
                pos = np.arange(c)
                blk, o = tables[i][pos // bs], pos % bs
                for kind, g in ((0, gk), (1, gv)):
                    d = np.abs(lattice_rank(g[blk, o]) - lattice_rank(pool[layer, kind, blk, o]))
                    diff += int((d > 0).sum())
                    far += int((d > 1).sum())
                    total += d.size
            cmp[layer] = (diff, far, total)

    res = test_gpu_tiny.run_schedule(tiny8, prompts, 6, chunk=chunk, bs=bs, nb=80, seed=bs,
                                     kv=TINY_KV, final=pools)
    test_gpu_tiny.check(res)
    worst = max(r[2] for r in res)
    print(f"tiny fp8 bs={bs} chunk={chunk}: {len(res)} steps, max abs logit error {worst:.2e}; "
          "pool codes differing from the oracle's (differing, more than one step apart, of): "
          + ", ".join(f"layer {l} {d}/{f}/{t}" for l, (d, f, t) in cmp.items()))
    # Layer 0 appends the same inputs on both sides (the embedding rows):
    # an fp32 and an fp64 evaluation, then one rounding each, so a code
    # differs at most by one step, and rarely. Deeper layers' inputs already
    # differ by the rounding below them (a flipped code moves the next
    # layer's keys by an absolute amount, several steps apart near zero);
    # they are checked through the logits, and their codes only for rarity.
    d0, f0, t0 = cmp[0]
    assert f0 == 0, f"layer 0: {f0} codes more than one step from the oracle's"
    assert d0 <= t0 // 1000
    for layer, (d, f, t) in cmp.items():
        assert d <= t // 100, f"layer {layer}: {d} of {t} codes differ"

# ------------------------------------------------------------- 8B layer

LAYER_KV = dict(kv_dtype=B.CBD_KV_FP8_E4M3, k_scale=0.25, v_scale=0.25)


@pytest.fixture(scope="module")
def big8():
    shape = configs.LLAMA8B_1L
    wg = synth.make_weights(shape, seed=0, device="cuda")
    wc = {k: ([t.cpu() for t in v] if isinstance(v, list) else v.cpu()) for k, v in wg.items()}
    om = O.Model(shape, wc, kv_fp8=True, k_scale=LAYER_KV["k_scale"],
                 v_scale=LAYER_KV["v_scale"])
    return wg, om, wc


# contexts U[512, 4096] run on the per-tile kernel; 32 rows over contexts
# up to 1023 keys run on the row kernel
@pytest.mark.parametrize("Bn,rows,hi", [(8, [0, 3, 7], 4096), (64, [0, 17, 40, 63], 4096),
                                        (32, [0, 15, 31], 1023)])
def test_8b_layer_fp8_decode_step(big8, Bn, rows, hi):
    wg, om, _ = big8
    ok, mx, res, g_tk, r_tk, own, all_tk, att = test_gpu_8b.decode_step(
        (wg, om), Bn, seed=100 + Bn, sample_rows=rows, lo=16 if hi < 4096 else 512, hi=hi,
        kv=LAYER_KV, om=om)
    print(f"8b fp8 B={Bn}: max abs logit error {mx:.4f}, decidable rows {int(res.sum())}/"
          f"{len(rows)}, attention of all {Bn} rows: largest error {att.max():.2e}")
    assert ok, f"max abs logit error {mx:.3g}"
    assert att.max() <= ATTN_TOL, f"attention rows {np.nonzero(att > ATTN_TOL)[0][:8].tolist()}"
    assert np.array_equal(g_tk[res], r_tk[res])
    assert np.array_equal(own, all_tk)


CHUNK_KV = dict(kv_dtype=B.CBD_KV_FP8_E4M3, k_scale=0.01, v_scale=0.005)


def test_8b_layer_fp8_chunk_appends(big8):
    """512 prompt rows at positions 1024..1535 (the first 1024 cached as
    codes): the appended codes against the oracle's fp64 stage values. The
    scales put K/scale at about 128 and V/scale at about 256 standard
    deviations, so some of both saturate at 448."""
    shape = configs.LLAMA8B_1L
    wg, _, wc = big8
    ks, vs = CHUNK_KV["k_scale"], CHUNK_KV["v_scale"]
    bs, off, n = 32, 1024, 512
    seed = 9
    nb = (off + n) // bs
    perm = synth.permutation(seed, "blocks", nb)
    table = perm.astype(np.int32)[None, :]
    prompt = synth.uniform_ints(seed, "prompt", off + n, 0, shape.vocab - 1)
    eng = Engine(shape, wg, block_size=bs, num_blocks=nb, max_blocks_per_seq=nb, max_slots=1,
                 max_rows=n, max_seqs=1, max_position=off + n, **CHUNK_KV)
    try:
        fill_pool(eng, seed, perm[:off // bs])
        meta = eng.upload_step(slots=[0], block_tables=table, ctx_lens=[off], n_new=[n],
                               tokens=prompt[off:], want_token=[1])
        lg = torch.empty((1, shape.vocab), dtype=torch.float32, device="cuda")
        tk = torch.empty(1, dtype=torch.int32, device="cuda")
        eng.step_forward(meta, lg, tk)
        torch.cuda.synchronize()
        assert eng.status() == 0
        g_lg = lg.cpu().numpy()
        att = attention_rows_vs_oracle(eng, table, [off], [n])
        k0, v0 = eng.kv_views(0)
        blocks = torch.as_tensor(perm[off // bs:].astype(np.int64), device="cuda")
        gk = k0[blocks].permute(0, 2, 1, 3).reshape(n, shape.n_kv_heads, shape.head_dim)
        gv = v0[blocks].permute(0, 3, 1, 2).reshape(n, shape.n_kv_heads, shape.head_dim)
        gk, gv = gk.contiguous().cpu().numpy(), gv.contiguous().cpu().numpy()
    finally:
        eng.close()
    print(f"8b fp8 chunk: attention of all {n} rows, largest error {att.max():.2e}")
    assert att.max() <= ATTN_TOL, f"attention rows {np.nonzero(att > ATTN_TOL)[0][:8].tolist()}"

    hd, hkv, hq = shape.head_dim, shape.n_kv_heads, shape.n_heads
    E = O.bf16_to_f64(O.as_u16(wc["embed"])[np.asarray(prompt[off:], np.int64)])
    Wqkv = O.bf16_to_f64(O.as_u16(wc["w_qkv"][0])).reshape(-1, shape.d_model)
    Wk, Wv = Wqkv[hq * hd:(hq + hkv) * hd], Wqkv[(hq + hkv) * hd:]
    g0 = O.as_u16(wc["attn_norm"][0])
    flips = sat = total = 0
    bad = []
    for i in range(n):
        h = O.rmsnorm(E[i], g0, shape.rms_eps)
        k, v = Wk @ h, Wv @ h
        # fp32 dot products within 2^-16 sum |w||h| (hi + lo operands, fp32
        # accumulation), the rotation adds its two inputs' bounds; the
        # division by the scale and the fp32 value add 2^-22 relative
        bk = 2.0 ** -16 * (np.abs(Wk) @ np.abs(h))
        bv = 2.0 ** -16 * (np.abs(Wv) @ np.abs(h))
        kr = np.concatenate([O.rope(k[g * hd:(g + 1) * hd], off + i, shape.rope_base)
                             for g in range(hkv)])
        bkr = np.concatenate([np.tile(bk[g * hd:g * hd + hd // 2] + bk[g * hd + hd // 2:(g + 1) * hd], 2)
                              for g in range(hkv)])
        for name, codes, exact, bound, scale in (("K", gk[i].reshape(-1), kr, bkr, ks),
                                                 ("V", gv[i].reshape(-1), v, bv, vs)):
            x = exact / scale
            b = bound / scale + np.abs(x) * 2.0 ** -22
            g = _DEC[codes.astype(np.int64)]
            dev = np.abs(g - np.clip(x, -448.0, 448.0))
            ok = np.isfinite(g) & (dev <= b + e4m3_half_spacing(g))
            want = np.array([O.float_to_e4m3(float(t)) for t in x], np.uint8)
            flips += int((codes != want).sum())
            sat += int((np.abs(x) > 448.0).sum())
            total += x.size
            for e in np.nonzero(~ok)[0][:4]:
                bad.append(f"row {i} {name}[{e}]: code {codes[e]:#04x} ({g[e]:.6g}) exact "
                           f"{x[e]:.8g}, rounding {want[e]:#04x}, bound {b[e]:.3g}")
    print(f"8b fp8 chunk appends: {flips} of {total} codes differ from the rounding of the "
          f"exact value, {sat} saturated, outside the bound: {len(bad)}")
    for line in bad[:16]:
        print("  " + line)
    assert not bad
    assert sat > 0  # the scales do reach the saturation path

    om = O.Model(shape, wc, kv_fp8=True, k_scale=ks, v_scale=vs)
    pool, compact = oracle_pool(shape, seed, [table[0]], [off], bs, [n], kv_fp8=True)
    ref_lg, ref_tk = O.paged_step(om, pool, compact, [off], [n], [int(t) for t in prompt[off:]],
                                  [1])
    ok_l, mx, row_err = compare_logits(g_lg, ref_lg)
    res = resolvable_rows(ref_lg, row_err)
    print(f"8b fp8 chunk: emitting row max abs logit error {mx:.2e}, decidable {int(res.sum())}")
    assert ok_l, f"max abs logit error {mx:.3g}"


# ------------------------------------------------------- long contexts

def test_long_context_b256_fp8():
    shape, wlc = configs.LLAMA8B_1L_V64K, configs.SAMPLE_8B_B256
    seed, Bn = 4, wlc.batch[0]
    wg = synth.make_weights(shape, seed=seed, device="cuda")
    wl = bench.build_workload(shape, Bn, seed, ctx_range=wlc.ctx_range, bs=wlc.block_size)
    eng = Engine(shape, wg, block_size=wl["bs"], num_blocks=wl["total"],
                 max_blocks_per_seq=wl["mbps"], max_slots=Bn, max_rows=Bn, max_seqs=Bn,
                 max_position=wl["max_position"], **LAYER_KV)
    try:
        bench.fill_pool(eng, seed, wl["perm"])
        meta = eng.upload_step(slots=list(range(Bn)), block_tables=wl["tables"],
                               ctx_lens=wl["ctx"], n_new=[1] * Bn, tokens=wl["tokens"],
                               want_token=[1] * Bn)
        lg = torch.empty((Bn, shape.vocab), dtype=torch.float32, device="cuda")
        tk = torch.empty(Bn, dtype=torch.int32, device="cuda")
        eng.step_forward(meta, lg, tk)
        torch.cuda.synchronize()
        assert eng.status() == 0
        g_lg, g_tk = lg.cpu().numpy(), tk.cpu().numpy()
        att = attention_rows_vs_oracle(eng, wl["tables"], wl["ctx"], [1] * Bn)
    finally:
        eng.close()
    print(f"long fp8 step: attention of all {Bn} rows, largest error {att.max():.2e}")
    assert att.max() <= ATTN_TOL, f"attention rows {np.nonzero(att > ATTN_TOL)[0][:8].tolist()}"
    assert np.array_equal(g_tk, [O.argmax_f32(r) for r in g_lg])
    rows = [int(r) for r in np.argsort(wl["ctx"])[:3]]
    wc = {k: ([t.cpu() for t in v] if isinstance(v, list) else v.cpu()) for k, v in wg.items()}
    om = O.Model(shape, wc, kv_fp8=True, k_scale=LAYER_KV["k_scale"],
                 v_scale=LAYER_KV["v_scale"])
    cached = [int(wl["ctx"][i]) for i in rows]
    pool, compact = oracle_pool(shape, seed, [wl["tables"][i] for i in rows], cached, wl["bs"],
                                [1] * len(rows), kv_fp8=True)
    ref_lg, ref_tk = O.paged_step(om, pool, compact, cached, [1] * len(rows),
                                  [int(wl["tokens"][i]) for i in rows], [1] * len(rows))
    ok, mx, row_err = compare_logits(g_lg[rows], ref_lg)
    res = resolvable_rows(ref_lg, row_err)
    print(f"long fp8 step: max abs logit error {mx:.2e} on rows with ctx {cached}")
    assert ok, f"max abs logit error {mx:.3g}"
    assert np.array_equal(g_tk[rows][res], ref_tk[res])

"""The mixed step at full size: the 8B shape with all 32 layers (d_model 4096,
32/8 heads, FFN 14336, vocab 128256), 48 decode rows with contexts uniform
in 1024..8192 over a shuffled 32-position block pool of synthetic N(0,1)
bf16 K/V, plus the first 512-token chunk of a 4096-token prompt: 560 rows in
one step.

Checks:
  * the two decode rows with the shortest contexts: logits within the stated
    tolerance of the oracle's paged step (all 32 layers) and the greedy id
    on decidable rows;
  * every appended K (after RoPE) and V of the chunk at layer 0, against the
    oracle's fp64 evaluation of the same stage (norm, projection, rotation):
    the GPU's bf16 value is the rounding of a value within the GPU's fp32
    error bound of the exact one (which forces the oracle's own rounding
    wherever that bound is below half a bf16 ulp);
  * greedy ids equal the argmax of the GPU's own fp32 logits on every row,
    and the device status stays clear."""
import numpy as np
import pytest
import torch

import bench
import oracle as O
from continuous_batching_decode_forward_amd import configs, synth
from continuous_batching_decode_forward_amd.engine import Engine

from gpu_util import compare_logits, oracle_pool, resolvable_rows

pytestmark = pytest.mark.gpu

SHAPE = configs.LLAMA8B


def bf16_bits_to_f64(u):
    return (np.asarray(u, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_half_ulp(g):
    """Half the bf16 spacing at |g| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(g), 2.0 ** -126)))
    return 2.0 ** (e - 8)


def neighbours_ok(g_bits, exact, bound):
    """g_bits (bf16) must be the bf16 rounding of some value within `bound`
    of `exact` (the GPU's fp32 value, then one rounding): |g - exact| <=
    bound + half a bf16 ulp of g. Where the bound is below half an ulp this
    leaves only the round-to-nearest of `exact`, or its neighbour when
    `exact` lies within the bound of the midpoint. Returns (ok mask, number
    of elements that differ from the rounding of `exact`, largest
    |g - exact| / (bound + half ulp))."""
    want = O.bf16_round(exact)
    g = bf16_bits_to_f64(g_bits)
    slack = bound + bf16_half_ulp(g)
    dev = np.abs(g - exact)
    return dev <= slack, int((g_bits != want).sum()), float((dev / slack).max())


def test_mixed_step_8b_32_layers():
    torch.cuda.set_device(0)
    seed = 0
    wg = synth.make_weights(SHAPE, seed=seed, device="cuda")
    wl = bench.build_mixed(SHAPE, seed)
    n_dec = len(wl["ctx"])
    eng = Engine(SHAPE, wg, block_size=wl["bs"], num_blocks=wl["total"],
                 max_blocks_per_seq=wl["mbps"], max_slots=n_dec + 1,
                 max_rows=wl["chunk"] + n_dec, max_seqs=n_dec + 1,
                 max_position=wl["max_position"])
    try:
        bench.fill_pool(eng, seed, wl["cached"])
        seqs, tab, ctx, nn, toks, want = bench.mixed_step(wl, 0)
        meta = eng.upload_step(slots=seqs, block_tables=tab, ctx_lens=ctx, n_new=nn,
                               tokens=toks, want_token=want)
        n_out = meta.n_out
        assert n_out == n_dec  # the first chunk emits nothing
        lg = torch.empty((n_out, SHAPE.vocab), dtype=torch.float32, device="cuda")
        tk = torch.empty(n_out, dtype=torch.int32, device="cuda")
        eng.step_forward(meta, lg, tk)
        torch.cuda.synchronize()
        assert eng.status() == 0
        g_lg, g_tk = lg.cpu().numpy(), tk.cpu().numpy()
        k0, v0 = eng.kv_views(0)
        blocks = torch.as_tensor(wl["tables"][0, :wl["chunk"] // wl["bs"]].astype(np.int64),
                                 device="cuda")
        # [blocks][Hkv][bs][hd] -> [positions][Hkv][hd]; V is [blocks][Hkv][hd][bs]
        gk = k0[blocks].permute(0, 2, 1, 3).reshape(wl["chunk"], SHAPE.n_kv_heads,
                                                    SHAPE.head_dim)
        gv = v0[blocks].permute(0, 3, 1, 2).reshape(wl["chunk"], SHAPE.n_kv_heads,
                                                    SHAPE.head_dim)
        gk = O.as_u16(gk.contiguous().cpu())
        gv = O.as_u16(gv.contiguous().cpu())
    finally:
        eng.close()

    assert np.array_equal(g_tk, [O.argmax_f32(r) for r in g_lg])

    wc = {k: ([t.cpu() for t in v] if isinstance(v, list) else v.cpu()) for k, v in wg.items()}
    del wg
    # chunk appends at layer 0: the oracle's pieces in fp64
    hd, hkv, hq = SHAPE.head_dim, SHAPE.n_kv_heads, SHAPE.n_heads
    E = O.bf16_to_f64(O.as_u16(wc["embed"])[np.asarray(wl["prompt"][:wl["chunk"]], np.int64)])
    Wqkv = O.bf16_to_f64(O.as_u16(wc["w_qkv"][0])).reshape(-1, SHAPE.d_model)
    Wk = Wqkv[hq * hd:(hq + hkv) * hd]
    Wv = Wqkv[(hq + hkv) * hd:]
    g0 = O.as_u16(wc["attn_norm"][0])
    flips, total, bad, n_bad, worst = 0, 0, [], {"K": 0, "V": 0}, 0.0
    for i in range(wl["chunk"]):
        x = E[i]
        h = O.rmsnorm(x, g0, SHAPE.rms_eps)
        k = Wk @ h
        v = Wv @ h
        # fp32 dot products: within 2^-16 * sum |h||w| (hi + lo operands, fp32
        # accumulation); the rotation adds the two inputs' bounds
        bk = 2.0 ** -16 * (np.abs(Wk) @ np.abs(h))
        bv = 2.0 ** -16 * (np.abs(Wv) @ np.abs(h))
        kr = np.concatenate([O.rope(k[g * hd:(g + 1) * hd], i, SHAPE.rope_base)
                             for g in range(hkv)])
        bkr = np.concatenate([np.tile(bk[g * hd:g * hd + hd // 2] + bk[g * hd + hd // 2:(g + 1) * hd], 2)
                              for g in range(hkv)])
        ok_k, fk, rk = neighbours_ok(gk[i].reshape(-1), kr, bkr)
        ok_v, fv, rv = neighbours_ok(gv[i].reshape(-1), v, bv)
        worst = max(worst, rk, rv)
        for name, ok_, gb, ex, bd in (("K", ok_k, gk[i].reshape(-1), kr, bkr),
                                      ("V", ok_v, gv[i].reshape(-1), v, bv)):
            for e in np.nonzero(~ok_)[0][:4]:
                bad.append(f"row {i} {name}[{e}]: gpu {bf16_bits_to_f64(gb[e]):.8g} "
                           f"exact {ex[e]:.8g} rounding {bf16_bits_to_f64(O.bf16_round(ex[e:e+1])[0]):.8g} "
                           f"bound {bd[e]:.3g}")
            n_bad[name] += int((~ok_).sum())
        flips += fk + fv
        total += kr.size + v.size
    print(f"chunk layer-0 appends outside the bound: {n_bad}; largest deviation "
          f"{worst:.3g} of the bound")
    for line in bad[:24]:
        print("  " + line)
    assert not bad, f"appended K/V outside the rounding bound: {n_bad}"
    # decode rows with the shortest contexts, through all 32 layers
    model = O.Model(SHAPE, wc)
    rows = [int(r) for r in np.argsort(wl["ctx"])[:2]]
    tabs = [wl["tables"][1 + r] for r in rows]
    cached = [int(wl["ctx"][r]) for r in rows]
    pool, compact = oracle_pool(SHAPE, seed, tabs, cached, wl["bs"], [1] * len(rows))
    ref_lg, ref_tok = O.paged_step(model, pool, compact, cached, [1] * len(rows),
                                   [int(wl["dec_tokens"][0][r]) for r in rows], [1] * len(rows))
    ok, mx, row_err = compare_logits(g_lg[rows], ref_lg)
    res = resolvable_rows(ref_lg, row_err)
    print(f"mixed 8B step: decode rows (ctx {cached}) max abs logit error {mx:.2e}, "
          f"{int(res.sum())} decidable; chunk layer-0 K/V appends: {flips} of {total} "
          f"differ from the rounding of the exact value, all within the bound "
          f"(largest {worst:.3g} of it)")
    assert ok, f"max abs logit error {mx:.3g}"
    assert np.array_equal(g_tk[rows][res], ref_tok[res])

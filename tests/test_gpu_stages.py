"""Stage-by-stage GPU parity on one 8B-shaped layer: every activation the
step stores (QKV projection, rotated queries, attention output, FFN input,
SwiGLU output, residual stream, final-norm rows) against the oracle's pieces
applied to the oracle's own previous stage, as the largest difference over
the vector's rms (one bf16 ulp at that scale is ~2^-8). Where both sides
round nearly the same real number to bf16 they may differ by one ulp when it
sits near a rounding boundary; anything larger, or widespread, is a defect."""
import numpy as np
import pytest
import torch

import oracle as O
from continuous_batching_decode_forward_amd import binding as B
from continuous_batching_decode_forward_amd import configs, synth

from gpu_util import fill_pool, make_engine

pytestmark = pytest.mark.gpu

SHAPE = configs.LLAMA8B_1L


def stage_error(gpu_bf16: torch.Tensor, ref_u16: np.ndarray):
    """(max |gpu - oracle| / rms(oracle), fraction of elements that differ).
    One bf16 ulp at the vector's own scale is about 2^-8 = 0.0039."""
    g = O.bf16_to_f64(gpu_bf16).reshape(-1)
    o = O.bf16_to_f64(ref_u16).reshape(-1)
    rms = float(np.sqrt(np.mean(o * o))) or 1.0
    d = np.abs(g - o)
    return float(d.max() / rms), float((d > 0).mean())


def to_u16(x):
    return np.array([O.f64_to_bf16(v) for v in x], np.uint16)


@pytest.fixture(scope="module")
def big():
    wg = synth.make_weights(SHAPE, seed=0, device="cuda")
    wc = {k: ([t.cpu() for t in v] if isinstance(v, list) else v.cpu()) for k, v in wg.items()}
    return wg, wc


def test_every_stage_of_an_8b_layer_within_bf16_rounding(big):
    wg, wc = big
    Bn, bs, seed = 4, 32, 11
    ctx = synth.uniform_ints(seed, "ctx", Bn, 512, 4096)
    need = [-(-(int(c) + 1) // bs) for c in ctx]
    perm = synth.permutation(seed, "blocks", sum(need))
    mbps = -(-4097 // bs)
    tables = np.full((Bn, mbps), -1, np.int32)
    o = 0
    for i in range(Bn):
        tables[i, :need[i]] = perm[o:o + need[i]]
        o += need[i]
    tokens = synth.uniform_ints(seed, "tok", Bn, 0, SHAPE.vocab - 1)
    eng = make_engine(SHAPE, wg, block_size=bs, num_blocks=len(perm), max_blocks_per_seq=mbps,
                      max_rows=16, max_seqs=16, max_position=4097)
    fill_pool(eng, seed, perm)
    meta = eng.upload_step(slots=list(range(Bn)), block_tables=tables, ctx_lens=ctx,
                           n_new=[1] * Bn, tokens=tokens, want_token=[1] * Bn)
    tk = torch.empty(Bn, dtype=torch.int32, device="cuda")
    eng.step_forward(meta, None, tk)
    torch.cuda.synchronize()
    assert eng.status() == 0
    hq, hkv, hd, d, F = (SHAPE.n_heads, SHAPE.n_kv_heads, SHAPE.head_dim, SHAPE.d_model,
                         SHAPE.ffn_dim)
    qkv_n = (hq + 2 * hkv) * hd
    gpu = {name: eng.debug_buffer(which, Bn, width) for name, which, width in [
        ("qkv", B.CBD_BUF_QKV, qkv_n), ("q", B.CBD_BUF_Q, hq * hd),
        ("attn", B.CBD_BUF_ATTN, hq * hd), ("h2", B.CBD_BUF_H, d), ("a", B.CBD_BUF_FFN, F),
        ("x2", B.CBD_BUF_X, d), ("hf", B.CBD_BUF_LM_IN, d)]}
    eng.close()
    # a second engine whose down projection is zero leaves x1 (the residual
    # after attention) in the residual buffer
    wz = dict(wg)
    wz["w_down"] = [torch.zeros_like(t) for t in wg["w_down"]]
    eng = make_engine(SHAPE, wz, block_size=bs, num_blocks=len(perm), max_blocks_per_seq=mbps,
                      max_rows=16, max_seqs=16, max_position=4097)
    fill_pool(eng, seed, perm)
    meta = eng.upload_step(slots=list(range(Bn)), block_tables=tables, ctx_lens=ctx,
                           n_new=[1] * Bn, tokens=tokens, want_token=[1] * Bn)
    eng.step_forward(meta, None, tk)
    torch.cuda.synchronize()
    gpu["x1"] = eng.debug_buffer(B.CBD_BUF_X, Bn, d)
    eng.close()
    stats = {k: [] for k in gpu}
    for i in range(Bn):
        x0 = O.as_u16(wc["embed"][int(tokens[i])])
        h = O.rmsnorm(x0, wc["attn_norm"][0], SHAPE.rms_eps)
        qkv = to_u16(O.linear(h, wc["w_qkv"][0]))
        stats["qkv"].append(stage_error(gpu["qkv"][i], qkv))
        pos = int(ctx[i])
        q = np.concatenate([O.rope(qkv[j * hd:(j + 1) * hd], pos, SHAPE.rope_base)
                            for j in range(hq)])
        stats["q"].append(stage_error(gpu["q"][i], q))
        k_new = np.concatenate([O.rope(qkv[(hq + j) * hd:(hq + j + 1) * hd], pos, SHAPE.rope_base)
                                for j in range(hkv)]).reshape(1, hkv, hd)
        v_new = qkv[(hq + hkv) * hd:].reshape(1, hkv, hd)
        Kc = O.as_u16(synth.logical_kv(seed, 0, 0, tables[i], pos, hkv, bs, hd))
        Vc = O.as_u16(synth.logical_kv(seed, 0, 1, tables[i], pos, hkv, bs, hd))
        K = np.concatenate([Kc, k_new])
        V = np.concatenate([Vc, v_new])
        attn = O.attention_dense(q, K, V, hq, hkv, hd)
        stats["attn"].append(stage_error(gpu["attn"][i], attn))
        t = to_u16(O.linear(attn, wc["w_o"][0]))
        x1 = to_u16(O.bf16_to_f64(x0) + O.bf16_to_f64(t))
        stats["x1"].append(stage_error(gpu["x1"][i], x1))
        dx = np.nonzero(O.as_u16(gpu["x1"][i]) != x1)[0]
        if len(dx):
            print(f"row {i}: x1 differs at {len(dx)} columns, by 64-column tile:",
                  np.bincount(dx // 64, minlength=d // 64).nonzero()[0][:20])
        h2 = O.rmsnorm(x1, wc["ffn_norm"][0], SHAPE.rms_eps)
        stats["h2"].append(stage_error(gpu["h2"][i], h2))
        g = O.bf16_to_f64(to_u16(O.linear(h2, wc["w_gate"][0])))
        u = O.bf16_to_f64(to_u16(O.linear(h2, wc["w_up"][0])))
        a = to_u16(g / (1.0 + np.exp(-g)) * u)
        stats["a"].append(stage_error(gpu["a"][i], a))
        dn = to_u16(O.linear(a, wc["w_down"][0]))
        x2 = to_u16(O.bf16_to_f64(x1) + O.bf16_to_f64(dn))
        stats["x2"].append(stage_error(gpu["x2"][i], x2))
        hf = O.rmsnorm(x2, wc["final_norm"], SHAPE.rms_eps)
        stats["hf"].append(stage_error(gpu["hf"][i], hf))
    report = {k: (max(e for e, _ in v), max(f for _, f in v)) for k, v in stats.items()}
    print("stage: (max error / rms, fraction of elements differing)", report)
    for k, (err, frac) in report.items():
        assert err <= 2.0 ** -6, f"{k}: max error {err:.3g} of the rms"
        assert frac < 0.02, f"{k}: {frac:.3%} of elements differ"

"""Pins for the oracle's whole step.

* Batched equals serial, byte for byte (the Kestrel page, "0.8MB 跑通 Qwen"
  14-1, section 3: batched outputs were identical to serial ones; section 1:
  only the compute is merged, the per-request state stays separate).
* Invariance to the order of sequences in a step and to the block-table
  permutation (Go under the hood 20.3.2: paging is addressing only).
* The layer's composition, through special weight sets that reduce it to
  library routines (numpy float64 products) and to the separately pinned
  pieces.
"""
import numpy as np
import pytest
import torch

import oracle as O
from continuous_batching_decode_forward_amd import configs, synth

CFG = configs.TINY


@pytest.fixture(scope="module")
def tiny_model():
    return O.Model(CFG, synth.make_weights(CFG, seed=0))


def make_sequences(seed, n_seq=4, lo=5, hi=40):
    lens = synth.uniform_ints(seed, "ctx", n_seq, lo, hi)
    return [synth.uniform_ints(seed, f"prompt.{i}", int(lens[i]), 0, CFG.vocab - 1)
            for i in range(n_seq)]


def serial_run(model, prompt, n_decode):
    """Serial ground truth: logits after the prompt, then after each greedy
    token fed back, one token per forward."""
    kv = model.dense_kv(len(prompt) + n_decode + 1)
    out = [O.serial_forward(model, kv, prompt, 0, last_only=False)[-1]]
    pos = len(prompt)
    for _ in range(n_decode):
        t = O.argmax_f64(out[-1])
        out.append(O.serial_forward(model, kv, [t], pos))
        pos += 1
    return out


def paged_run(model, prompts, n_decode, block_perm, chunk=None, order=None, bs=4, nb=64):
    """The same sequences through paged-batched steps. The prompts are
    prefilled in chunks of `chunk` rows (all sequences' chunks share a step),
    then every sequence decodes one row per step. `order` permutes the
    sequences inside every step."""
    n = len(prompts)
    order = list(range(n)) if order is None else list(order)
    per_seq = nb // n
    tables = np.full((n, per_seq), -1, np.int32)
    for i in range(n):
        tables[i] = block_perm[i * per_seq:(i + 1) * per_seq]
    pool = model.paged_pool(nb, bs)
    ctx = [0] * n
    logits = [[] for _ in range(n)]
    chunk = chunk or max(len(p) for p in prompts)
    while any(ctx[i] < len(prompts[i]) for i in range(n)):
        seqs = [i for i in order if ctx[i] < len(prompts[i])]
        nn = [min(chunk, len(prompts[i]) - ctx[i]) for i in seqs]
        toks = np.concatenate([prompts[i][ctx[i]:ctx[i] + k] for i, k in zip(seqs, nn)])
        want = [int(ctx[i] + k == len(prompts[i])) for i, k in zip(seqs, nn)]
        lg, _ = O.paged_step(model, pool, tables[seqs], [ctx[i] for i in seqs], nn, toks, want)
        o = 0
        for i, k, w in zip(seqs, nn, want):
            ctx[i] += k
            if w:
                logits[i].append(lg[o])
                o += 1
    for _ in range(n_decode):
        toks = [O.argmax_f64(logits[i][-1]) for i in order]
        lg, g = O.paged_step(model, pool, tables[order], [ctx[i] for i in order], [1] * n,
                             toks, [1] * n)
        for o, i in enumerate(order):
            logits[i].append(lg[o])
            ctx[i] += 1
    return logits


def test_paged_batched_equals_serial_byte_for_byte(tiny_model):
    prompts = make_sequences(0)
    perm = synth.permutation(0, "blocks", 64)
    paged = paged_run(tiny_model, prompts, 20, perm)
    for i, p in enumerate(prompts):
        ser = serial_run(tiny_model, p, 20)
        assert len(ser) == len(paged[i]) == 21
        for step, (a, b) in enumerate(zip(ser, paged[i])):
            assert np.array_equal(a, b), f"seq {i} step {step}"


def test_chunking_order_and_block_permutation_change_nothing(tiny_model):
    prompts = make_sequences(1)
    ref = paged_run(tiny_model, prompts, 6, synth.permutation(1, "blocks", 64))
    alt = paged_run(tiny_model, prompts, 6, synth.permutation(2, "blocks", 64), chunk=7,
                    order=[2, 0, 3, 1])
    for i in range(len(prompts)):
        for a, b in zip(ref[i], alt[i]):
            assert np.array_equal(a, b)


def test_paged_step_rejects_bad_metadata(tiny_model):
    pool = tiny_model.paged_pool(8, 4)
    table = np.array([[0, 1]], np.int32)
    with pytest.raises(ValueError):      # ctx + n_new beyond the table
        O.paged_step(tiny_model, pool, table, [6], [3], [1, 2, 3], [1])
    with pytest.raises(ValueError):      # block id outside the pool
        O.paged_step(tiny_model, pool, np.array([[0, 9]], np.int32), [4], [1], [1], [1])
    with pytest.raises(ValueError):      # token outside the vocabulary
        O.paged_step(tiny_model, pool, table, [0], [1], [CFG.vocab], [1])


# --------------------------------------------------- layer composition pins

def one_layer(seed, zero=()):
    cfg = CFG.with_layers(1)
    w = synth.make_weights(cfg, seed)
    for k in zero:
        w[k] = [torch.zeros_like(t) for t in w[k]]
    return cfg, w


def lm(w, cfg, hf):
    """The LM head as a bf16 contraction: its input rounded to bf16 (nearest
    even), then a double product with the bf16 weights."""
    hb = O.bf16_to_f64(O.bf16_round(hf))
    return O.bf16_to_f64(w["lm_head"]).reshape(cfg.vocab, cfg.d_model) @ hb


def test_zero_projections_make_the_layer_identity():
    """W_o = 0 and W_down = 0: both residual branches add zero, so the logits
    are the LM head applied to the final norm of the token's embedding."""
    cfg, w = one_layer(3, zero=("w_o", "w_down"))
    m = O.Model(cfg, w)
    tok = 123
    lg = O.serial_forward(m, m.dense_kv(4), [tok], 0)
    h = O.rmsnorm(O.bf16_to_f64(w["embed"][tok]), w["final_norm"], cfg.rms_eps)
    assert np.allclose(lg, lm(w, cfg, h), rtol=0, atol=1e-12)


def test_ffn_branch_is_silu_gate_times_up_then_down():
    """With W_o = 0 only the FFN branch changes x; compare the logits with the
    branch built from numpy products and the pinned pieces. Swapping gate and
    up, or dropping the residual, fails this."""
    cfg, w = one_layer(4, zero=("w_o",))
    m = O.Model(cfg, w)
    tok = 77
    lg = O.serial_forward(m, m.dense_kv(4), [tok], 0)
    x = O.bf16_to_f64(w["embed"][tok])
    h = O.rmsnorm(x, w["ffn_norm"][0], cfg.rms_eps)
    g = O.bf16_to_f64(w["w_gate"][0]).reshape(cfg.ffn_dim, cfg.d_model) @ h
    u = O.bf16_to_f64(w["w_up"][0]).reshape(cfg.ffn_dim, cfg.d_model) @ h
    a = g / (1.0 + np.exp(-g)) * u
    down = O.bf16_to_f64(w["w_down"][0]).reshape(cfg.d_model, cfg.ffn_dim) @ a
    hf = O.rmsnorm(x + down, w["final_norm"], cfg.rms_eps)
    assert np.allclose(lg, lm(w, cfg, hf), rtol=0, atol=1e-9)
    # the swapped SwiGLU and the dropped residual give visibly different logits
    a_sw = u / (1.0 + np.exp(-u)) * g
    assert np.max(np.abs(a_sw - a)) > 1e-3
    no_res = lm(w, cfg, O.rmsnorm(down, w["final_norm"], cfg.rms_eps))
    assert np.max(np.abs(no_res - lg)) > 1e-2


def test_attention_branch_reads_the_cached_prefix():
    """With W_gate = 0 the FFN adds silu(0)*u = 0. Feed two tokens: the second
    token's attention must average over both positions; compare with the
    dense brute-force attention over the K/V the first forward cached."""
    cfg, w = one_layer(5, zero=("w_gate",))
    m = O.Model(cfg, w)
    kv = m.dense_kv(4)
    toks = [11, 2222]
    lg = O.serial_forward(m, kv, toks, 0, last_only=False)
    hq, hkv, hd = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    wqkv = O.bf16_to_f64(w["w_qkv"][0]).reshape(-1, cfg.d_model)
    x = O.bf16_to_f64(w["embed"][toks[1]])
    qkv = wqkv @ O.rmsnorm(x, w["attn_norm"][0], cfg.rms_eps)
    q = np.concatenate([O.rope(qkv[i * hd:(i + 1) * hd], 1, cfg.rope_base) for i in range(hq)])
    K = kv[0, 0, :2].copy()
    V = kv[0, 1, :2].copy()
    # the cached K of position 1 is this token's rotated k rounded to bf16,
    # its V the plain v rounded to bf16
    k1 = np.concatenate([O.rope(qkv[(hq + i) * hd:(hq + i + 1) * hd], 1, cfg.rope_base)
                         for i in range(hkv)])
    assert np.array_equal(K[1].reshape(-1), O.bf16_round(k1))
    assert np.array_equal(V[1].reshape(-1), O.bf16_round(qkv[(hq + hkv) * hd:]))
    # and position 0 holds token 0's, rotated by angle 0
    x0 = O.bf16_to_f64(w["embed"][toks[0]])
    qkv0 = wqkv @ O.rmsnorm(x0, w["attn_norm"][0], cfg.rms_eps)
    assert np.array_equal(K[0].reshape(-1), O.bf16_round(qkv0[hq * hd:(hq + hkv) * hd]))
    o = O.attention_dense(q, K, V, hq, hkv, hd)
    t = O.bf16_to_f64(w["w_o"][0]).reshape(cfg.d_model, hq * hd) @ o
    hf = O.rmsnorm(x + t, w["final_norm"], cfg.rms_eps)
    assert np.allclose(lg[1], lm(w, cfg, hf), rtol=0, atol=1e-9)


def test_layers_apply_in_order_with_their_own_weights():
    """A 2-layer model whose layer 1 (then layer 0) has zero output
    projections equals the 1-layer model made of the other layer alone."""
    cfg2 = CFG.with_layers(2)
    w = synth.make_weights(cfg2, 6)
    toks = [5, 900, 17]

    def run(cfg, weights):
        m = O.Model(cfg, weights)
        return O.serial_forward(m, m.dense_kv(8), toks, 0, last_only=False)

    for keep in (0, 1):
        wz = {k: (list(v) if isinstance(v, list) else v) for k, v in w.items()}
        for k in ("w_o", "w_down"):
            wz[k][1 - keep] = torch.zeros_like(wz[k][1 - keep])
        w1 = {k: ([v[keep]] if isinstance(v, list) else v) for k, v in w.items()}
        assert np.array_equal(run(cfg2, wz), run(CFG.with_layers(1), w1))


def test_in_step_greedy_takes_the_lowest_id_of_planted_ties():
    """Exact ties planted in the step's logits: a row of the LM head copied
    onto another id gives that id the same dot product, summed in the same
    order, so its logit equals the original's bit for bit. The step's greedy
    id must be the lowest id among the maxima of the binary32 logits, i.e.
    numpy's first-index argmax (the batched-equals-serial claim of the
    Kestrel page, "0.8MB 跑通 Qwen" 14-1 section 3, covers greedy ids).
    Copies land both above and below the original maximum, and on ids 0 and
    V - 1, so a highest-id rule (>=) or a first-row-only rule fails."""
    cfg = CFG.with_layers(1)
    w = synth.make_weights(cfg, seed=8)
    prompts = [synth.uniform_ints(8, f"tie.{i}", n, 0, cfg.vocab - 1)
               for i, n in enumerate((3, 7, 5, 2))]
    nn = [len(p) for p in prompts]
    toks = np.concatenate(prompts)
    tables = np.arange(16, dtype=np.int32).reshape(4, 4)

    def step(weights):
        m = O.Model(cfg, weights)
        return O.paged_step(m, m.paged_pool(16, 4), tables, [0] * 4, nn, toks, [1] * 4)

    lg, g = step(w)
    assert np.array_equal(g, np.argmax(lg.astype(np.float32), axis=1))
    best = [int(i) for i in np.argmax(lg, axis=1)]
    assert len(set(best)) == 4, "choose another seed: two rows share their maximum"
    V = cfg.vocab
    # partner ids: above, below, the first and the last id of the vocabulary
    partners = [best[0] + 1, best[1] - 1, 0, V - 1]
    taken = set(best)
    for r, j in enumerate(partners):
        while j in taken or not 0 <= j < V:
            j = (j + 17) % V
        partners[r] = j
        taken.add(j)
    wt = dict(w)
    lm_head = w["lm_head"].clone()
    for r, j in enumerate(partners):
        lm_head[j] = lm_head[best[r]]
    wt["lm_head"] = lm_head
    lg2, g2 = step(wt)
    for r, j in enumerate(partners):
        assert lg2[r, j] == lg2[r, best[r]] == lg[r, best[r]], f"row {r}: no exact tie"
        assert int(g2[r]) == min(j, best[r]), f"row {r}: ties must go to the lowest id"
    assert any(j > b for j, b in zip(partners, best)) and any(j < b for j, b in zip(partners, best))
    assert np.array_equal(g2, np.argmax(lg2.astype(np.float32), axis=1))

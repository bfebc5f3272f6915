"""Greedy ids on exactly tied logits, on the GPU: ties go to the lowest id.

The batched step must give the serial decode's greedy ids (the Kestrel page,
"0.8MB 跑通 Qwen" 14-1 section 3), and with ties that decision needs a fixed
rule; the rule here is the lowest id among the maxima. Random fp32 logits
almost never tie, so the ties are planted: on the 8B-shaped layer + LM head
(vocab 128256), the LM-head row of each step row's maximum is copied onto
other ids, which then compute the same dot product in the same order and tie
with the maximum bit for bit. The partner ids put the tie
  * in the same 16-column fragment (one above, one below the maximum),
  * across the 256-column workgroups of the stream path and the dense path's
    tiles (ids 255/256 and 511/512, the first and the last workgroup),
  * 16 and 256 columns away (other lanes, other waves),
and the step runs at 1, 8, 64 rows (the stream kernel's three row shapes)
and at 96 and 256 rows (the dense kernel). Every row's token must equal the
lowest id among its row maximum in the step's own logits, and the planted
ties must be present there (rows whose maximum is the same id share each
other's copies)."""
import numpy as np
import pytest
import torch

from continuous_batching_decode_forward_amd import configs, synth

from gpu_util import fill_pool, make_engine

pytestmark = pytest.mark.gpu

SHAPE = configs.LLAMA8B_1L
N_ROWS = 256
BS = 32


def _workload(seed):
    ctx = synth.uniform_ints(seed, "ctx", N_ROWS, 1, 200)
    need = [-(-(int(c) + 1) // BS) for c in ctx]
    perm = synth.permutation(seed, "blocks", int(sum(need)))
    mbps = max(need)
    tables = np.full((N_ROWS, mbps), -1, np.int32)
    o = 0
    for i in range(N_ROWS):
        tables[i, :need[i]] = perm[o:o + need[i]]
        o += need[i]
    tokens = synth.uniform_ints(seed, "tok", N_ROWS, 0, SHAPE.vocab - 1)
    return ctx, tables, perm, tokens, mbps


def _run(wg, wl, seed, batches):
    ctx, tables, perm, tokens, mbps = wl
    eng = make_engine(SHAPE, wg, block_size=BS, num_blocks=len(perm), max_blocks_per_seq=mbps,
                      max_rows=N_ROWS, max_seqs=N_ROWS, max_position=256)
    out = {}
    try:
        fill_pool(eng, seed, perm)
        for B in batches:
            meta = eng.upload_step(slots=list(range(B)), block_tables=tables[:B], ctx_lens=ctx[:B],
                                   n_new=[1] * B, tokens=tokens[:B], want_token=[1] * B)
            lg = torch.empty((B, SHAPE.vocab), dtype=torch.float32, device="cuda")
            tk = torch.full((B,), -1, dtype=torch.int32, device="cuda")
            eng.step_forward(meta, lg, tk)
            torch.cuda.synchronize()
            assert eng.status() == 0
            out[B] = (lg.cpu().numpy(), tk.cpu().numpy())
    finally:
        eng.close()
    return out


def _partners(best, V):
    """Planted tie ids per row (each id used once, never another row's
    maximum): boundary ids for the first rows, then offsets that put the
    copy in the same fragment, another lane group, another wave or another
    workgroup, above and below."""
    special = [255, 256, 511, 512, 0, V - 1, 16, 4095, 4096, V - 256]
    offsets = [1, -1, 16, -16, 256, -256, 3, -5, 1024, -4096]
    taken = set(int(b) for b in best)
    out = []
    for r, b in enumerate(best):
        want = [special[r]] if r < len(special) else [b + offsets[r % len(offsets)]]
        if r % 3 == 0:  # a three-way tie on some rows
            want.append(b + offsets[(r + 1) % len(offsets)])
        ids = []
        for j in want:
            while j in taken or not 0 <= j < V:
                j = (j + 7919) % V
            taken.add(j)
            ids.append(int(j))
        out.append(ids)
    return out


def test_greedy_ties_go_to_the_lowest_id_on_both_gemm_paths():
    torch.cuda.set_device(0)
    seed = 21
    batches = (1, 8, 64, 96, 256)
    wg = synth.make_weights(SHAPE, seed=seed, device="cuda")
    wl = _workload(seed)
    base = _run(wg, wl, seed, (N_ROWS,))
    lg0, tk0 = base[N_ROWS]
    best = np.argmax(lg0, axis=1)  # numpy: first index of the maximum
    assert np.array_equal(tk0, best)
    print(f"rows sharing their maximum's id with another row: "
          f"{N_ROWS - len(set(best.tolist()))} of {N_ROWS}")
    partners = _partners(best, SHAPE.vocab)
    lm = wg["lm_head"].clone()
    for r, ids in enumerate(partners):
        for j in ids:
            lm[j] = wg["lm_head"][int(best[r])]
    wt = dict(wg)
    wt["lm_head"] = lm
    runs = _run(wt, wl, seed, batches)
    # rows whose maximum sits on the same id share each other's copies
    tied = {}
    for r, ids in enumerate(partners):
        tied.setdefault(int(best[r]), {int(best[r])}).update(ids)
    planted_at_max = 0
    for B in batches:
        lg, tk = runs[B]
        expect = np.argmax(lg, axis=1)
        assert np.array_equal(tk, expect), \
            f"B={B}: rows {np.nonzero(tk != expect)[0][:8].tolist()} differ from the lowest-id maximum"
        for r in range(B):
            b = int(best[r])
            for j in partners[r]:
                assert lg[r, j] == lg[r, b], f"B={B} row {r}: ids {b} and {j} do not tie"
            if lg[r, b] == lg[r].max():
                planted_at_max += 1
                assert tk[r] == min(tied[b]), f"B={B} row {r}: {tk[r]} for ties at {sorted(tied[b])}"
    # nearly every row's planted tie is at its maximum (the logits of a row
    # may move by rounding between the stream and dense paths)
    assert planted_at_max >= 0.9 * sum(batches)
    print(f"planted ties at the row maximum: {planted_at_max} of {sum(batches)} rows")

"""Pins for the composer's reference model on the scaled-down constants of
the interactive figure in Go under the hood section 20.3.2 (4 slots,
4-position blocks, 8-token prefill chunks, at most 12 rows per step, 7
requests arriving one after another), driven by a fake model whose tokens
are a hash of (request, position).

What the section fixes: admission that reserves the answer's blocks lets
every admitted request finish; admission on a free slot alone can leave every
slot busy, the pool empty and no sequence able to grow; prefill chunks come
before decode rows; a sequence that does not fit waits and is never evicted.
"""
import pytest

from oracle.composer_ref import (FINISH_EOS, FINISH_LENGTH, FREE_SLOT, REQUEST_LEVEL,
                                 RESERVE, ComposerRef, ceil_div)

# (arrival step, prompt length, max_new); the figure's own values are not in
# the text, these are chosen so that four concurrent answers overflow the pool.
REQUESTS = [(0, 10, 30), (0, 14, 26), (1, 6, 34), (2, 16, 22), (3, 9, 28), (5, 12, 30),
            (6, 7, 31)]
POOL = 24


def fake_token(rid, pos, eos_at=None, n_generated=0):
    if eos_at is not None and n_generated + 1 == eos_at:
        return 0
    return 1 + (rid * 7919 + pos * 104729) % 997


def drive(policy, requests=REQUESTS, pool=POOL, eos=None, max_steps=400, block_order=None):
    c = ComposerRef(max_slots=4, block_size=4, num_blocks=pool, max_rows=12, chunk_size=8,
                    eos_id=0, policy=policy, block_order=block_order)
    eos = eos or {}
    ttft, done, trace = {}, {}, []
    pending = sorted(range(len(requests)), key=lambda i: requests[i][0])
    for step in range(max_steps):
        while pending and requests[pending[0]][0] <= step:
            i = pending.pop(0)
            _, plen, mx = requests[i]
            c.submit(i, [1 + (i * 31 + j) % 50 for j in range(plen)], mx)
        held_before = {r.request_id: list(r.blocks) for r in c.active.values()}
        p = c.plan()
        # no eviction: blocks held before the plan are still held, in order
        for r in c.active.values():
            if r.request_id in held_before:
                assert r.blocks[:len(held_before[r.request_id])] == held_before[r.request_id]
        held = sum(len(r.blocks) for r in c.active.values())
        assert held + len(c.free_blocks) == pool
        assert p.n_rows <= 12
        trace.append((step, p, held, len(c.free_blocks), len(c.active)))
        if p.stalled:
            return ttft, done, trace, c
        if not p.n_new:
            if not pending and not c.queue and not c.active:
                break
            c.commit([])
            continue
        # prefill chunks strictly before decode rows
        kinds = [ (p.n_new[i] > 1 or not p.want_token[i] or p.step_ids[i] == 0)
                  and p.ctx_lens[i] < requests[p.request_ids[i]][1] for i in range(len(p.slots))]
        assert kinds == sorted(kinds, reverse=True)
        toks = []
        for i, rid in enumerate(p.request_ids):
            if p.want_token[i]:
                pos = p.ctx_lens[i] + p.n_new[i] - 1
                toks.append(fake_token(rid, pos, eos.get(rid), p.step_ids[i]))
                if p.step_ids[i] == 0:
                    ttft[rid] = step - requests[rid][0]
        c.commit(toks)
        for rid, why, gen in c.finished:
            done.setdefault(rid, (step - requests[rid][0], why, len(gen)))
    return ttft, done, trace, c


def test_reservation_finishes_every_request():
    ttft, done, trace, c = drive(RESERVE)
    assert sorted(done) == list(range(len(REQUESTS)))
    for rid, (_, why, n) in done.items():
        assert why == FINISH_LENGTH and n == REQUESTS[rid][2]
    assert not any(t[1].stalled for t in trace)
    # reservation never over-commits: what admitted requests hold fits the pool
    for step, p, held, free, n_active in trace:
        assert held <= POOL


def test_free_slot_admission_exhausts_the_pool():
    _, done, trace, c = drive(FREE_SLOT)
    step, p, held, free, n_active = trace[-1]
    assert p.stalled
    assert n_active == 4 and free == 0
    for r in c.active.values():      # nobody can take one more position
        assert r.ctx + 1 > len(r.blocks) * 4 or r.prefilled < len(r.prompt)
    assert len(done) < len(REQUESTS)


def test_request_level_batching_delays_late_arrivals():
    ttft_cb, done_cb, _, _ = drive(RESERVE, pool=200)
    ttft_rl, done_rl, _, _ = drive(REQUEST_LEVEL, pool=200)
    assert sorted(done_rl) == sorted(done_cb) == list(range(len(REQUESTS)))
    late = [4, 5, 6]
    assert sum(ttft_rl[r] for r in late) > sum(ttft_cb[r] for r in late)


def test_eos_retires_early_and_frees_slot_and_blocks():
    ttft, done, trace, c = drive(RESERVE, eos={0: 3, 2: 1}, pool=200)
    assert done[0][1] == FINISH_EOS and done[0][2] == 3
    assert done[2][1] == FINISH_EOS and done[2][2] == 1
    assert len(c.free_blocks) == 200 and not c.active


def test_deferred_decode_rows_run_next_step():
    """Eight slots, a 6-row budget: decode rows that do not fit one step are
    the first candidates' complement, and every decoding sequence is served
    within two steps (lowest slots first, none dropped)."""
    c = ComposerRef(max_slots=8, block_size=4, num_blocks=200, max_rows=6, chunk_size=8,
                    eos_id=0, policy=RESERVE)
    for i in range(8):
        c.submit(i, [5], 20)
    served = []
    for step in range(12):
        p = c.plan()
        assert p.n_rows <= 6
        served.append(set(p.request_ids))
        c.commit([7] * sum(p.want_token))
    # after prefill, every sequence appears at least once in any two steps
    for a, b in zip(served[3:], served[4:]):
        assert a | b == set(range(8))


def test_block_order_is_fifo_from_the_given_permutation():
    order = [5, 3, 9, 0, 1, 2, 4, 6, 7, 8, 10, 11]
    c = ComposerRef(max_slots=2, block_size=4, num_blocks=12, max_rows=12, chunk_size=8,
                    eos_id=0, policy=RESERVE, block_order=order)
    c.submit(0, [1] * 5, 3)          # 8 positions -> 2 blocks
    c.submit(1, [1] * 9, 3)          # 12 positions -> 3 blocks
    p = c.plan()
    assert p.block_tables == [[5, 3], [9, 0, 1]]
    assert p.slots == [0, 1]
    assert ceil_div(9 + 3, 4) == 3

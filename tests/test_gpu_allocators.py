"""The engine's slot and block allocators through the C ABI (Go under the
hood 20.3.2: fixed-size KV blocks from one shared pool, taken at admission;
a request that does not fit waits, nothing is evicted). An engine needs
device buffers, so these run with the GPU tests; the allocators themselves
are host code and enqueue nothing but the slot reset."""
import numpy as np
import pytest
import torch

from continuous_batching_decode_forward_amd import binding as B
from continuous_batching_decode_forward_amd import configs, synth

from gpu_util import make_engine, weights_to

pytestmark = pytest.mark.gpu

N_BLOCKS = 10


@pytest.fixture(scope="module")
def eng():
    torch.cuda.set_device(0)
    w = weights_to(synth.make_weights(configs.TINY, seed=2), "cuda")
    order = synth.permutation(31, "blocks", N_BLOCKS).astype(np.int32)
    e = make_engine(configs.TINY, w, block_size=4, num_blocks=N_BLOCKS, max_blocks_per_seq=8,
                    max_rows=16, max_seqs=4, max_position=32, max_slots=3, block_order=order)
    yield e, [int(b) for b in order]
    e.close()


def test_block_alloc_is_fifo_all_or_nothing_and_free_appends(eng):
    e, order = eng
    h = e.handle
    assert B.cbd_blocks_available(h) == N_BLOCKS
    assert B.cbd_block_alloc(h, 0) == []
    a = B.cbd_block_alloc(h, 3)
    assert a == order[:3]                       # the front of the seeded order
    assert B.cbd_blocks_available(h) == 7
    with pytest.raises(B.CbdError) as ei:       # more than the pool holds: takes none
        B.cbd_block_alloc(h, 8)
    assert ei.value.code == B.CBD_E_NOBLOCKS
    assert B.cbd_blocks_available(h) == 7
    b = B.cbd_block_alloc(h, 2)
    assert b == order[3:5]                      # the failed call took nothing
    B.cbd_block_free(h, [a[1], a[0]])           # appended to the back, in the given order
    assert B.cbd_blocks_available(h) == 7
    rest = B.cbd_block_alloc(h, 7)
    assert rest == order[5:] + [a[1], a[0]]
    assert B.cbd_blocks_available(h) == 0
    with pytest.raises(B.CbdError) as ei:
        B.cbd_block_alloc(h, 1)
    assert ei.value.code == B.CBD_E_NOBLOCKS
    B.cbd_block_free(h, a[2:] + b + rest)
    assert B.cbd_blocks_available(h) == N_BLOCKS


def test_block_free_rejects_double_and_foreign_ids_and_frees_none(eng):
    e, order = eng
    h = e.handle
    ids = B.cbd_block_alloc(h, 2)
    B.cbd_block_free(h, [ids[0]])
    for bad in ([ids[1], ids[0]],                # ids[0] is already free: a double free
                [ids[1], N_BLOCKS],              # outside the pool
                [ids[1], -1]):
        with pytest.raises(B.CbdError) as ei:
            B.cbd_block_free(h, bad)
        assert ei.value.code == B.CBD_E_INVAL
        assert B.cbd_blocks_available(h) == N_BLOCKS - 1   # ids[1] is still allocated
    B.cbd_block_free(h, [ids[1]])
    assert B.cbd_blocks_available(h) == N_BLOCKS
    with pytest.raises(B.CbdError) as ei:
        B.cbd_block_alloc(h, -1)
    assert ei.value.code == B.CBD_E_INVAL
    # put the free list back in seeded order for the next test
    got = B.cbd_block_alloc(h, N_BLOCKS)
    B.cbd_block_free(h, sorted(got, key=order.index))


def test_slots_go_lowest_free_first_and_run_out(eng):
    e, _ = eng
    h = e.handle
    s = [B.cbd_slot_alloc(h, None, 100 + i) for i in range(3)]
    assert s == [0, 1, 2]
    with pytest.raises(B.CbdError) as ei:
        B.cbd_slot_alloc(h, None, 200)
    assert ei.value.code == B.CBD_E_NOSLOT
    B.cbd_slot_free(h, 1)
    assert B.cbd_slot_alloc(h, None, 201) == 1
    with pytest.raises(B.CbdError) as ei:
        B.cbd_slot_free(h, 7)
    assert ei.value.code == B.CBD_E_INVAL
    for x in (0, 1, 2):
        B.cbd_slot_free(h, x)
    with pytest.raises(B.CbdError) as ei:        # already free
        B.cbd_slot_free(h, 0)
    assert ei.value.code == B.CBD_E_INVAL
    torch.cuda.synchronize()


def test_composer_rejects_an_engine_it_could_overrun(eng):
    e, _ = eng
    c = B.cbd_sched_config()
    c.max_slots, c.block_size, c.num_blocks = 3, 4, N_BLOCKS
    c.max_blocks_per_seq, c.max_rows, c.chunk_size, c.eos_id, c.policy = 8, 16, 8, 0, 0
    s = B.cbd_sched_create(c, e.handle)
    B.cbd_sched_destroy(s)
    for field, value in (("max_slots", 4),            # above the engine's slots and sequences
                         ("max_blocks_per_seq", 9),   # past the engine's table
                         ("max_rows", 17), ("block_size", 8), ("num_blocks", 9)):
        bad = B.cbd_sched_config()
        for k, _ in B.cbd_sched_config._fields_:
            setattr(bad, k, getattr(c, k))
        setattr(bad, field, value)
        with pytest.raises(B.CbdError) as ei:
            B.cbd_sched_create(bad, e.handle)
        assert ei.value.code == B.CBD_E_INVAL, field


def test_slot_alloc_checks_the_forbidden_ids(eng):
    e, _ = eng
    h = e.handle
    for n, ids in ((9, [1] * 8), (1, [configs.TINY.vocab]), (2, [3, -1]), (-1, [])):
        c = B.cbd_sampling()
        c.temperature, c.top_p, c.penalty_decay = 1.0, 1.0, 1.0
        c.n_forbidden = n
        for i, t in enumerate(ids[:8]):
            c.forbidden[i] = t
        with pytest.raises(B.CbdError) as ei:
            B.cbd_slot_alloc(h, c, 1)
        assert ei.value.code == B.CBD_E_INVAL
    c = B.cbd_sampling()
    c.temperature, c.top_p, c.penalty_decay, c.n_forbidden = 1.0, 1.0, 1.0, 8
    for i in range(8):
        c.forbidden[i] = configs.TINY.vocab - 1 - i
    s = B.cbd_slot_alloc(h, c, 2)
    B.cbd_slot_free(h, s)
    torch.cuda.synchronize()

"""The C-ABI library loads without a GPU and exports every function that
include/cbd.h declares; host-side argument checks and size queries work."""
import ctypes as C
import os
import re

import pytest

from continuous_batching_decode_forward_amd import binding as B
from continuous_batching_decode_forward_amd import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "cbd.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(cbd_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported_and_bound():
    L = B.lib()
    names = declared_functions()
    assert len(names) >= 20
    bound = {n for n, _, _ in B.SIGNATURES}
    for n in names:
        assert hasattr(L, n), f"{n} not exported"
        assert n in bound, f"{n} has no binding"


def make_cfg(shape=configs.LLAMA8B_1L, **kw):
    c = B.cbd_config()
    c.n_layers, c.d_model, c.n_heads = shape.n_layers, shape.d_model, shape.n_heads
    c.n_kv_heads, c.head_dim, c.ffn_dim, c.vocab = (shape.n_kv_heads, shape.head_dim,
                                                    shape.ffn_dim, shape.vocab)
    c.block_size, c.num_blocks, c.max_blocks_per_seq = 32, 1000, 129
    c.max_slots, c.max_rows, c.max_seqs, c.max_position = 64, 64, 64, 4200
    c.rms_eps, c.rope_base = 1e-5, 10000.0
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_size_queries_follow_the_documented_layout():
    c = make_cfg()
    kv = B.cbd_kv_pool_bytes(c)
    assert kv == 1 * 2 * 1000 * 8 * 32 * 128 * 2
    assert B.cbd_slot_state_bytes(c) >= 64 * 128256 * 4
    assert B.cbd_workspace_bytes(c) > 64 * 4096 * 2


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 96, B.CBD_E_UNSUPPORTED), ("block_size", 12, B.CBD_E_UNSUPPORTED),
    ("n_kv_heads", 3, B.CBD_E_INVAL), ("n_kv_heads", 1, B.CBD_E_UNSUPPORTED),
    ("d_model", 4100, B.CBD_E_UNSUPPORTED), ("num_blocks", 0, B.CBD_E_INVAL),
    ("max_seqs", 65, B.CBD_E_INVAL)])
def test_config_errors(field, value, code):
    c = make_cfg(**{field: value})
    with pytest.raises(B.CbdError) as ei:
        B.cbd_workspace_bytes(c)
    assert ei.value.code == code
    assert B.cbd_last_error()


def test_engine_create_rejects_null_buffers():
    c = make_cfg()
    w = B.cbd_weights()
    h = C.c_void_p()
    rc = B.lib().cbd_engine_create(C.byref(c), C.byref(w), None, None, None, None, None, None,
                                   C.byref(h))
    assert rc == B.CBD_E_INVAL


def test_step_rejects_null_engine():
    st = B.cbd_step()
    assert B.lib().cbd_step_forward(None, C.byref(st), None, None, None) == B.CBD_E_INVAL


@pytest.mark.parametrize("buf,nbytes,out,blocks", [(None, 16, 256, 1), (256, 16, None, 1),
                                                  (256, 16, 256, 0), (264, 16, 256, 1),
                                                  (256, 24, 256, 1)])
def test_read_probe_rejects_bad_arguments(buf, nbytes, out, blocks):
    """NULL pointers, no workgroups, a buffer not 16-byte aligned or a size
    not a multiple of 16: refused before any launch (no device memory is
    touched, the addresses are never dereferenced)."""
    rc = B.lib().cbd_read_probe(buf, nbytes, out, blocks, None)
    assert rc == B.CBD_E_INVAL


@pytest.mark.parametrize("rows,width", [(37, 688), (16, 256), (1, 4096), (560, 128)])
def test_operand_tile_layout_reader_inverts_the_documented_layout(rows, width):
    # The layout cbd.h documents for "tiled" split planes: element (r, k) at
    # ((r / 16 * KB + k / 32) * 64 + (k / 8 % 4) * 16 + r % 16) * 8 + k % 8.
    import numpy as np
    from continuous_batching_decode_forward_amd.engine import untile_plane
    r16, w32 = -(-rows // 16) * 16, -(-width // 32) * 32
    kb = w32 // 32
    vals = np.arange(rows * width, dtype=np.float64).reshape(rows, width) + 1.0
    flat = np.zeros(r16 * w32)
    for r in range(rows):
        for k in range(width):
            at = ((r // 16 * kb + k // 32) * 64 + (k // 8 % 4) * 16 + r % 16) * 8 + k % 8
            assert flat[at] == 0.0
            flat[at] = vals[r, k]
    assert np.array_equal(untile_plane(flat, rows, width), vals)

"""ctypes binding of libcbd.so: the C ABI declared in include/cbd.h, under the
same names, with argument marshalling only. Every computation runs in the
library's HIP kernels; there is no fallback path. If the library has not been
built this module raises on import of the library (call build() first)."""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcbd.so")

CBD_OK = 0
CBD_E_INVAL = -1
CBD_E_NOSLOT = -2
CBD_E_NOBLOCKS = -3
CBD_E_UNSUPPORTED = -4
CBD_E_DEVICE = -5
ERROR_NAMES = {-1: "CBD_E_INVAL", -2: "CBD_E_NOSLOT", -3: "CBD_E_NOBLOCKS",
               -4: "CBD_E_UNSUPPORTED", -5: "CBD_E_DEVICE"}

CBD_STATUS_BAD_BLOCK = 0x1
CBD_STATUS_BAD_TOKEN = 0x2
CBD_STATUS_BAD_SLOT = 0x4
CBD_STATUS_BAD_SHAPE = 0x8

CBD_KV_BF16 = 0
CBD_KV_FP8_E4M3 = 1
CBD_W_BF16 = 0
CBD_W_INT8 = 1

CBD_GRAPH_CACHE = 16

CBD_MODE_GREEDY = 0
CBD_MODE_SAMPLE = 1

CBD_ADMIT_RESERVE = 0
CBD_ADMIT_FREE_SLOT = 1
CBD_ADMIT_REQUEST_LEVEL = 2

CBD_PACE_PREFILL_FIRST = 0
CBD_PACE_ALBATROSS = 1
CBD_PACE_SEPARATE = 2

CBD_KERNEL_QKV = 1
CBD_KERNEL_ROPE = 2
CBD_KERNEL_ATTN = 3
CBD_KERNEL_O = 4
CBD_KERNEL_GATEUP = 5
CBD_KERNEL_DOWN = 6
CBD_KERNEL_LM_HEAD = 7
CBD_KERNEL_SAMPLE = 8
CBD_KERNEL_NORM = 9

CBD_BUF_X = 1
CBD_BUF_H = 2
CBD_BUF_QKV = 3
CBD_BUF_Q = 4
CBD_BUF_ATTN = 5
CBD_BUF_FFN = 6
CBD_BUF_LM_IN = 7

CBD_FINISH_EOS = 1
CBD_FINISH_LENGTH = 2
CBD_FINISH_ABORT = 3

I32P = C.POINTER(C.c_int32)
U64P = C.POINTER(C.c_uint64)
VP = C.c_void_p


class CbdError(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        super().__init__(f"{where}: {ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code


class cbd_config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn_dim", C.c_int32),
                ("vocab", C.c_int32), ("block_size", C.c_int32), ("num_blocks", C.c_int32),
                ("max_blocks_per_seq", C.c_int32), ("max_slots", C.c_int32),
                ("max_rows", C.c_int32), ("max_seqs", C.c_int32), ("max_position", C.c_int32),
                ("rms_eps", C.c_float), ("pad0_", C.c_float), ("rope_base", C.c_double),
                ("kv_dtype", C.c_int32), ("k_scale", C.c_float), ("v_scale", C.c_float),
                ("weight_dtype", C.c_int32)]


class cbd_weights(C.Structure):
    _fields_ = [("embed", VP), ("final_norm", VP), ("lm_head", VP),
                ("attn_norm", C.POINTER(VP)), ("w_qkv", C.POINTER(VP)), ("w_o", C.POINTER(VP)),
                ("ffn_norm", C.POINTER(VP)), ("w_gate", C.POINTER(VP)), ("w_up", C.POINTER(VP)),
                ("w_down", C.POINTER(VP)),
                ("lm_head_scale", VP), ("s_qkv", C.POINTER(VP)), ("s_o", C.POINTER(VP)),
                ("s_gate", C.POINTER(VP)), ("s_up", C.POINTER(VP)), ("s_down", C.POINTER(VP))]


CBD_MAX_FORBIDDEN = 8


class cbd_sampling(C.Structure):
    _fields_ = [("temperature", C.c_float), ("top_p", C.c_float), ("top_k", C.c_int32),
                ("freq_penalty", C.c_float), ("presence_penalty", C.c_float),
                ("penalty_decay", C.c_float), ("seed", C.c_uint64),
                ("n_forbidden", C.c_int32), ("forbidden", C.c_int32 * CBD_MAX_FORBIDDEN)]

    @classmethod
    def from_params(cls, sp) -> "cbd_sampling":
        """From any object with the fields' names (forbidden: a sequence)."""
        c = cls()
        c.temperature, c.top_p, c.top_k = sp.temperature, sp.top_p, sp.top_k
        c.freq_penalty, c.presence_penalty = sp.freq_penalty, sp.presence_penalty
        c.penalty_decay, c.seed = sp.penalty_decay, sp.seed
        ids = list(getattr(sp, "forbidden", ()))
        c.n_forbidden = len(ids)
        for i, t in enumerate(ids):
            c.forbidden[i] = int(t)
        return c


class cbd_step(C.Structure):
    _fields_ = [("n_seqs", C.c_int32), ("n_rows", C.c_int32), ("n_out", C.c_int32),
                ("max_ctx", C.c_int32), ("max_blocks_per_seq", C.c_int32), ("mode", C.c_int32),
                ("slots", VP), ("block_tables", VP), ("ctx_lens", VP), ("n_new", VP),
                ("tokens", VP), ("want_token", VP), ("step_ids", VP)]


class cbd_sched_config(C.Structure):
    _fields_ = [("max_slots", C.c_int32), ("block_size", C.c_int32), ("num_blocks", C.c_int32),
                ("max_blocks_per_seq", C.c_int32), ("max_rows", C.c_int32),
                ("chunk_size", C.c_int32), ("eos_id", C.c_int32), ("policy", C.c_int32),
                ("pacing", C.c_int32), ("max_prefill", C.c_int32),
                ("decode_prefill_ratio", C.c_int32), ("min_forward_seq_len", C.c_int32),
                ("ctx_round", C.c_int32), ("graph_decode", C.c_int32)]


class cbd_plan(C.Structure):
    _fields_ = [("n_seqs", C.c_int32), ("n_rows", C.c_int32), ("n_out", C.c_int32),
                ("max_ctx", C.c_int32), ("max_blocks_per_seq", C.c_int32),
                ("n_prefill_rows", C.c_int32), ("n_decode_rows", C.c_int32),
                ("stalled", C.c_int32),
                ("slots", I32P), ("block_tables", I32P), ("ctx_lens", I32P), ("n_new", I32P),
                ("tokens", I32P), ("want_token", I32P), ("step_ids", I32P),
                ("request_ids", U64P)]


class cbd_sched_stats(C.Structure):
    _fields_ = [("queued", C.c_int32), ("active", C.c_int32), ("free_slots", C.c_int32),
                ("free_blocks", C.c_int32), ("steps", C.c_int64), ("finished", C.c_int64)]


# (name, restype, argtypes) for every exported symbol of include/cbd.h
SIGNATURES = [
    ("cbd_kv_pool_bytes", C.c_int, [C.POINTER(cbd_config), C.POINTER(C.c_size_t)]),
    ("cbd_slot_state_bytes", C.c_int, [C.POINTER(cbd_config), C.POINTER(C.c_size_t)]),
    ("cbd_workspace_bytes", C.c_int, [C.POINTER(cbd_config), C.POINTER(C.c_size_t)]),
    ("cbd_packed_weights_bytes", C.c_int, [C.POINTER(cbd_config), C.POINTER(C.c_size_t)]),
    ("cbd_engine_create", C.c_int, [C.POINTER(cbd_config), C.POINTER(cbd_weights), VP, VP, VP,
                                    VP, I32P, VP, C.POINTER(VP)]),
    ("cbd_engine_destroy", C.c_int, [VP]),
    ("cbd_slot_alloc", C.c_int, [VP, C.POINTER(cbd_sampling), C.c_uint64, I32P]),
    ("cbd_slot_free", C.c_int, [VP, C.c_int32]),
    ("cbd_block_alloc", C.c_int, [VP, C.c_int32, I32P]),
    ("cbd_block_free", C.c_int, [VP, C.c_int32, I32P]),
    ("cbd_blocks_available", C.c_int, [VP]),
    ("cbd_step_forward", C.c_int, [VP, C.POINTER(cbd_step), VP, VP, VP]),
    ("cbd_step_forward_graph", C.c_int, [VP, C.POINTER(cbd_step), VP, VP, VP]),
    ("cbd_graph_stats", C.c_int, [VP, C.POINTER(C.c_int64)]),
    ("cbd_read_probe", C.c_int, [VP, C.c_size_t, VP, C.c_int32, VP]),
    ("cbd_sample_logits", C.c_int, [VP, VP, C.c_int32, VP, VP, VP, VP]),
    ("cbd_sample_logits_noalloc", C.c_int, [VP, VP, C.c_int32, VP, VP, VP, VP]),
    ("cbd_engine_status", C.c_int, [VP, VP, C.POINTER(C.c_uint32)]),
    ("cbd_last_error", C.c_char_p, []),
    ("cbd_debug_buffer", C.c_int, [VP, C.c_int32, C.POINTER(VP), C.POINTER(C.c_size_t)]),
    ("cbd_profile_begin", C.c_int, [VP, C.c_int32]),
    ("cbd_profile_end", C.c_int, [VP, C.POINTER(C.c_double), I32P]),
    ("cbd_sched_create", C.c_int, [C.POINTER(cbd_sched_config), VP, I32P, C.POINTER(VP)]),
    ("cbd_sched_destroy", C.c_int, [VP]),
    ("cbd_sched_submit", C.c_int, [VP, I32P, C.c_int32, C.c_int32, C.POINTER(cbd_sampling),
                                   C.c_uint64]),
    ("cbd_sched_plan", C.c_int, [VP, C.POINTER(cbd_plan)]),
    ("cbd_sched_commit", C.c_int, [VP, I32P, C.c_int32]),
    ("cbd_sched_abort", C.c_int, [VP, C.c_uint64]),
    ("cbd_sched_pop_finished", C.c_int, [VP, U64P, I32P, I32P]),
    ("cbd_sched_stats_get", C.c_int, [VP, C.POINTER(cbd_sched_stats)]),
    ("cbd_sched_meta_ints", C.c_int, [C.POINTER(cbd_sched_config), C.POINTER(C.c_size_t)]),
    ("cbd_sched_step", C.c_int, [VP, C.c_int32, VP, VP, VP, VP, VP, C.POINTER(cbd_plan)]),
]

_lib = None


def lib():
    """The loaded libcbd.so. Raises if it has not been built: there is no
    other implementation to fall back to."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m continuous_batching_decode_forward_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(rc: int, where: str) -> int:
    if rc < 0:
        raise CbdError(rc, where, lib().cbd_last_error().decode())
    return rc


def _call(name, *args):
    return _check(getattr(lib(), name)(*args), name)


# ------------------------------------------------------- same-name wrappers

def cbd_kv_pool_bytes(cfg: cbd_config) -> int:
    n = C.c_size_t()
    _call("cbd_kv_pool_bytes", C.byref(cfg), C.byref(n))
    return n.value


def cbd_slot_state_bytes(cfg: cbd_config) -> int:
    n = C.c_size_t()
    _call("cbd_slot_state_bytes", C.byref(cfg), C.byref(n))
    return n.value


def cbd_workspace_bytes(cfg: cbd_config) -> int:
    n = C.c_size_t()
    _call("cbd_workspace_bytes", C.byref(cfg), C.byref(n))
    return n.value


def cbd_packed_weights_bytes(cfg: cbd_config) -> int:
    n = C.c_size_t()
    _call("cbd_packed_weights_bytes", C.byref(cfg), C.byref(n))
    return n.value


def cbd_engine_create(cfg, weights, packed, kv_pool, slot_state, workspace, block_order,
                      stream) -> int:
    h = VP()
    order = None
    if block_order is not None:
        order = (C.c_int32 * len(block_order))(*[int(b) for b in block_order])
    _call("cbd_engine_create", C.byref(cfg), C.byref(weights), packed, kv_pool, slot_state,
          workspace,
          C.cast(order, I32P) if order is not None else None, stream, C.byref(h))
    return h.value


def cbd_engine_destroy(engine) -> None:
    _call("cbd_engine_destroy", engine)


def cbd_slot_alloc(engine, params, request_id: int) -> int:
    s = C.c_int32()
    _call("cbd_slot_alloc", engine, C.byref(params) if params is not None else None,
          int(request_id), C.byref(s))
    return s.value


def cbd_slot_free(engine, slot: int) -> None:
    _call("cbd_slot_free", engine, int(slot))


def cbd_block_alloc(engine, n: int) -> list:
    buf = (C.c_int32 * max(n, 1))()
    _call("cbd_block_alloc", engine, int(n), buf)
    return list(buf[:n])


def cbd_block_free(engine, ids) -> None:
    buf = (C.c_int32 * max(len(ids), 1))(*[int(i) for i in ids])
    _call("cbd_block_free", engine, len(ids), buf)


def cbd_blocks_available(engine) -> int:
    return _call("cbd_blocks_available", engine)


def cbd_step_forward(engine, step: cbd_step, logits_out, tokens_out, stream) -> None:
    _call("cbd_step_forward", engine, C.byref(step), logits_out, tokens_out, stream)


def cbd_step_forward_graph(engine, step: cbd_step, logits_out, tokens_out, stream) -> None:
    _call("cbd_step_forward_graph", engine, C.byref(step), logits_out, tokens_out, stream)


def cbd_read_probe(buf, nbytes: int, out, blocks: int, stream) -> None:
    _call("cbd_read_probe", buf, int(nbytes), out, int(blocks), stream)


def cbd_graph_stats(engine) -> tuple:
    """(graphs recorded, graphs replayed, graphs cached)."""
    out = (C.c_int64 * 3)()
    _call("cbd_graph_stats", engine, out)
    return tuple(int(v) for v in out)


def cbd_sample_logits(engine, logits, n: int, slots, step_ids, tokens_out, stream) -> None:
    _call("cbd_sample_logits", engine, logits, int(n), slots, step_ids, tokens_out, stream)


def cbd_sample_logits_noalloc(engine, logits, n: int, slots, step_ids, tokens_out,
                              stream) -> None:
    _call("cbd_sample_logits_noalloc", engine, logits, int(n), slots, step_ids, tokens_out,
          stream)


def cbd_engine_status(engine, stream) -> int:
    f = C.c_uint32()
    _call("cbd_engine_status", engine, stream, C.byref(f))
    return f.value


def cbd_last_error() -> str:
    return lib().cbd_last_error().decode()


def cbd_debug_buffer(engine, which: int):
    p, n = VP(), C.c_size_t()
    _call("cbd_debug_buffer", engine, int(which), C.byref(p), C.byref(n))
    return p.value, n.value


def cbd_profile_begin(engine, kernel_class: int) -> None:
    _call("cbd_profile_begin", engine, int(kernel_class))


def cbd_profile_end(engine):
    ms, n = C.c_double(), C.c_int32()
    _call("cbd_profile_end", engine, C.byref(ms), C.byref(n))
    return ms.value, n.value


def cbd_sched_create(cfg: cbd_sched_config, engine=None, block_order=None) -> int:
    h = VP()
    order = None
    if block_order is not None:
        order = (C.c_int32 * len(block_order))(*[int(b) for b in block_order])
    _call("cbd_sched_create", C.byref(cfg), engine,
          C.cast(order, I32P) if order is not None else None, C.byref(h))
    return h.value


def cbd_sched_destroy(sched) -> None:
    _call("cbd_sched_destroy", sched)


def cbd_sched_submit(sched, prompt, max_new: int, params, request_id: int) -> None:
    buf = (C.c_int32 * max(len(prompt), 1))(*[int(t) for t in prompt])
    _call("cbd_sched_submit", sched, buf, len(prompt), int(max_new),
          C.byref(params) if params is not None else None, int(request_id))


def cbd_sched_plan(sched) -> cbd_plan:
    p = cbd_plan()
    _call("cbd_sched_plan", sched, C.byref(p))
    return p


def cbd_sched_commit(sched, tokens) -> None:
    buf = (C.c_int32 * max(len(tokens), 1))(*[int(t) for t in tokens])
    _call("cbd_sched_commit", sched, buf, len(tokens))


def cbd_sched_abort(sched, request_id: int) -> None:
    _call("cbd_sched_abort", sched, int(request_id))


def cbd_sched_pop_finished(sched):
    rid, why, n = C.c_uint64(), C.c_int32(), C.c_int32()
    got = _call("cbd_sched_pop_finished", sched, C.byref(rid), C.byref(why), C.byref(n))
    return (rid.value, why.value, n.value) if got else None


def cbd_sched_stats_get(sched) -> cbd_sched_stats:
    s = cbd_sched_stats()
    _call("cbd_sched_stats_get", sched, C.byref(s))
    return s


def cbd_sched_meta_ints(cfg: cbd_sched_config) -> int:
    n = C.c_size_t()
    _call("cbd_sched_meta_ints", C.byref(cfg), C.byref(n))
    return n.value


def cbd_sched_step(sched, mode: int, meta_dev, host_stage, tokens_dev, logits_out,
                   stream) -> cbd_plan:
    """Pointers are integers or None (device / host addresses)."""
    p = cbd_plan()
    _call("cbd_sched_step", sched, int(mode), meta_dev, host_stage, tokens_dev, logits_out,
          stream, C.byref(p))
    return p

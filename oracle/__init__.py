"""CPU oracle for the continuous-batching decode forward step (ctypes wrapper).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg import this package. The product path never does, and this
package imports nothing from the product.

The arithmetic lives in oracle.c (plain C loops, double activations and
accumulation; bf16 only for the weights and the KV cache); composer_ref.py
holds the scheduling policy as a plain Python simulation.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (fp contraction off, OpenMP on)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math",
                               "-fopenmp", "-fPIC", "-shared", "-std=c11", SRC,
                               "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = C.CDLL(build())
        _declare(_lib)
    return _lib


U16P = C.POINTER(C.c_uint16)
I32P = C.POINTER(C.c_int32)
F64P = C.POINTER(C.c_double)
F32P = C.POINTER(C.c_float)
U64P = C.POINTER(C.c_uint64)


class OrModel(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn_dim", C.c_int32),
                ("vocab", C.c_int32), ("kv_fp8", C.c_int32),
                ("rms_eps", C.c_double), ("rope_base", C.c_double),
                ("embed", U16P), ("final_norm", U16P), ("lm_head", U16P),
                ("attn_norm", C.POINTER(U16P)), ("w_qkv", C.POINTER(U16P)),
                ("w_o", C.POINTER(U16P)), ("ffn_norm", C.POINTER(U16P)),
                ("w_gate", C.POINTER(U16P)), ("w_up", C.POINTER(U16P)),
                ("w_down", C.POINTER(U16P)),
                ("k_scale", C.c_double), ("v_scale", C.c_double),
                ("w_int8", C.c_int32), ("pad_", C.c_int32), ("lm_head_scale", F32P),
                ("s_qkv", C.POINTER(F32P)), ("s_o", C.POINTER(F32P)),
                ("s_gate", C.POINTER(F32P)), ("s_up", C.POINTER(F32P)),
                ("s_down", C.POINTER(F32P))]


class OrSampling(C.Structure):
    _fields_ = [("temperature", C.c_float), ("top_p", C.c_float), ("top_k", C.c_int32),
                ("freq_penalty", C.c_float), ("presence_penalty", C.c_float),
                ("penalty_decay", C.c_float), ("seed", C.c_uint64),
                ("n_forbidden", C.c_int32), ("forbidden", C.c_int32 * 8)]


class OrSampleInfo(C.Structure):
    _fields_ = [("token", C.c_int32), ("n_kept", C.c_int32), ("sum_all", C.c_float),
                ("sum_topk", C.c_float), ("target", C.c_float), ("cum_before", C.c_float),
                ("cum_after", C.c_float), ("sum_kept", C.c_float), ("r", C.c_float),
                ("cdf_lo", C.c_float), ("cdf_hi", C.c_float), ("p1", C.c_float),
                ("p2", C.c_float), ("u", C.c_float), ("n_cut", C.c_int32),
                ("n_before", C.c_int32)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


def _declare(L):
    L.or_bf16_to_f64.argtypes = [C.c_uint16]
    L.or_bf16_to_f64.restype = C.c_double
    L.or_f64_to_bf16.argtypes = [C.c_double]
    L.or_f64_to_bf16.restype = C.c_uint16
    L.or_rmsnorm.argtypes = [F64P, U16P, C.c_int32, C.c_double, F64P]
    L.or_linear.argtypes = [F64P, C.c_int32, U16P, C.c_int32, F64P]
    L.or_linear_i8.argtypes = [F64P, C.c_int32, C.c_void_p, F32P, C.c_int32, F64P]
    L.or_rope.argtypes = [F64P, C.c_int32, C.c_int32, C.c_double]
    L.or_attention_dense.argtypes = [F64P, U16P, U16P, C.c_int32, C.c_int32, C.c_int32,
                                     C.c_int32, F64P]
    L.or_attention_dense_kv.argtypes = [F64P, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32,
                                        C.c_int32, C.c_int32, C.c_int32, C.c_double,
                                        C.c_double, F64P]
    L.or_serial_forward.argtypes = [C.POINTER(OrModel), C.c_void_p, C.c_int32, I32P, C.c_int32,
                                    C.c_int32, C.c_int32, F64P]
    L.or_paged_step.argtypes = [C.POINTER(OrModel), C.c_void_p, C.c_int32, C.c_int32, C.c_int32,
                                I32P, C.c_int32, I32P, I32P, I32P, I32P, F64P, I32P]
    L.or_e4m3_to_f64.argtypes = [C.c_uint8]
    L.or_e4m3_to_f64.restype = C.c_double
    L.or_f64_to_e4m3.argtypes = [C.c_double]
    L.or_f64_to_e4m3.restype = C.c_uint8
    L.or_argmax_f32.argtypes = [F32P, C.c_int32]
    L.or_argmax_f32.restype = C.c_int32
    L.or_argmax_f64.argtypes = [F64P, C.c_int32]
    L.or_argmax_f64.restype = C.c_int32
    L.or_philox4x64_10.argtypes = [U64P, U64P, U64P]
    L.or_uniform24.argtypes = [C.c_uint64, C.c_uint64, C.c_uint32]
    L.or_uniform24.restype = C.c_float
    L.or_sample_f32.argtypes = [F32P, C.c_int32, F32P, C.POINTER(OrSampling), C.c_uint64,
                                C.c_uint32, C.POINTER(OrSampleInfo)]
    L.or_sample_f32.restype = C.c_int32
    L.or_num_threads.restype = C.c_int32
    L.or_set_num_threads.argtypes = [C.c_int32]


def _p(a: np.ndarray, t):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(t)


def as_u16(t) -> np.ndarray:
    """bf16 torch tensor or uint16 array -> contiguous uint16 numpy array."""
    if isinstance(t, np.ndarray):
        return np.ascontiguousarray(t.view(np.uint16))
    import torch
    return np.ascontiguousarray(t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))


def bf16_to_f64(a) -> np.ndarray:
    u = as_u16(a).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ model

PROJ = ("w_qkv", "w_o", "w_gate", "w_up", "w_down")
SCALES = {"w_qkv": "s_qkv", "w_o": "s_o", "w_gate": "s_gate", "w_up": "s_up", "w_down": "s_down",
          "lm_head": "lm_head_scale"}


def _as_np(x, dtype):
    if isinstance(x, np.ndarray):
        return np.ascontiguousarray(x, dtype=dtype)
    return np.ascontiguousarray(x.detach().cpu().contiguous().numpy().astype(dtype, copy=False))


class Model:
    """Holds the oracle's view of a weight set (uint16 bf16 arrays, or int8
    codes with float32 row scales for the projections) and the ctypes
    struct pointing at them. Keep the object alive while in use."""

    def __init__(self, shape, weights: dict, kv_fp8: bool = False, k_scale: float = 1.0,
                 v_scale: float = 1.0):
        """kv_fp8: the KV cache holds E4M3 codes of value / scale (else bf16).
        Weights with "s_qkv" etc. entries are int8 codes read as q * scale
        per matrix row (the LM head's scales under "lm_head_scale")."""
        self.shape = shape
        self.kv_fp8 = bool(kv_fp8)
        self.w_int8 = "s_qkv" in weights
        self.arrays = {}
        for k, v in weights.items():
            if self.w_int8 and (k in PROJ or k == "lm_head"):
                conv = lambda x: _as_np(x, np.int8)
            elif self.w_int8 and k in SCALES.values():
                conv = lambda x: _as_np(x, np.float32)
            else:
                conv = as_u16
            self.arrays[k] = [conv(x) for x in v] if isinstance(v, list) else conv(v)
        m = OrModel()
        m.n_layers, m.d_model, m.n_heads = shape.n_layers, shape.d_model, shape.n_heads
        m.n_kv_heads, m.head_dim, m.ffn_dim = shape.n_kv_heads, shape.head_dim, shape.ffn_dim
        m.vocab, m.rms_eps, m.rope_base = shape.vocab, shape.rms_eps, shape.rope_base
        m.kv_fp8, m.k_scale, m.v_scale = int(self.kv_fp8), float(k_scale), float(v_scale)
        m.embed = _p(self.arrays["embed"], U16P)
        m.final_norm = _p(self.arrays["final_norm"], U16P)
        m.lm_head = C.cast(self.arrays["lm_head"].ctypes.data, U16P)
        self._ptr_arrays = {}
        for k in ("attn_norm", "w_qkv", "w_o", "ffn_norm", "w_gate", "w_up", "w_down"):
            arr = (U16P * shape.n_layers)(*[C.cast(a.ctypes.data, U16P) for a in self.arrays[k]])
            self._ptr_arrays[k] = arr
            setattr(m, k, C.cast(arr, C.POINTER(U16P)))
        m.w_int8 = int(self.w_int8)
        if self.w_int8:
            m.lm_head_scale = _p(self.arrays["lm_head_scale"], F32P)
            for k in PROJ:
                sk = SCALES[k]
                arr = (F32P * shape.n_layers)(*[_p(a, F32P) for a in self.arrays[sk]])
                self._ptr_arrays[sk] = arr
                setattr(m, sk, C.cast(arr, C.POINTER(F32P)))
        self.struct = m

    @property
    def kv_dtype(self):
        return np.uint8 if self.kv_fp8 else np.uint16

    def dense_kv(self, max_pos: int) -> np.ndarray:
        s = self.shape
        return np.zeros((s.n_layers, 2, max_pos, s.n_kv_heads, s.head_dim), self.kv_dtype)

    def paged_pool(self, num_blocks: int, block_size: int) -> np.ndarray:
        s = self.shape
        return np.zeros((s.n_layers, 2, num_blocks, block_size, s.n_kv_heads, s.head_dim),
                        self.kv_dtype)


def serial_forward(model: Model, kv_dense: np.ndarray, tokens, start_pos: int,
                   last_only: bool = True) -> np.ndarray:
    """Decode one sequence alone, one token per forward. Returns logits
    (double): [vocab] if last_only else [n][vocab]."""
    toks = np.ascontiguousarray(tokens, dtype=np.int32)
    n = len(toks)
    V = model.shape.vocab
    out = np.empty((V,) if last_only else (n, V), np.float64)
    assert kv_dense.dtype == model.kv_dtype and kv_dense.flags["C_CONTIGUOUS"]
    rc = lib().or_serial_forward(C.byref(model.struct), kv_dense.ctypes.data, kv_dense.shape[2],
                                 _p(toks, I32P), n, start_pos, int(last_only), _p(out, F64P))
    if rc != 0:
        raise ValueError(f"or_serial_forward failed ({rc})")
    return out


def paged_step(model: Model, pool: np.ndarray, block_tables: np.ndarray, ctx_lens,
               n_new, tokens, want_token):
    """One paged-batched step. Returns (logits [n_out][vocab] double,
    greedy ids [n_out])."""
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    nn = np.ascontiguousarray(n_new, dtype=np.int32)
    tk = np.ascontiguousarray(tokens, dtype=np.int32)
    wt = np.ascontiguousarray(want_token, dtype=np.int32)
    n_out = int(wt.astype(bool).sum())
    V = model.shape.vocab
    logits = np.empty((max(n_out, 1), V), np.float64)
    greedy = np.empty(max(n_out, 1), np.int32)
    assert pool.dtype == model.kv_dtype and pool.flags["C_CONTIGUOUS"]
    rc = lib().or_paged_step(C.byref(model.struct), pool.ctypes.data, pool.shape[2], pool.shape[3],
                             len(ctx), _p(bt, I32P), bt.shape[1], _p(ctx, I32P), _p(nn, I32P),
                             _p(tk, I32P), _p(wt, I32P), _p(logits, F64P), _p(greedy, I32P))
    if rc != 0:
        raise ValueError(f"or_paged_step failed ({rc})")
    return logits[:n_out], greedy[:n_out]


# ---------------------------------------------------------------- pieces

def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64).reshape(-1)


def rmsnorm(x, g, eps: float) -> np.ndarray:
    """x (double [d]) normalised and scaled by the bf16 gain g."""
    x, g = _f64(x), as_u16(g)
    y = np.empty_like(x)
    lib().or_rmsnorm(_p(x, F64P), _p(g, U16P), x.size, eps, _p(y, F64P))
    return y


def linear(x, W) -> np.ndarray:
    """W (bf16 [N][K]) times x (double [K])."""
    x, W = _f64(x), as_u16(W)
    assert W.shape[1] == x.size
    y = np.empty(W.shape[0], np.float64)
    lib().or_linear(_p(x, F64P), W.shape[1], _p(W, U16P), W.shape[0], _p(y, F64P))
    return y


def linear_i8(x, Q, scale) -> np.ndarray:
    """Q (int8 [N][K]) with row scales (float32 [N]) times x (double [K])."""
    x = _f64(x)
    Q = np.ascontiguousarray(Q, dtype=np.int8)
    scale = np.ascontiguousarray(scale, dtype=np.float32)
    assert Q.shape[1] == x.size and scale.size == Q.shape[0]
    y = np.empty(Q.shape[0], np.float64)
    lib().or_linear_i8(_p(x, F64P), Q.shape[1], Q.ctypes.data, _p(scale, F32P), Q.shape[0],
                       _p(y, F64P))
    return y


def rope(v, pos: int, base: float) -> np.ndarray:
    v = _f64(v).copy()
    lib().or_rope(_p(v, F64P), v.size, pos, base)
    return v


def attention_dense(q, K, V, n_heads: int, n_kv_heads: int, head_dim: int) -> np.ndarray:
    """q [Hq*hd] double, K/V [n][Hkv][hd] bf16 -> [Hq*hd] double."""
    q, K, V = _f64(q), as_u16(K), as_u16(V)
    out = np.empty(n_heads * head_dim, np.float64)
    n = K.shape[0]
    rc = lib().or_attention_dense(_p(q, F64P), _p(K, U16P), _p(V, U16P), n, n_heads,
                                  n_kv_heads, head_dim, _p(out, F64P))
    if rc != 0:
        raise ValueError("or_attention_dense failed")
    return out


def attention_dense_fp8(q, K, V, n_heads: int, n_kv_heads: int, head_dim: int,
                        k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """q [Hq*hd] double, K/V [n][Hkv][hd] E4M3 codes of value / scale."""
    q = _f64(q)
    K = np.ascontiguousarray(K, dtype=np.uint8)
    V = np.ascontiguousarray(V, dtype=np.uint8)
    out = np.empty(n_heads * head_dim, np.float64)
    rc = lib().or_attention_dense_kv(_p(q, F64P), K.ctypes.data, V.ctypes.data, K.shape[0],
                                     n_heads, n_kv_heads, head_dim, 1, k_scale, v_scale,
                                     _p(out, F64P))
    if rc != 0:
        raise ValueError("or_attention_dense_kv failed")
    return out


def e4m3_to_float(code: int) -> float:
    return lib().or_e4m3_to_f64(int(code))


def float_to_e4m3(x: float) -> int:
    return lib().or_f64_to_e4m3(float(x))


def bf16_round(x) -> np.ndarray:
    """Round doubles to bf16 (nearest even) and return the bf16 bits."""
    a = _f64(x)
    return np.array([lib().or_f64_to_bf16(float(v)) for v in a], np.uint16)


def f64_to_bf16(x: float) -> int:
    return lib().or_f64_to_bf16(float(x))


def bf16_to_float(h: int) -> float:
    return lib().or_bf16_to_f64(int(h))


def argmax_f32(x) -> int:
    a = np.ascontiguousarray(x, dtype=np.float32)
    return lib().or_argmax_f32(_p(a, F32P), a.size)


def argmax_f64(x) -> int:
    a = np.ascontiguousarray(x, dtype=np.float64)
    return lib().or_argmax_f64(_p(a, F64P), a.size)


def philox4x64_10(ctr, key) -> list:
    c = np.ascontiguousarray(ctr, dtype=np.uint64)
    k = np.ascontiguousarray(key, dtype=np.uint64)
    o = np.empty(4, np.uint64)
    lib().or_philox4x64_10(_p(c, U64P), _p(k, U64P), _p(o, U64P))
    return [int(v) for v in o]


def uniform24(seed: int, request_id: int, step_id: int) -> float:
    return lib().or_uniform24(seed, request_id, step_id)


def sampling_struct(sp) -> OrSampling:
    s = OrSampling()
    s.temperature, s.top_p, s.top_k = sp.temperature, sp.top_p, sp.top_k
    s.freq_penalty, s.presence_penalty = sp.freq_penalty, sp.presence_penalty
    s.penalty_decay, s.seed = sp.penalty_decay, sp.seed
    ids = list(getattr(sp, "forbidden", ()))
    assert len(ids) <= 8
    s.n_forbidden = len(ids)
    for i, t in enumerate(ids):
        s.forbidden[i] = int(t)
    return s


def sample(logits, counts, sp, request_id: int, step_id: int):
    """One sampler row in fp32. counts (float32 [V]) is updated in place
    when given. Returns (token, info dict)."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    info = OrSampleInfo()
    s = sampling_struct(sp)
    cp = None
    if counts is not None:
        assert counts.dtype == np.float32 and counts.flags["C_CONTIGUOUS"]
        cp = _p(counts, F32P)
    tok = lib().or_sample_f32(_p(lg, F32P), lg.size, cp, C.byref(s), request_id, step_id,
                              C.byref(info))
    return tok, info.as_dict()


def num_threads() -> int:
    return lib().or_num_threads()


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops (rows, heads, vocabulary)."""
    lib().or_set_num_threads(int(n))

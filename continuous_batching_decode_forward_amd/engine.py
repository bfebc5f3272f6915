"""Python-side plumbing around the C ABI: device buffers come from PyTorch
(memory and streams only), everything else goes through libcbd.so.

    eng = Engine(shape, weights, block_size=32, num_blocks=..., ...)
    meta = eng.upload_step(slots, tables, ctx_lens, n_new, tokens, want, step_ids)
    eng.step_forward(meta, logits_out, tokens_out)
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import numpy as np
import torch

from . import binding as B


def _ptr(t: torch.Tensor | None):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream_ptr(stream) -> C.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


@dataclass
class StepMeta:
    """Device copy of one step's metadata (one int32 buffer) + host scalars."""
    buf: torch.Tensor
    step: B.cbd_step
    n_seqs: int
    n_rows: int
    n_out: int


def untile_plane(flat: np.ndarray, rows: int, width: int) -> np.ndarray:
    """[rows][width] from one plane in operand tiles (1 KB tiles of 16 rows x
    32 columns, rows padded to 16 and columns to 32; see cbd.h)."""
    kb = (width + 31) // 32
    f = flat.size // (kb * 512)
    # [fragment][k-block][8-column group][row in fragment][8] -> [row][column]
    v = flat.reshape(f, kb, 4, 16, 8).transpose(0, 3, 1, 2, 4).reshape(f * 16, kb * 32)
    return v[:rows, :width]


class Engine:
    def __init__(self, shape, weights: dict, *, block_size: int, num_blocks: int,
                 max_blocks_per_seq: int, max_slots: int, max_rows: int, max_seqs: int,
                 max_position: int, block_order=None, device="cuda", stream=None,
                 kv_dtype: int = B.CBD_KV_BF16, k_scale: float = 0.0, v_scale: float = 0.0):
        self.shape = shape
        self.device = torch.device(device)
        cfg = B.cbd_config()
        cfg.n_layers, cfg.d_model, cfg.n_heads = shape.n_layers, shape.d_model, shape.n_heads
        cfg.n_kv_heads, cfg.head_dim, cfg.ffn_dim = shape.n_kv_heads, shape.head_dim, shape.ffn_dim
        cfg.vocab, cfg.block_size, cfg.num_blocks = shape.vocab, block_size, num_blocks
        cfg.max_blocks_per_seq, cfg.max_slots, cfg.max_rows = max_blocks_per_seq, max_slots, max_rows
        cfg.max_seqs, cfg.max_position = max_seqs, max_position
        cfg.rms_eps, cfg.rope_base = shape.rms_eps, shape.rope_base
        cfg.kv_dtype, cfg.k_scale, cfg.v_scale = kv_dtype, k_scale, v_scale
        # int8 projections: weights with per-row scales (synth.make_weights_int8)
        self.w_int8 = "s_qkv" in weights
        cfg.weight_dtype = B.CBD_W_INT8 if self.w_int8 else B.CBD_W_BF16
        self.cfg = cfg
        self.kv_fp8 = kv_dtype == B.CBD_KV_FP8_E4M3
        self.block_size, self.num_blocks = block_size, num_blocks
        self.max_blocks_per_seq = max_blocks_per_seq
        self.packed = torch.empty(B.cbd_packed_weights_bytes(cfg), dtype=torch.uint8,
                                  device=self.device)
        self.kv_pool = torch.empty(B.cbd_kv_pool_bytes(cfg), dtype=torch.uint8, device=self.device)
        self.slot_state = torch.empty(B.cbd_slot_state_bytes(cfg), dtype=torch.uint8,
                                      device=self.device)
        self.workspace = torch.empty(B.cbd_workspace_bytes(cfg), dtype=torch.uint8,
                                     device=self.device)
        self.weights = weights  # keep alive
        w = B.cbd_weights()
        w.embed, w.final_norm, w.lm_head = (weights["embed"].data_ptr(),
                                            weights["final_norm"].data_ptr(),
                                            weights["lm_head"].data_ptr())
        self._arrs = {}
        per_layer = ["attn_norm", "w_qkv", "w_o", "ffn_norm", "w_gate", "w_up", "w_down"]
        if self.w_int8:
            per_layer += ["s_qkv", "s_o", "s_gate", "s_up", "s_down"]
            w.lm_head_scale = weights["lm_head_scale"].data_ptr()
        for k in per_layer:
            arr = (C.c_void_p * shape.n_layers)(*[t.data_ptr() for t in weights[k]])
            self._arrs[k] = arr
            setattr(w, k, C.cast(arr, C.POINTER(C.c_void_p)))
        self._w = w
        self.stream = stream
        self.handle = B.cbd_engine_create(cfg, w, _ptr(self.packed), _ptr(self.kv_pool),
                                          _ptr(self.slot_state),
                                          _ptr(self.workspace), block_order,
                                          _stream_ptr(stream))

    # ---------------------------------------------------------- pool views
    def kv_views(self, layer: int):
        """(K, V) views of one layer's pool regions, bf16 (or uint8 E4M3 codes
        for an 8-bit cache): K [num_blocks][Hkv][block_size][hd],
        V [num_blocks][Hkv][hd][block_size]."""
        s = self.shape
        per = self.num_blocks * s.n_kv_heads * self.block_size * s.head_dim
        flat = self.kv_pool if self.kv_fp8 else self.kv_pool.view(torch.bfloat16)
        k = flat[(2 * layer) * per:(2 * layer + 1) * per].view(
            self.num_blocks, s.n_kv_heads, self.block_size, s.head_dim)
        v = flat[(2 * layer + 1) * per:(2 * layer + 2) * per].view(
            self.num_blocks, s.n_kv_heads, s.head_dim, self.block_size)
        return k, v

    # ---------------------------------------------------------------- step
    def upload_step(self, slots, block_tables, ctx_lens, n_new, tokens, want_token,
                    step_ids=None, mode=B.CBD_MODE_GREEDY, max_ctx=None, stream=None) -> StepMeta:
        """Copy host metadata into one device int32 buffer and describe it."""
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        n = len(ctx_lens)
        parts = [np.asarray(slots, np.int32), bt.reshape(-1), np.asarray(ctx_lens, np.int32),
                 np.asarray(n_new, np.int32), np.asarray(tokens, np.int32),
                 np.asarray(want_token, np.int32),
                 np.asarray(step_ids if step_ids is not None else np.zeros(n), np.int32)]
        host = np.concatenate(parts)
        buf = torch.from_numpy(host).to(self.device, non_blocking=False)
        offs = np.cumsum([0] + [len(p) for p in parts])
        st = B.cbd_step()
        st.n_seqs = n
        st.n_rows = int(np.sum(n_new))
        st.n_out = int(np.count_nonzero(want_token))
        ctx = np.asarray(ctx_lens, np.int64) + np.asarray(n_new, np.int64)
        st.max_ctx = int(max_ctx if max_ctx is not None else ctx.max())
        st.max_blocks_per_seq = bt.shape[1]
        st.mode = mode
        base = buf.data_ptr()
        names = ["slots", "block_tables", "ctx_lens", "n_new", "tokens", "want_token", "step_ids"]
        for name, o in zip(names, offs[:-1]):
            setattr(st, name, base + 4 * int(o))
        return StepMeta(buf, st, n, st.n_rows, st.n_out)

    def step_forward(self, meta: StepMeta, logits_out: torch.Tensor | None,
                     tokens_out: torch.Tensor, stream=None) -> None:
        B.cbd_step_forward(self.handle, meta.step, _ptr(logits_out), _ptr(tokens_out),
                           _stream_ptr(stream))

    def step_forward_graph(self, meta: StepMeta, logits_out: torch.Tensor | None,
                           tokens_out: torch.Tensor, stream) -> None:
        """The step replayed from a recorded HIP graph (one per step shape);
        `stream` must be a side stream, not the null stream."""
        B.cbd_step_forward_graph(self.handle, meta.step, _ptr(logits_out), _ptr(tokens_out),
                                 _stream_ptr(stream))

    def graph_stats(self) -> tuple:
        return B.cbd_graph_stats(self.handle)

    def sample_logits(self, logits: torch.Tensor, slots: torch.Tensor, step_ids: torch.Tensor,
                      tokens_out: torch.Tensor, stream=None) -> None:
        B.cbd_sample_logits(self.handle, _ptr(logits), logits.shape[0], _ptr(slots),
                            _ptr(step_ids), _ptr(tokens_out), _stream_ptr(stream))

    def status(self, stream=None) -> int:
        return B.cbd_engine_status(self.handle, _stream_ptr(stream))

    def slot_counts(self) -> torch.Tensor:
        """The per-slot penalty counts [max_slots][vocab] fp32 (a view)."""
        s = self.cfg
        params_bytes = (s.max_slots * 80 + 255) // 256 * 256  # 80-byte slot parameters
        return self.slot_state[params_bytes:params_bytes + s.max_slots * s.vocab * 4].view(
            torch.float32).view(s.max_slots, s.vocab)

    # Buffers that hold fp32 values as two bf16 planes (hi, then lo), and
    # those of them whose planes are in operand tiles (16 x 32 tiles of 1 KB).
    _SPLIT = (B.CBD_BUF_H, B.CBD_BUF_Q, B.CBD_BUF_ATTN, B.CBD_BUF_FFN, B.CBD_BUF_LM_IN)
    _TILED = (B.CBD_BUF_H, B.CBD_BUF_ATTN, B.CBD_BUF_FFN, B.CBD_BUF_LM_IN)

    def debug_buffer(self, which: int, rows: int, width: int) -> np.ndarray:
        """The first `rows` rows of an internal activation buffer as float64
        values (a split buffer's value is hi + lo, summed exactly)."""
        ptr, nbytes = B.cbd_debug_buffer(self.handle, which)
        off = ptr - self.workspace.data_ptr()
        assert 0 <= off and off + nbytes <= self.workspace.numel() and rows * width * 4 <= nbytes
        buf = self.workspace[off:off + nbytes]
        if which not in self._SPLIT:
            return buf[:rows * width * 4].view(torch.float32).view(rows, width).cpu().numpy() \
                .astype(np.float64)
        plane = nbytes // 2
        def part(o, n):
            u = buf[o:o + n * 2].view(torch.int16).cpu().numpy().view(np.uint16)
            return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        if which not in self._TILED:
            return (part(0, rows * width) + part(plane, rows * width)).reshape(rows, width)
        n = plane // 2  # elements per plane: rows padded to 16, columns to 32
        return untile_plane(part(0, n) + part(plane, n), rows, width)

    def close(self):
        if getattr(self, "handle", None):
            B.cbd_engine_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class ComposerLoop:
    """The host step composer attached to an engine and stepped natively:
    each step() is one cbd_sched_step (plan, upload, step, tokens back,
    commit). The staging buffers are allocated here with torch: the device
    metadata buffer, page-locked host staging and the device token row."""

    def __init__(self, eng: Engine, *, max_rows: int, chunk_size: int, eos_id: int,
                 policy: int = B.CBD_ADMIT_RESERVE, max_slots: int | None = None,
                 max_blocks_per_seq: int | None = None, pacing: int = B.CBD_PACE_PREFILL_FIRST,
                 max_prefill: int = 0, decode_prefill_ratio: int = 0,
                 min_forward_seq_len: int = 0, ctx_round: int = 0, graph_decode: bool = False):
        cfg = B.cbd_sched_config()
        cfg.max_slots = max_slots or eng.cfg.max_slots
        cfg.block_size, cfg.num_blocks = eng.block_size, eng.num_blocks
        cfg.max_blocks_per_seq = max_blocks_per_seq or eng.max_blocks_per_seq
        cfg.max_rows, cfg.chunk_size, cfg.eos_id, cfg.policy = max_rows, chunk_size, eos_id, policy
        cfg.pacing, cfg.max_prefill = pacing, max_prefill
        cfg.decode_prefill_ratio, cfg.min_forward_seq_len = decode_prefill_ratio, min_forward_seq_len
        cfg.ctx_round, cfg.graph_decode = ctx_round, int(graph_decode)
        self.cfg, self.eng = cfg, eng
        self.handle = B.cbd_sched_create(cfg, eng.handle)
        n = B.cbd_sched_meta_ints(cfg)
        self.meta_dev = torch.empty(n, dtype=torch.int32, device=eng.device)
        self.host = torch.empty(n, dtype=torch.int32, pin_memory=True)
        self.tokens_dev = torch.empty(cfg.max_slots, dtype=torch.int32, device=eng.device)
        # graph replay records by stream capture, which the null stream does
        # not allow: such a loop steps on its own side stream by default
        self.stream = torch.cuda.Stream(device=eng.device) if graph_decode else None

    def submit(self, prompt, max_new: int, params=None, request_id: int = 0) -> None:
        B.cbd_sched_submit(self.handle, prompt, max_new, params, request_id)

    def step(self, mode=B.CBD_MODE_GREEDY, logits_out: torch.Tensor | None = None,
             stream=None) -> B.cbd_plan:
        return B.cbd_sched_step(self.handle, mode, self.meta_dev.data_ptr(),
                                self.host.data_ptr(), self.tokens_dev.data_ptr(),
                                None if logits_out is None else logits_out.data_ptr(),
                                _stream_ptr(stream if stream is not None else self.stream).value)

    def last_tokens(self, n: int) -> np.ndarray:
        """The tokens the last step committed (host staging copy)."""
        return self.host[:n].numpy().copy()

    def pop_finished(self) -> list:
        out = []
        while (f := B.cbd_sched_pop_finished(self.handle)) is not None:
            out.append(f)
        return out

    def stats(self) -> B.cbd_sched_stats:
        return B.cbd_sched_stats_get(self.handle)

    def close(self):
        if getattr(self, "handle", None):
            B.cbd_sched_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

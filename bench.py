#!/usr/bin/env python3
"""Benchmark of one continuous-batching decode step on one MI355X.

Workload (default): one 8B-shaped decoder layer + LM head (d_model 4096,
32/8 heads, head_dim 128, FFN 14336, vocab 128256), bf16 random-init weights
~N(0, 0.02), B decode rows with contexts uniform in 512..4096 held as
synthetic N(0,1) bf16 KV in 32-position blocks through shuffled block
tables, greedy argmax. A step is one cbd_step_forward over all B rows with
every input already in HBM. The headline is B = 64; B in {1, 8, 32, 128,
256} is also reported.

Prints one JSON line: decode tokens/s, ms per step, achieved HBM GB/s under
the (W + B*A)/beta cost model, the dominant kernel's roofline (timed with HIP
events on the step's stream during the timed steps), and the CPU oracle timed
on a bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kv_bytes_per_pos(shape, elem=2):
    """K and V bytes of one position over all layers (elem: bytes per value,
    2 for bf16, 1 for E4M3)."""
    return 2 * shape.n_kv_heads * shape.head_dim * elem * shape.n_layers


def step_bytes(shape, ctx, n_out, kv_elem=2, w_int8=False):
    """Algorithmic HBM bytes of one decode step: every weight once (int8
    codes and their row scales for int8 weights), the embedding rows, each
    row's cached KV (ctx + 1 positions read, one appended) and the fp32
    logits written."""
    from continuous_batching_decode_forward_amd import synth
    W = synth.weight_bytes(shape, w_int8) + len(ctx) * shape.d_model * 2
    kvb = kv_bytes_per_pos(shape, kv_elem)
    A = sum((int(c) + 1) * kvb + kvb for c in ctx)
    return W + A + n_out * shape.vocab * 4


def class_bytes(shape, ctx, n_out):
    """Algorithmic HBM bytes per step of each kernel class of the decode step:
    each projection's bf16 weights (every layer), the batch's K/V read and
    appended for attention, the LM head's weights and fp32 logits."""
    from continuous_batching_decode_forward_amd import synth
    ws = synth.weight_shapes(shape)
    L = shape.n_layers
    mat = lambda *names: L * sum(2 * int(np.prod(ws[k])) for k in names)
    kvb = 2 * shape.n_kv_heads * shape.head_dim * 2  # K and V of one position, one layer
    return {"qkv": mat("w_qkv"), "o": mat("w_o"), "gateup": mat("w_gate", "w_up"),
            "down": mat("w_down"), "attn": L * sum((int(c) + 2) * kvb for c in ctx),
            "lm_head": lm_head_bytes(shape, n_out)}


def lm_head_bytes(shape, n_out):
    """LM head per launch: the bf16 weight once, the activation rows (the
    final norm's output, read as bf16) and the fp32 logits written."""
    return shape.vocab * shape.d_model * 2 + n_out * shape.d_model * 2 + n_out * shape.vocab * 4


# The dominant kernel's HBM traffic comes from rocprofv3 counter runs kept in
# profiles/ (FETCH_SIZE and WRITE_SIZE per dispatch, scaled by what the same
# counters read for a device-to-device copy of known size). It is reported
# only while the sources it was measured on are unchanged.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lm_head_gemm_8b_b64_traffic.md")
TRAFFIC_SOURCES = ["continuous_batching_decode_forward_amd/csrc/gemm.hip",
                   "continuous_batching_decode_forward_amd/csrc/common.h",
                   "continuous_batching_decode_forward_amd/csrc/kernels.h"]


def sources_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(batch):
    try:
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if line.startswith('{"traffic"'):
                    rec = json.loads(line)["traffic"]
                    if rec.get("sources") == sources_digest() and rec.get("batch") == batch:
                        return rec["bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        pass
    return None


def build_workload(shape, B, seed, ctx_range=(512, 4096), bs=32):
    """B decode rows with contexts uniform in ctx_range (inclusive), their
    blocks drawn from a seeded permutation of a pool that holds exactly
    their contexts plus the appended position."""
    from continuous_batching_decode_forward_amd import synth
    ctx = synth.uniform_ints(seed, "ctx", B, ctx_range[0], ctx_range[1])
    need = [-(-(int(c) + 1) // bs) for c in ctx]
    total = int(sum(need))
    perm = synth.permutation(seed, "blocks", total)
    mbps = -(-(ctx_range[1] + 1) // bs)
    tables = np.full((B, mbps), -1, np.int32)
    o = 0
    for i in range(B):
        tables[i, :need[i]] = perm[o:o + need[i]]
        o += need[i]
    tokens = synth.uniform_ints(seed, "tok", B, 0, shape.vocab - 1)
    return dict(bs=bs, ctx=ctx, tables=tables, perm=perm, total=total, mbps=mbps,
                tokens=tokens, max_position=ctx_range[1] + 1)


def fill_pool(eng, seed, blocks):
    """Seeded cached K/V in the engine's pool layout: N(0, 1) bf16 values, or
    E4M3 codes (magnitudes 0..7.5) for an 8-bit cache."""
    import torch
    from continuous_batching_decode_forward_amd import synth
    gen = synth.kv_codes_fp8 if eng.kv_fp8 else synth.kv_values
    s = eng.shape
    bs, hkv, hd = eng.block_size, s.n_kv_heads, s.head_dim
    dev = eng.kv_pool.device
    blocks = torch.as_tensor(np.asarray(blocks, np.int64), device=dev)
    kh = torch.arange(hkv, device=dev)
    off = torch.arange(bs, device=dev)
    dim = torch.arange(hd, device=dev)
    for layer in range(s.n_layers):
        k, v = eng.kv_views(layer)
        for c0 in range(0, len(blocks), 2048):
            b = blocks[c0:c0 + 2048]
            k[b] = gen(seed, layer, 0, b.view(-1, 1, 1, 1), kh.view(1, -1, 1, 1),
                       off.view(1, 1, -1, 1), dim.view(1, 1, 1, -1), hkv, bs, hd)
            v[b] = gen(seed, layer, 1, b.view(-1, 1, 1, 1), kh.view(1, -1, 1, 1),
                       off.view(1, 1, 1, -1), dim.view(1, 1, -1, 1), hkv, bs, hd)


def time_steps(eng, meta, lg, tk, steps, warmup, stream, profile_class=None):
    import torch
    from continuous_batching_decode_forward_amd import binding as B
    for _ in range(warmup):
        eng.step_forward(meta, lg, tk, stream)
    torch.cuda.synchronize()
    if profile_class is not None:
        B.cbd_profile_begin(eng.handle, profile_class)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    t0 = time.perf_counter()
    for _ in range(steps):
        eng.step_forward(meta, lg, tk, stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / steps
    kern = None
    if profile_class is not None:
        tot, n = B.cbd_profile_end(eng.handle)
        kern = (tot / max(n, 1), n)
    return ms, wall, kern


def hbm_read_probe(nbytes=4 << 30, blocks=512, reps=10, rounds=3):
    """The bandwidth a plain streaming read of a 4 GiB buffer reaches
    (cbd_read_probe: 512 x 1024 threads, non-temporal 16-byte loads), timed
    with HIP events on the current stream, the best of a few rounds: the
    practical ceiling beside the published 8 TB/s peak."""
    import torch
    from continuous_batching_decode_forward_amd import binding as B
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(blocks * 1024, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    B.cbd_read_probe(buf.data_ptr(), nbytes, out.data_ptr(), blocks, st.cuda_stream)
    best = None
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            B.cbd_read_probe(buf.data_ptr(), nbytes, out.data_ptr(), blocks, st.cuda_stream)
        e1.record(st)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        best = ms if best is None else min(best, ms)
    del buf, out
    torch.cuda.empty_cache()
    gbs = nbytes / (best * 1e-3) / 1e9
    return {"gbs": gbs, "frac_of_peak": gbs / PEAK_HBM_GBS, "bytes": nbytes, "ms": best,
            "blocks": blocks, "threads_per_block": 1024, "reps": reps, "rounds": rounds}


def cpu_info():
    """The host CPU's model name and the cores this process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return model, os.cpu_count(), usable


def oracle_kv_pool(shape, seed, tables, n_cached, n_new, bs, device):
    """The oracle's pool ([L][2][blocks][bs][Hkv][hd] bf16 bits, host) for
    the given sequences, blocks renumbered 0.. in table order, holding the
    same synthetic cached K/V as the engine's pool (values keyed by the
    physical block), generated on `device`; returns (pool, compact tables)."""
    import torch
    import oracle as O
    from continuous_batching_decode_forward_amd import synth
    hkv, hd = shape.n_kv_heads, shape.head_dim
    need = [-(-(int(c) + int(n)) // bs) for c, n in zip(n_cached, n_new)]
    pool = np.zeros((shape.n_layers, 2, max(sum(need), 1), bs, hkv, hd), np.uint16)
    compact = np.full((len(need), max(need)), -1, np.int32)
    kh = torch.arange(hkv, device=device).view(1, 1, -1, 1)
    off = torch.arange(bs, device=device).view(1, -1, 1, 1)
    dim = torch.arange(hd, device=device).view(1, 1, 1, -1)
    nxt = 0
    for i, (tab, c) in enumerate(zip(tables, n_cached)):
        ids = np.arange(nxt, nxt + need[i], dtype=np.int32)
        compact[i, :need[i]] = ids
        nxt += need[i]
        nbc = -(-int(c) // bs)
        if nbc == 0:
            continue
        phys = torch.as_tensor(np.asarray(tab[:nbc], np.int64), device=device).view(-1, 1, 1, 1)
        for layer in range(shape.n_layers):
            for kind in (0, 1):
                vals = synth.kv_values(seed, layer, kind, phys, kh, off, dim, hkv, bs, hd)
                pool[layer, kind, ids[:nbc]] = O.as_u16(vals.cpu()).reshape(nbc, bs, hkv, hd)
    return pool, compact


def cpu_baseline(shape, wg, wl, seed, B, budget_s):
    """The oracle, as it stands, on the same step: all B decode rows of the
    8B layer + LM head step in one paged step on every core the oracle's
    OpenMP loops use (rows, heads and vocabulary in parallel), then a
    bounded 1-thread sample (rows one at a time) for the per-core rate."""
    import oracle as O
    wc = {k: ([t.cpu() for t in v] if isinstance(v, list) else v.cpu()) for k, v in wg.items()}
    om = O.Model(shape, wc)
    ctx = [int(c) for c in wl["ctx"][:B]]
    toks = [int(t) for t in wl["tokens"][:B]]
    pool, compact = oracle_kv_pool(shape, seed, list(wl["tables"][:B]), ctx, [1] * B, wl["bs"],
                                   "cuda")
    threads = O.num_threads()
    t0 = time.perf_counter()
    O.paged_step(om, pool, compact, ctx, [1] * B, toks, [1] * B)
    whole = time.perf_counter() - t0
    # one thread: rows alone, until about a third of the budget
    O.set_num_threads(1)
    done, spent = 0, 0.0
    try:
        for i in range(B):
            t0 = time.perf_counter()
            O.paged_step(om, pool, compact[i:i + 1], [ctx[i]], [1], [toks[i]], [1])
            spent += time.perf_counter() - t0
            done += 1
            if spent >= budget_s / 3:
                break
    finally:
        O.set_num_threads(threads)
    model, n_cpu, usable = cpu_info()
    return {"value": B / whole, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole B={B} step (8B layer + LM head, contexts U[512,4096]) in one "
                      f"oracle paged step on {threads} threads: {whole:.1f} s",
            "ms_per_step": whole * 1e3,
            "single_thread": {"value": done / spent, "unit": "tokens/s", "cores": 1,
                              "sample": f"{done} rows of the same step, each alone, "
                                        f"{spent:.1f} s"},
            "cpu_model": model, "nproc": n_cpu, "usable_cores": usable}


def penalty_history(seed, B, V, n_hist, decay):
    """Per-row penalty counts after a seeded history of n_hist generated
    tokens: each step c <- fl(c * decay), then c[token] += 1."""
    from continuous_batching_decode_forward_amd import synth
    counts = np.zeros((B, V), np.float32)
    hist = synth.uniform_ints(seed, "history", B * n_hist, 0, V - 1).reshape(B, n_hist)
    d = np.float32(decay)
    rows = np.arange(B)
    for t in range(n_hist):
        counts *= d
        counts[rows, hist[:, t]] += np.float32(1.0)
    return counts


def bench_sampled(args):
    print(json.dumps(run_sampled(args.steps, args.warmup, kv_fp8=args.kv_fp8)), flush=True)


# The 8-bit cache's scales for the seeded codes (magnitudes 0..7.5): keys
# and values of about unit size after dequantisation.
FP8_KV = {"k_scale": 0.25, "v_scale": 0.25}


def run_sampled(steps, warmup, kv_fp8=False):
    """The KV-dominated sampled step: one 8B-shaped layer + LM head over a
    65536-token vocabulary, B = 256 decode rows with contexts uniform in
    8192..32768, sampler T = 1.0, top_p = 0.3, top_k = 0, frequency penalty
    1.0, decay 0.996 on a seeded 64-token history per row. kv_fp8: the same
    step over an 8-bit (E4M3) cache, half the KV bytes."""
    import torch
    from continuous_batching_decode_forward_amd import binding as B
    from continuous_batching_decode_forward_amd import configs, synth
    from continuous_batching_decode_forward_amd.engine import Engine
    shape, wlc = configs.LLAMA8B_1L_V64K, configs.SAMPLE_8B_B256
    seed, Bn = 0, wlc.batch[0]
    stream = torch.cuda.current_stream()
    log(f"[bench] weights {shape.name} on GPU")
    wg = synth.make_weights(shape, seed=seed, device="cuda")
    wl = build_workload(shape, Bn, seed, ctx_range=wlc.ctx_range, bs=wlc.block_size)
    elem = 1 if kv_fp8 else 2
    kv_args = dict(kv_dtype=B.CBD_KV_FP8_E4M3, **FP8_KV) if kv_fp8 else {}
    eng = Engine(shape, wg, block_size=wl["bs"], num_blocks=wl["total"],
                 max_blocks_per_seq=wl["mbps"], max_slots=Bn, max_rows=Bn, max_seqs=Bn,
                 max_position=wl["max_position"], **kv_args)
    log(f"[bench] filling {wl['total']} KV blocks "
        f"({wl['total'] * kv_bytes_per_pos(shape, elem) * wl['bs'] / 1e9:.1f} GB"
        f"{', E4M3' if kv_fp8 else ''})")
    fill_pool(eng, seed, wl["perm"])
    sp = wlc.sampling
    params = B.cbd_sampling.from_params(sp)
    slots = [B.cbd_slot_alloc(eng.handle, params, r) for r in range(Bn)]
    counts0 = torch.from_numpy(penalty_history(seed, Bn, shape.vocab, 64, sp.penalty_decay))
    counts0 = counts0.to("cuda")
    eng.slot_counts()[slots] = counts0
    meta = eng.upload_step(slots=slots, block_tables=wl["tables"], ctx_lens=wl["ctx"],
                           n_new=[1] * Bn, tokens=wl["tokens"], want_token=[1] * Bn,
                           step_ids=[64] * Bn, mode=B.CBD_MODE_SAMPLE)
    tk = torch.empty(Bn, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    ms, wall, kern = time_steps(eng, meta, None, tk, steps, warmup, stream)
    times = {}
    for name in ("ATTN", "LM_HEAD", "SAMPLE", "GATEUP", "DOWN", "QKV", "O"):
        _, _, k = time_steps(eng, meta, None, tk, 5, 1, stream,
                             profile_class=getattr(B, "CBD_KERNEL_" + name))
        times[name.lower() + "_us"] = round(k[0] * 1e3, 1)
    if eng.status():
        raise RuntimeError("device status set")
    byts = step_bytes(shape, wl["ctx"], Bn, elem) + 3 * Bn * shape.vocab * 4  # + sampler r/w
    kv = sum((int(c) + 1) * kv_bytes_per_pos(shape, elem) for c in wl["ctx"])
    out = {"workload": wlc.name + ("-e4m3kv" if kv_fp8 else ""), "batch": Bn,
           "ctx_range": list(wlc.ctx_range), "kv_cache": "e4m3" if kv_fp8 else "bf16",
           "ms_per_step": ms, "tokens_per_s": Bn / (ms * 1e-3),
           "step_algorithmic_bytes": byts, "hbm_gbs": byts / (ms * 1e-3) / 1e9,
           "roofline_frac": byts / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
           "kv_bytes": kv, "attention_gbs": kv / (times["attn_us"] * 1e-6) / 1e9,
           "sampler_gbs": 3 * Bn * shape.vocab * 4 / (times["sample_us"] * 1e-6) / 1e9,
           "kernel_us": times, "steps": steps, "warmup": warmup}
    eng.close()
    del eng, wg
    torch.cuda.empty_cache()
    return out


def build_mixed(shape, seed, n_dec=48, ctx_range=(1024, 8192), prompt=4096, chunk=512, bs=32):
    """The mixed step's inputs: n_dec decode rows with contexts uniform in
    ctx_range (blocks for their cached positions and the positions the
    prompt's steps append), and one prompt of `prompt` uniform ids prefilled
    in chunks of `chunk` rows, one chunk per step (offsets 0, chunk, ...).
    Blocks come from one seeded permutation of the pool; sequence 0 is the
    prompt, sequences 1..n_dec the decode rows."""
    from continuous_batching_decode_forward_amd import synth
    n_steps = prompt // chunk
    ctx = synth.uniform_ints(seed, "ctx", n_dec, ctx_range[0], ctx_range[1])
    need = [-(-prompt // bs)] + [-(-(int(c) + n_steps) // bs) for c in ctx]
    total = int(sum(need))
    perm = synth.permutation(seed, "blocks", total)
    mbps = max(need)
    tables = np.full((n_dec + 1, mbps), -1, np.int32)
    o = 0
    for i in range(n_dec + 1):
        tables[i, :need[i]] = perm[o:o + need[i]]
        o += need[i]
    cached = perm[need[0]:]  # the decode rows' blocks hold synthetic K/V
    prompt_ids = synth.uniform_ints(seed, "prompt", prompt, 0, shape.vocab - 1)
    dec_tokens = synth.uniform_ints(seed, "dectok", n_dec * n_steps, 0,
                                    shape.vocab - 1).reshape(n_steps, n_dec)
    return dict(bs=bs, ctx=ctx, tables=tables, total=total, mbps=mbps, cached=cached,
                prompt=prompt_ids, dec_tokens=dec_tokens, chunk=chunk, n_steps=n_steps,
                max_position=max(prompt, int(ctx.max()) + n_steps))


def mixed_step(wl, j, with_chunk=True):
    """Step j of the mixed workload: (slots, tables, ctx_lens, n_new, tokens,
    want_token) -- the chunk at offset j * chunk first, then every decode row
    at its context + j."""
    n_dec, ch = len(wl["ctx"]), wl["chunk"]
    seqs = ([0] if with_chunk else []) + list(range(1, n_dec + 1))
    ctx = ([j * ch] if with_chunk else []) + [int(c) + j for c in wl["ctx"]]
    nn = ([ch] if with_chunk else []) + [1] * n_dec
    toks = (list(wl["prompt"][j * ch:(j + 1) * ch]) if with_chunk else []) + \
        [int(t) for t in wl["dec_tokens"][j]]
    want = ([int(j == wl["n_steps"] - 1)] if with_chunk else []) + [1] * n_dec
    return seqs, wl["tables"][seqs], ctx, nn, toks, want


def bench_mixed8b(args):
    print(json.dumps(run_mixed8b(max(args.steps, 8))), flush=True)


def run_int8_weights(steps, warmup, batches=(1, 8, 32, 64)):
    """The headline step (one 8B-shaped layer + LM head, contexts U[512,
    4096], greedy) with int8 weights: every projection and the LM head as
    int8 codes with a float32 scale per row, the same KV cache. W falls from
    1.49 to 0.74 GB per step."""
    import torch
    from continuous_batching_decode_forward_amd import binding as B
    from continuous_batching_decode_forward_amd import configs, synth
    from continuous_batching_decode_forward_amd.engine import Engine
    shape, seed = configs.LLAMA8B_1L, 0
    stream = torch.cuda.current_stream()
    log(f"[bench] int8 weights {shape.name} on GPU")
    wg = synth.make_weights_int8(shape, seed=seed, device="cuda")
    Bmax = max(batches)
    wl = build_workload(shape, Bmax, seed)
    eng = Engine(shape, wg, block_size=wl["bs"], num_blocks=wl["total"],
                 max_blocks_per_seq=wl["mbps"], max_slots=Bmax, max_rows=Bmax, max_seqs=Bmax,
                 max_position=4097)
    fill_pool(eng, seed, wl["perm"])
    torch.cuda.synchronize()
    out = {"workload": "8b-layer+lmhead-decode-int8-weights", "weights": "int8 + fp32 row scales",
           "weight_bytes": synth.weight_bytes(shape, True), "sweep": []}
    for Bn in batches:
        meta = eng.upload_step(slots=list(range(Bn)), block_tables=wl["tables"][:Bn],
                               ctx_lens=wl["ctx"][:Bn], n_new=[1] * Bn, tokens=wl["tokens"][:Bn],
                               want_token=[1] * Bn)
        lg = torch.empty((Bn, shape.vocab), dtype=torch.float32, device="cuda")
        tk = torch.empty(Bn, dtype=torch.int32, device="cuda")
        ms, _, _ = time_steps(eng, meta, lg, tk, steps, warmup, stream)
        _, _, k = time_steps(eng, meta, lg, tk, 5, 1, stream, profile_class=B.CBD_KERNEL_LM_HEAD)
        if eng.status():
            raise RuntimeError("device status set")
        byts = step_bytes(shape, wl["ctx"][:Bn], Bn, w_int8=True)
        gbs = byts / (ms * 1e-3) / 1e9
        out["sweep"].append({"batch": Bn, "ms_per_step": ms, "tokens_per_s": Bn / (ms * 1e-3),
                             "step_algorithmic_bytes": byts, "hbm_gbs": gbs,
                             "roofline_frac": gbs / PEAK_HBM_GBS,
                             "lm_head_us": round(k[0] * 1e3, 1)})
        log(f"[bench] int8 weights B={Bn}: {ms:.3f} ms/step, {Bn / (ms * 1e-3):.0f} tok/s, "
            f"{gbs:.0f} GB/s; LM head {k[0] * 1e3:.1f} us")
    eng.close()
    del eng, wg
    torch.cuda.empty_cache()
    return out


def vendor_gemm_reference(shape, rows, reps=20):
    """The vendor BLAS (torch.nn.functional.linear on bf16 operands, which
    ROCm serves with hipBLASLt) at the layer projections' shapes, timed with HIP
    events at `rows` rows and at twice as many. The second is the executed
    MFMA work of this library's dense GEMM over `rows` rows, whose fp32
    activations enter as two bf16 planes (hi + lo). A comparison point for
    the dense path only; nothing of the step runs through it."""
    import torch
    import torch.nn.functional as F
    d, hd = shape.d_model, shape.head_dim
    shapes = {"qkv": ((shape.n_heads + 2 * shape.n_kv_heads) * hd, d),
              "o": (d, shape.n_heads * hd), "gateup": (2 * shape.ffn_dim, d),
              "down": (d, shape.ffn_dim)}
    out = {}
    g = torch.Generator(device="cuda").manual_seed(0)
    for name, (N, K) in shapes.items():
        w = (torch.randn(N, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        for M in (rows, 2 * rows):
            x = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
            for _ in range(3):
                y = F.linear(x, w)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                y = F.linear(x, w)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / reps * 1e3
            out[f"{name}_{M}rows_us"] = round(us, 1)
            out[f"{name}_{M}rows_pflops"] = round(2 * M * N * K / (us * 1e-6) / 1e15, 3)
            del x, y
        del w
    torch.cuda.empty_cache()
    return out


def run_mixed8b(reps):
    """The mixed step on the full 8B shape (32 layers, d_model 4096, 32/8
    heads, FFN 14336, vocab 128256): 48 decode rows with contexts uniform in
    1024..8192 plus one 512-token chunk of a 4096-token prompt, 560 rows per
    step, 32-position blocks; the prompt runs as 8 consecutive steps
    (offsets 0..3584). Each step is timed as it is and without its chunk (the
    same 48 decode rows alone); the difference is the chunk's time."""
    import torch
    from continuous_batching_decode_forward_amd import binding as B
    from continuous_batching_decode_forward_amd import configs, synth
    from continuous_batching_decode_forward_amd.engine import Engine
    shape, wlc = configs.LLAMA8B, configs.MIXED_8B
    seed = 0
    stream = torch.cuda.current_stream()
    log(f"[bench] weights {shape.name} on GPU")
    wg = synth.make_weights(shape, seed=seed, device="cuda")
    wl = build_mixed(shape, seed, n_dec=wlc.batch[0], ctx_range=wlc.ctx_range, bs=wlc.block_size)
    n_dec = len(wl["ctx"])
    eng = Engine(shape, wg, block_size=wl["bs"], num_blocks=wl["total"],
                 max_blocks_per_seq=wl["mbps"], max_slots=n_dec + 1, max_rows=wl["chunk"] + n_dec,
                 max_seqs=n_dec + 1, max_position=wl["max_position"])
    log(f"[bench] filling {len(wl['cached'])} KV blocks "
        f"({len(wl['cached']) * shape.kv_bytes_per_pos * wl['bs'] / 1e9:.1f} GB)")
    fill_pool(eng, seed, wl["cached"])
    tk = torch.empty(n_dec + 1, dtype=torch.int32, device="cuda")
    d, hq, hd, L = shape.d_model, shape.n_heads, shape.head_dim, shape.n_layers
    ws = synth.weight_shapes(shape)
    lin = 2 * L * sum(int(np.prod(ws[k])) for k in ("w_qkv", "w_o", "w_gate", "w_up", "w_down"))
    rows = []
    for j in range(wl["n_steps"]):
        seqs, tab, ctx, nn, toks, want = mixed_step(wl, j)
        meta = eng.upload_step(slots=seqs, block_tables=tab, ctx_lens=ctx, n_new=nn, tokens=toks,
                               want_token=want)
        ms_mixed, _, _ = time_steps(eng, meta, None, tk, reps, 1, stream)
        seqs_d, tab_d, ctx_d, nn_d, toks_d, want_d = mixed_step(wl, j, with_chunk=False)
        meta_d = eng.upload_step(slots=seqs_d, block_tables=tab_d, ctx_lens=ctx_d, n_new=nn_d,
                                 tokens=toks_d, want_token=want_d)
        ms_dec, _, _ = time_steps(eng, meta_d, None, tk, reps, 1, stream)
        kern = None
        if j in (0, wl["n_steps"] - 1):  # per-step time of each kernel class, all layers
            kern = {}
            for name in ("ATTN", "QKV", "O", "GATEUP", "DOWN", "ROPE", "NORM", "LM_HEAD"):
                _, _, k = time_steps(eng, meta, None, tk, 3, 0, stream,
                                     profile_class=getattr(B, "CBD_KERNEL_" + name))
                kern[name.lower() + "_ms"] = round(k[0] * k[1] / 3, 3)
        # redo the mixed step last, so the chunk's K/V is in place for step j + 1
        eng.step_forward(meta, None, tk, stream)
        o = j * wl["chunk"]
        attn = sum(4 * hq * hd * (o + i + 1) for i in range(wl["chunk"])) * L
        chunk_flops = wl["chunk"] * lin + attn + (2 * shape.vocab * d if want[0] else 0)
        dec_bytes = step_bytes(shape, ctx_d, n_dec)
        chunk_ms = ms_mixed - ms_dec
        rows.append({"offset": o, "ms_mixed": ms_mixed, "ms_decode_only": ms_dec,
                     "chunk_ms": chunk_ms, "chunk_tflop": chunk_flops / 1e12,
                     "chunk_mfma_util": chunk_flops / (chunk_ms * 1e-3) / 2.5e15 if chunk_ms > 0 else None,
                     "decode_gbs": dec_bytes / (ms_dec * 1e-3) / 1e9})
        if kern:
            rows[-1]["kernel_ms"] = kern
        log(f"[bench] offset {o}: mixed {ms_mixed:.2f} ms, decode-only {ms_dec:.2f} ms")
    torch.cuda.synchronize()
    if eng.status():
        raise RuntimeError("device status set")
    mean = lambda k: float(np.mean([r[k] for r in rows]))
    out = {"workload": wlc.name, "decode_rows": n_dec, "chunk": wl["chunk"], "rows": wl["chunk"] + n_dec,
           "ms_per_step_mean": mean("ms_mixed"), "ms_decode_only_mean": mean("ms_decode_only"),
           "chunk_ms_mean": mean("chunk_ms"),
           "chunk_mfma_util_mean": float(np.mean([r["chunk_mfma_util"] or 0 for r in rows])),
           "decode_gbs_mean": mean("decode_gbs"),
           "decode_roofline_frac": mean("decode_gbs") / PEAK_HBM_GBS,
           "decode_tokens_per_s_mixed": n_dec / (mean("ms_mixed") * 1e-3),
           "reps_per_offset": reps, "steps": rows}
    eng.close()
    del eng, wg
    torch.cuda.empty_cache()
    # This library's dense GEMMs per layer at the step's rows (first offset;
    # gate/up with its split-K sum + SwiGLU pass), beside the vendor BLAS.
    k0 = rows[0]["kernel_ms"]
    out["dense_gemm_per_layer_us"] = {k: round(k0[k + "_ms"] / L * 1e3, 1)
                                      for k in ("qkv", "o", "gateup", "down")}
    out["vendor_gemm_reference"] = vendor_gemm_reference(shape, wl["chunk"] + n_dec)
    return out


def cb_requests(seed, n, vocab, prompt_range=(16, 512), new_range=(2, 300)):
    """A seeded closed-loop request stream: prompt lengths and answer budgets
    uniform in the given ranges, prompt ids uniform over the vocabulary."""
    from continuous_batching_decode_forward_amd import synth
    lens = synth.uniform_ints(seed, "plen", n, *prompt_range)
    news = synth.uniform_ints(seed, "maxnew", n, *new_range)
    return [(i, synth.uniform_ints(seed, f"prompt{i}", int(lens[i]), 0, vocab - 1),
             int(news[i])) for i in range(n)]


def bench_cb2b(args):
    runs = [(int(x), False, 0) for x in args.cb_pacing.split(",")]
    if args.cb_graph:  # graph replay against the same loop eagerly, both with max_ctx rounded
        runs += [(0, False, 256), (0, True, 256)]
    for line in run_cb2b([int(b) for b in args.cb_slots.split(",")], args.cb_steps, runs):
        print(json.dumps(line), flush=True)


def host_enqueue_cost(eng, Bn, ctx=256, n=8):
    """Host time to enqueue one decode step of B rows (contexts `ctx`),
    eagerly (every launch) and as one graph launch (after its recording),
    each over n steps queued back to back; the GPU work is then drained.
    Block contents are whatever the pool holds: only the host side is timed."""
    import torch
    bs = eng.block_size
    nb = -(-(ctx + 1) // bs)
    tables = np.arange(Bn * nb, dtype=np.int32).reshape(Bn, nb) % eng.num_blocks
    meta = eng.upload_step(slots=list(range(Bn)), block_tables=tables, ctx_lens=[ctx] * Bn,
                           n_new=[1] * Bn, tokens=[1] * Bn, want_token=[1] * Bn)
    tk = torch.empty(Bn, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    res = {"workload": "2b-28layer host enqueue cost", "slots": Bn, "ctx": ctx, "steps": n}
    with torch.cuda.stream(s):
        eng.step_forward_graph(meta, None, tk, s)  # recorded here, outside the timing
        s.synchronize()
        for name, fn in (("eager", eng.step_forward), ("graph", eng.step_forward_graph)):
            fn(meta, None, tk, s)
            s.synchronize()
            t0 = time.perf_counter()
            for _ in range(n):
                fn(meta, None, tk, s)
            t1 = time.perf_counter()
            s.synchronize()
            t2 = time.perf_counter()
            res[f"{name}_enqueue_us_per_step"] = 1e6 * (t1 - t0) / n
            res[f"{name}_ms_per_step"] = 1e3 * (t2 - t0) / n
    log(f"[bench] 2B B={Bn} host enqueue per step: eager {res['eager_enqueue_us_per_step']:.0f} us, "
        f"graph {res['graph_enqueue_us_per_step']:.0f} us; queued steps {res['eager_ms_per_step']:.3f} "
        f"vs {res['graph_ms_per_step']:.3f} ms")
    return res


def run_cb2b(slot_counts, n_steps, runs):
    """Continuous batching on the full 2B-shaped decoder (28 layers, d_model
    2048, 16/8 heads, FFN 6144, vocab 151936): B slots, prompts 16..512,
    answers 2..300 tokens (EOS id 0), 32-position blocks, 16 blocks per slot,
    answer blocks reserved at admission, 512-token chunks, 512 + B rows per
    step, a closed-loop queue (never empty), greedy. Each step is one native
    cbd_sched_step (plan, upload, step, tokens back, commit), timed on the
    host clock around the call. Each pacing of prefill against decode runs
    the same request stream: time to first token is taken from a request's
    submission to the end of the step that emitted its first token.
    runs: (pacing, graph replay of decode-only steps, max_ctx rounding of
    decode-only steps). With a graph run, the host's enqueue cost of one
    decode step, eager and graph, is measured too."""
    import torch
    from continuous_batching_decode_forward_amd import configs, synth
    from continuous_batching_decode_forward_amd.engine import ComposerLoop, Engine
    shape, wlc = configs.QWEN2B, configs.CB_2B
    seed, bs, chunk = 0, wlc.block_size, 512
    names = {0: "prefill-first", 1: "albatross", 2: "separate"}
    log(f"[bench] weights {shape.name} on GPU")
    wg = synth.make_weights(shape, seed=seed, device="cuda")
    mbps = -(-(wlc.ctx_range[1] + 300) // bs)
    out = []
    for Bn in slot_counts:
        pool = 16 * Bn
        order = synth.permutation(seed, "blocks", pool).astype(np.int32)
        eng = Engine(shape, wg, block_size=bs, num_blocks=pool, max_blocks_per_seq=mbps,
                     max_slots=Bn, max_rows=chunk + Bn, max_seqs=Bn, max_position=mbps * bs,
                     block_order=order)
        reqs = cb_requests(seed + Bn, 4096, shape.vocab)

        def run(steps, first, pacing, graph, ctx_round):
            loop = ComposerLoop(eng, max_rows=chunk + Bn, chunk_size=chunk, eos_id=0,
                                pacing=pacing, ctx_round=ctx_round, graph_decode=graph)
            if loop.stream is None:  # eager loops step on a side stream too
                loop.stream = torch.cuda.Stream()
            nxt, rec, submitted, ttft = first, [], {}, []
            try:
                for _ in range(steps):
                    while loop.stats().queued < Bn:  # closed loop: the queue never empties
                        rid, prompt, mx = reqs[nxt % len(reqs)]
                        loop.submit(prompt, mx, None, nxt)
                        submitted[nxt] = time.perf_counter()
                        nxt += 1
                    t0 = time.perf_counter()
                    p = loop.step()
                    t1 = time.perf_counter()
                    n = p.n_seqs
                    for i in range(n):
                        if p.want_token[i] and p.step_ids[i] == 0:
                            ttft.append(t1 - submitted.pop(int(p.request_ids[i])))
                    ctx = list(p.ctx_lens[:n]) if p.n_prefill_rows == 0 else []
                    rec.append((t1 - t0, p.n_prefill_rows, p.n_decode_rows, p.n_out, ctx))
                fin = loop.pop_finished()
            finally:
                loop.close()
            return rec, fin, ttft

        for pacing, graph, ctx_round in runs:
            # warm-up on its own composer; closing it frees every slot and block
            run(8, 10_000, pacing, graph, ctx_round)
            torch.cuda.synchronize()
            g0 = eng.graph_stats()
            t0 = time.perf_counter()
            rec, fin, ttft = run(n_steps, 0, pacing, graph, ctx_round)
            wall = time.perf_counter() - t0
            if eng.status():
                raise RuntimeError("device status set")
            gen = sum(r[3] for r in rec)
            dec = [r for r in rec if r[1] == 0 and r[2] > 0]
            mixed = [r for r in rec if r[1] > 0]
            d_time = sum(r[0] for r in dec)
            d_rows = sum(r[2] for r in dec)
            d_bytes = sum(step_bytes(shape, r[4], r[3]) for r in dec)
            tt = np.array(ttft) * 1e3
            g1 = eng.graph_stats()
            line = {"workload": wlc.name, "slots": Bn, "pacing": names[pacing], "steps": n_steps,
                    "graph_replay": bool(graph), "ctx_round": ctx_round,
                    "graphs_recorded": g1[0] - g0[0], "graph_replays": g1[1] - g0[1],
                    "wall_s": wall, "generated_tokens": gen, "tokens_per_s": gen / wall,
                    "finished_requests": len(fin),
                    "ttft_ms": {"n": int(tt.size), "mean": float(tt.mean()) if tt.size else None,
                                "p50": float(np.percentile(tt, 50)) if tt.size else None,
                                "p90": float(np.percentile(tt, 90)) if tt.size else None},
                    "decode_only_steps": len(dec),
                    "decode_ms_per_step": 1e3 * d_time / max(len(dec), 1),
                    "decode_tokens_per_s": d_rows / d_time if d_time else None,
                    "decode_hbm_gbs": d_bytes / d_time / 1e9 if d_time else None,
                    "decode_roofline_frac": d_bytes / d_time / 1e9 / PEAK_HBM_GBS if d_time else None,
                    "mixed_steps": len(mixed),
                    "mixed_ms_per_step": 1e3 * sum(r[0] for r in mixed) / max(len(mixed), 1),
                    "prefill_rows": sum(r[1] for r in rec)}
            log(f"[bench] 2B loop B={Bn} {names[pacing]}{' graph' if graph else ''}"
                f"{f' ctx_round {ctx_round}' if ctx_round else ''}: {line['tokens_per_s']:.0f} tok/s, "
                f"decode {line['decode_ms_per_step']:.3f} ms/step, "
                f"ttft p50 {line['ttft_ms']['p50']}")
            out.append(line)
        if any(g for _, g, _ in runs):
            out.append(host_enqueue_cost(eng, Bn))
        eng.close()
    del wg
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--batch", type=int, default=64)
    ap.add_argument("--sweep", default="1,8,32,64,128,256")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the long-context sampled and the mixed 32-layer workloads")
    ap.add_argument("--mixed-reps", type=int, default=8,
                    help="timed repetitions per chunk offset of the mixed workload")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one 1 GiB device-to-device copy (counter calibration)")
    ap.add_argument("--print-sources-digest", action="store_true")
    ap.add_argument("--workload", default="8b-layer+lmhead-decode",
                    choices=["8b-layer+lmhead-decode", "8b-layer+lmhead65536-b256-sampled",
                             "2b-28layer-continuous-batching",
                             "8b-32layer-mixed-48dec+512chunk"],
                    help="the headline decode sweep (default) or another configured workload")
    ap.add_argument("--kv-fp8", action="store_true",
                    help="the sampled workload over an 8-bit (E4M3) KV cache")
    ap.add_argument("--cb-slots", default="8,32", help="slot counts of the 2B loop workload")
    ap.add_argument("--cb-steps", type=int, default=256, help="steps of the 2B loop workload")
    ap.add_argument("--cb-graph", type=int, default=1,
                    help="also run the loop with graph replay of decode-only steps, against the "
                         "same loop eagerly (both with max_ctx rounded up to 256)")
    ap.add_argument("--cb-pacing", default="0,1,2",
                    help="pacings of the 2B loop workload: 0 prefill first, 1 Albatross, "
                         "2 prefill apart from decode")
    args = ap.parse_args()
    if args.print_sources_digest:
        print(sources_digest())
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the step runs on a single MI355X and this "
              "build has no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from continuous_batching_decode_forward_amd import binding as B
    from continuous_batching_decode_forward_amd import configs, synth
    from continuous_batching_decode_forward_amd.engine import Engine

    if args.workload == "8b-layer+lmhead65536-b256-sampled":
        torch.cuda.set_device(0)
        return bench_sampled(args)
    if args.workload == "8b-32layer-mixed-48dec+512chunk":
        torch.cuda.set_device(0)
        return bench_mixed8b(args)
    if args.workload == "2b-28layer-continuous-batching":
        torch.cuda.set_device(0)
        return bench_cb2b(args)

    shape = configs.LLAMA8B_1L
    seed = 0
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    if args.calibrate_copy:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration copy: 1073741824 bytes read, 1073741824 written")
        del src, dst
        torch.cuda.empty_cache()
    log(f"[bench] weights {shape.name} on GPU")
    wg = synth.make_weights(shape, seed=seed, device="cuda")
    Bmax = max([args.batch] + [int(b) for b in args.sweep.split(",") if b])
    wl = build_workload(shape, Bmax, seed)
    eng = Engine(shape, wg, block_size=wl["bs"], num_blocks=wl["total"],
                 max_blocks_per_seq=wl["mbps"], max_slots=Bmax, max_rows=Bmax, max_seqs=Bmax,
                 max_position=4097)
    log(f"[bench] filling {wl['total']} KV blocks")
    fill_pool(eng, seed, wl["perm"])
    torch.cuda.synchronize()

    def run(Bn, steps, warmup, profile_class=None):
        meta = eng.upload_step(slots=list(range(Bn)), block_tables=wl["tables"][:Bn],
                               ctx_lens=wl["ctx"][:Bn], n_new=[1] * Bn,
                               tokens=wl["tokens"][:Bn], want_token=[1] * Bn)
        lg = torch.empty((Bn, shape.vocab), dtype=torch.float32, device="cuda")
        tk = torch.empty(Bn, dtype=torch.int32, device="cuda")
        ms, wall, kern = time_steps(eng, meta, lg, tk, steps, warmup, stream, profile_class)
        st = eng.status()
        if st:
            raise RuntimeError(f"device status {st:#x}")
        byts = step_bytes(shape, wl["ctx"][:Bn], Bn)
        return ms, wall, kern, byts

    sweep = []
    for b in [int(x) for x in args.sweep.split(",") if x]:
        if b == args.batch:
            continue
        ms, wall, _, byts = run(b, max(10, args.steps // 2), args.warmup)
        gbs = byts / (ms * 1e-3) / 1e9
        sweep.append({"batch": b, "tokens_per_s": b / (ms * 1e-3), "ms_per_step": ms,
                      "hbm_gbs": gbs, "roofline_frac": gbs / PEAK_HBM_GBS})
        log(f"[bench] B={b}: {ms:.3f} ms/step, {b / (ms * 1e-3):.0f} tok/s, {gbs:.0f} GB/s")

    Bn = args.batch
    log(f"[bench] timed: B={Bn}, {args.warmup} warmup + {args.steps} steps")
    ms, wall, kern, byts = run(Bn, args.steps, args.warmup, profile_class=B.CBD_KERNEL_LM_HEAD)
    tokps = Bn / (ms * 1e-3)
    gbs = byts / (ms * 1e-3) / 1e9
    sweep.append({"batch": Bn, "tokens_per_s": tokps, "ms_per_step": ms, "hbm_gbs": gbs,
                  "roofline_frac": gbs / PEAK_HBM_GBS})
    sweep.sort(key=lambda r: r["batch"])
    lm_ms, lm_n = kern
    lm_bytes = lm_head_bytes(shape, Bn)
    # Each kernel class of the same step timed on its own (HIP events around
    # its launches, 10 steps), with its algorithmic bytes where it streams.
    cb = class_bytes(shape, wl["ctx"][:Bn], Bn)
    classes = {}
    for name in ("QKV", "ROPE", "ATTN", "O", "GATEUP", "DOWN", "LM_HEAD", "SAMPLE", "NORM"):
        _, _, k, _ = run(Bn, 10, 2, profile_class=getattr(B, "CBD_KERNEL_" + name))
        key = name.lower()
        us = k[0] * 1e3 * k[1] / 10  # per step
        rec = {"us_per_step": us}
        if key in cb:
            rec["bytes"] = cb[key]
            rec["gbs"] = cb[key] / (us * 1e-6) / 1e9
            rec["frac"] = rec["gbs"] / PEAK_HBM_GBS
        classes[key] = rec
    lm_gbs = lm_bytes / (lm_ms * 1e-3) / 1e9
    log(f"[bench] B={Bn}: {ms:.3f} ms/step ({wall / args.steps * 1e3:.3f} ms wall), "
        f"{tokps:.0f} tok/s, {gbs:.0f} GB/s; LM head {lm_ms * 1e3:.1f} us, {lm_gbs:.0f} GB/s")

    eng.close()
    del eng
    torch.cuda.empty_cache()
    probe = hbm_read_probe()
    log(f"[bench] streaming-read probe: {probe['gbs']:.0f} GB/s "
        f"({probe['frac_of_peak']:.3f} of the 8 TB/s peak)")
    for rec in sweep:
        rec["frac_of_read_probe"] = rec["hbm_gbs"] / probe["gbs"]

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(shape, wg, wl, seed, Bn, args.cpu_seconds)
        log(f"[bench] CPU oracle: {cpu['value']:.3f} tokens/s on {cpu['cores']} threads, "
            f"{cpu['single_thread']['value']:.3f} tokens/s on one ({cpu['cpu_model']})")

    out = {
        "metric": "decode tokens/s per step and HBM GB/s vs (W+B*A)/beta roofline, 8B-shape, 1 GPU",
        "value": tokps,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "8b-layer+lmhead-decode", "batch": Bn, "ctx_range": [512, 4096],
                   "block_size": 32, "greedy": True, "d_model": 4096, "n_heads": 32,
                   "n_kv_heads": 8, "head_dim": 128, "ffn_dim": 14336, "vocab": 128256,
                   "n_layers": 1},
        "hbm_gbs": gbs,
        "step_algorithmic_bytes": byts,
        "step_roofline_frac": gbs / PEAK_HBM_GBS,
        # the same step against the bandwidth a plain stream reaches here
        "step_frac_of_read_probe": gbs / probe["gbs"],
        "roofline": {"bound": "hbm", "kernel": "lm_head_gemm", "achieved": lm_gbs,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": lm_gbs / PEAK_HBM_GBS,
                     "traffic": measured_traffic(Bn), "avg_launch_us": lm_ms * 1e3,
                     "launches": lm_n,
                     "bytes_per_launch": lm_bytes,
                     "frac_of_read_probe": lm_gbs / probe["gbs"]},
        "hbm_read_probe": probe,
        "cpu_baseline": cpu,
        "kernel_classes": classes,
        "sweep": sweep,
    }
    del wg
    torch.cuda.empty_cache()
    if not args.headline_only:
        # The other measured workloads, each timed on its own stream with HIP
        # events like the headline: the KV-dominated sampled step and the
        # 32-layer mixed step (decode rows + a prefill chunk).
        log("[bench] long-context sampled step (B=256, contexts 8k..32k, vocab 65536)")
        out["long_context_sampled"] = run_sampled(max(10, args.steps // 2), 3)
        log(f"[bench] long-context sampled: {out['long_context_sampled']['ms_per_step']:.3f} ms/step, "
            f"{out['long_context_sampled']['roofline_frac']:.3f} of peak")
        log("[bench] the same step over an 8-bit (E4M3) KV cache")
        out["long_context_sampled_e4m3kv"] = run_sampled(max(10, args.steps // 2), 3,
                                                         kv_fp8=True)
        log(f"[bench] long-context sampled, E4M3 cache: "
            f"{out['long_context_sampled_e4m3kv']['ms_per_step']:.3f} ms/step, "
            f"{out['long_context_sampled_e4m3kv']['roofline_frac']:.3f} of peak")
        log("[bench] the headline step with int8 weights")
        out["decode_8b_layer_int8_weights"] = run_int8_weights(max(10, args.steps // 2), 3)
        log("[bench] 32-layer 8B mixed step (48 decode rows + 512-token chunk)")
        out["mixed_8b_32layer"] = run_mixed8b(args.mixed_reps)
        log(f"[bench] mixed: {out['mixed_8b_32layer']['ms_per_step_mean']:.2f} ms/step mean, "
            f"chunk MFMA use {out['mixed_8b_32layer']['chunk_mfma_util_mean']:.3f}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Seeded request streams and composer constants shared by the continuous-
batching tests (the GPU loop tests and the host replay of their attention
schedule), so that both see the same plans."""
from __future__ import annotations

from continuous_batching_decode_forward_amd import configs, synth

# The 2B-shaped 28-layer loop at 8 slots with the workload's constants:
# 32-position blocks, 512-token chunks, 16 blocks per slot, prompts 16..512,
# answers 2..300, EOS id 0, rows = one chunk + every slot.
QWEN = configs.QWEN2B
Q_SLOTS, Q_BS, Q_CHUNK = 8, 32, 512
Q_POOL = 16 * Q_SLOTS
Q_MBPS = -(-(512 + 300) // Q_BS)
Q_ROWS = Q_CHUNK + Q_SLOTS
Q_SEED, Q_REQUESTS, Q_STEPS = 4, 24, 48


def request_stream(seed, n, prompt_range, new_range, vocab, first_prompt=None):
    """n requests (id, prompt ids, max_new): prompt lengths and answer budgets
    uniform over the given inclusive ranges, prompt ids uniform."""
    lens = synth.uniform_ints(seed, "plen", n, *prompt_range)
    if first_prompt is not None:
        lens[0] = first_prompt
    news = synth.uniform_ints(seed, "maxnew", n, *new_range)
    out = []
    for i in range(n):
        toks = synth.uniform_ints(seed, f"prompt{i}", int(lens[i]), 0, vocab - 1)
        out.append((i, [int(t) for t in toks], int(news[i])))
    return out


def qwen_loop_stream():
    """The request stream of the full-size 2B loop test."""
    return request_stream(Q_SEED, Q_REQUESTS, (16, 512), (2, 300), QWEN.vocab, first_prompt=16)

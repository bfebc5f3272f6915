"""Model shapes and synthetic workloads.

Each workload is named by what it is. The model shapes are the
decoder sizes the workloads are quoted on; the step constants (32-position
blocks, 512-token prefill chunks) are Forma's, as Go under the hood
section 20.3.2 reports them, and the scaled-down figure constants
(4 slots, 4-position blocks, 8-token chunks, at most 12 rows per step)
come from the same section's interactive figure.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    rms_eps: float = 1e-5
    rope_base: float = 10000.0

    def with_layers(self, n: int) -> "ModelShape":
        return replace(self, n_layers=n, name=f"{self.name}-L{n}")

    @property
    def kv_bytes_per_pos(self) -> int:
        """K and V bytes of one position across all layers (bf16)."""
        return 2 * self.n_kv_heads * self.head_dim * 2 * self.n_layers


TINY = ModelShape("tiny-2L", 2, 256, 4, 2, 64, 688, 4096)
LLAMA8B_1L = ModelShape("8b-1layer", 1, 4096, 32, 8, 128, 14336, 128256)
LLAMA8B_1L_V64K = ModelShape("8b-1layer-v65536", 1, 4096, 32, 8, 128, 14336, 65536)
QWEN2B = ModelShape("2b-28layer", 28, 2048, 16, 8, 128, 6144, 151936)
LLAMA8B = ModelShape("8b-32layer", 32, 4096, 32, 8, 128, 14336, 128256)


@dataclass(frozen=True)
class SamplingParams:
    temperature: float = 1.0
    top_p: float = 0.3
    top_k: int = 0
    freq_penalty: float = 1.0
    presence_penalty: float = 0.0
    penalty_decay: float = 0.996
    seed: int = 0
    forbidden: tuple = ()  # ids the sampler never draws


@dataclass(frozen=True)
class Workload:
    name: str
    model: ModelShape
    batch: tuple
    ctx_range: tuple
    block_size: int
    greedy: bool = True
    steps: int = 1
    sampling: SamplingParams = field(default_factory=SamplingParams)
    seed: int = 0


# Tiny 2-layer decoder: 4 sequences, prompts of 5..40 tokens, 4-position
# blocks over a shuffled 64-block pool, 20 greedy decode steps.
TINY_DECODE = Workload("tiny-2layer-b4-greedy20", TINY, (4,), (5, 40), 4, steps=20)

# One 8B-shaped layer + LM head, B in {1,8,32,64}, contexts 512..4096,
# 32-position blocks, greedy.
DECODE_8B_LAYER = Workload("8b-layer+lmhead-decode", LLAMA8B_1L, (1, 8, 32, 64),
                           (512, 4096), 32)

# Full 2B-shaped decoder under continuous batching: B in {8, 32} slots,
# prompts 16..512, answers of 2..300 tokens, 256 steps.
CB_2B = Workload("2b-28layer-continuous-batching", QWEN2B, (8, 32), (16, 512), 32,
                 steps=256)

# Full 8B shape, 48 decode rows (contexts 1k..8k) + one 512-token chunk of a
# 4096-token prompt per step, at most 560 rows.
MIXED_8B = Workload("8b-32layer-mixed-48dec+512chunk", LLAMA8B, (48,), (1024, 8192), 32)

# KV-dominated decode: 8B layer + LM head over vocab 65536, B=256, contexts
# 8k..32k, sampler T=1.0, top_p=0.3, top_k=0, freq 1.0, decay 0.996.
SAMPLE_8B_B256 = Workload("8b-layer+lmhead65536-b256-sampled", LLAMA8B_1L_V64K, (256,),
                          (8192, 32768), 32, greedy=False)

WORKLOADS = {w.name: w for w in (TINY_DECODE, DECODE_8B_LAYER, CB_2B, MIXED_8B, SAMPLE_8B_B256)}

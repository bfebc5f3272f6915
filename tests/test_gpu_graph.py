"""The step under HIP graph capture: cbd_step_forward enqueues only kernel
launches on the caller's stream (no allocation, no memset, no host
synchronisation), so a caller can capture one step per shape class and
replay it (the CUDAGraph decode path the RWKV-Runner Albatross article lists
as a follow-up). The captured step is replayed several times, with the
program's own eager work and synchronisations between replays, and every
replay must give the eager step's logits and tokens bit for bit (the step is
idempotent: the same metadata appends the same K/V at the same positions)."""
import numpy as np
import pytest
import torch

import bench
from continuous_batching_decode_forward_amd import configs, synth
from continuous_batching_decode_forward_amd.engine import Engine

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape,B,ctx_range", [(configs.LLAMA8B_1L, 64, (512, 4096)),
                                               (configs.TINY, 6, (5, 300))],
                         ids=["8b-layer-b64", "tiny-b6"])
def test_captured_step_replays_equal_the_eager_step(shape, B, ctx_range):
    torch.cuda.set_device(0)
    wg = synth.make_weights(shape, seed=2, device="cuda")
    wl = bench.build_workload(shape, B, 2, ctx_range=ctx_range, bs=32)
    eng = Engine(shape, wg, block_size=32, num_blocks=wl["total"], max_blocks_per_seq=wl["mbps"],
                 max_slots=B, max_rows=B, max_seqs=B, max_position=wl["max_position"])
    try:
        bench.fill_pool(eng, 2, wl["perm"])
        meta = eng.upload_step(slots=list(range(B)), block_tables=wl["tables"], ctx_lens=wl["ctx"],
                               n_new=[1] * B, tokens=wl["tokens"], want_token=[1] * B)
        s = torch.cuda.Stream()
        lg = torch.empty((B, shape.vocab), dtype=torch.float32, device="cuda")
        tk = torch.empty(B, dtype=torch.int32, device="cuda")
        with torch.cuda.stream(s):
            eng.step_forward(meta, lg, tk, s)  # eager (also sets up every kernel attribute)
        torch.cuda.synchronize()
        ref_lg, ref_tk = lg.clone(), tk.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            eng.step_forward(meta, lg, tk, s)
        torch.cuda.synchronize()
        for rep in range(4):
            lg.fill_(float("nan"))
            tk.fill_(-1)
            junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
            torch.cuda.synchronize()
            with torch.cuda.stream(s):
                g.replay()
            torch.cuda.synchronize()
            assert torch.equal(lg, ref_lg), f"replay {rep}: logits differ"
            assert torch.equal(tk, ref_tk), f"replay {rep}: tokens differ"
            assert float(junk) == float(junk)
        assert eng.status() == 0
    finally:
        eng.close()

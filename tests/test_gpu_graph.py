"""A denoising step captured in a HIP graph (torch.cuda.CUDAGraph on the handle's own
stream) and replayed: every replay, with eager work and synchronisations between the
replays, gives x and v bit for bit equal to the eager step.  The step's kernels take
their arguments (timesteps, pointers, sizes) at capture, so a graph is one step of the
schedule; the boundary and reference passes run eagerly before."""
import numpy as np
import pytest
import torch

import synth
from synth import Grid
from tests.gpu_util import device

pytestmark = pytest.mark.gpu

MINI_BF16 = synth.config(2, cid=212, L=2, D=256, H=2, dh=128, d_a=64, M=7,
                         chunk=Grid(0, 3, 10, 13), ref=Grid(-2, 1, 10, 13), bnd=Grid(-1, 1, 10, 13),
                         steps=2)


@pytest.mark.parametrize("cfg", [synth.TINY_FP32, MINI_BF16], ids=["config1_fp32", "mini_bf16"])
def test_graph_replay_equals_eager_step(cfg):
    from chunked_streaming_dit_amd import DitChunk
    from chunked_streaming_dit_amd.workload import chunk_config, f32, grid_of, upload_weights
    dev = device()
    P = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg, 0)
    s = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(s):
        h = DitChunk(chunk_config(cfg), upload_weights(P, cfg.dtype, dev), dev)
        h.ref_kv_precompute(f32(inp["ref"], dev), grid_of(cfg.ref))
        b = cfg.bnd
        h.boundary_kv_carry(f32(inp["bnd"], dev), grid_of(Grid(0, 1, b.h, b.w)))
        audio = f32(inp["audio"], dev)
        x0 = f32(inp["x_init"], dev)
        x = torch.empty_like(x0)
        v = torch.empty_like(x0)
        g_chunk = grid_of(cfg.chunk)
        t0, t1 = cfg.t_start, cfg.t_start + (cfg.t_end - cfg.t_start) / cfg.steps
        # eager reference
        x.copy_(x0)
        h.step(x, t0, t1, g_chunk, audio=audio, v_out=v)
    s.synchronize()
    x_ref, v_ref = x.clone(), v.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        x.copy_(x0)
    s.synchronize()
    with torch.cuda.graph(graph, stream=s):
        h.step(x, t0, t1, g_chunk, audio=audio, v_out=v)
    for rep in range(3):
        with torch.cuda.stream(s):
            x.copy_(x0)
            v.fill_(float("nan"))
            graph.replay()
        s.synchronize()
        assert torch.equal(x, x_ref), rep
        assert torch.equal(v, v_ref), rep
        # eager work between replays
        with torch.cuda.stream(s):
            x.copy_(x0)
            h.step(x, t0, t1, g_chunk, audio=audio, v_out=v)
        s.synchronize()
        assert torch.equal(x, x_ref), rep
    assert not torch.equal(x_ref, x0)
    h.close()

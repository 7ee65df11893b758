"""Per-block weight streaming (dit_weight_stream): block weights read from pinned host
memory through a device ring of nslot slots give the same results, bit for bit, as the
resident weight table, and match the oracle.

The mini workload has L = 3 blocks, so nslot = 2 cycles a slot through different blocks
within a pass and carries the prefetch across passes (reference, boundary and every
denoising step are passes).
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from synth import Grid
from chunked_streaming_dit_amd import torch_dtype
from tests.gpu_util import TOL, device, rel_err, run_standalone_gpu, schedule

pytestmark = pytest.mark.gpu

MINI = synth.config(2, cid=211, L=3, D=256, H=2, dh=128, d_a=64, M=7,
                    chunk=Grid(0, 3, 10, 13), ref=Grid(-2, 1, 10, 13), bnd=Grid(-1, 1, 10, 13),
                    steps=2)


def _pinned_blocks(P, cfg):
    """Block weights as new pinned host tensors of the compute dtype."""
    td = torch_dtype(cfg.dtype)
    out = {}
    for name, a in P.items():
        if not name.startswith("blk"):
            continue
        t = torch.empty(a.shape, dtype=td, pin_memory=True)
        t.copy_(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(td))
        out[name] = t
    return out


@pytest.fixture(scope="module")
def mini():
    from chunked_streaming_dit_amd.workload import upload_weights
    dev = device()
    P = synth.make_weights(MINI)
    inp = synth.make_inputs(MINI, 0)
    W = upload_weights(P, MINI.dtype, dev)
    x_res, v_res, h = run_standalone_gpu(MINI, P, inp, dev, weights=W)
    h.close()
    return dev, P, inp, W, x_res, v_res


@pytest.mark.parametrize("nslot", [1, 2, 3])
def test_streamed_equals_resident_bitwise(mini, nslot):
    from chunked_streaming_dit_amd import DitChunk
    from chunked_streaming_dit_amd.workload import chunk_config
    dev, P, inp, W, x_res, v_res = mini
    h = DitChunk(chunk_config(MINI), W, dev)
    h.weight_stream(_pinned_blocks(P, MINI), nslot=nslot)
    for rep in range(2):  # the second run starts from a ring left by the first
        x, vs, _ = run_standalone_gpu(MINI, P, inp, dev, handle=h)
        assert np.array_equal(x, x_res), (nslot, rep)
        for a, b in zip(vs, v_res):
            assert np.array_equal(a, b), (nslot, rep)
    h.close()


def test_streamed_modulation_table(mini):
    """The modulation table computed while the block weights stream through the ring
    (it is one more pass over the blocks): the same results, bit for bit, as the
    resident run with the table."""
    from chunked_streaming_dit_amd import DitChunk
    from chunked_streaming_dit_amd.workload import chunk_config
    dev, P, inp, W, _, _ = mini
    table = schedule(MINI)[:-1] + [0.0]
    x_res, v_res, hr = run_standalone_gpu(MINI, P, inp, dev, weights=W, table=table)
    hr.close()
    h = DitChunk(chunk_config(MINI), W, dev)
    h.weight_stream(_pinned_blocks(P, MINI), nslot=2)
    for rep in range(2):
        x, vs, _ = run_standalone_gpu(MINI, P, inp, dev, handle=h, table=table)
        assert np.array_equal(x, x_res), rep
        for a, b in zip(vs, v_res):
            assert np.array_equal(a, b), rep
    h.close()


def test_stream_switching_and_oracle(mini):
    """Streaming on, off, on again with another ring depth: every run equals the
    resident one; the streamed run also matches the oracle."""
    from chunked_streaming_dit_amd import DitChunk
    from chunked_streaming_dit_amd.workload import chunk_config
    dev, P, inp, W, x_res, v_res = mini
    host = _pinned_blocks(P, MINI)
    h = DitChunk(chunk_config(MINI), W, dev)
    for mode in (2, None, 3, 2):
        h.weight_stream(host if mode else None, nslot=mode or 2)
        x, _, _ = run_standalone_gpu(MINI, P, inp, dev, handle=h)
        assert np.array_equal(x, x_res), mode
    h.close()
    ref_kv = O.ref_context(P, MINI, inp["ref"], MINI.ref)
    bkv = O.bnd_context(P, MINI, ref_kv, inp["bnd"], MINI.bnd.h, MINI.bnd.w)
    ctx = [[ref_kv[l], bkv[l]] for l in range(MINI.L)]
    xo, vo = O.chunk_denoise(P, MINI, inp["x_init"], ctx, inp["audio"], None, steps=MINI.steps, record=True)
    errs = [rel_err(a, b) for a, b in zip(v_res, vo)]
    dx = rel_err(x_res - inp["x_init"], xo - inp["x_init"])
    assert max(errs) <= TOL[MINI.dtype] and dx <= TOL[MINI.dtype], (errs, dx)


@pytest.mark.parametrize("audio_first", [True, False], ids=["before_context", "after_context"])
def test_streamed_held_audio(mini, audio_first):
    """Held audio with streamed weights: audio_kv_precompute only holds the features,
    and each block's audio K/V is computed when the next pass (a context pass, or the
    first step) brings the block's weights into the ring.  The chunk equals, bit for bit,
    the resident run with the audio given to every step."""
    from chunked_streaming_dit_amd import AUDIO_HELD, DitChunk
    from chunked_streaming_dit_amd.workload import chunk_config, f32, grid_of
    dev, P, inp, W, x_res, v_res = mini
    h = DitChunk(chunk_config(MINI), W, dev)
    h.weight_stream(_pinned_blocks(P, MINI), nslot=2)
    audio = f32(inp["audio"], dev)
    ts = schedule(MINI)
    for rep in range(2):
        if audio_first:
            h.audio_kv_precompute(audio)
        h.ref_kv_precompute(f32(inp["ref"], dev), grid_of(MINI.ref))
        b = MINI.bnd
        h.boundary_kv_carry(f32(inp["bnd"], dev), grid_of(Grid(0, 1, b.h, b.w)))
        if not audio_first:
            h.audio_kv_precompute(audio)
        x = f32(inp["x_init"], dev)
        v = torch.empty_like(x)
        for k in range(MINI.steps):
            h.step(x, ts[k], ts[k + 1], grid_of(MINI.chunk), audio=AUDIO_HELD, v_out=v)
            torch.cuda.synchronize()
            assert np.array_equal(v.cpu().numpy(), v_res[k]), (rep, k)
        assert np.array_equal(x.cpu().numpy(), x_res), rep
    h.close()

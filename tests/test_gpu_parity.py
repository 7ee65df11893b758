"""End-to-end parity of the C-ABI path (ref_kv_precompute, boundary_kv_carry,
dit_chunk_step) against the f64 oracle on the same seeded inputs.

Compared: the velocity of every step and dx = x_S - x_0 (x itself is dominated by its
exact initial value), max-abs normalised; <= 1e-4 for fp32, <= 2e-2 for bf16.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
import synth
from synth import Grid
from tests.gpu_util import TOL, device, rel_err, run_standalone_gpu, schedule

pytestmark = pytest.mark.gpu

# Small variants that still span several 64/128 tiles with ragged tails.
MINI_BF16 = synth.config(2, cid=202, L=2, D=256, H=2, dh=128, d_a=64, M=7,
                         chunk=Grid(0, 3, 10, 13), ref=Grid(-2, 1, 10, 13), bnd=Grid(-1, 1, 10, 13),
                         steps=2)
MINI_F32 = dataclasses.replace(MINI_BF16, cid=203, dtype="f32", H=4, dh=64)
MINI_F32_DH64 = synth.config(1, cid=204, L=2, chunk=Grid(0, 3, 7, 9), ref=Grid(-2, 1, 7, 9),
                             bnd=Grid(-1, 1, 5, 9), M=5, steps=2, t_start=0.9, t_end=0.3)
MINI_SR = synth.config(4, cid=205, L=2, D=256, H=2, dh=128,
                       chunk=Grid(0, 2, 12, 14), ref=Grid(-2, 1, 12, 14), bnd=Grid(-1, 1, 12, 14),
                       steps=2)


def _check(cfg, steps=None, table=None):
    """GPU chunk vs the oracle; table: timesteps of a modulation table set first."""
    dev = device()
    P = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg, 0)
    xg, vg, _ = run_standalone_gpu(cfg, P, inp, dev, steps=steps, table=table)
    S = cfg.steps if steps is None else steps
    g = cfg.chunk
    ref_kv = O.ref_context(P, cfg, inp["ref"], cfg.ref)
    ctx = [[ref_kv[l]] for l in range(cfg.L)]
    if cfg.bnd is not None:
        bkv = O.bnd_context(P, cfg, ref_kv, inp["bnd"], cfg.bnd.h, cfg.bnd.w)
        ctx = [[ref_kv[l], bkv[l]] for l in range(cfg.L)]
    cond = None
    if cfg.C_c > 0:
        cond = O.upsample2_tokens(inp["cond_lr"], g.frames, g.h, g.w) if cfg.cond_up == 2 else inp["cond"]
    xo, vo = O.chunk_denoise(P, cfg, inp["x_init"], ctx, inp.get("audio"), cond, steps=S, record=True)
    tol = TOL[cfg.dtype]
    errs = [rel_err(a, b) for a, b in zip(vg, vo)]
    dx = rel_err(xg - inp["x_init"], xo - inp["x_init"])
    print(f"{cfg.name} cid={cfg.cid} table={table}: v errs {['%.2e' % e for e in errs]}, dx err {dx:.2e}")
    assert max(errs) <= tol and dx <= tol, (errs, dx)
    return xg, vg


def test_config1_tiny_fp32():
    _check(synth.TINY_FP32)


def test_mini_fp32_multi_tile():
    _check(MINI_F32)


def test_mini_fp32_dh64_partial_boundary():
    _check(MINI_F32_DH64)


def test_mini_bf16_multi_tile():
    _check(MINI_BF16)


def test_mini_super_resolution_bf16():
    _check(MINI_SR)


def test_mini_super_resolution_single_step_bf16():
    """The super-resolution stage in one Euler step 1 -> 0 (x_1 = x_0 - v)."""
    assert MINI_SR.t_start == 1.0 and MINI_SR.t_end == 0.0
    _check(MINI_SR, steps=1)


@pytest.mark.parametrize("cfg", [synth.TINY_FP32, MINI_F32, MINI_F32_DH64, MINI_BF16, MINI_SR],
                         ids=["config1", "mini_f32", "mini_f32_dh64", "mini_bf16", "mini_sr"])
def test_modulation_table_parity(cfg):
    """dit_modulation_table for the schedule and t = 0 (every pass takes its adaLN
    vectors from the table), and a partial table (the context passes and the second step
    from the table, the other steps computed per pass): the chunk matches the oracle."""
    ts = schedule(cfg)
    _check(cfg, table=ts[:-1] + [0.0])
    _check(cfg, table=[0.0] + ts[1:2])


@pytest.mark.parametrize("base", [MINI_BF16, MINI_F32])
def test_modulation_table_bitwise_equals_per_pass(base):
    """The table's vectors are computed with the per-pass arithmetic: the same x and v,
    bit for bit, with the table for the schedule, a partial table, a table holding other
    timesteps only, the cleared table and the schedule in another order."""
    from chunked_streaming_dit_amd.workload import upload_weights
    dev = device()
    P = synth.make_weights(base)
    inp = synth.make_inputs(base, 0)
    W = upload_weights(P, base.dtype, dev)
    x_ref, v_ref, h = run_standalone_gpu(base, P, inp, dev, weights=W)
    ts = schedule(base)
    for table in (ts[:-1] + [0.0], ts[1:2], [0.0, 0.123, 0.7], [], [0.0] + ts[::-1]):
        x, vs, _ = run_standalone_gpu(base, P, inp, dev, handle=h, table=table)
        assert np.array_equal(x, x_ref), table
        for k, (a, b) in enumerate(zip(vs, v_ref)):
            assert np.array_equal(a, b), (table, k)
    h.close()


@pytest.mark.parametrize("base", [MINI_BF16, MINI_F32])
def test_held_audio_kv_bitwise_equals_per_step_audio(base):
    """audio_kv_precompute once per chunk, then every step with DIT_AUDIO_HELD: the same
    x and v, bit for bit, as passing the audio to every step (which the parity tests
    above check against the oracle)."""
    from chunked_streaming_dit_amd import AUDIO_HELD, DitChunk
    from chunked_streaming_dit_amd.workload import chunk_config, f32, grid_of, upload_weights
    dev = device()
    P = synth.make_weights(base)
    inp = synth.make_inputs(base, 0)
    W = upload_weights(P, base.dtype, dev)
    x_ref, v_ref, h = run_standalone_gpu(base, P, inp, dev, weights=W)
    audio = f32(inp["audio"], dev)
    for rep in range(2):
        h.ref_kv_precompute(f32(inp["ref"], dev), grid_of(base.ref))
        b = base.bnd
        h.boundary_kv_carry(f32(inp["bnd"], dev), grid_of(Grid(0, 1, b.h, b.w)))
        h.audio_kv_precompute(audio)
        x = f32(inp["x_init"], dev)
        v = torch.empty_like(x)
        ts = [base.t_start + (base.t_end - base.t_start) * k / base.steps for k in range(base.steps + 1)]
        for k in range(base.steps):
            h.step(x, ts[k], ts[k + 1], grid_of(base.chunk), audio=AUDIO_HELD, v_out=v)
            torch.cuda.synchronize()
            assert np.array_equal(v.cpu().numpy(), v_ref[k]), (rep, k)
        assert np.array_equal(x.cpu().numpy(), x_ref), rep
    h.audio_kv_precompute(None)
    with pytest.raises(Exception):
        h.step(x, 1.0, 0.5, grid_of(base.chunk), audio=AUDIO_HELD)
    h.close()


def test_mini_stream_bf16():
    """Chunked streaming: chunk 0 has no boundary; each later chunk's boundary is the
    previous chunk's final last frame (carried on the GPU)."""
    from chunked_streaming_dit_amd import DitChunk
    from chunked_streaming_dit_amd.workload import chunk_config, f32, grid_of, upload_weights
    dev = device()
    cfg = dataclasses.replace(MINI_BF16, cid=206, bnd=None, n_chunks=3)
    P = synth.make_weights(cfg)
    chunks = [synth.make_inputs(cfg, c) for c in range(cfg.n_chunks)]
    outs = O.stream(P, cfg, chunks, chunks[0]["ref"])
    h = DitChunk(chunk_config(cfg), upload_weights(P, cfg.dtype, dev), dev)
    h.ref_kv_precompute(f32(chunks[0]["ref"], dev), grid_of(cfg.ref))
    g = cfg.chunk
    ts = O.schedule(cfg.steps, cfg.t_start, cfg.t_end)
    prev = None
    for c, inp in enumerate(chunks):
        if prev is None:
            h.boundary_kv_carry(None, grid_of(Grid(0, 0, 0, 0)))
        else:
            h.boundary_kv_carry(prev, grid_of(g))
        x = f32(inp["x_init"], dev)
        for k in range(cfg.steps):
            h.step(x, ts[k], ts[k + 1], grid_of(g), audio=f32(inp["audio"], dev))
        prev = x
        torch.cuda.synchronize()
        err = rel_err(x.cpu().numpy() - inp["x_init"], outs[c] - inp["x_init"])
        print(f"chunk {c}: dx err {err:.2e}")
        assert err <= TOL["bf16"], (c, err)


@pytest.mark.parametrize("base", ["bf16", "f32"])
def test_mini_interp_stream(base):
    """N- and I-chunks in the order N0, N1, I0, N2, I1: I_k attends to
    [reference | N_k's last frame at t = -1 | N_k+1's first frame at t = frames | chunk];
    the boundary call before each N-chunk clears the anchor."""
    from chunked_streaming_dit_amd import DitChunk
    from chunked_streaming_dit_amd.workload import chunk_config, f32, grid_of, upload_weights
    dev = device()
    cfg = dataclasses.replace(MINI_BF16 if base == "bf16" else MINI_F32, cid=207 if base == "bf16" else 208,
                              bnd=None)
    P = synth.make_weights(cfg)
    n_in = [synth.make_inputs(cfg, c) for c in range(3)]
    i_in = [synth.make_inputs(cfg, 100 + k) for k in range(2)]
    n_ref, i_ref = O.interp_stream(P, cfg, n_in, i_in, n_in[0]["ref"])
    h = DitChunk(chunk_config(cfg), upload_weights(P, cfg.dtype, dev), dev)
    h.ref_kv_precompute(f32(n_in[0]["ref"], dev), grid_of(cfg.ref))
    g = cfg.chunk
    ts = O.schedule(cfg.steps, cfg.t_start, cfg.t_end)

    def denoise(inp):
        x = f32(inp["x_init"], dev)
        for k in range(cfg.steps):
            h.step(x, ts[k], ts[k + 1], grid_of(g), audio=f32(inp["audio"], dev))
        return x

    n_gpu, i_gpu = [], []
    for c in range(3):
        if c == 0:
            h.boundary_kv_carry(None, grid_of(Grid(0, 0, 0, 0)))
        else:
            h.boundary_kv_carry(n_gpu[-1], grid_of(g))  # also clears the anchor
        n_gpu.append(denoise(n_in[c]))
        if c >= 1:
            k = c - 1
            h.boundary_kv_carry(n_gpu[k], grid_of(g))
            h.interp_anchor_kv(n_gpu[k + 1], grid_of(g), g.frames)
            i_gpu.append(denoise(i_in[k]))
    torch.cuda.synchronize()
    tol = TOL[cfg.dtype]
    for name, got, want, inps in (("N", n_gpu, n_ref, n_in), ("I", i_gpu, i_ref, i_in)):
        for k, (a, b) in enumerate(zip(got, want)):
            err = rel_err(a.cpu().numpy() - inps[k]["x_init"], b - inps[k]["x_init"])
            print(f"{name}{k}: dx err {err:.2e}")
            assert err <= tol, (name, k, err)


@pytest.mark.parametrize("base", ["bf16", "f32"])
def test_mini_interp_window_stream(base):
    """N0, N1, I0, N2, I1 with the I-chunks under the window reading: I_k is a window of
    F + 2 frames at t = -1 .. F whose first and last frames are reset before every step
    to N_k's last and N_k+1's first frame carried to the step's time (fm_noise_to), seen
    with the reference only; its F middle frames are kept."""
    from chunked_streaming_dit_amd import DitChunk, fm_noise_to
    from chunked_streaming_dit_amd.workload import chunk_config, f32, grid_of, upload_weights
    dev = device()
    cfg = dataclasses.replace(MINI_BF16 if base == "bf16" else MINI_F32, cid=209 if base == "bf16" else 210,
                              bnd=None)
    P = synth.make_weights(cfg)
    n_in = [synth.make_inputs(cfg, c) for c in range(3)]
    i_in = [synth.make_inputs(cfg, 100 + k) for k in range(2)]
    eps = [synth.anchor_noise(cfg, 100 + k) for k in range(2)]
    n_ref, i_ref = O.interp_window_stream(P, cfg, n_in, i_in, eps, n_in[0]["ref"])
    g = cfg.chunk
    hw = g.h * g.w
    F = g.frames
    h = DitChunk(chunk_config(cfg, max_tokens=(F + 2) * hw), upload_weights(P, cfg.dtype, dev), dev)
    h.ref_kv_precompute(f32(n_in[0]["ref"], dev), grid_of(cfg.ref))
    ts = O.schedule(cfg.steps, cfg.t_start, cfg.t_end)
    win = grid_of(Grid(-1, F + 2, g.h, g.w))

    def denoise(inp):
        x = f32(inp["x_init"], dev)
        for k in range(cfg.steps):
            h.step(x, ts[k], ts[k + 1], grid_of(g), audio=f32(inp["audio"], dev))
        return x

    def window(inp, z0, z1, e):
        x = torch.zeros(((F + 2) * hw, cfg.C_p), device=dev)
        x[hw:(F + 1) * hw] = f32(inp["x_init"], dev)
        ed = f32(e, dev)
        audio = f32(inp["audio"], dev)
        for k in range(cfg.steps):
            fm_noise_to(x[:hw], z0, ed[:hw], ts[k])
            fm_noise_to(x[(F + 1) * hw:], z1, ed[hw:], ts[k])
            h.step(x, ts[k], ts[k + 1], win, audio=audio)
        return x[hw:(F + 1) * hw].clone()

    n_gpu, i_gpu = [], []
    for c in range(3):
        if c == 0:
            h.boundary_kv_carry(None, grid_of(Grid(0, 0, 0, 0)))
        else:
            h.boundary_kv_carry(n_gpu[-1], grid_of(g))
        n_gpu.append(denoise(n_in[c]))
        if c >= 1:
            k = c - 1
            h.boundary_kv_carry(None, grid_of(Grid(0, 0, 0, 0)))  # the window sees the reference only
            z0 = n_gpu[k][(F - 1) * hw:].contiguous()
            z1 = n_gpu[k + 1][:hw].contiguous()
            i_gpu.append(window(i_in[k], z0, z1, eps[k]))
    torch.cuda.synchronize()
    tol = TOL[cfg.dtype]
    for name, got, want, inps in (("N", n_gpu, n_ref, n_in), ("I", i_gpu, i_ref, i_in)):
        for k, (a, b) in enumerate(zip(got, want)):
            err = rel_err(a.cpu().numpy() - inps[k]["x_init"], b - inps[k]["x_init"])
            print(f"{name}{k}: dx err {err:.2e}")
            assert err <= tol, (name, k, err)


@pytest.mark.parametrize("base", ["bf16", "f32"])
def test_mini_stream_boundary_by_reuse(base):
    """Three chunks, each chunk's last step carrying its last frame's K/V forward as the
    next boundary (dit_chunk_step_carry), against oracle.stream_reuse."""
    from chunked_streaming_dit_amd import DitChunk
    from chunked_streaming_dit_amd.workload import chunk_config, f32, grid_of, upload_weights
    dev = device()
    cfg = dataclasses.replace(MINI_BF16 if base == "bf16" else MINI_F32, cid=209 if base == "bf16" else 210,
                              bnd=None, n_chunks=3)
    P = synth.make_weights(cfg)
    chunks = [synth.make_inputs(cfg, c) for c in range(cfg.n_chunks)]
    want = O.stream_reuse(P, cfg, chunks, chunks[0]["ref"])
    h = DitChunk(chunk_config(cfg), upload_weights(P, cfg.dtype, dev), dev)
    h.ref_kv_precompute(f32(chunks[0]["ref"], dev), grid_of(cfg.ref))
    h.boundary_kv_carry(None, grid_of(Grid(0, 0, 0, 0)))
    g = cfg.chunk
    ts = O.schedule(cfg.steps, cfg.t_start, cfg.t_end)
    tol = TOL[cfg.dtype]
    for c, inp in enumerate(chunks):
        x = f32(inp["x_init"], dev)
        for k in range(cfg.steps):
            h.step(x, ts[k], ts[k + 1], grid_of(g), audio=f32(inp["audio"], dev),
                   carry_boundary=k == cfg.steps - 1)
        torch.cuda.synchronize()
        err = rel_err(x.cpu().numpy() - inp["x_init"], want[c] - inp["x_init"])
        print(f"chunk {c}: dx err {err:.2e}")
        assert err <= tol, (c, err)


def test_config2_full_size_first_step():
    """The base low-res chunk at its full shape (7800 tokens, keys 1560|1560|7800,
    4 blocks, hidden 1536, 12x128 heads, 50 audio tokens): the first denoising step."""
    _check(synth.BASE_CHUNK, steps=1)


def test_gemm_and_elementwise_timing_counts_every_launch():
    """dit_timing kinds DIT_TIME_GEMM and DIT_TIME_ELEM (with DIT_TIME_ATTN on as well):
    every block Linear and every RMSNorm pass / final layer of the passes is counted with
    its 2 M N K flop or its bytes, with positive durations; results are unchanged bit for
    bit.  (MINI_BF16: bf16, dh 128, 7 audio tokens, so the cross-attention is folded:
    its out-projection has K = H*64; its q Linear carries the softmax epilogue.)"""
    from chunked_streaming_dit_amd.workload import upload_weights
    cfg = MINI_BF16
    dev = device()
    P = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg, 0)
    W = upload_weights(P, cfg.dtype, dev)
    x_ref, v_ref, h = run_standalone_gpu(cfg, P, inp, dev, weights=W)
    h.timing_enable(7)
    x, vs, _ = run_standalone_gpu(cfg, P, inp, dev, handle=h)
    n_att = h.timing_read(0)[0]
    ng, msg, fg = h.timing_read(1)
    ne, mse, be = h.timing_read(2)
    h.timing_enable(False)
    h.close()
    D, L, F, HK, N = cfg.D, cfg.L, cfg.F, cfg.H * 64, cfg.chunk.n
    ctx_n = [cfg.ref.n, cfg.bnd.n]
    # context pass: QKV, out, MLP in, MLP out for blocks 0..L-2, QKV only for the last
    g_ctx = sum((L - 1) * (2 * n * 3 * D * D + 2 * n * D * D + 4 * n * F * D) + 2 * n * 3 * D * D for n in ctx_n)
    g_step = L * (2 * N * 3 * D * D + 2 * N * D * D + 2 * N * D * D + 2 * N * D * HK + 4 * N * F * D)
    assert n_att == 2 * (L - 1) + cfg.steps * L
    assert ng == 2 * (4 * (L - 1) + 1) + cfg.steps * L * 6
    assert fg == g_ctx + cfg.steps * g_step
    elt = 2
    e_ctx = sum((L - 1) * 2 * (n * D * (4 + elt) + 2 * D * 4) + n * D * (4 + elt) + 2 * D * 4 for n in ctx_n)
    e_norms = L * (2 * (N * D * (4 + elt) + 2 * D * 4) + N * D * (4 + elt))
    e_final = N * D * 4 + N * 64 * 4 * 3 + 64 * (D + 1) * elt + 2 * D * 4
    assert ne == 2 * (2 * (L - 1) + 1) + cfg.steps * (3 * L + 1)
    assert be == e_ctx + cfg.steps * (e_norms + e_final)
    assert msg > 0 and mse > 0
    assert np.array_equal(x, x_ref)
    for a, b in zip(vs, v_ref):
        assert np.array_equal(a, b)


def test_attention_timing_counts_every_launch():
    """dit_timing: with timing on, every self-attention launch of a chunk (the context
    passes run blocks 0..L-2, the steps all L blocks) is counted with its 4 n_q n_kv D
    flop and a positive duration, and the chunk's x and v are bit for bit those of an
    untimed run (the timed launch is the same kernel)."""
    from chunked_streaming_dit_amd.workload import upload_weights
    cfg = MINI_BF16
    dev = device()
    P = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg, 0)
    W = upload_weights(P, cfg.dtype, dev)
    x_ref, v_ref, h = run_standalone_gpu(cfg, P, inp, dev, weights=W)
    h.timing_enable(True)
    x, vs, _ = run_standalone_gpu(cfg, P, inp, dev, handle=h)
    count, ms, flop = h.timing_read()
    n_ref, n_bnd, N = cfg.ref.n, cfg.bnd.n, cfg.chunk.n
    D, L = cfg.D, cfg.L
    assert count == 2 * (L - 1) + cfg.steps * L
    want = 4.0 * D * ((L - 1) * (n_ref * n_ref + n_bnd * (n_ref + n_bnd)) + cfg.steps * L * N * (n_ref + n_bnd + N))
    assert flop == want
    assert ms > 0 and ms / count < 100.0
    assert h.timing_read()[0] == 0  # the read opened a new window
    h.timing_enable(False)
    h.close()
    assert np.array_equal(x, x_ref)
    for a, b in zip(vs, v_ref):
        assert np.array_equal(a, b)

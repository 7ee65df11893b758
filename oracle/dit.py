"""Plain float64 implementation of one chunk's flow-matching DiT denoising pass.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Everything is numpy
float64 on the host: no blocking, fusion or reordering beyond what each
definition states, so that every function can be read against its definition.

Page references are to HeyGen, "Avatar inference at scale":
  [arch]  section "The underlying model architecture": a DiT trained with flow
          matching, conditioned on rich reference tokens; long videos are made
          chunk by chunk, the first chunk relying on the static reference only
          and later chunks on boundary data from the previous segment.
  [loop]  section "The streaming framework and pipeline loop": the reference is
          encoded once per request; the audio-to-video stage runs a multi-step
          diffusion pass per chunk, conditioned on the previous chunk's boundary
          frames; the super-resolution stage upscales in a single step.
  [mem]   section "Constant memory over duration": only the static reference
          conditioning and a minimal anchor set persist between chunks.
  [bnd]   section "Boundary continuity and chunk consistency": ordinary N-chunks make
          the timeline and interpolation (I) chunks smooth the transitions; the
          order is N0, N1, I0, N2, I1, ...; an I-chunk is made once the N-chunks on
          both sides are done, from the last frame of the earlier and an early
          frame of the later one as anchors, whose predictions are then discarded.
Readings the pages leave open (they give no block internals) are marked
"reading:".
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "rms_norm", "modulate", "silu", "gelu_tanh", "linear", "timestep_features",
    "conditioning", "block_modulation", "final_modulation", "rope_split",
    "grid_positions", "rope_angles", "rope_apply", "qk_norm", "softmax",
    "attention", "upsample2_tokens", "patch_input", "block_forward",
    "context_pass", "dit_velocity", "euler", "schedule", "chunk_denoise",
    "last_frame", "stream", "W", "ref_context", "bnd_context", "standalone", "velocity_rows",
    "first_frame", "anchor_context", "interp_stream",
    "bnd_reuse_context", "stream_reuse", "mlp", "interp_window", "interp_window_stream",
]

Weights = Dict[str, np.ndarray]


def W(P: Weights, name: str) -> np.ndarray:
    """Fetch a parameter as float64."""
    return np.asarray(P[name], dtype=np.float64)


# ------------------------------------------------------------------ primitives


def rms_norm(x: np.ndarray, eps: float) -> np.ndarray:
    """reading: RMSNorm over the last axis, x / sqrt(mean(x^2) + eps), no affine."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def modulate(u: np.ndarray, shift: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """reading: adaLN modulation u * (1 + scale) + shift, one vector per step."""
    return u * (1.0 + scale) + shift


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def gelu_tanh(x: np.ndarray) -> np.ndarray:
    """reading: GELU, tanh form 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))


def linear(x: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """y = x W^T + b with W stored [out, in]."""
    return x @ w.T + b


# ------------------------------------------------------------------ timestep conditioning


def timestep_features(t: float, width: int = 256) -> np.ndarray:
    """reading: sinusoid of s = 1000 t, [cos(s w_i) || sin(s w_i)], w_i = 10000^(-i/half)."""
    half = width // 2
    s = 1000.0 * float(t)
    freqs = 10000.0 ** (-np.arange(half, dtype=np.float64) / half)
    return np.concatenate([np.cos(s * freqs), np.sin(s * freqs)])


def conditioning(P: Weights, t: float) -> np.ndarray:
    """reading: c = SiLU(Linear(SiLU(Linear(phi(t))))); one global t per step."""
    e = silu(linear(timestep_features(t), W(P, "t1.w"), W(P, "t1.b")))
    return silu(linear(e, W(P, "t2.w"), W(P, "t2.b")))


def block_modulation(P: Weights, l: int, c: np.ndarray) -> List[np.ndarray]:
    """reading: Linear_{D->6D}(c) split into shift_msa, scale_msa, gate_msa,
    shift_mlp, scale_mlp, gate_mlp (in that order)."""
    m = linear(c, W(P, f"blk{l}.mod.w"), W(P, f"blk{l}.mod.b"))
    return list(np.split(m, 6))


def final_modulation(P: Weights, c: np.ndarray) -> List[np.ndarray]:
    """reading: Linear_{D->2D}(c) split into shift_f, scale_f."""
    m = linear(c, W(P, "fmod.w"), W(P, "fmod.b"))
    return list(np.split(m, 2))


# ------------------------------------------------------------------ 3D rotary positions


def rope_split(dh: int) -> Tuple[int, int, int]:
    """reading: head dims per axis (t, h, w): d_h = d_w = 2 floor(dh/6), d_t = rest."""
    d_hw = 2 * (dh // 6)
    return dh - 2 * d_hw, d_hw, d_hw


def grid_positions(t0: int, frames: int, h: int, w: int) -> np.ndarray:
    """(t, y, x) of every token of a frames x h x w grid, row-major; t = t0 + frame.

    reading: positions are chunk-local; the boundary frame sits at t = -1 and the
    reference frame at t = -2, each on its own (y, x) grid."""
    f, y, x = np.meshgrid(np.arange(frames), np.arange(h), np.arange(w), indexing="ij")
    return np.stack([f.ravel() + t0, y.ravel(), x.ravel()], axis=1).astype(np.int64)


def rope_angles(pos: np.ndarray, dh: int, theta: float) -> np.ndarray:
    """Angle of every rotated pair: [n, dh/2].

    reading: pair i of an axis with d_a dims turns by p * theta^(-2i/d_a); the
    first d_t/2 pairs follow t, the next d_h/2 follow y, the last d_w/2 follow x."""
    parts = []
    for axis, d in enumerate(rope_split(dh)):
        i = np.arange(d // 2, dtype=np.float64)
        inv = theta ** (-2.0 * i / d)
        parts.append(pos[:, axis:axis + 1].astype(np.float64) * inv[None, :])
    return np.concatenate(parts, axis=1)


def rope_apply(x: np.ndarray, ang: np.ndarray) -> np.ndarray:
    """Rotate adjacent pairs (2i, 2i+1) of every head: x [n, H, dh], ang [n, dh/2]."""
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def qk_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """reading: per-head RMSNorm over dh times a learned gamma shared by all heads."""
    return rms_norm(x, eps) * gamma


# ------------------------------------------------------------------ attention


def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


QUERY_GROUP = 2048  # query rows per score matrix (bounds memory at full-size workloads)
HEAD_THREADS = 1    # heads computed concurrently (scripts that run full-size workloads raise it)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Per head softmax(q k^T / sqrt(dh)) v.  q [n, H, dh], k/v [m, H, dh] -> [n, H, dh].

    Every query row is its own softmax over all m keys, so the rows are taken
    QUERY_GROUP at a time: the arithmetic of each row is the same, only the size of
    the score matrix held at once changes.  Heads are independent; with HEAD_THREADS > 1
    they are computed by that many threads (one BLAS thread each), with the same
    arithmetic per head."""
    n, H, dh = q.shape
    out = np.empty((n, H, dh), dtype=np.float64)

    def head(hh: int) -> None:
        for r0 in range(0, n, QUERY_GROUP):
            r1 = min(n, r0 + QUERY_GROUP)
            s = (q[r0:r1, hh, :] @ k[:, hh, :].T) / np.sqrt(dh)
            out[r0:r1, hh, :] = softmax(s, axis=1) @ v[:, hh, :]

    if HEAD_THREADS > 1 and H > 1:
        from concurrent.futures import ThreadPoolExecutor

        from threadpoolctl import threadpool_limits
        with threadpool_limits(1), ThreadPoolExecutor(min(HEAD_THREADS, H)) as ex:
            list(ex.map(head, range(H)))
    else:
        for hh in range(H):
            head(hh)
    return out


def _heads(x: np.ndarray, H: int) -> np.ndarray:
    return x.reshape(x.shape[0], H, -1)


# ------------------------------------------------------------------ inputs to the patch embed


def upsample2_tokens(z: np.ndarray, frames: int, h: int, w: int) -> np.ndarray:
    """Nearest 2x upsample in (y, x) of half-resolution latent tokens.

    Tokens carry a (1, 2, 2) patch of channels laid out (c, dy, dx).  Upsampling the
    pixel grid by 2 and re-patchifying gives token (f, y, x), channel (c, dy, dx) =
    low-res token (f, y//2, x//2), channel (c, y%2, x%2), for every dy, dx.
    reading: the super-resolution stage is conditioned on the low-resolution
    latents by channel concatenation."""
    hl, wl = h // 2, w // 2
    C = z.shape[1]
    zc = z.reshape(frames, hl, wl, C // 4, 2, 2)
    out = np.empty((frames, h, w, C // 4, 2, 2), dtype=np.float64)
    for y in range(h):
        for x in range(w):
            src = zc[:, y // 2, x // 2, :, y % 2, x % 2]            # [frames, C/4]
            out[:, y, x, :, :, :] = src[:, :, None, None]
    return out.reshape(frames * h * w, C)


def patch_input(x: np.ndarray, cond: Optional[np.ndarray], C_c: int) -> np.ndarray:
    """[x || cond]; context tokens (cond None) get a zero conditioning half."""
    x = np.asarray(x, dtype=np.float64)
    if C_c == 0:
        return x
    if cond is None:
        cond = np.zeros((x.shape[0], C_c))
    return np.concatenate([x, np.asarray(cond, dtype=np.float64)], axis=1)


# ------------------------------------------------------------------ one DiT block


def block_forward(P: Weights, cfg, l: int, h: np.ndarray, mod: Sequence[np.ndarray],
                  pos: np.ndarray, ctx_kv: Sequence[Tuple[np.ndarray, np.ndarray]],
                  audio: Optional[np.ndarray], kv_only: bool = False):
    """One DiT block over token states h [n, D].

    Keys/values are the read-only context K/V (reference, then boundary), followed
    by the block's own tokens.  Returns (h_out, k, v), with k normalised and rotated.
    With kv_only the block stops after producing k and v (h_out is None).
    reading: self-attention, then audio cross-attention (skipped without audio),
    then the MLP, each pre-normed with a residual; adaLN shift/scale on the
    self-attention and MLP inputs and gates on their outputs [arch, loop]."""
    D, H, eps = cfg.D, cfg.H, cfg.eps
    p = f"blk{l}."
    sh1, sc1, g1, sh2, sc2, g2 = mod
    u = modulate(rms_norm(h, eps), sh1, sc1)
    qkv = linear(u, W(P, p + "qkv.w"), W(P, p + "qkv.b"))
    q, k, v = (_heads(a, H) for a in np.split(qkv, 3, axis=1))
    ang = rope_angles(pos, cfg.dh, cfg.rope_theta)
    q = rope_apply(qk_norm(q, W(P, p + "gq"), eps), ang)
    k = rope_apply(qk_norm(k, W(P, p + "gk"), eps), ang)
    if kv_only:
        return None, k, v
    K = np.concatenate([kk for kk, _ in ctx_kv] + [k], axis=0)
    V = np.concatenate([vv for _, vv in ctx_kv] + [v], axis=0)
    o = attention(q, K, V).reshape(h.shape[0], D)
    h = h + g1 * linear(o, W(P, p + "o.w"), W(P, p + "o.b"))
    if audio is not None and audio.shape[0] > 0:
        a = np.asarray(audio, dtype=np.float64)
        uc = rms_norm(h, eps)
        qc = qk_norm(_heads(linear(uc, W(P, p + "cq.w"), W(P, p + "cq.b")), H), W(P, p + "gcq"), eps)
        kc = qk_norm(_heads(linear(a, W(P, p + "ck.w"), W(P, p + "ck.b")), H), W(P, p + "gck"), eps)
        vc = _heads(linear(a, W(P, p + "cv.w"), W(P, p + "cv.b")), H)
        oc = attention(qc, kc, vc).reshape(h.shape[0], D)
        h = h + linear(oc, W(P, p + "co.w"), W(P, p + "co.b"))
    u = modulate(rms_norm(h, eps), sh2, sc2)
    h = h + g2 * mlp(u, W(P, p + "fc1.w"), W(P, p + "fc1.b"), W(P, p + "fc2.w"), W(P, p + "fc2.b"))
    return h, k, v


MLP_ROW_GROUP = 8192  # token rows per MLP hidden matrix (bounds memory at full-size workloads)


def mlp(u: np.ndarray, w1: np.ndarray, b1: np.ndarray, w2: np.ndarray, b2: np.ndarray) -> np.ndarray:
    """The per-token MLP fc2(GELU(fc1(u))).  Each row is its own computation, so rows
    are taken MLP_ROW_GROUP at a time: only the size of the hidden matrix held at once
    changes."""
    y = np.empty((u.shape[0], w2.shape[0]), dtype=np.float64)
    for r0 in range(0, u.shape[0], MLP_ROW_GROUP):
        r1 = min(u.shape[0], r0 + MLP_ROW_GROUP)
        y[r0:r1] = linear(gelu_tanh(linear(u[r0:r1], w1, b1)), w2, b2)
    return y


# ------------------------------------------------------------------ context K/V passes


def context_pass(P: Weights, cfg, z: np.ndarray, pos: np.ndarray,
                 prior: Sequence[Sequence[Tuple[np.ndarray, np.ndarray]]]):
    """Per-block K/V of clean context tokens z [n, C_p] (reference or boundary).

    reading: context tokens run through the same blocks at t = 0; they see the
    earlier context segments (``prior[l]``: list of (K, V) per block) and
    themselves, never the chunk; no audio.  Their K/V do not depend on the chunk
    or the step, so they are computed once and kept read-only: the reference once
    per request [loop], the boundary once per chunk [arch, loop]."""
    c = conditioning(P, 0.0)
    h = linear(patch_input(z, None, cfg.C_c), W(P, "pe.w"), W(P, "pe.b"))
    out = []
    for l in range(cfg.L):
        mod = block_modulation(P, l, c)
        last = l == cfg.L - 1
        h_next, k, v = block_forward(P, cfg, l, h, mod, pos, list(prior[l]), None, kv_only=last)
        out.append((k, v))
        h = h_next
    return out


# ------------------------------------------------------------------ velocity and Euler


def dit_velocity(P: Weights, cfg, x: np.ndarray, t: float, pos: np.ndarray,
                 ctx: Sequence[Sequence[Tuple[np.ndarray, np.ndarray]]],
                 audio: Optional[np.ndarray], cond: Optional[np.ndarray] = None) -> np.ndarray:
    """Velocity v = DiT(x, t) for the chunk's latent tokens x [N, C_p] [arch].

    ``ctx[l]`` lists the read-only (K, V) of block l's context segments."""
    c = conditioning(P, t)
    h = linear(patch_input(x, cond, cfg.C_c), W(P, "pe.w"), W(P, "pe.b"))
    for l in range(cfg.L):
        h, _, _ = block_forward(P, cfg, l, h, block_modulation(P, l, c), pos, list(ctx[l]), audio)
    sh, sc = final_modulation(P, c)
    u = modulate(rms_norm(h, cfg.eps), sh, sc)
    return linear(u, W(P, "fin.w"), W(P, "fin.b"))


def euler(x: np.ndarray, v: np.ndarray, t: float, t_next: float) -> np.ndarray:
    """Flow-matching Euler update x + (t_next - t) v."""
    return x + (float(t_next) - float(t)) * v


def schedule(steps: int, t_start: float, t_end: float) -> np.ndarray:
    """reading: linear schedule t_k = t_start + (t_end - t_start) k / steps, k = 0..steps."""
    k = np.arange(steps + 1, dtype=np.float64)
    return t_start + (t_end - t_start) * k / steps


def chunk_denoise(P: Weights, cfg, x0: np.ndarray, ctx, audio, cond=None, grid=None,
                  steps: Optional[int] = None, t_start=None, t_end=None, record=False):
    """The multi-step diffusion pass over one chunk [loop]: Euler on the schedule.

    Returns the final latent (and, with record, the list of per-step velocities)."""
    g = grid if grid is not None else cfg.chunk
    pos = grid_positions(0, g.frames, g.h, g.w)
    S = cfg.steps if steps is None else steps
    ts = schedule(S, cfg.t_start if t_start is None else t_start,
                  cfg.t_end if t_end is None else t_end)
    x = np.asarray(x0, dtype=np.float64)
    vs = []
    for k in range(S):
        v = dit_velocity(P, cfg, x, ts[k], pos, ctx, audio, cond)
        vs.append(v)
        x = euler(x, v, ts[k], ts[k + 1])
    return (x, vs) if record else x


def last_frame(x: np.ndarray, frames: int, h: int, w: int) -> np.ndarray:
    """Tokens of the last latent frame of a chunk (the boundary carried forward)."""
    n = h * w
    return np.asarray(x, dtype=np.float64)[(frames - 1) * n:frames * n]


def first_frame(x: np.ndarray, frames: int, h: int, w: int) -> np.ndarray:
    """Tokens of the first latent frame of a chunk (the later interpolation anchor) [bnd].

    reading: of the later N-chunk's first frames, the anchor is its frame 0."""
    n = h * w
    return np.asarray(x, dtype=np.float64)[:n]


def ref_context(P: Weights, cfg, ref: np.ndarray, ref_grid):
    """Reference K/V per block: the reference sees only itself."""
    pos = grid_positions(ref_grid.t0, ref_grid.frames, ref_grid.h, ref_grid.w)
    return context_pass(P, cfg, ref, pos, [[] for _ in range(cfg.L)])


def bnd_context(P: Weights, cfg, ref_kv, bnd: np.ndarray, h: int, w: int):
    """Boundary K/V per block: one frame at t = -1, seeing the reference and itself."""
    pos = grid_positions(-1, 1, h, w)
    return context_pass(P, cfg, bnd, pos, [[ref_kv[l]] for l in range(cfg.L)])


def bnd_reuse_context(P: Weights, cfg, x: np.ndarray, t: float, pos: np.ndarray,
                      ctx: Sequence[Sequence[Tuple[np.ndarray, np.ndarray]]],
                      audio: Optional[np.ndarray], grid, cond: Optional[np.ndarray] = None):
    """Boundary K/V by reuse [arch, loop]: the per-block K and V that a chunk's final
    denoising step (input latent x at time t, context ctx) forms for the tokens of its
    last frame, with K at positions (-1, y, x).

    reading: the alternative to bnd_context.  The pages say the next chunk is
    conditioned on the previous chunk's boundary frames without saying how their K/V
    are formed; here they are not recomputed by a clean pass at t = 0 but taken from
    the last step's own forward pass (input latent and timestep of that step), K
    placed at the boundary's time position.  Block l's K/V are formed from that block's
    input states, exactly as block_forward forms the keys of those rows."""
    g = grid
    D, H, eps = cfg.D, cfg.H, cfg.eps
    c = conditioning(P, t)
    h = linear(patch_input(x, cond, cfg.C_c), W(P, "pe.w"), W(P, "pe.b"))
    hw = g.h * g.w
    rows = slice((g.frames - 1) * hw, g.frames * hw)
    ang_b = rope_angles(grid_positions(-1, 1, g.h, g.w), cfg.dh, cfg.rope_theta)
    out = []
    for l in range(cfg.L):
        mod = block_modulation(P, l, c)
        p = f"blk{l}."
        u = modulate(rms_norm(h[rows], eps), mod[0], mod[1])
        qkv = linear(u, W(P, p + "qkv.w"), W(P, p + "qkv.b"))
        k = rope_apply(qk_norm(_heads(qkv[:, D:2 * D], H), W(P, p + "gk"), eps), ang_b)
        v = _heads(qkv[:, 2 * D:], H)
        out.append((k, v))
        if l + 1 < cfg.L:  # the next block's input states (the last block's output is unused)
            h, _, _ = block_forward(P, cfg, l, h, mod, pos, list(ctx[l]), audio)
    return out


def anchor_context(P: Weights, cfg, ref_kv, bnd_kv, anchor: np.ndarray, h: int, w: int,
                   t_pos: int):
    """Interpolation-anchor K/V per block [bnd]: one frame at t = t_pos, seeing the
    reference, the boundary (if given) and itself.

    reading: both anchors of an I-chunk are context segments like the boundary: the
    earlier N-chunk's last frame is the boundary (t = -1), the later N-chunk's first
    frame is this anchor, placed at t = t_pos = the I-chunk's frame count (the frame
    after the I-chunk's own).  Anchors are never denoised, so the "discarded anchor
    predictions" are simply never formed."""
    pos = grid_positions(t_pos, 1, h, w)
    prior = [[ref_kv[l]] + ([bnd_kv[l]] if bnd_kv is not None else []) for l in range(cfg.L)]
    return context_pass(P, cfg, anchor, pos, prior)


def stream(P: Weights, cfg, chunks: Sequence[Dict[str, np.ndarray]], ref: np.ndarray,
           record: bool = False):
    """Chunked generation [arch, loop, mem]: reference K/V once, then per chunk the
    boundary K/V from the previous chunk's last frame (none for chunk 0), then the
    multi-step pass.  Returns the final latent of every chunk (with record, also the
    list of every chunk's per-step velocities)."""
    g = cfg.chunk
    ref_kv = ref_context(P, cfg, ref, cfg.ref)
    outs, vels = [], []
    prev = None
    for inp in chunks:
        if prev is None:
            ctx = [[ref_kv[l]] for l in range(cfg.L)]
        else:
            bkv = bnd_context(P, cfg, ref_kv, last_frame(prev, g.frames, g.h, g.w), g.h, g.w)
            ctx = [[ref_kv[l], bkv[l]] for l in range(cfg.L)]
        cond = None
        if cfg.C_c > 0:
            cond = (upsample2_tokens(inp["cond_lr"], g.frames, g.h, g.w)
                    if cfg.cond_up == 2 else inp["cond"])
        x, vs = chunk_denoise(P, cfg, inp["x_init"], ctx, inp.get("audio"), cond, record=True)
        outs.append(x)
        vels.append(vs)
        prev = x
    return (outs, vels) if record else outs


def stream_reuse(P: Weights, cfg, chunks: Sequence[Dict[str, np.ndarray]], ref: np.ndarray):
    """stream() with the boundary carried by reuse: chunk c > 0 is conditioned on the K/V
    that chunk c-1's last denoising step formed for its last frame (bnd_reuse_context).
    Returns the final latent of every chunk."""
    g = cfg.chunk
    pos = grid_positions(0, g.frames, g.h, g.w)
    ref_kv = ref_context(P, cfg, ref, cfg.ref)
    ts = schedule(cfg.steps, cfg.t_start, cfg.t_end)
    outs = []
    carried = None
    for inp in chunks:
        ctx = [[ref_kv[l]] + ([carried[l]] if carried is not None else []) for l in range(cfg.L)]
        cond = None
        if cfg.C_c > 0:
            cond = (upsample2_tokens(inp["cond_lr"], g.frames, g.h, g.w)
                    if cfg.cond_up == 2 else inp["cond"])
        audio = inp.get("audio")
        x = np.asarray(inp["x_init"], dtype=np.float64)
        for k in range(cfg.steps):
            if k == cfg.steps - 1:
                carried = bnd_reuse_context(P, cfg, x, ts[k], pos, ctx, audio, g, cond)
            x = euler(x, dit_velocity(P, cfg, x, ts[k], pos, ctx, audio, cond), ts[k], ts[k + 1])
        outs.append(x)
    return outs


def interp_stream(P: Weights, cfg, n_chunks: Sequence[Dict[str, np.ndarray]],
                  i_chunks: Sequence[Dict[str, np.ndarray]], ref: np.ndarray):
    """N- and I-chunks in the order N0, N1, I0, N2, I1, ... [bnd].

    N-chunks run as in stream() (boundary from the previous N-chunk's last frame).
    I-chunk k runs once N_k and N_k+1 are done: boundary = last frame of N_k
    (t = -1), anchor = first frame of N_k+1 (t = frames), keys
    [reference | boundary | anchor | chunk].  i_chunks[k] supplies x_init / audio /
    conditioning of I_k; needs len(i_chunks) == len(n_chunks) - 1.
    Returns (N-chunk finals, I-chunk finals)."""
    g = cfg.chunk
    ref_kv = ref_context(P, cfg, ref, cfg.ref)
    n_out, i_out = [], []

    def cond_of(inp):
        if cfg.C_c == 0:
            return None
        return upsample2_tokens(inp["cond_lr"], g.frames, g.h, g.w) if cfg.cond_up == 2 else inp["cond"]

    for c, inp in enumerate(n_chunks):
        if c == 0:
            ctx = [[ref_kv[l]] for l in range(cfg.L)]
        else:
            bkv = bnd_context(P, cfg, ref_kv, last_frame(n_out[-1], g.frames, g.h, g.w), g.h, g.w)
            ctx = [[ref_kv[l], bkv[l]] for l in range(cfg.L)]
        n_out.append(chunk_denoise(P, cfg, inp["x_init"], ctx, inp.get("audio"), cond_of(inp)))
        if c >= 1:
            k = c - 1
            bkv = bnd_context(P, cfg, ref_kv, last_frame(n_out[k], g.frames, g.h, g.w), g.h, g.w)
            akv = anchor_context(P, cfg, ref_kv, bkv, first_frame(n_out[k + 1], g.frames, g.h, g.w),
                                 g.h, g.w, g.frames)
            ctx = [[ref_kv[l], bkv[l], akv[l]] for l in range(cfg.L)]
            ic = i_chunks[k]
            i_out.append(chunk_denoise(P, cfg, ic["x_init"], ctx, ic.get("audio"), cond_of(ic)))
    return n_out, i_out


def interp_window(P: Weights, cfg, ref_kv, z_prev: np.ndarray, z_next: np.ndarray,
                  ic: Dict[str, np.ndarray], eps: np.ndarray, record: bool = False):
    """An I-chunk under the window reading of the anchors [bnd].

    reading (the alternative to anchor_context): the anchors are frames of the I-chunk's
    own generation window [earlier N-chunk's last frame | F new frames | later N-chunk's
    first frame], at t = -1, 0..F-1, F.  Before every step the two anchor frames are
    set to their known latents carried to the step's time on the flow-matching path,
    (1 - t) z + t eps (eps: [2 h w, C_p] fixed noise, earlier anchor first); the window
    is denoised as one chunk that sees the reference and itself (no boundary segment);
    at the end the anchor frames, i.e. the model's predictions for them, are dropped.
    Returns the F new frames (with record, also the per-step window velocities)."""
    g = cfg.chunk
    n = g.h * g.w
    F = g.frames
    pos = grid_positions(-1, F + 2, g.h, g.w)
    ctx = [[ref_kv[l]] for l in range(cfg.L)]
    ts = schedule(cfg.steps, cfg.t_start, cfg.t_end)
    z0 = np.asarray(z_prev, dtype=np.float64)
    z1 = np.asarray(z_next, dtype=np.float64)
    e = np.asarray(eps, dtype=np.float64)
    x = np.concatenate([np.zeros((n, cfg.C_p)), np.asarray(ic["x_init"], dtype=np.float64),
                        np.zeros((n, cfg.C_p))], axis=0)
    vs = []
    for k in range(cfg.steps):
        t = float(ts[k])
        x[:n] = (1.0 - t) * z0 + t * e[:n]
        x[(F + 1) * n:] = (1.0 - t) * z1 + t * e[n:]
        v = dit_velocity(P, cfg, x, ts[k], pos, ctx, ic.get("audio"))
        vs.append(v)
        x = euler(x, v, ts[k], ts[k + 1])
    out = x[n:(F + 1) * n]
    return (out, vs) if record else out


def interp_window_stream(P: Weights, cfg, n_chunks: Sequence[Dict[str, np.ndarray]],
                         i_chunks: Sequence[Dict[str, np.ndarray]], eps: Sequence[np.ndarray],
                         ref: np.ndarray):
    """interp_stream() with the I-chunks under the window reading (interp_window): N-chunks
    as in stream(); I-chunk k, once N_k and N_k+1 are done, from N_k's last frame and
    N_k+1's first frame with anchor noise eps[k].  Returns (N-chunk finals, I-chunk
    finals)."""
    assert cfg.C_c == 0, "the window reading is built for chunks without conditioning"
    g = cfg.chunk
    ref_kv = ref_context(P, cfg, ref, cfg.ref)
    n_out, i_out = [], []
    for c, inp in enumerate(n_chunks):
        if c == 0:
            ctx = [[ref_kv[l]] for l in range(cfg.L)]
        else:
            bkv = bnd_context(P, cfg, ref_kv, last_frame(n_out[-1], g.frames, g.h, g.w), g.h, g.w)
            ctx = [[ref_kv[l], bkv[l]] for l in range(cfg.L)]
        n_out.append(chunk_denoise(P, cfg, inp["x_init"], ctx, inp.get("audio")))
        if c >= 1:
            k = c - 1
            i_out.append(interp_window(P, cfg, ref_kv, last_frame(n_out[k], g.frames, g.h, g.w),
                                       first_frame(n_out[k + 1], g.frames, g.h, g.w), i_chunks[k], eps[k]))
    return n_out, i_out


def standalone(P: Weights, cfg, inp: Dict[str, np.ndarray], record: bool = True):
    """One self-contained chunk: reference K/V, the seeded boundary frame's K/V (if the
    workload has one), then the chunk's multi-step pass.

    Returns (x_final, velocities, ref_kv, bnd_kv)."""
    g = cfg.chunk
    ref_kv = ref_context(P, cfg, inp["ref"], cfg.ref)
    bnd_kv = None
    if cfg.bnd is not None:
        bnd_kv = bnd_context(P, cfg, ref_kv, inp["bnd"], cfg.bnd.h, cfg.bnd.w)
        ctx = [[ref_kv[l], bnd_kv[l]] for l in range(cfg.L)]
    else:
        ctx = [[ref_kv[l]] for l in range(cfg.L)]
    cond = None
    if cfg.C_c > 0:
        cond = (upsample2_tokens(inp["cond_lr"], g.frames, g.h, g.w)
                if cfg.cond_up == 2 else inp["cond"])
    x, vs = chunk_denoise(P, cfg, inp["x_init"], ctx, inp.get("audio"), cond, record=True)
    return x, vs, ref_kv, bnd_kv


def velocity_rows(P: Weights, cfg, x: np.ndarray, t: float, pos: np.ndarray,
                  ctx: Sequence[Sequence[Tuple[np.ndarray, np.ndarray]]],
                  audio: Optional[np.ndarray], rows: np.ndarray,
                  cond: Optional[np.ndarray] = None) -> np.ndarray:
    """dit_velocity(...)[rows] for a single-block model (cfg.L == 1), computing the
    query-side path only for the requested rows.

    With one block, a row's velocity depends on the other tokens only through that
    block's keys and values, so K and V are formed for every token while queries,
    attention, MLP and the final layer run for the requested rows alone.  This makes
    sampled checks affordable at full token counts."""
    assert cfg.L == 1, "row-restricted evaluation is exact only for one block"
    D, H, eps = cfg.D, cfg.H, cfg.eps
    c = conditioning(P, t)
    sh1, sc1, g1, sh2, sc2, g2 = block_modulation(P, 0, c)
    h_all = linear(patch_input(x, cond, cfg.C_c), W(P, "pe.w"), W(P, "pe.b"))
    u_all = modulate(rms_norm(h_all, eps), sh1, sc1)
    wqkv, bqkv = W(P, "blk0.qkv.w"), W(P, "blk0.qkv.b")
    ang_all = rope_angles(pos, cfg.dh, cfg.rope_theta)
    k = rope_apply(qk_norm(_heads(linear(u_all, wqkv[D:2 * D], bqkv[D:2 * D]), H), W(P, "blk0.gk"), eps),
                   ang_all)
    v = _heads(linear(u_all, wqkv[2 * D:], bqkv[2 * D:]), H)
    h = h_all[rows]
    q = rope_apply(qk_norm(_heads(linear(u_all[rows], wqkv[:D], bqkv[:D]), H), W(P, "blk0.gq"), eps),
                   ang_all[rows])
    K = np.concatenate([kk for kk, _ in ctx[0]] + [k], axis=0)
    V = np.concatenate([vv for _, vv in ctx[0]] + [v], axis=0)
    o = attention(q, K, V).reshape(len(rows), D)
    h = h + g1 * linear(o, W(P, "blk0.o.w"), W(P, "blk0.o.b"))
    if audio is not None and audio.shape[0] > 0:
        a = np.asarray(audio, dtype=np.float64)
        qc = qk_norm(_heads(linear(rms_norm(h, eps), W(P, "blk0.cq.w"), W(P, "blk0.cq.b")), H),
                     W(P, "blk0.gcq"), eps)
        kc = qk_norm(_heads(linear(a, W(P, "blk0.ck.w"), W(P, "blk0.ck.b")), H), W(P, "blk0.gck"), eps)
        vc = _heads(linear(a, W(P, "blk0.cv.w"), W(P, "blk0.cv.b")), H)
        h = h + linear(attention(qc, kc, vc).reshape(len(rows), D), W(P, "blk0.co.w"), W(P, "blk0.co.b"))
    u = modulate(rms_norm(h, eps), sh2, sc2)
    h = h + g2 * linear(gelu_tanh(linear(u, W(P, "blk0.fc1.w"), W(P, "blk0.fc1.b"))),
                        W(P, "blk0.fc2.w"), W(P, "blk0.fc2.b"))
    shf, scf = final_modulation(P, c)
    return linear(modulate(rms_norm(h, eps), shf, scf), W(P, "fin.w"), W(P, "fin.b"))

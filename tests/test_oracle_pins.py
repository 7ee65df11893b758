"""Pins of the f64 oracle against facts that do not come from the oracle itself.

Each test checks one oracle function against a brute-force formulation, a closed
form, an identity of the mathematics, or an independent library routine, on
tiny shapes.  A plausible slip in the oracle (a dropped term, a wrong sign,
index or operand order) should fail at least one of them.
"""
import dataclasses
import itertools

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O
import synth
from synth import Grid

# A tiny workload with every segment present: 2 blocks, 2 heads of 8, audio.
TINY = synth.config(1, cid=101, L=2, D=16, H=2, dh=8, C_p=8, d_a=6, M=3,
                    chunk=Grid(0, 2, 2, 3), ref=Grid(-2, 1, 2, 3), bnd=Grid(-1, 1, 2, 3),
                    steps=3, t_start=1.0, t_end=0.0)
# Same with half-resolution conditioning (super-resolution form), no audio.
TINY_SR = synth.config(4, cid=104, L=2, D=16, H=2, dh=8, C_p=8, C_c=8, d_a=0, M=0,
                       chunk=Grid(0, 2, 4, 6), ref=Grid(-2, 1, 4, 6), bnd=Grid(-1, 1, 4, 6),
                       steps=2, t_start=1.0, t_end=0.0, dtype="f32")


@pytest.fixture(scope="module")
def tiny():
    return synth.make_weights(TINY), synth.make_inputs(TINY, 0)


def _rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- P1 / P2 attention


def test_p1_attention_matches_triple_loop():
    r = _rng(1)
    n, m, H, dh = 5, 7, 2, 3
    q, k, v = r.standard_normal((n, H, dh)), r.standard_normal((m, H, dh)), r.standard_normal((m, H, dh))
    ref = np.zeros((n, H, dh))
    for h in range(H):
        for i in range(n):
            s = [sum(q[i, h, d] * k[j, h, d] for d in range(dh)) / dh ** 0.5 for j in range(m)]
            mx = max(s)
            e = [np.exp(x - mx) for x in s]
            z = sum(e)
            for d in range(dh):
                ref[i, h, d] = sum(e[j] * v[j, h, d] for j in range(m)) / z
    assert np.abs(O.attention(q, k, v) - ref).max() <= 1e-13


def test_p2_softmax_rows_sum_to_one_and_match_scipy():
    s = _rng(2).standard_normal((9, 13)) * 30.0
    p = O.softmax(s, axis=1)
    assert np.abs(p.sum(axis=1) - 1.0).max() <= 1e-14
    assert np.abs(p - scipy.special.softmax(s, axis=1)).max() <= 1e-15
    assert (p >= 0).all()


def test_attention_heads_in_threads_and_query_groups_change_nothing(monkeypatch):
    """The oracle's attention with heads computed by several threads and queries taken in
    groups smaller than the query count gives the same result as one head and one group
    at a time (each row's arithmetic is the same)."""
    r = _rng(5)
    q, k, v = r.standard_normal((37, 5, 8)), r.standard_normal((23, 5, 8)), r.standard_normal((23, 5, 8))
    want = O.attention(q, k, v)
    import oracle.dit as OD
    monkeypatch.setattr(OD, "HEAD_THREADS", 3)
    monkeypatch.setattr(OD, "QUERY_GROUP", 8)
    got = O.attention(q, k, v)
    assert np.abs(got - want).max() <= 1e-14


def test_mlp_row_groups_change_nothing(monkeypatch):
    """The oracle's MLP taken in row groups smaller than the token count (with a ragged
    last group) gives the same rows as all rows at once, and both are fc2(GELU(fc1(u)))
    row by row."""
    r = _rng(6)
    u = r.standard_normal((29, 12))
    w1, b1 = r.standard_normal((20, 12)), r.standard_normal(20)
    w2, b2 = r.standard_normal((12, 20)), r.standard_normal(12)
    want = O.mlp(u, w1, b1, w2, b2)
    import oracle.dit as OD
    monkeypatch.setattr(OD, "MLP_ROW_GROUP", 8)
    got = O.mlp(u, w1, b1, w2, b2)
    assert np.abs(got - want).max() <= 1e-13
    for i in (0, 7, 8, 28):
        x = u[i] @ w1.T + b1
        g = 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))
        assert np.abs(g @ w2.T + b2 - got[i]).max() <= 1e-12


def test_attention_matches_torch_sdpa_f64():
    r = _rng(3)
    q, k, v = r.standard_normal((6, 3, 4)), r.standard_normal((11, 3, 4)), r.standard_normal((11, 3, 4))
    t = lambda a: torch.from_numpy(a).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v))[0].permute(1, 0, 2).numpy()
    assert np.abs(O.attention(q, k, v) - ref).max() <= 1e-13


# ---------------------------------------------------------------- primitives vs library routines


def test_rmsnorm_p9_and_torch():
    x = _rng(4).standard_normal((7, 33)) * 3.0
    eps = 1e-6
    y = O.rms_norm(x, eps)
    ms = np.mean(x * x, axis=1)
    assert np.abs(np.mean(y * y, axis=1) - ms / (ms + eps)).max() <= 1e-14
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (33,), eps=eps).numpy()
    assert np.abs(y - ref).max() <= 1e-14


def test_gelu_silu_against_library_and_identities():
    x = np.linspace(-8, 8, 4001)
    tx = torch.from_numpy(x)
    assert np.abs(O.gelu_tanh(x) - torch.nn.functional.gelu(tx, approximate="tanh").numpy()).max() <= 1e-14
    assert np.abs(O.gelu_tanh(x) - O.gelu_tanh(-x) - x).max() <= 1e-13
    exact = 0.5 * x * (1 + scipy.special.erf(x / np.sqrt(2)))
    assert np.abs(O.gelu_tanh(x) - exact).max() < 5e-4
    assert np.abs(O.silu(x) - x * scipy.special.expit(x)).max() <= 1e-14
    assert np.abs(O.silu(x) - torch.nn.functional.silu(tx).numpy()).max() <= 1e-14


def test_timestep_features_known_values():
    phi0 = O.timestep_features(0.0)
    assert phi0.shape == (256,)
    assert np.array_equal(phi0[:128], np.ones(128)) and np.array_equal(phi0[128:], np.zeros(128))
    t = 0.37
    phi = O.timestep_features(t)
    # frequency 0 is 1, so the first cos/sin pair is cos(1000 t), sin(1000 t)
    assert abs(phi[0] - np.cos(370.0)) < 1e-12 and abs(phi[128] - np.sin(370.0)) < 1e-12
    # the last frequency is 10000^(-127/128)
    f = 10000.0 ** (-127 / 128)
    assert abs(phi[127] - np.cos(370.0 * f)) < 1e-12 and abs(phi[255] - np.sin(370.0 * f)) < 1e-12
    assert np.abs(phi[:128] ** 2 + phi[128:] ** 2 - 1).max() < 1e-14


def test_block_modulation_split_order():
    D = 4
    c = np.arange(D, dtype=np.float64)
    P = {"blk0.mod.w": np.zeros((6 * D, D)), "blk0.mod.b": np.arange(6 * D, dtype=np.float64)}
    parts = O.block_modulation(P, 0, c)
    for i, p in enumerate(parts):  # shift_msa, scale_msa, gate_msa, shift_mlp, scale_mlp, gate_mlp
        assert np.array_equal(p, np.arange(i * D, (i + 1) * D))
    P = {"fmod.w": np.zeros((2 * D, D)), "fmod.b": np.arange(2 * D, dtype=np.float64)}
    sh, sc = O.final_modulation(P, c)
    assert np.array_equal(sh, np.arange(D)) and np.array_equal(sc, np.arange(D, 2 * D))


# ---------------------------------------------------------------- P8 RoPE


def test_rope_split_values():
    assert O.rope_split(128) == (44, 42, 42)
    assert O.rope_split(64) == (24, 20, 20)
    assert O.rope_split(8) == (4, 2, 2)


def test_grid_positions_enumeration():
    pos = O.grid_positions(-1, 2, 3, 4)
    want = [(t - 1, y, x) for t in range(2) for y in range(3) for x in range(4)]
    assert [tuple(p) for p in pos] == want


def test_p8_rope_axis_pairs_and_identities():
    dh, theta = 64, 10000.0
    dt, dy, dx = O.rope_split(dh)
    # unit vector in one pair; rotate by a position on one axis only
    def rot(pair, pos):
        x = np.zeros((1, 1, dh))
        x[0, 0, 2 * pair] = 1.0
        return O.rope_apply(x, O.rope_angles(np.array([pos]), dh, theta))[0, 0]
    # pair 0 of each axis has frequency 1: the angle equals the coordinate on that axis
    for pair, pos, ang in [(0, (3, 0, 0), 3.0), (dt // 2, (0, 5, 0), 5.0),
                           (dt // 2 + dy // 2, (0, 0, 7), 7.0)]:
        out = rot(pair, pos)
        assert abs(out[2 * pair] - np.cos(ang)) < 1e-14 and abs(out[2 * pair + 1] - np.sin(ang)) < 1e-14
        # another axis's coordinate leaves this pair alone
        other = tuple(0 if i == np.argmax(pos) else 9 for i in range(3))
        assert abs(rot(pair, other)[2 * pair] - 1.0) < 1e-14
    # second t pair turns at theta^(-2/d_t)
    out = rot(1, (4, 0, 0))
    assert abs(out[2] - np.cos(4 * theta ** (-2 / dt))) < 1e-14
    r = _rng(5)
    q = r.standard_normal((10, 3, dh))
    pos = r.integers(-3, 40, size=(10, 3))
    ang = O.rope_angles(pos, dh, theta)
    rq = O.rope_apply(q, ang)
    assert np.abs(np.linalg.norm(rq, axis=-1) - np.linalg.norm(q, axis=-1)).max() < 1e-12
    assert np.abs(O.rope_apply(q, O.rope_angles(np.zeros((10, 3), int), dh, theta)) - q).max() == 0
    # scores depend only on position differences
    k = r.standard_normal((10, 3, dh))
    pk = r.integers(-3, 40, size=(10, 3))
    s1 = np.einsum("nhd,nhd->nh", rq, O.rope_apply(k, O.rope_angles(pk, dh, theta)))
    s2 = np.einsum("nhd,nhd->nh", O.rope_apply(q, O.rope_angles(pos - pk, dh, theta)), k)
    assert np.abs(s1 - s2).max() < 1e-11


def test_upsample2_matches_pixel_space():
    frames, h, w, C = 2, 4, 6, 8
    z = _rng(6).standard_normal((frames * (h // 2) * (w // 2), C))
    # tokens -> low-res pixels [c, f, Y, X]; token (f, Y, X) channel (c, dy, dx) = pixel (c, f, 2Y+dy, 2X+dx)
    c4 = C // 4
    pix = np.zeros((c4, frames, h, w))
    zz = z.reshape(frames, h // 2, w // 2, c4, 2, 2)
    for f, Y, X, c, a, b in itertools.product(range(frames), range(h // 2), range(w // 2), range(c4), range(2), range(2)):
        pix[c, f, 2 * Y + a, 2 * X + b] = zz[f, Y, X, c, a, b]
    up = pix.repeat(2, axis=2).repeat(2, axis=3)          # nearest 2x in pixel space
    tok = np.zeros((frames, h, w, c4, 2, 2))
    for f, y, x, c, a, b in itertools.product(range(frames), range(h), range(w), range(c4), range(2), range(2)):
        tok[f, y, x, c, a, b] = up[c, f, 2 * y + a, 2 * x + b]
    assert np.array_equal(O.upsample2_tokens(z, frames, h, w), tok.reshape(frames * h * w, C))


# ---------------------------------------------------------------- P5 Euler closed form


@pytest.mark.parametrize("lam", [0.0, -0.7, 1.3])
def test_p5_euler_closed_form(lam):
    S, t0, t1 = 8, 1.0, 0.0
    ts = O.schedule(S, t0, t1)
    assert np.allclose(np.diff(ts), (t1 - t0) / S, atol=1e-16, rtol=0)
    x0 = _rng(7).standard_normal(5)
    c = _rng(8).standard_normal(5)
    x = x0.copy()
    for k in range(S):
        x = O.euler(x, lam * x + c, ts[k], ts[k + 1])
    d = (t1 - t0) / S
    if lam == 0.0:
        want = x0 + (t1 - t0) * c
    else:
        g = (1 + lam * d) ** S
        want = g * x0 + c * (g - 1) / lam
    assert np.abs(x - want).max() <= 1e-14 * max(1.0, np.abs(want).max())


# ---------------------------------------------------------------- whole-model pins


def _ctx(P, cfg, inp):
    ref_kv = O.ref_context(P, cfg, inp["ref"], cfg.ref)
    bnd_kv = O.bnd_context(P, cfg, ref_kv, inp["bnd"], cfg.bnd.h, cfg.bnd.w)
    return ref_kv, bnd_kv, [[ref_kv[l], bnd_kv[l]] for l in range(cfg.L)]


def _pos(g):
    return O.grid_positions(g.t0, g.frames, g.h, g.w)


def joint_velocity(P, cfg, segs, audio, t, L=None):
    """Monolithic form: one sequence [ref; bnd; (anchor;) chunk] with a per-token
    timestep (0 for context tokens) and a block-causal mask (a segment sees the
    segments with ids up to its own; the chunk, the highest id, sees everything);
    audio only for chunk rows; every block runs on every token.
    segs: list of (tokens [n, C_in], positions, seg_id, t)."""
    L = cfg.L if L is None else L
    D, H, dh, eps = cfg.D, cfg.H, cfg.dh, cfg.eps
    X = np.concatenate([s[0] for s in segs])
    pos = np.concatenate([s[1] for s in segs])
    seg = np.concatenate([np.full(len(s[0]), s[2]) for s in segs])
    tt = np.concatenate([np.full(len(s[0]), s[3]) for s in segs])
    n = len(X)
    is_chunk = seg == seg.max()
    h = X @ O.W(P, "pe.w").T + O.W(P, "pe.b")
    cvec = {tv: O.conditioning(P, tv) for tv in set(tt.tolist())}
    allowed = seg[None, :] <= seg[:, None]
    ang = O.rope_angles(pos, dh, cfg.rope_theta)
    for l in range(L):
        p = f"blk{l}."
        rows = np.stack([np.concatenate(O.block_modulation(P, l, cvec[tv])) for tv in tt])
        sh1, sc1, g1, sh2, sc2, g2 = (rows[:, i * D:(i + 1) * D] for i in range(6))
        u = O.rms_norm(h, eps) * (1 + sc1) + sh1
        qkv = u @ O.W(P, p + "qkv.w").T + O.W(P, p + "qkv.b")
        q = O.rope_apply(O.qk_norm(qkv[:, :D].reshape(n, H, dh), O.W(P, p + "gq"), eps), ang)
        k = O.rope_apply(O.qk_norm(qkv[:, D:2 * D].reshape(n, H, dh), O.W(P, p + "gk"), eps), ang)
        v = qkv[:, 2 * D:].reshape(n, H, dh)
        o = np.zeros((n, H, dh))
        for hh in range(H):
            s = q[:, hh] @ k[:, hh].T / np.sqrt(dh)
            s = np.where(allowed, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            e = np.exp(s)
            o[:, hh] = (e / e.sum(axis=1, keepdims=True)) @ v[:, hh]
        h = h + g1 * (o.reshape(n, D) @ O.W(P, p + "o.w").T + O.W(P, p + "o.b"))
        if audio is not None:
            hc = h[is_chunk]
            qc = O.qk_norm((O.rms_norm(hc, eps) @ O.W(P, p + "cq.w").T + O.W(P, p + "cq.b")).reshape(-1, H, dh),
                           O.W(P, p + "gcq"), eps)
            kc = O.qk_norm((audio @ O.W(P, p + "ck.w").T + O.W(P, p + "ck.b")).reshape(-1, H, dh),
                           O.W(P, p + "gck"), eps)
            vc = (audio @ O.W(P, p + "cv.w").T + O.W(P, p + "cv.b")).reshape(-1, H, dh)
            oc = np.zeros((len(hc), H, dh))
            for hh in range(H):
                s = qc[:, hh] @ kc[:, hh].T / np.sqrt(dh)
                e = np.exp(s - s.max(axis=1, keepdims=True))
                oc[:, hh] = (e / e.sum(axis=1, keepdims=True)) @ vc[:, hh]
            h[is_chunk] = hc + oc.reshape(-1, D) @ O.W(P, p + "co.w").T + O.W(P, p + "co.b")
        u = O.rms_norm(h, eps) * (1 + sc2) + sh2
        y = O.gelu_tanh(u @ O.W(P, "blk%d.fc1.w" % l).T + O.W(P, p + "fc1.b"))
        h = h + g2 * (y @ O.W(P, p + "fc2.w").T + O.W(P, p + "fc2.b"))
    hc = h[is_chunk]
    c = cvec[segs[-1][3]]
    fm = O.linear(c, O.W(P, "fmod.w"), O.W(P, "fmod.b"))
    u = O.rms_norm(hc, eps) * (1 + fm[D:]) + fm[:D]
    return u @ O.W(P, "fin.w").T + O.W(P, "fin.b")


def test_p3_cached_context_equals_joint_masked(tiny):
    P, inp = tiny
    cfg = TINY
    _, _, ctx = _ctx(P, cfg, inp)
    t = 0.63
    v = O.dit_velocity(P, cfg, inp["x_init"], t, _pos(cfg.chunk), ctx, inp["audio"])
    segs = [(inp["ref"], _pos(cfg.ref), 0, 0.0), (inp["bnd"], _pos(cfg.bnd), 1, 0.0),
            (inp["x_init"], _pos(cfg.chunk), 2, t)]
    vj = joint_velocity(P, cfg, segs, inp["audio"].astype(np.float64), t)
    assert np.abs(v - vj).max() <= 1e-12 * np.abs(vj).max()


def test_p3_super_resolution_form():
    cfg = TINY_SR
    P, inp = synth.make_weights(cfg), synth.make_inputs(cfg, 0)
    _, _, ctx = _ctx(P, cfg, inp)
    g = cfg.chunk
    cond = O.upsample2_tokens(inp["cond_lr"], g.frames, g.h, g.w)
    t = 0.5
    v = O.dit_velocity(P, cfg, inp["x_init"], t, _pos(g), ctx, None, cond)
    z = np.zeros((cfg.N_ref, cfg.C_c))
    segs = [(np.concatenate([inp["ref"], z], 1), _pos(cfg.ref), 0, 0.0),
            (np.concatenate([inp["bnd"], z], 1), _pos(cfg.bnd), 1, 0.0),
            (np.concatenate([inp["x_init"], cond], 1), _pos(g), 2, t)]
    vj = joint_velocity(P, cfg, segs, None, t)
    assert np.abs(v - vj).max() <= 1e-12 * np.abs(vj).max()


def test_p4_single_chunk_stream_equals_unchunked(tiny):
    """One chunk covering every frame, no boundary, through stream(): equals the
    monolithic [ref; all frames] computation integrated with the same Euler loop."""
    P, inp = tiny
    cfg = dataclasses.replace(TINY, bnd=None)
    x_stream = O.stream(P, cfg, [inp], inp["ref"])[0]
    ts = O.schedule(cfg.steps, cfg.t_start, cfg.t_end)
    x = inp["x_init"].astype(np.float64)
    for k in range(cfg.steps):
        segs = [(inp["ref"], _pos(cfg.ref), 0, 0.0), (x, _pos(cfg.chunk), 2, ts[k])]
        x = x + (ts[k + 1] - ts[k]) * joint_velocity(P, cfg, segs, inp["audio"].astype(np.float64), ts[k])
    assert np.abs(x_stream - x).max() <= 1e-12 * np.abs(x).max()


def test_stream_boundary_is_previous_last_frame(tiny):
    """Chunk 1 of a stream equals a standalone chunk whose boundary frame is chunk 0's
    final last frame."""
    P, _ = tiny
    cfg = dataclasses.replace(TINY, bnd=None, steps=2)
    chunks = [synth.make_inputs(TINY, c) for c in range(2)]
    outs = O.stream(P, cfg, chunks, chunks[0]["ref"])
    g = cfg.chunk
    ref_kv = O.ref_context(P, cfg, chunks[0]["ref"], cfg.ref)
    bnd = outs[0][(g.frames - 1) * g.h * g.w:]
    bkv = O.bnd_context(P, cfg, ref_kv, bnd, g.h, g.w)
    x1 = O.chunk_denoise(P, cfg, chunks[1]["x_init"], [[ref_kv[l], bkv[l]] for l in range(cfg.L)],
                         chunks[1]["audio"])
    assert np.abs(x1 - outs[1]).max() == 0.0


def test_p6_constant_velocity_model(tiny):
    P, inp = tiny
    P = dict(P)
    P["fin.w"] = np.zeros_like(P["fin.w"])
    _, _, ctx = _ctx(P, TINY, inp)
    x, vs = O.chunk_denoise(P, TINY, inp["x_init"], ctx, inp["audio"], record=True)
    b = P["fin.b"].astype(np.float64)
    for v in vs:
        assert np.abs(v - b).max() == 0.0
    want = inp["x_init"] + (TINY.t_end - TINY.t_start) * b
    assert np.abs(x - want).max() <= 1e-14


def _gated(P, l, D, gate_msa, gate_mlp):
    P = dict(P)
    P[f"blk{l}.mod.w"] = np.zeros_like(P[f"blk{l}.mod.w"])
    b = np.zeros(6 * D)
    b[2 * D:3 * D] = gate_msa
    b[5 * D:6 * D] = gate_mlp
    P[f"blk{l}.mod.b"] = b
    return P


def test_p7_uniform_attention_counts_each_segment_once(tiny):
    """q = 0 makes every score equal, so attention returns the mean of all value rows
    (reference, boundary and the block's own tokens, each exactly once)."""
    P, inp = tiny
    cfg, D = TINY, TINY.D
    ref_kv, bnd_kv, ctx = _ctx(P, cfg, inp)
    P = _gated(P, 0, D, 1.0, 0.0)            # only the self-attention branch contributes
    w = P["blk0.qkv.w"].astype(np.float64).copy()
    bq = P["blk0.qkv.b"].astype(np.float64).copy()
    w[:D] = 0
    bq[:D] = 0
    P["blk0.qkv.w"], P["blk0.qkv.b"] = w, bq
    h = _rng(9).standard_normal((cfg.N, D))
    mod = O.block_modulation(P, 0, np.zeros(D))
    out, _, _ = O.block_forward(P, cfg, 0, h, mod, _pos(cfg.chunk), ctx[0], None)
    own_v = O.rms_norm(h, cfg.eps) @ w[2 * D:].T + bq[2 * D:]
    allv = np.concatenate([ref_kv[0][1].reshape(-1, D), bnd_kv[0][1].reshape(-1, D), own_v])
    assert len(allv) == cfg.N_ref + cfg.N_bnd + cfg.N
    want = h + allv.mean(axis=0) @ P["blk0.o.w"].astype(np.float64).T + P["blk0.o.b"]
    assert np.abs(out - want).max() <= 1e-12


def test_p10_zero_gates_are_identity(tiny):
    P, inp = tiny
    cfg, D = TINY, TINY.D
    _, _, ctx = _ctx(P, cfg, inp)
    P = _gated(P, 1, D, 0.0, 0.0)
    P["blk1.co.w"] = np.zeros_like(P["blk1.co.w"])
    P["blk1.co.b"] = np.zeros_like(P["blk1.co.b"])
    h = _rng(10).standard_normal((cfg.N, D))
    out, _, _ = O.block_forward(P, cfg, 1, h, O.block_modulation(P, 1, np.ones(D)), _pos(cfg.chunk),
                                ctx[1], inp["audio"])
    assert np.array_equal(out, h)


# ---------------------------------------------------------------- interpolation chunks


def _anchor_pos(cfg):
    g = cfg.chunk
    return O.grid_positions(g.frames, 1, g.h, g.w)


def test_interp_cached_context_equals_joint_masked(tiny):
    """An I-chunk's cached [ref | bnd | anchor] K/V give the velocity of the monolithic
    block-causal sequence [ref; bnd; anchor; chunk] (anchor at t = frames, seeing
    ref, bnd and itself)."""
    P, inp = tiny
    cfg = TINY
    anchor = synth.make_inputs(TINY, 5)["bnd"]  # any frame of the grid's h x w size
    ref_kv, bnd_kv, _ = _ctx(P, cfg, inp)
    akv = O.anchor_context(P, cfg, ref_kv, bnd_kv, anchor, cfg.chunk.h, cfg.chunk.w, cfg.chunk.frames)
    ctx = [[ref_kv[l], bnd_kv[l], akv[l]] for l in range(cfg.L)]
    t = 0.41
    v = O.dit_velocity(P, cfg, inp["x_init"], t, _pos(cfg.chunk), ctx, inp["audio"])
    segs = [(inp["ref"], _pos(cfg.ref), 0, 0.0), (inp["bnd"], _pos(cfg.bnd), 1, 0.0),
            (anchor, _anchor_pos(cfg), 2, 0.0), (inp["x_init"], _pos(cfg.chunk), 3, t)]
    vj = joint_velocity(P, cfg, segs, inp["audio"].astype(np.float64), t)
    assert np.abs(v - vj).max() <= 1e-12 * np.abs(vj).max()
    # the anchor matters: without it the velocity differs
    v_no = O.dit_velocity(P, cfg, inp["x_init"], t, _pos(cfg.chunk), [c[:2] for c in ctx], inp["audio"])
    assert np.abs(v - v_no).max() > 1e-6 * np.abs(v).max()


def test_interp_time_shift_invariance(tiny):
    """Shifting every time coordinate (reference, boundary, anchor, chunk) together
    leaves an I-chunk's velocity unchanged."""
    P, inp = tiny
    cfg = TINY
    anchor = synth.make_inputs(TINY, 5)["bnd"]
    def vel(shift):
        sh = np.array([shift, 0, 0])
        rkv = O.context_pass(P, cfg, inp["ref"], _pos(cfg.ref) + sh, [[] for _ in range(cfg.L)])
        bkv = O.context_pass(P, cfg, inp["bnd"], _pos(cfg.bnd) + sh, [[rkv[l]] for l in range(cfg.L)])
        akv = O.context_pass(P, cfg, anchor, _anchor_pos(cfg) + sh, [[rkv[l], bkv[l]] for l in range(cfg.L)])
        ctx = [[rkv[l], bkv[l], akv[l]] for l in range(cfg.L)]
        return O.dit_velocity(P, cfg, inp["x_init"], 0.3, _pos(cfg.chunk) + sh, ctx, inp["audio"])
    v0, v1 = vel(0), vel(-9)
    assert np.abs(v0 - v1).max() <= 1e-11 * np.abs(v0).max()


def test_interp_stream_schedule_and_anchor_frames(tiny):
    """N0, N1, I0, N2, I1: the N-chunks equal stream(); I_k equals one chunk whose
    boundary is N_k's last frame and whose anchor is N_k+1's first frame (rows picked
    here by their grid coordinates), placed at t = frames."""
    P, _ = tiny
    cfg = dataclasses.replace(TINY, bnd=None, steps=1)
    g = cfg.chunk
    n_in = [synth.make_inputs(TINY, c) for c in range(3)]
    i_in = [synth.make_inputs(TINY, 100 + k) for k in range(2)]
    n_out, i_out = O.interp_stream(P, cfg, n_in, i_in, n_in[0]["ref"])
    assert len(n_out) == 3 and len(i_out) == 2
    for a, b in zip(n_out, O.stream(P, cfg, n_in, n_in[0]["ref"])):
        assert np.abs(a - b).max() == 0.0
    pos = _pos(g)
    ref_kv = O.ref_context(P, cfg, n_in[0]["ref"], cfg.ref)
    for k in range(2):
        last = n_out[k][pos[:, 0] == g.frames - 1]
        first = n_out[k + 1][pos[:, 0] == 0]
        bkv = O.context_pass(P, cfg, last, O.grid_positions(-1, 1, g.h, g.w), [[ref_kv[l]] for l in range(cfg.L)])
        akv = O.context_pass(P, cfg, first, O.grid_positions(g.frames, 1, g.h, g.w),
                             [[ref_kv[l], bkv[l]] for l in range(cfg.L)])
        x = O.chunk_denoise(P, cfg, i_in[k]["x_init"], [[ref_kv[l], bkv[l], akv[l]] for l in range(cfg.L)],
                            i_in[k]["audio"])
        assert np.abs(x - i_out[k]).max() == 0.0


# ---------------------------------------------------------------- boundary by reuse


# ---------------------------------------------------------------- I-chunk, window reading

def _window_cfg(steps, t_start):
    return dataclasses.replace(TINY, bnd=None, steps=steps, t_start=t_start, t_end=0.0)


def test_window_velocity_equals_joint_sequence(tiny):
    """The first step of a window I-chunk: its velocity is the monolithic sequence
    [ref; window] with the window at t = -1 .. F (one segment seeing itself and the
    reference) whose anchor frames hold (1 - t) z + t eps; the velocities of the anchor
    rows exist and are then dropped."""
    P, inp = tiny
    cfg = _window_cfg(2, 0.7)
    g = cfg.chunk
    n = g.h * g.w
    z0, z1 = synth.make_inputs(TINY, 5)["bnd"], synth.make_inputs(TINY, 6)["bnd"]
    eps = synth.anchor_noise(TINY, 3)
    ref_kv = O.ref_context(P, cfg, inp["ref"], cfg.ref)
    out, vs = O.interp_window(P, cfg, ref_kv, z0, z1, inp, eps, record=True)
    t = 0.7
    z0, z1, e = (a.astype(np.float64) for a in (z0, z1, eps))
    xw = np.concatenate([(1 - t) * z0 + t * e[:n], inp["x_init"].astype(np.float64), (1 - t) * z1 + t * e[n:]])
    pos = np.concatenate([O.grid_positions(-1, 1, g.h, g.w), _pos(g), O.grid_positions(g.frames, 1, g.h, g.w)])
    segs = [(inp["ref"], _pos(cfg.ref), 0, 0.0), (xw, pos, 1, t)]
    vj = joint_velocity(P, cfg, segs, inp["audio"].astype(np.float64), t)
    assert vs[0].shape == ((g.frames + 2) * n, cfg.C_p)
    assert np.abs(vs[0] - vj).max() <= 1e-12 * np.abs(vj).max()
    assert out.shape == (g.frames * n, cfg.C_p)


def test_window_at_t1_sees_only_anchor_noise(tiny):
    """One step from t = 1: the anchors are pure noise then, so the new frames do not
    depend on the anchor latents; from t = 0.5 they do."""
    P, inp = tiny
    g = TINY.chunk
    z0, z1 = synth.make_inputs(TINY, 5)["bnd"], synth.make_inputs(TINY, 6)["bnd"]
    eps = synth.anchor_noise(TINY, 3)
    for t0, moves in ((1.0, False), (0.5, True)):
        cfg = _window_cfg(1, t0)
        ref_kv = O.ref_context(P, cfg, inp["ref"], cfg.ref)
        a = O.interp_window(P, cfg, ref_kv, z0, z1, inp, eps)
        b = O.interp_window(P, cfg, ref_kv, 3.0 * z1, -z0, inp, eps)
        c = O.interp_window(P, cfg, ref_kv, z0, z1, inp, 2.0 * eps)
        assert (np.abs(a - b).max() > 1e-9) == moves
        assert np.abs(a - c).max() > 1e-9
        assert a.shape == (g.frames * g.h * g.w, cfg.C_p)


def test_window_without_attention_is_per_token(tiny):
    """With every block gated off (the model is then patch embed + final layer, token by
    token) the new frames equal the plain multi-step pass of the I-chunk's own noise:
    the window keeps their rows and order, and the anchors do not reach them."""
    P, inp = tiny
    cfg = _window_cfg(3, 1.0)
    P0 = P
    for l in range(cfg.L):
        P0 = _gated(P0, l, cfg.D, 0.0, 0.0)
    z0, z1 = synth.make_inputs(TINY, 5)["bnd"], synth.make_inputs(TINY, 6)["bnd"]
    eps = synth.anchor_noise(TINY, 3)
    ref_kv = O.ref_context(P0, cfg, inp["ref"], cfg.ref)
    got = O.interp_window(P0, cfg, ref_kv, z0, z1, inp, eps)
    want = O.chunk_denoise(P0, cfg, inp["x_init"], [[ref_kv[l]] for l in range(cfg.L)], inp["audio"])
    assert np.abs(got - want).max() <= 1e-13 * np.abs(want).max()


def test_interp_window_stream_order_and_anchor_frames(tiny):
    """N0, N1, I0, N2, I1 under the window reading: the N-chunks equal stream(); I_k equals
    interp_window with N_k's last frame and N_k+1's first frame (rows picked here by their
    grid coordinates) and its own anchor noise."""
    P, _ = tiny
    cfg = _window_cfg(2, 1.0)
    g = cfg.chunk
    n_in = [synth.make_inputs(TINY, c) for c in range(3)]
    i_in = [synth.make_inputs(TINY, 100 + k) for k in range(2)]
    eps = [synth.anchor_noise(TINY, 100 + k) for k in range(2)]
    n_out, i_out = O.interp_window_stream(P, cfg, n_in, i_in, eps, n_in[0]["ref"])
    assert len(n_out) == 3 and len(i_out) == 2
    for a, b in zip(n_out, O.stream(P, cfg, n_in, n_in[0]["ref"])):
        assert np.abs(a - b).max() == 0.0
    pos = _pos(g)
    ref_kv = O.ref_context(P, cfg, n_in[0]["ref"], cfg.ref)
    for k in range(2):
        last = n_out[k][pos[:, 0] == g.frames - 1]
        first = n_out[k + 1][pos[:, 0] == 0]
        want = O.interp_window(P, cfg, ref_kv, last, first, i_in[k], eps[k])
        assert np.abs(i_out[k] - want).max() == 0.0


def test_bnd_reuse_special_case_equals_clean_boundary_pass(tiny):
    """A one-frame chunk at t0 = 0 whose reference sits one frame earlier (t = -1), run at
    t = 0 without audio, has the relative positions, visibility, timestep and inputs of a
    boundary context pass (frame at -1, reference at -2): its reused K/V equal
    bnd_context's."""
    P, inp = tiny
    cfg = TINY
    g = cfg.chunk
    frame = inp["bnd"]
    ref_kv = O.ref_context(P, cfg, inp["ref"], cfg.ref)                       # reference at t = -2
    want = O.bnd_context(P, cfg, ref_kv, frame, g.h, g.w)                     # frame at t = -1
    ref_m1 = O.ref_context(P, cfg, inp["ref"], Grid(-1, 1, cfg.ref.h, cfg.ref.w))
    g1 = Grid(0, 1, g.h, g.w)
    got = O.bnd_reuse_context(P, cfg, frame, 0.0, _pos(g1), [[ref_m1[l]] for l in range(cfg.L)], None, g1)
    for (k1, v1), (k2, v2) in zip(got, want):
        assert np.abs(k1 - k2).max() <= 1e-12 * np.abs(k2).max()
        assert np.abs(v1 - v2).max() <= 1e-12 * np.abs(v2).max()


def test_bnd_reuse_rows_and_time_shift(tiny):
    """Multi-frame chunk: the reused K/V are the last frame's rows of the keys and values
    each block forms in the step's own forward pass, K turned by -frames on the time axis
    (rope_apply with the angles of a (-frames, 0, 0) offset)."""
    P, inp = tiny
    cfg = TINY
    g = cfg.chunk
    _, _, ctx = _ctx(P, cfg, inp)
    t = 0.37
    got = O.bnd_reuse_context(P, cfg, inp["x_init"], t, _pos(g), ctx, inp["audio"], g)
    c = O.conditioning(P, t)
    h = O.linear(O.patch_input(inp["x_init"], None, cfg.C_c), O.W(P, "pe.w"), O.W(P, "pe.b"))
    hw = g.h * g.w
    shift = O.rope_angles(np.tile([[-g.frames, 0, 0]], (hw, 1)), cfg.dh, cfg.rope_theta)
    for l in range(cfg.L):
        mod = O.block_modulation(P, l, c)
        h_next, k, v = O.block_forward(P, cfg, l, h, mod, _pos(g), list(ctx[l]), inp["audio"])
        k_last = O.rope_apply(k[(g.frames - 1) * hw:], shift)
        assert np.abs(got[l][0] - k_last).max() <= 1e-12 * np.abs(k_last).max()
        assert np.abs(got[l][1] - v[(g.frames - 1) * hw:]).max() == 0.0
        h = h_next


def test_stream_reuse_carries_last_step_input(tiny):
    """stream_reuse, composed by hand: chunk c is chunk_denoise with the context
    [reference, bnd_reuse_context(x_{S-1}, t_{S-1})], where x_{S-1} is chunk c-1's input
    to its LAST denoising step (S-1 Euler steps from its x_init) and t_{S-1} that step's
    time.  A carry from any other step (e.g. the first: x_init at t_0) fails."""
    P, _ = tiny
    cfg = dataclasses.replace(TINY, bnd=None, steps=3)
    chunks = [synth.make_inputs(TINY, c) for c in range(3)]
    got = O.stream_reuse(P, cfg, chunks, chunks[0]["ref"])
    g = cfg.chunk
    pos = _pos(g)
    ts = O.schedule(cfg.steps, cfg.t_start, cfg.t_end)
    ref_kv = O.ref_context(P, cfg, chunks[0]["ref"], cfg.ref)
    carried = None
    for c, inp in enumerate(chunks):
        ctx = [[ref_kv[l]] + ([carried[l]] if carried is not None else []) for l in range(cfg.L)]
        want = O.chunk_denoise(P, cfg, inp["x_init"], ctx, inp["audio"])
        assert np.abs(got[c] - want).max() <= 1e-12 * np.abs(want).max(), c
        x = inp["x_init"].astype(np.float64)
        for k in range(cfg.steps - 1):
            x = x + (ts[k + 1] - ts[k]) * O.dit_velocity(P, cfg, x, ts[k], pos, ctx, inp["audio"])
        carried = O.bnd_reuse_context(P, cfg, x, ts[-2], pos, ctx, inp["audio"], g)
        if c == 0:
            # the carry of the first step's input differs: chunk 1 would change
            first = O.bnd_reuse_context(P, cfg, inp["x_init"], ts[0], pos, ctx, inp["audio"], g)
            other = O.chunk_denoise(P, cfg, chunks[1]["x_init"], [[ref_kv[l], first[l]] for l in range(cfg.L)],
                                    chunks[1]["audio"])
            assert np.abs(other - got[1]).max() > 1e-6 * np.abs(got[1]).max()


def test_qk_norm_per_head_and_gamma_after_normalisation():
    """qk_norm on its own: each head of each row is RMS-normalised over dh, then
    multiplied elementwise by gamma (shared by the heads).
      - scaling one head's input leaves every output unchanged up to eps (a per-head
        normalisation: no other head moves at all);
      - with gamma = g for every entry, mean(y^2) over a head = g^2 ms / (ms + eps);
      - non-uniform gamma against the per-element formula written out with scalar
        loops; a gamma applied before the normalisation (rms_norm(x * gamma)) fails it."""
    r = _rng(31)
    n, H, dh, eps = 3, 4, 6, 1e-6
    x = r.standard_normal((n, H, dh)) * 2.0
    gamma = 1.0 + 0.5 * r.standard_normal(dh)
    y = O.qk_norm(x, gamma, eps)
    x2 = x.copy()
    x2[:, 1, :] *= 7.0
    y2 = O.qk_norm(x2, gamma, eps)
    assert np.abs(np.delete(y2, 1, axis=1) - np.delete(y, 1, axis=1)).max() == 0.0
    assert np.abs(y2[:, 1] - y[:, 1]).max() <= 1e-6 * np.abs(y).max()
    g = 1.7
    yg = O.qk_norm(x, np.full(dh, g), eps)
    ms = np.mean(x * x, axis=-1)
    assert np.abs(np.mean(yg * yg, axis=-1) - g * g * ms / (ms + eps)).max() <= 1e-13
    want = np.empty_like(x)
    for i in range(n):
        for hh in range(H):
            ss = 0.0
            for d in range(dh):
                ss += x[i, hh, d] * x[i, hh, d]
            rinv = 1.0 / (ss / dh + eps) ** 0.5
            for d in range(dh):
                want[i, hh, d] = x[i, hh, d] * rinv * gamma[d]
    assert np.abs(y - want).max() <= 1e-14 * np.abs(want).max()
    slip = O.rms_norm(x * gamma, eps)
    assert np.abs(slip - want).max() > 1e-3


def test_stream_reuse_first_chunk_and_carry(tiny):
    """stream_reuse: chunk 0 equals stream()'s; chunk 1 is conditioned on the K/V of chunk
    0's last step (not on a clean pass), so it differs from stream()'s chunk 1."""
    P, _ = tiny
    cfg = dataclasses.replace(TINY, bnd=None, steps=2)
    chunks = [synth.make_inputs(TINY, c) for c in range(2)]
    a = O.stream_reuse(P, cfg, chunks, chunks[0]["ref"])
    b = O.stream(P, cfg, chunks, chunks[0]["ref"])
    assert np.abs(a[0] - b[0]).max() == 0.0
    assert np.abs(a[1] - b[1]).max() > 1e-6 * np.abs(b[1]).max()


def test_p11_context_key_permutation_invariance(tiny):
    P, inp = tiny
    cfg = TINY
    _, _, ctx = _ctx(P, cfg, inp)
    perm = _rng(11).permutation(cfg.N_ref)
    ctx_p = [[(k[perm], v[perm]) for (k, v) in seg[:1]] + seg[1:] for seg in ctx]
    t = 0.4
    v1 = O.dit_velocity(P, cfg, inp["x_init"], t, _pos(cfg.chunk), ctx, inp["audio"])
    v2 = O.dit_velocity(P, cfg, inp["x_init"], t, _pos(cfg.chunk), ctx_p, inp["audio"])
    assert np.abs(v1 - v2).max() <= 1e-12 * np.abs(v1).max()


def test_p8_time_shift_invariance(tiny):
    """Shifting every token's time coordinate (reference, boundary, chunk) together
    leaves the velocity unchanged: only position differences enter the scores."""
    P, inp = tiny
    cfg = TINY
    def vel(shift):
        sh = np.array([shift, 0, 0])
        rp, bp, cp = _pos(cfg.ref) + sh, _pos(cfg.bnd) + sh, _pos(cfg.chunk) + sh
        rkv = O.context_pass(P, cfg, inp["ref"], rp, [[] for _ in range(cfg.L)])
        bkv = O.context_pass(P, cfg, inp["bnd"], bp, [[rkv[l]] for l in range(cfg.L)])
        ctx = [[rkv[l], bkv[l]] for l in range(cfg.L)]
        return O.dit_velocity(P, cfg, inp["x_init"], 0.7, cp, ctx, inp["audio"])
    v0, v1 = vel(0), vel(17)
    assert np.abs(v0 - v1).max() <= 1e-11 * np.abs(v0).max()


def test_conditioning_structure_special_case():
    """With t1.w = 0 and t2 the identity, c = SiLU(SiLU(t1.b)) for every t, and with
    t1 picking feature 0 (cos 1000 t) the first entry follows that feature."""
    D = 5
    b = np.linspace(-2, 2, D)
    P = {"t1.w": np.zeros((D, 256)), "t1.b": b, "t2.w": np.eye(D), "t2.b": np.zeros(D)}
    for t in (0.0, 0.3, 1.0):
        assert np.abs(O.conditioning(P, t) - O.silu(O.silu(b))).max() == 0.0
    P["t1.w"] = np.zeros((D, 256))
    P["t1.w"][0, 0] = 1.0
    P["t1.b"] = np.zeros(D)
    t = 0.123
    assert abs(O.conditioning(P, t)[0] - O.silu(O.silu(np.cos(123.0)))) < 1e-15


@pytest.mark.parametrize("sr", [False, True])
def test_velocity_rows_equals_full_velocity_one_block(sr):
    """The row-restricted single-block evaluation equals the full computation's rows."""
    cfg = dataclasses.replace(TINY_SR if sr else TINY, L=1)
    P, inp = synth.make_weights(cfg), synth.make_inputs(cfg, 0)
    _, _, ctx = _ctx(P, cfg, inp)
    g = cfg.chunk
    cond = O.upsample2_tokens(inp["cond_lr"], g.frames, g.h, g.w) if sr else None
    audio = None if sr else inp["audio"]
    pos = _pos(g)
    full = O.dit_velocity(P, cfg, inp["x_init"], 0.55, pos, ctx, audio, cond)
    rows = np.array([0, 3, cfg.N - 1, 5])
    part = O.velocity_rows(P, cfg, inp["x_init"], 0.55, pos, ctx, audio, rows, cond)
    assert np.abs(part - full[rows]).max() <= 1e-13 * np.abs(full).max()

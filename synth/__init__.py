"""Seeded synthetic inputs and workload shapes for the chunked streaming DiT step.

This module is shared by the CPU oracle and the GPU path, so it holds no
arithmetic of the method itself: only workload shapes, the tensor catalogue
(names and shapes), seeded Gaussian draws, and the f64 -> f32 -> bf16
round-to-nearest-even cast that turns a draw into the value both sides consume.

The pages (HeyGen, "Avatar inference at scale", section on the model
architecture) describe a flow-matching DiT conditioned on rich reference
tokens, audio features and the previous chunk's boundary frames, but give no
sizes and no weights.  The five workloads below are synthetic stand-ins whose
shapes follow the stated chunk/reference/boundary/audio token counts; values are
N(0, 1/fan_in) weights and N(0, 1) latents and audio features.
"""
from __future__ import annotations

import collections.abc
import dataclasses
import zlib
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = [
    "Grid", "Config", "CONFIGS", "config", "round_bf16", "to_bf16_bits",
    "weight_catalogue", "make_weights", "make_inputs", "GLOBAL_NAMES",
    "BLOCK_NAMES", "Bf16Weights", "from_bf16_bits",
]

# --------------------------------------------------------------------------------------
# workload shapes
# --------------------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Grid:
    """A token grid: frames x h x w tokens, row-major over (frame, y, x).

    ``t0`` is the time coordinate of frame 0.  Token (f, y, x) sits at time
    ``t0 + f``.
    """

    t0: int
    frames: int
    h: int
    w: int

    @property
    def n(self) -> int:
        return self.frames * self.h * self.w


@dataclasses.dataclass(frozen=True)
class Config:
    cid: int
    name: str
    dtype: str            # "f32" or "bf16": storage/compute type of weights and activations
    L: int                # DiT blocks
    D: int                # hidden size
    H: int                # heads
    dh: int               # head dim
    mlp_ratio: int
    C_p: int              # latent channels per token (the velocity has this many)
    C_c: int              # conditioning channels concatenated to the latent (0: none)
    cond_up: int          # 1: cond given per token; 2: given at half (h, w) and upsampled
    d_a: int              # audio feature dim (0: no audio cross-attention weights)
    M: int                # audio tokens per chunk
    chunk: Grid
    ref: Grid
    bnd: Optional[Grid]   # standalone boundary frame (None: first chunk, no boundary)
    steps: int
    t_start: float
    t_end: float
    n_chunks: int = 1
    eps: float = 1e-6
    rope_theta: float = 10000.0

    @property
    def C_in(self) -> int:
        return self.C_p + self.C_c

    @property
    def N(self) -> int:
        return self.chunk.n

    @property
    def N_ref(self) -> int:
        return self.ref.n

    @property
    def N_bnd(self) -> int:
        return 0 if self.bnd is None else self.bnd.n

    @property
    def F(self) -> int:
        return self.D * self.mlp_ratio


_C2_CHUNK = Grid(0, 5, 30, 52)

CONFIGS: Dict[int, Config] = {
    1: Config(1, "tiny single block, fp32", "f32", L=1, D=256, H=4, dh=64, mlp_ratio=4,
              C_p=64, C_c=0, cond_up=1, d_a=64, M=16,
              chunk=Grid(0, 2, 8, 8), ref=Grid(-2, 1, 8, 8), bnd=Grid(-1, 1, 4, 8),
              steps=1, t_start=0.5, t_end=0.45),
    2: Config(2, "base low-res chunk, bf16", "bf16", L=4, D=1536, H=12, dh=128, mlp_ratio=4,
              C_p=64, C_c=0, cond_up=1, d_a=768, M=50,
              chunk=_C2_CHUNK, ref=Grid(-2, 1, 30, 52), bnd=Grid(-1, 1, 30, 52),
              steps=8, t_start=1.0, t_end=0.0),
    3: Config(3, "streaming sequence of 6 base chunks, bf16", "bf16", L=4, D=1536, H=12, dh=128,
              mlp_ratio=4, C_p=64, C_c=0, cond_up=1, d_a=768, M=50,
              chunk=_C2_CHUNK, ref=Grid(-2, 1, 30, 52), bnd=None,
              steps=8, t_start=1.0, t_end=0.0, n_chunks=6),
    4: Config(4, "super-resolution chunk, bf16", "bf16", L=2, D=1536, H=12, dh=128, mlp_ratio=4,
              C_p=64, C_c=64, cond_up=2, d_a=0, M=0,
              chunk=Grid(0, 5, 60, 104), ref=Grid(-2, 1, 60, 104), bnd=Grid(-1, 1, 60, 104),
              steps=4, t_start=1.0, t_end=0.0),
    5: Config(5, "large base chunk, bf16", "bf16", L=30, D=3072, H=24, dh=128, mlp_ratio=4,
              C_p=64, C_c=0, cond_up=1, d_a=768, M=200,
              chunk=Grid(0, 21, 30, 52), ref=Grid(-2, 1, 30, 52), bnd=Grid(-1, 1, 30, 52),
              steps=1, t_start=1.0, t_end=0.875),
}


# The workloads by name (the integer keys above seed their tensors).
TINY_FP32 = CONFIGS[1]
BASE_CHUNK = CONFIGS[2]
STREAM_6_CHUNKS = CONFIGS[3]
SUPER_RES = CONFIGS[4]
LARGE_CHUNK = CONFIGS[5]


def config(base: int, **overrides) -> Config:
    """Return workload ``base``, optionally with fields replaced (small test variants;
    give a variant its own ``cid`` so that its seeds differ)."""
    c = CONFIGS[base]
    return dataclasses.replace(c, **overrides) if overrides else c


# --------------------------------------------------------------------------------------
# casts (data preparation, not method arithmetic)
# --------------------------------------------------------------------------------------


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of float32 values that are already bf16-exact."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# --------------------------------------------------------------------------------------
# tensor catalogue.  Linear weights are stored [out, in] (row-major, input-contiguous).
# --------------------------------------------------------------------------------------

GLOBAL_NAMES = ("pe.w", "pe.b", "t1.w", "t1.b", "t2.w", "t2.b",
                "fmod.w", "fmod.b", "fin.w", "fin.b")
BLOCK_NAMES = ("mod.w", "mod.b", "qkv.w", "qkv.b", "gq", "gk", "o.w", "o.b",
               "cq.w", "cq.b", "ck.w", "ck.b", "cv.w", "cv.b", "gcq", "gck",
               "co.w", "co.b", "fc1.w", "fc1.b", "fc2.w", "fc2.b")
T_FREQ = 256  # width of the sinusoidal timestep feature


def weight_catalogue(cfg: Config) -> Dict[str, Tuple[Tuple[int, ...], int, str]]:
    """name -> (shape, fan_in, kind) where kind is "w" (N(0,1/fan_in)) or "g" (1+0.1 N(0,1))."""
    D, dh, C = cfg.D, cfg.dh, cfg
    cat: Dict[str, Tuple[Tuple[int, ...], int, str]] = {
        "pe.w": ((D, C.C_in), C.C_in, "w"), "pe.b": ((D,), C.C_in, "w"),
        "t1.w": ((D, T_FREQ), T_FREQ, "w"), "t1.b": ((D,), T_FREQ, "w"),
        "t2.w": ((D, D), D, "w"), "t2.b": ((D,), D, "w"),
        "fmod.w": ((2 * D, D), D, "w"), "fmod.b": ((2 * D,), D, "w"),
        "fin.w": ((C.C_p, D), D, "w"), "fin.b": ((C.C_p,), D, "w"),
    }
    F = cfg.F
    for l in range(cfg.L):
        p = f"blk{l}."
        blk = {
            "mod.w": ((6 * D, D), D, "w"), "mod.b": ((6 * D,), D, "w"),
            "qkv.w": ((3 * D, D), D, "w"), "qkv.b": ((3 * D,), D, "w"),
            "gq": ((dh,), 1, "g"), "gk": ((dh,), 1, "g"),
            "o.w": ((D, D), D, "w"), "o.b": ((D,), D, "w"),
            "fc1.w": ((F, D), D, "w"), "fc1.b": ((F,), D, "w"),
            "fc2.w": ((D, F), F, "w"), "fc2.b": ((D,), F, "w"),
        }
        if cfg.d_a > 0:
            blk.update({
                "cq.w": ((D, D), D, "w"), "cq.b": ((D,), D, "w"),
                "ck.w": ((D, cfg.d_a), cfg.d_a, "w"), "ck.b": ((D,), cfg.d_a, "w"),
                "cv.w": ((D, cfg.d_a), cfg.d_a, "w"), "cv.b": ((D,), cfg.d_a, "w"),
                "gcq": ((dh,), 1, "g"), "gck": ((dh,), 1, "g"),
                "co.w": ((D, D), D, "w"), "co.b": ((D,), D, "w"),
            })
        for k, v in blk.items():
            cat[p + k] = v
    return cat


# --------------------------------------------------------------------------------------
# seeded draws
# --------------------------------------------------------------------------------------

_PART = 1 << 22   # elements per independently seeded part of a large tensor
_GLOBAL_BLOCK = 65535


def _seed(cid: int, block: int, name: str, chunk: int, part: int) -> np.random.SeedSequence:
    return np.random.SeedSequence([cid, block, zlib.crc32(name.encode()), chunk, part])


def _normal(cid: int, block: int, name: str, chunk: int, n: int) -> np.ndarray:
    """n standard normal draws (float64), generated in independently seeded parts."""
    out = np.empty(n, dtype=np.float64)
    for p, s in enumerate(range(0, n, _PART)):
        e = min(n, s + _PART)
        out[s:e] = np.random.default_rng(_seed(cid, block, name, chunk, p)).standard_normal(e - s)
    return out


def _finish(a64: np.ndarray, dtype: str) -> np.ndarray:
    a = a64.astype(np.float32)  # RNE
    return round_bf16(a) if dtype == "bf16" else a


def _one_weight(cfg: Config, name: str, spec) -> np.ndarray:
    shape, fan_in, kind = spec
    if name.startswith("blk"):
        block = int(name[3:name.index(".")])
        base = name[name.index(".") + 1:]
    else:
        block, base = _GLOBAL_BLOCK, name
    n = int(np.prod(shape))
    z = _normal(cfg.cid, block, base, 0, n)
    if kind == "w":
        z *= 1.0 / np.sqrt(fan_in)
    else:
        z = 1.0 + 0.1 * z
    return _finish(z, cfg.dtype).reshape(shape)


def from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """float32 values of bf16 bit patterns (uint16)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


class Bf16Weights(collections.abc.Mapping):
    """A bf16 workload's parameters held as bf16 bit patterns (half the memory of float32:
    10.5 GB instead of 21 GB for the large chunk); indexing returns the float32 values,
    the same values make_weights returns."""

    def __init__(self, bits: Dict[str, np.ndarray]):
        self.bits = bits

    def __getitem__(self, name: str) -> np.ndarray:
        return from_bf16_bits(self.bits[name])

    def __iter__(self):
        return iter(self.bits)

    def __len__(self) -> int:
        return len(self.bits)


def make_weights(cfg: Config, threads: int = 8, compact: bool = False):
    """All parameters of workload ``cfg`` as float32 arrays (bf16-exact for bf16 workloads).

    compact (bf16 workloads only): a Bf16Weights mapping that stores the bit patterns."""
    cat = weight_catalogue(cfg)
    names = list(cat)
    if compact and cfg.dtype != "bf16":
        raise ValueError("compact weights need a bf16 workload")
    one = (lambda nm: to_bf16_bits(_one_weight(cfg, nm, cat[nm]))) if compact else \
        (lambda nm: _one_weight(cfg, nm, cat[nm]))
    with ThreadPoolExecutor(max(1, threads)) as ex:
        arrs = list(ex.map(one, names))
    d = dict(zip(names, arrs))
    return Bf16Weights(d) if compact else d


def _tokens(cfg: Config, name: str, chunk: int, shape, dtype: str) -> np.ndarray:
    z = _normal(cfg.cid, 0, name, chunk, int(np.prod(shape)))
    return _finish(z, dtype).reshape(shape)


def anchor_noise(cfg: Config, chunk: int = 0) -> np.ndarray:
    """Seeded noise of the two anchor frames of an interpolation window, [2 h w, C_p]
    float32 (the earlier anchor's frame first)."""
    g = cfg.chunk
    return _tokens(cfg, "anchor_eps", chunk, (2 * g.h * g.w, cfg.C_p), "f32")


def make_inputs(cfg: Config, chunk: int = 0) -> Dict[str, np.ndarray]:
    """Seeded per-chunk inputs (all float32).

    x_init  [N, C_p]      initial noise of the chunk (fp32 latent)
    audio   [M, d_a]      audio feature tokens (bf16-exact for bf16 workloads)
    ref     [N_ref, C_p]  clean reference latent tokens (one frame)
    bnd     [N_bnd, C_p]  standalone boundary frame (only when the workload has one)
    cond_lr [N/4, C_c]    half-resolution conditioning latent tokens (cond_up == 2)
    cond    [N, C_c]      per-token conditioning (C_c > 0 and cond_up == 1)
    """
    out = {"x_init": _tokens(cfg, "x_init", chunk, (cfg.N, cfg.C_p), "f32")}
    if cfg.M > 0:
        out["audio"] = _tokens(cfg, "audio", chunk, (cfg.M, cfg.d_a), cfg.dtype)
    out["ref"] = _tokens(cfg, "ref", 0, (cfg.N_ref, cfg.C_p), "f32")
    if cfg.bnd is not None:
        out["bnd"] = _tokens(cfg, "bnd", chunk, (cfg.N_bnd, cfg.C_p), "f32")
    if cfg.C_c > 0:
        g = cfg.chunk
        if cfg.cond_up == 2:
            n_lr = g.frames * (g.h // 2) * (g.w // 2)
            out["cond_lr"] = _tokens(cfg, "cond_lr", chunk, (n_lr, cfg.C_c), "f32")
        else:
            out["cond"] = _tokens(cfg, "cond", chunk, (cfg.N, cfg.C_c), "f32")
    return out

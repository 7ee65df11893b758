"""Glue between the seeded synthetic workloads (package ``synth``) and the library:
config translation and host -> device upload.  No arithmetic of the method."""
from __future__ import annotations

from typing import Dict

import numpy as np
import torch

from .dit import ChunkConfig, grid, torch_dtype


def chunk_config(cfg, max_tokens=None, max_ref=None, max_bnd=None, max_audio=None) -> ChunkConfig:
    """ChunkConfig sized for a synth.Config workload (capacities default to its sizes)."""
    nb = cfg.N_bnd if cfg.bnd is not None else cfg.chunk.h * cfg.chunk.w
    return ChunkConfig(L=cfg.L, D=cfg.D, H=cfg.H, dh=cfg.dh, mlp_ratio=cfg.mlp_ratio, c_p=cfg.C_p,
                       c_c=cfg.C_c, cond_up=cfg.cond_up, d_a=cfg.d_a, dtype=cfg.dtype,
                       max_tokens=max_tokens or cfg.N, max_ref=max_ref or cfg.N_ref,
                       max_bnd=max_bnd if max_bnd is not None else nb,
                       max_audio=max_audio if max_audio is not None else cfg.M,
                       eps=cfg.eps, rope_theta=cfg.rope_theta)


def upload_weights(P, dtype: str, device) -> Dict[str, torch.Tensor]:
    """float32 arrays (bf16-exact for bf16 workloads) -> device tensors of the compute dtype.
    A mapping that holds bf16 bit patterns (``bits``: name -> uint16 array) is uploaded
    as those bits."""
    td = torch_dtype(dtype)
    bits = getattr(P, "bits", None)
    if bits is not None:
        if td != torch.bfloat16:
            raise ValueError("bf16 bit patterns need the bf16 compute dtype")
        return {k: torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).to(device).view(torch.bfloat16)
                for k, v in bits.items()}
    return {k: torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(device).to(td)
            for k, v in P.items()}


def f32(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def grid_of(g) -> "grid":
    return grid(g.t0, g.frames, g.h, g.w)

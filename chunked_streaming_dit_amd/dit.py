"""Python face of libditchunk: a handle class for the chunk step and thin op wrappers.

Tensors must already live on the GPU, be contiguous and have the documented dtype;
this module only checks that and passes pointers and the current HIP stream.
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Dict, Optional, Sequence, Tuple

import torch

from . import _lib as C

__all__ = ["ChunkConfig", "DitChunk", "grid", "fm_euler_step", "fm_noise_to", "ops", "torch_dtype"]


def torch_dtype(dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def _dt_code(dtype: str) -> int:
    return {"f32": C.DIT_F32, "bf16": C.DIT_BF16}[dtype]


def grid(t0: int, frames: int, h: int, w: int) -> C.DitGrid:
    return C.DitGrid(t0, frames, h, w)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(t: Optional[torch.Tensor], name: str, dtype: Optional[torch.dtype] = None) -> None:
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


@dataclasses.dataclass(frozen=True)
class ChunkConfig:
    L: int
    D: int
    H: int
    dh: int
    mlp_ratio: int
    c_p: int
    c_c: int
    cond_up: int
    d_a: int
    dtype: str
    max_tokens: int
    max_ref: int
    max_bnd: int
    max_audio: int
    eps: float = 1e-6
    rope_theta: float = 10000.0

    def c_struct(self) -> C.DitConfig:
        return C.DitConfig(self.L, self.D, self.H, self.dh, self.mlp_ratio, self.c_p, self.c_c,
                           self.cond_up, self.d_a, _dt_code(self.dtype), self.max_tokens,
                           self.max_ref, self.max_bnd, self.max_audio, self.eps, self.rope_theta)

    def state_bytes(self) -> int:
        cs = self.c_struct()
        n = C.lib().dit_state_bytes(ctypes.byref(cs))
        if n == 0:
            raise C.DitError(C.DIT_EINVAL, C.last_error())
        return n

    def workspace_bytes(self) -> int:
        cs = self.c_struct()
        n = C.lib().dit_workspace_bytes(ctypes.byref(cs))
        if n == 0:
            raise C.DitError(C.DIT_EINVAL, C.last_error())
        return n

    def block_weight_bytes(self) -> int:
        """Bytes of one block slot of the weight-streaming ring."""
        cs = self.c_struct()
        n = C.lib().dit_block_weight_bytes(ctypes.byref(cs))
        if n == 0:
            raise C.DitError(C.DIT_EINVAL, C.last_error())
        return n

    def weight_names(self):
        names = list(C.GLOBAL_ORDER)
        for l in range(self.L):
            names += [f"blk{l}.{b}" for b in C.BLOCK_ORDER]
        return names


AUDIO_HELD = object()  # step(audio=AUDIO_HELD): use the audio K/V held by audio_kv_precompute


class DitChunk:
    """A libditchunk handle with its state and workspace allocated as torch tensors.

    weights: name -> GPU tensor in the config's dtype (names of the ditchunk.h table:
    "pe.w", ..., "blk{l}.qkv.w", ...); cross-attention entries may be absent when d_a == 0.
    """

    def __init__(self, cfg: ChunkConfig, weights: Dict[str, torch.Tensor],
                 device: Optional[torch.device] = None):
        self.cfg = cfg
        self.device = device or torch.device("cuda", torch.cuda.current_device())
        dt = torch_dtype(cfg.dtype)
        names = cfg.weight_names()
        ptrs = (C.P * len(names))()
        self._weights = []
        for i, nm in enumerate(names):
            t = weights.get(nm)
            if t is None:
                ptrs[i] = None
                continue
            _dev(t, nm, dt)
            self._weights.append(t)
            ptrs[i] = t.data_ptr()
        self.state = torch.empty(cfg.state_bytes(), dtype=torch.uint8, device=self.device)
        self.workspace = torch.empty(cfg.workspace_bytes(), dtype=torch.uint8, device=self.device)
        h = C.P()
        cs = cfg.c_struct()
        C.check(C.lib().dit_create(ctypes.byref(cs), ptrs, self.state.data_ptr(), self.state.numel(),
                                   self.workspace.data_ptr(), self.workspace.numel(), _stream(),
                                   ctypes.byref(h)))
        self._h = h

    def close(self) -> None:
        """Release the handle.  Teardown order: weight streaming is switched off (its
        copies finish), the device is synchronised, the handle is destroyed, and only
        then are the ring and the pinned host blocks released, so that no copy or kernel
        can still touch memory that is being freed."""
        if getattr(self, "_h", None):
            if getattr(self, "_stream_keep", None) is not None:
                C.lib().dit_weight_stream(self._h, None, None, 0, 0)
            torch.cuda.synchronize(self.device)
            C.lib().dit_destroy(self._h)
            self._h = None
        self._stream_keep = None
        self._ring = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def weight_stream(self, host_blocks: Optional[Dict[str, torch.Tensor]], nslot: int = 2) -> None:
        """Stream the block weights from pinned host tensors (names "blk{l}.<entry>",
        shapes and dtype of the weight table) through a device ring of nslot block slots
        (dit_weight_stream); None switches back to the resident weights."""
        # Work already enqueued may still read the ring (or, on the library's copy
        # stream, write it) when streaming is switched off or moves to other host
        # blocks: synchronise first.  The ring itself stays allocated across switches, so
        # switching streaming on again (the hand-over between two stages) needs no wait
        # and the prefetch of the first blocks overlaps the work still running.
        if getattr(self, "_stream_keep", None) is not None or host_blocks is None:
            torch.cuda.synchronize(self.device)
        if host_blocks is None:
            C.check(C.lib().dit_weight_stream(self._h, None, None, 0, 0))
            self._stream_keep = None
            return
        dt = torch_dtype(self.cfg.dtype)
        names = [f"blk{l}.{b}" for l in range(self.cfg.L) for b in C.BLOCK_ORDER]
        ptrs = (C.P * len(names))()
        keep = []
        for i, nm in enumerate(names):
            t = host_blocks.get(nm)
            if t is None:
                ptrs[i] = None
                continue
            if t.is_cuda or not t.is_pinned() or not t.is_contiguous() or t.dtype != dt:
                raise ValueError(f"{nm} must be a contiguous pinned host tensor of {dt}")
            keep.append(t)
            ptrs[i] = t.data_ptr()
        need = nslot * self.cfg.block_weight_bytes()
        ring = getattr(self, "_ring", None)
        if ring is None or ring.numel() < need:
            # A new ring comes from torch's caching allocator, which may hand back memory
            # that kernels still enqueued on torch's stream were using; the library's copy
            # stream would not wait for them, so synchronise once before copying into it.
            self._ring = None
            ring = torch.empty(need, dtype=torch.uint8, device=self.device)
            torch.cuda.synchronize(self.device)
            self._ring = ring
        C.check(C.lib().dit_weight_stream(self._h, ptrs, ring.data_ptr(), ring.numel(), nslot))
        self._stream_keep = keep

    def ref_kv_precompute(self, ref: torch.Tensor, g: C.DitGrid) -> None:
        _dev(ref, "ref", torch.float32)
        C.check(C.lib().ref_kv_precompute(self._h, ref.data_ptr(), g))

    def boundary_kv_carry(self, x_prev: Optional[torch.Tensor], g: C.DitGrid) -> None:
        _dev(x_prev, "x_prev", torch.float32)
        C.check(C.lib().boundary_kv_carry(self._h, _ptr(x_prev), g))

    def interp_anchor_kv(self, x_next: Optional[torch.Tensor], g: C.DitGrid, t_pos: int) -> None:
        """Anchor K/V of an interpolation chunk from frame 0 of the next chunk's final
        latent x_next (grid g), placed at time position t_pos; g.frames == 0 clears it."""
        _dev(x_next, "x_next", torch.float32)
        C.check(C.lib().interp_anchor_kv(self._h, _ptr(x_next), g, int(t_pos)))

    def audio_kv_precompute(self, audio: Optional[torch.Tensor]) -> None:
        """Hold the chunk's audio K/V of every block (audio_kv_precompute); steps given
        audio=AUDIO_HELD reuse them.  None clears them."""
        _dev(audio, "audio", torch.float32)
        C.check(C.lib().audio_kv_precompute(self._h, _ptr(audio), 0 if audio is None else audio.shape[0]))

    def modulation_table(self, ts: Optional[Sequence[float]]) -> None:
        """Hold the adaLN vectors of the timesteps ts (at most DIT_MOD_TABLE_MAX; a
        request's schedule plus 0.0 for the context passes): passes at one of these exact
        timesteps reuse them (dit_modulation_table).  None or [] clears the table."""
        ts = [] if ts is None else [float(t) for t in ts]
        arr = (ctypes.c_double * max(len(ts), 1))(*ts)
        C.check(C.lib().dit_modulation_table(self._h, arr, len(ts)))

    def step(self, x: torch.Tensor, t: float, t_next: float, g: C.DitGrid,
             cond: Optional[torch.Tensor] = None, audio=None,
             v_out: Optional[torch.Tensor] = None, carry_boundary: bool = False) -> None:
        """One denoising step; audio: features [M, d_a], None, or AUDIO_HELD (the K/V held
        by audio_kv_precompute); carry_boundary: the chunk's last step, which also leaves
        its last frame's K/V as the next boundary (dit_chunk_step_carry)."""
        _dev(x, "x", torch.float32)
        _dev(cond, "cond", torch.float32)
        _dev(v_out, "v_out", torch.float32)
        if audio is AUDIO_HELD:
            M, audio = C.DIT_AUDIO_HELD, None
        else:
            _dev(audio, "audio", torch.float32)
            M = 0 if audio is None else audio.shape[0]
        fn = C.lib().dit_chunk_step_carry if carry_boundary else C.lib().dit_chunk_step
        C.check(fn(self._h, x.data_ptr(), _ptr(cond), _ptr(audio), M, g, float(t), float(t_next),
                   _ptr(v_out)))

    def timing_enable(self, on=True) -> None:
        """Time kernel launches with dispatch-stamped events (dit_timing_enable): True or
        a mask of 1 << DIT_TIME_* kinds (True: self-attention only); False: none."""
        mask = (1 if on else 0) if isinstance(on, bool) else int(on)
        C.check(C.lib().dit_timing_enable(self._h, mask))

    def timing_read(self, kind: int = C.DIT_TIME_ATTN) -> Tuple[int, float, float]:
        """(launches, summed ms, summed work) of a timing kind since the last read: work is
        algorithmic flop for DIT_TIME_ATTN and DIT_TIME_GEMM, bytes for DIT_TIME_ELEM."""
        n = ctypes.c_int()
        ms = ctypes.c_double()
        fl = ctypes.c_double()
        C.check(C.lib().dit_timing_read(self._h, int(kind), ctypes.byref(n), ctypes.byref(ms),
                                        ctypes.byref(fl)))
        return n.value, ms.value, fl.value


def fm_euler_step(x: torch.Tensor, v: torch.Tensor, dt: float) -> None:
    _dev(x, "x", torch.float32)
    _dev(v, "v", torch.float32)
    if x.numel() != v.numel():
        raise ValueError("x and v differ in size")
    C.check(C.lib().fm_euler_step(x.data_ptr(), v.data_ptr(), float(dt), x.numel(), _stream()))


def fm_noise_to(x: torch.Tensor, z: torch.Tensor, eps: torch.Tensor, t: float) -> None:
    """x = (1 - t) z + t eps (fm_noise_to); x may be z or eps."""
    for a, name in ((x, "x"), (z, "z"), (eps, "eps")):
        _dev(a, name, torch.float32)
    if not (x.numel() == z.numel() == eps.numel()):
        raise ValueError("x, z and eps differ in size")
    C.check(C.lib().fm_noise_to(x.data_ptr(), z.data_ptr(), eps.data_ptr(), float(t), x.numel(), _stream()))


class ops:
    """Kernel-level entry points (ditchunk_ops.h)."""

    @staticmethod
    def linear(A, W, b, act: int, out, dtype: str) -> None:
        M, K = A.shape
        N = W.shape[0]
        for t, n in ((A, "A"), (W, "W"), (b, "b"), (out, "out")):
            _dev(t, n)
        C.check(C.lib().ditk_linear(_dt_code(dtype), A.data_ptr(), W.data_ptr(), b.data_ptr(), M, N, K,
                                    act, out.data_ptr(), _stream()))

    @staticmethod
    def linear_residual(A, W, b, gate, h, dtype: str, workspace: Optional[torch.Tensor] = None) -> None:
        """workspace: optional fp32 tensor for the split-K launch (ditk_linear_residual)."""
        M, K = A.shape
        N = W.shape[0]
        for t, n in ((A, "A"), (W, "W"), (b, "b"), (h, "h")):
            _dev(t, n)
        _dev(gate, "gate", torch.float32)
        _dev(workspace, "workspace", torch.float32)
        C.check(C.lib().ditk_linear_residual(_dt_code(dtype), A.data_ptr(), W.data_ptr(), b.data_ptr(),
                                             _ptr(gate), M, N, K, h.data_ptr(), _ptr(workspace),
                                             0 if workspace is None else workspace.numel(), _stream()))

    @staticmethod
    def rmsnorm_modulate(h, shift, scale, eps, out, dtype: str) -> None:
        _dev(h, "h", torch.float32)
        _dev(out, "out")
        n, D = h.shape
        C.check(C.lib().ditk_rmsnorm_modulate(_dt_code(dtype), h.data_ptr(), n, D, _ptr(shift),
                                              _ptr(scale), eps, out.data_ptr(), _stream()))

    @staticmethod
    def qknorm_rope(dtype: str, dh: int, H: int, n: int, q_in, k_in, v_in, ld_in: int, gq, gk,
                    rope: bool, g: C.DitGrid, eps: float, theta: float, q_out, k_out, vt_out,
                    cap: int, q_scale: float = 1.0) -> None:
        C.check(C.lib().ditk_qknorm_rope(_dt_code(dtype), dh, H, n, _ptr(q_in), _ptr(k_in), _ptr(v_in),
                                         ld_in, _ptr(gq), _ptr(gk), 1 if rope else 0, g, eps, theta,
                                         q_scale, _ptr(q_out), _ptr(k_out), _ptr(vt_out), cap,
                                         _stream()))

    @staticmethod
    def attention(dtype: str, dh: int, H: int, q, segs: Sequence[Tuple[torch.Tensor, torch.Tensor, int, int]],
                  o, nsplit: int = 1, partial: Optional[torch.Tensor] = None,
                  q_prescaled: bool = False, gq: Optional[torch.Tensor] = None,
                  gk: Optional[torch.Tensor] = None, q_fold: float = 0.0, unsplit_rows: int = 0) -> None:
        """gq, gk: QK-norm gammas of normed q (times q_fold) and k: lets the kernel bound
        the logits and drop the running max.  unsplit_rows: leading queries (a multiple of
        256, or >= nq) that take the whole key range unsplit (ditk_attention)."""
        ns = len(segs)
        kp = (C.P * ns)(*[s[0].data_ptr() for s in segs])
        vp = (C.P * ns)(*[s[1].data_ptr() for s in segs])
        nn = (ctypes.c_int * ns)(*[s[2] for s in segs])
        cp = (ctypes.c_int * ns)(*[s[3] for s in segs])
        C.check(C.lib().ditk_attention(_dt_code(dtype), dh, H, q.data_ptr(), q.shape[0], ns, kp, vp, nn,
                                       cp, nsplit, _ptr(partial), int(unsplit_rows),
                                       1 if q_prescaled else 0, _ptr(gq),
                                       _ptr(gk), float(q_fold), o.data_ptr(), _stream()))

    @staticmethod
    def attention_probs(H: int, q, k, n: int, p, q_prescaled: bool = False) -> None:
        """Softmax probabilities of one short key segment, p [nq, H*64] (ditk_attention_probs)."""
        C.check(C.lib().ditk_attention_probs(H, q.data_ptr(), q.shape[0], k.data_ptr(), n, k.shape[0],
                                             1 if q_prescaled else 0, p.data_ptr(), _stream()))

    @staticmethod
    def modulation(dtype: str, cfg: ChunkConfig, weights: Dict[str, torch.Tensor], t: float,
                   mod_out, fmod_out, tmp) -> None:
        names = cfg.weight_names()
        ptrs = (C.P * len(names))(*[(weights[n].data_ptr() if n in weights else None) for n in names])
        C.check(C.lib().ditk_modulation(_dt_code(dtype), cfg.D, cfg.L, float(t), ptrs,
                                        mod_out.data_ptr(), fmod_out.data_ptr(), tmp.data_ptr(),
                                        _stream()))

    @staticmethod
    def patch_input(dtype: str, x, c_p: int, cond, c_c: int, mode: int, g: C.DitGrid, xin) -> None:
        C.check(C.lib().ditk_patch_input(_dt_code(dtype), x.data_ptr(), x.shape[0], c_p, _ptr(cond), c_c,
                                         mode, g, xin.data_ptr(), _stream()))

    @staticmethod
    def patch_embed(x, c_p: int, cond, c_c: int, mode: int, g: C.DitGrid, w, b, out) -> None:
        C.check(C.lib().ditk_patch_embed(x.data_ptr(), x.shape[0], c_p, _ptr(cond), c_c, mode, g,
                                         w.data_ptr(), b.data_ptr(), out.data_ptr(), out.shape[1],
                                         _stream()))

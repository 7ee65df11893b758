"""C-ABI checks that need no GPU: the library loads, exports every declared symbol,
sizes its buffers, and rejects bad arguments on the host before any HIP call.

Fake (never dereferenced) device addresses stand in for buffers: every call below
fails validation before it could launch anything.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
from chunked_streaming_dit_amd import _lib as C
from chunked_streaming_dit_amd.workload import chunk_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000  # 256-byte aligned, never touched


def _declared():
    names = set()
    for h in ("ditchunk.h", "ditchunk_ops.h"):
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", src, flags=re.M))
    return names


def test_library_exports_every_declared_symbol():
    lib = C.lib()
    declared = _declared()
    assert {"dit_chunk_step", "ref_kv_precompute", "boundary_kv_carry", "interp_anchor_kv", "fm_euler_step",
            "dit_create", "ditk_attention"} <= declared
    for n in declared:
        assert hasattr(lib, n), n
    assert declared == set(C.EXPORTS)


def _cs(cid=1, **kw):
    cs = chunk_config(synth.CONFIGS[cid]).c_struct()
    for k, v in kw.items():
        setattr(cs, k, v)
    return cs


def test_sizes_and_weight_count():
    lib = C.lib()
    for cid in range(1, 6):
        cs = _cs(cid)
        cfg = synth.CONFIGS[cid]
        assert lib.dit_weight_count(ctypes.byref(cs)) == 10 + 22 * cfg.L
        sb = lib.dit_state_bytes(ctypes.byref(cs))
        # per block K and V of the reference, the boundary, the interpolation anchor and
        # (with audio weights) the held audio
        aud = (max(cfg.M, 1) + 63) // 64 * 64 if cfg.d_a > 0 else 0
        elt = 2 if cfg.dtype == "bf16" else 4
        kv = cfg.L * 2 * cfg.D * elt * (
            (cfg.N_ref + 63) // 64 * 64 + 2 * ((cfg.chunk.h * cfg.chunk.w + 63) // 64 * 64) + aud)
        kv += aud * cfg.d_a * elt  # the held audio features
        if cfg.dtype == "bf16" and cfg.dh == 128 and 0 < cfg.M <= 64 and cfg.d_a > 0:
            kv += cfg.L * cfg.D * cfg.H * 64 * elt  # the folded cross-attention values
        # plus the modulation table: DIT_MOD_TABLE_MAX entries of (6 L + 2) D fp32
        kv += 16 * (6 * cfg.L + 2) * cfg.D * 4
        assert kv <= sb <= kv + (8 * cfg.L + 1) * 256
        assert lib.dit_workspace_bytes(ctypes.byref(cs)) > 0


@pytest.mark.parametrize("field,value", [("D", 300), ("dh", 96), ("dtype", 7), ("L", 0),
                                         ("cond_up", 3), ("c_c", 10), ("eps", 0.0),
                                         ("rope_theta", float("inf")), ("max_tokens", 0)])
def test_bad_config_rejected(field, value):
    cs = _cs(1, **{field: value})
    assert C.lib().dit_state_bytes(ctypes.byref(cs)) == 0
    assert C.last_error()


@pytest.mark.parametrize("D,H,mlp,max_tokens", [(4096, 32, 8, 70000), (3072, 24, 4, 180000),
                                                 (4096, 32, 4, 140000)])
def test_config_beyond_32bit_operand_offsets_rejected(D, H, mlp, max_tokens):
    """A token capacity whose activations [cap, max(3D, mlp D)] reach 2^31 elements, or
    whose V^T [D, cap] reaches 2^31 bytes, is an error (the kernels address those
    operands with 32-bit offsets); the large chunk's own capacity is accepted."""
    cs = _cs(5, D=D, H=H, mlp_ratio=mlp, max_tokens=max_tokens)
    assert C.lib().dit_state_bytes(ctypes.byref(cs)) == 0
    assert "2^31" in C.last_error()
    ok = _cs(5)
    assert C.lib().dit_state_bytes(ctypes.byref(ok)) > 0
    ok.max_tokens = 65536
    assert C.lib().dit_workspace_bytes(ctypes.byref(ok)) > 0


def test_ops_beyond_32bit_operand_offsets_rejected():
    lib = C.lib()
    # A [M, K] of 2^31 elements
    assert lib.ditk_linear(C.DIT_BF16, FAKE, FAKE, FAKE, 1 << 18, 256, 8192, 0, FAKE, None) == C.DIT_ESHAPE
    assert lib.ditk_linear_residual(C.DIT_BF16, FAKE, FAKE, FAKE, None, 1 << 18, 256, 8192, FAKE, None, 0,
                                    None) == C.DIT_ESHAPE
    # V^T [H*dh, cap] of 2^31 bytes
    P = ctypes.c_void_p
    k = (P * 1)(FAKE)
    n = (ctypes.c_int * 1)(1 << 19)
    cap = (ctypes.c_int * 1)(1 << 19)
    rc = lib.ditk_attention(C.DIT_BF16, 128, 16, FAKE, 256, 1, k, k, n, cap, 1, None, 0, 1, None, None, 0.0,
                            FAKE, None)
    assert rc == C.DIT_ESHAPE and "2^31" in C.last_error()


def test_probe_validation():
    lib = C.lib()
    fl = ctypes.c_double()
    assert lib.ditk_probe_mfma(None, 10, FAKE, C.DITK_PROBE_SINK_FLOATS, ctypes.byref(fl), None) == C.DIT_EINVAL
    assert lib.ditk_probe_mfma(FAKE, 0, FAKE, C.DITK_PROBE_SINK_FLOATS, ctypes.byref(fl), None) == C.DIT_EINVAL
    assert lib.ditk_probe_mfma(FAKE, 10, FAKE, C.DITK_PROBE_SINK_FLOATS - 1, ctypes.byref(fl),
                               None) == C.DIT_EWORKSPACE
    assert lib.ditk_probe_copy(FAKE, FAKE, 24, None) == C.DIT_EINVAL
    assert lib.ditk_probe_copy(FAKE + 8, FAKE, 32, None) == C.DIT_EINVAL
    assert lib.ditk_probe_copy(None, None, 0, None) == C.DIT_OK


def _handle(cid=1):
    cs = _cs(cid)
    lib = C.lib()
    n = lib.dit_weight_count(ctypes.byref(cs))
    w = (C.P * n)(*([FAKE] * n))
    h = C.P()
    rc = lib.dit_create(ctypes.byref(cs), w, FAKE, lib.dit_state_bytes(ctypes.byref(cs)), FAKE + (1 << 20),
                        lib.dit_workspace_bytes(ctypes.byref(cs)), None, ctypes.byref(h))
    assert rc == C.DIT_OK, C.last_error()
    return lib, cs, h


def test_create_validation():
    lib = C.lib()
    cs = _cs(1)
    n = lib.dit_weight_count(ctypes.byref(cs))
    w = (C.P * n)(*([FAKE] * n))
    h = C.P()
    sb, wb = lib.dit_state_bytes(ctypes.byref(cs)), lib.dit_workspace_bytes(ctypes.byref(cs))
    assert lib.dit_create(ctypes.byref(cs), w, FAKE, sb - 1, FAKE, wb, None, ctypes.byref(h)) == C.DIT_EWORKSPACE
    assert lib.dit_create(ctypes.byref(cs), w, FAKE, sb, FAKE, wb - 1, None, ctypes.byref(h)) == C.DIT_EWORKSPACE
    assert lib.dit_create(ctypes.byref(cs), w, FAKE + 8, sb, FAKE, wb, None, ctypes.byref(h)) == C.DIT_EINVAL
    w2 = (C.P * n)(*([FAKE] * n))
    w2[3] = None
    assert lib.dit_create(ctypes.byref(cs), w2, FAKE, sb, FAKE, wb, None, ctypes.byref(h)) == C.DIT_EINVAL
    assert lib.dit_create(ctypes.byref(cs), None, FAKE, sb, FAKE, wb, None, ctypes.byref(h)) == C.DIT_EINVAL
    assert "NULL" in C.last_error()


def test_call_order_and_shape_errors():
    lib, cs, h = _handle(1)
    g = C.DitGrid(0, 2, 8, 8)
    # step before the reference exists
    assert lib.dit_chunk_step(h, FAKE, None, FAKE, 16, g, 0.5, 0.45, None) == C.DIT_ESTATE
    assert "ref_kv_precompute" in C.last_error()
    assert lib.boundary_kv_carry(h, FAKE, C.DitGrid(0, 1, 4, 8)) == C.DIT_ESTATE
    # argument errors win over state errors and never launch
    assert lib.dit_chunk_step(h, None, None, None, 0, g, 0.5, 0.45, None) == C.DIT_EINVAL
    assert lib.dit_chunk_step(h, FAKE, None, None, 0, g, float("nan"), 0.45, None) == C.DIT_EINVAL
    assert lib.dit_chunk_step(h, FAKE, None, None, 0, C.DitGrid(0, 3, 8, 8), 0.5, 0.4, None) == C.DIT_ESHAPE
    assert lib.dit_chunk_step(h, FAKE, None, None, 0, C.DitGrid(0, 0, 8, 8), 0.5, 0.4, None) == C.DIT_ESHAPE
    assert lib.dit_chunk_step(h, FAKE, None, FAKE, 17, g, 0.5, 0.4, None) == C.DIT_ESHAPE
    assert lib.dit_chunk_step(h, FAKE, None, None, 3, g, 0.5, 0.4, None) == C.DIT_EINVAL
    assert lib.dit_chunk_step(h, FAKE, FAKE, None, 0, g, 0.5, 0.4, None) == C.DIT_EINVAL  # no cond channels
    assert lib.ref_kv_precompute(h, None, C.DitGrid(-2, 1, 8, 8)) == C.DIT_EINVAL
    assert lib.ref_kv_precompute(h, FAKE, C.DitGrid(-2, 1, 8, 9)) == C.DIT_ESHAPE
    assert lib.boundary_kv_carry(h, FAKE, C.DitGrid(0, 1, 8, 8)) == C.DIT_ESHAPE  # 64 > max_bnd 32
    assert lib.boundary_kv_carry(h, None, C.DitGrid(0, 2, 4, 8)) == C.DIT_EINVAL
    assert lib.boundary_kv_carry(h, None, C.DitGrid(0, 0, 0, 0)) == C.DIT_OK      # clear: no launch
    # the boundary-carrying last step: the step's checks, and the frame must fit max_bnd
    g32 = C.DitGrid(0, 4, 4, 8)  # 32 tokens per frame: fits max_bnd
    assert lib.dit_chunk_step_carry(h, FAKE, None, FAKE, 16, g32, 0.5, 0.45, None) == C.DIT_ESTATE
    assert lib.dit_chunk_step_carry(h, None, None, None, 0, g, 0.5, 0.45, None) == C.DIT_EINVAL
    assert lib.dit_chunk_step_carry(h, FAKE, None, None, 0, C.DitGrid(0, 3, 8, 8), 0.5, 0.4, None) == C.DIT_ESHAPE
    assert lib.dit_chunk_step_carry(h, FAKE, None, None, 0, C.DitGrid(0, 1, 8, 8), 0.5, 0.4, None) == C.DIT_ESHAPE
    assert "max_bnd" in C.last_error()  # 64 tokens per frame > max_bnd 32
    # interpolation anchor: same checks as the boundary
    assert lib.interp_anchor_kv(h, FAKE, C.DitGrid(0, 2, 4, 8), 2) == C.DIT_ESTATE
    assert "ref_kv_precompute" in C.last_error()
    assert lib.interp_anchor_kv(h, FAKE, C.DitGrid(0, 1, 8, 8), 2) == C.DIT_ESHAPE  # 64 > max_bnd 32
    assert lib.interp_anchor_kv(h, None, C.DitGrid(0, 2, 4, 8), 2) == C.DIT_EINVAL
    assert lib.interp_anchor_kv(h, FAKE, C.DitGrid(0, 1, 0, 8), 2) == C.DIT_ESHAPE
    assert lib.interp_anchor_kv(h, None, C.DitGrid(0, 0, 0, 0), 2) == C.DIT_OK     # clear: no launch
    assert lib.interp_anchor_kv(None, FAKE, C.DitGrid(0, 1, 4, 8), 2) == C.DIT_EINVAL
    # modulation table: checked before any launch; nt = 0 clears without a launch
    ts = (ctypes.c_double * 17)(*[1.0 - k / 16 for k in range(17)])
    assert lib.dit_modulation_table(h, ts, 17) == C.DIT_EINVAL  # > DIT_MOD_TABLE_MAX
    assert lib.dit_modulation_table(h, ts, -1) == C.DIT_EINVAL
    assert lib.dit_modulation_table(h, None, 2) == C.DIT_EINVAL
    ts[1] = float("inf")
    assert lib.dit_modulation_table(h, ts, 2) == C.DIT_EINVAL
    assert "not finite" in C.last_error()
    assert lib.dit_modulation_table(h, None, 0) == C.DIT_OK
    assert lib.dit_modulation_table(None, ts, 1) == C.DIT_EINVAL
    assert lib.dit_destroy(h) == C.DIT_OK
    assert lib.dit_destroy(None) == C.DIT_OK


def test_cond_and_audio_validation_sr_config():
    lib, cs, h = _handle(4)
    g = C.DitGrid(0, 5, 60, 104)
    assert lib.dit_chunk_step(h, FAKE, None, None, 0, g, 1.0, 0.75, None) == C.DIT_EINVAL   # cond missing
    assert lib.dit_chunk_step(h, FAKE, FAKE, None, 0, C.DitGrid(0, 1, 59, 104), 1.0, 0.75, None) == C.DIT_ESHAPE
    assert lib.dit_chunk_step(h, FAKE, FAKE, FAKE, 1, g, 1.0, 0.75, None) == C.DIT_ESHAPE    # max_audio 0
    lib.dit_destroy(h)


def test_euler_and_ops_validation():
    lib = C.lib()
    assert lib.fm_euler_step(FAKE, FAKE, 0.1, 0, None) == C.DIT_OK
    assert lib.fm_euler_step(None, FAKE, 0.1, 10, None) == C.DIT_EINVAL
    assert lib.fm_euler_step(FAKE, FAKE, float("inf"), 10, None) == C.DIT_EINVAL
    assert lib.fm_euler_step(FAKE, FAKE, 0.1, -1, None) == C.DIT_EINVAL
    assert lib.fm_euler_step(FAKE + 4, FAKE, 0.1, 8, None) == C.DIT_EINVAL
    assert lib.fm_noise_to(FAKE, FAKE, FAKE, 0.5, 0, None) == C.DIT_OK
    assert lib.fm_noise_to(FAKE, None, FAKE, 0.5, 8, None) == C.DIT_EINVAL
    assert lib.fm_noise_to(FAKE, FAKE, FAKE, float("nan"), 8, None) == C.DIT_EINVAL
    assert lib.fm_noise_to(FAKE, FAKE, FAKE, 0.5, -1, None) == C.DIT_EINVAL
    assert lib.fm_noise_to(FAKE, FAKE, FAKE + 8, 0.5, 8, None) == C.DIT_EINVAL
    assert lib.ditk_linear(1, FAKE, FAKE, FAKE, 10, 64, 100, 0, FAKE, None) == C.DIT_ESHAPE  # K % 64
    assert lib.ditk_linear(1, FAKE, FAKE, FAKE, 10, 66, 128, 0, FAKE, None) == C.DIT_ESHAPE  # N % 4
    assert lib.ditk_linear(5, FAKE, FAKE, FAKE, 10, 64, 128, 0, FAKE, None) == C.DIT_EINVAL
    assert lib.ditk_linear(1, FAKE, FAKE, FAKE, 10, 64, 128, 9, FAKE, None) == C.DIT_EINVAL
    assert lib.ditk_rmsnorm_modulate(1, FAKE, 4, 300, None, None, 1e-6, FAKE, None) == C.DIT_ESHAPE
    assert lib.ditk_rmsnorm_modulate(1, FAKE, 4, 256, FAKE, None, 1e-6, FAKE, None) == C.DIT_EINVAL
    g = C.DitGrid(0, 1, 2, 2)
    assert lib.ditk_qknorm_rope(1, 128, 2, 5, None, FAKE, None, 256, None, FAKE, 1, g, 1e-6, 1e4,
                                1.0, None, FAKE, None, 64, None) == C.DIT_ESHAPE  # grid covers 4 < 5
    assert lib.ditk_qknorm_rope(1, 128, 2, 65, None, FAKE, None, 256, None, FAKE, 0, g, 1e-6, 1e4,
                                1.0, None, FAKE, None, 64, None) == C.DIT_ESHAPE  # cap < round_up(n)
    g2 = C.DitGrid(0, 1, 4, 4)
    assert lib.ditk_qknorm_rope(1, 128, 2, 5, None, FAKE, None, 256, None, FAKE, 0, g2, 1e-6, 1e4,
                                0.0, None, FAKE, None, 64, None) == C.DIT_EINVAL  # q_scale <= 0
    k = (C.P * 1)(FAKE)
    n = (ctypes.c_int * 1)(70)
    cap = (ctypes.c_int * 1)(64)
    assert lib.ditk_attention(1, 128, 2, FAKE, 10, 1, k, k, n, cap, 1, None, 0, 0, None, None, 0.0, FAKE, None) == C.DIT_ESHAPE
    n[0] = 40
    assert lib.ditk_attention(1, 128, 2, FAKE, 10, 1, k, k, n, cap, 2, None, 0, 0, None, None, 0.0, FAKE, None) == C.DIT_EINVAL
    assert lib.ditk_attention(1, 128, 2, FAKE, 10, 1, k, k, n, cap, 9, FAKE, 0, 0, None, None, 0.0, FAKE, None) == C.DIT_EINVAL
    assert lib.ditk_attention(0, 128, 2, FAKE, 10, 1, k, k, n, cap, 1, None, 0, 0, None, None, 0.0, FAKE, None) == C.DIT_EINVAL
    assert lib.ditk_linear_residual(1, FAKE, FAKE, FAKE, None, 64, 256, 64, FAKE, None, 5, None) == C.DIT_EINVAL
    assert lib.ditk_linear_residual(1, FAKE, FAKE, FAKE, None, 64, 256, 64, FAKE, FAKE, -1, None) == C.DIT_EINVAL
    assert lib.ditk_attention_probs(2, FAKE, 10, FAKE, 65, 128, 1, FAKE, None) == C.DIT_ESHAPE  # n > 64
    assert lib.ditk_attention_probs(2, FAKE, 10, FAKE, 0, 64, 1, FAKE, None) == C.DIT_ESHAPE
    assert lib.ditk_attention_probs(2, FAKE, 10, FAKE, 50, 32, 1, FAKE, None) == C.DIT_ESHAPE  # cap < 64
    assert lib.ditk_attention_probs(2, None, 10, FAKE, 50, 64, 1, FAKE, None) == C.DIT_EINVAL
    # unsplit_rows: negative, or neither a multiple of the 256-query tile nor >= nq
    assert lib.ditk_attention(1, 128, 2, FAKE, 300, 1, k, k, n, cap, 2, FAKE, -1, 0, None, None, 0.0, FAKE,
                              None) == C.DIT_EINVAL
    assert lib.ditk_attention(1, 128, 2, FAKE, 300, 1, k, k, n, cap, 2, FAKE, 100, 0, None, None, 0.0, FAKE,
                              None) == C.DIT_EINVAL
    # rows 256..299 are still split, so the partial buffer is required
    assert lib.ditk_attention(1, 128, 2, FAKE, 300, 1, k, k, n, cap, 2, None, 256, 0, None, None, 0.0, FAKE,
                              None) == C.DIT_EINVAL
    n[0] = 0
    assert lib.ditk_attention(1, 128, 2, FAKE, 10, 1, k, k, n, cap, 1, None, 0, 0, None, None, 0.0, FAKE, None) == C.DIT_ESHAPE  # no keys
    gp = C.DitGrid(0, 2, 4, 6)
    assert lib.ditk_patch_embed(FAKE, 0, 64, None, 0, 0, gp, FAKE, FAKE, FAKE, 256, None) == C.DIT_OK  # empty
    assert lib.ditk_patch_embed(FAKE, 48, 64, None, 0, 0, gp, FAKE, FAKE, FAKE, 320, None) == C.DIT_ESHAPE  # D % 256
    assert lib.ditk_patch_embed(FAKE, 48, 60, None, 4, 0, gp, FAKE, FAKE, FAKE, 256, None) == C.DIT_ESHAPE  # c_p % 8
    assert lib.ditk_patch_embed(FAKE, 48, 64, None, 32, 0, gp, FAKE, FAKE, FAKE, 256, None) == C.DIT_ESHAPE  # K % 64
    assert lib.ditk_patch_embed(FAKE, 48, 64, None, 64, 2, gp, FAKE, FAKE, FAKE, 256, None) == C.DIT_EINVAL  # no cond
    assert lib.ditk_patch_embed(FAKE, 47, 64, FAKE, 64, 2, gp, FAKE, FAKE, FAKE, 256, None) == C.DIT_ESHAPE  # grid != n
    assert lib.ditk_patch_embed(FAKE, 30, 64, FAKE, 64, 2, C.DitGrid(0, 2, 3, 5), FAKE, FAKE, FAKE, 256,
                                None) == C.DIT_ESHAPE  # odd grid
    assert lib.ditk_patch_embed(FAKE, 48, 64, FAKE, 64, 3, gp, FAKE, FAKE, FAKE, 256, None) == C.DIT_ESHAPE


def test_block_weight_bytes_matches_the_weight_catalogue():
    """The streaming slot holds the block entries of the weight table, 256-byte aligned."""
    lib = C.lib()
    for cid in range(1, 6):
        cfg = synth.CONFIGS[cid]
        elt = 2 if cfg.dtype == "bf16" else 4
        cat = synth.weight_catalogue(cfg)
        want = 0
        for b in C.BLOCK_ORDER:
            spec = cat.get(f"blk0.{b}")
            nbytes = 0 if spec is None else elt * int(np.prod(spec[0]))
            want += (nbytes + 255) // 256 * 256
        assert lib.dit_block_weight_bytes(ctypes.byref(_cs(cid))) == want
    assert lib.dit_block_weight_bytes(ctypes.byref(_cs(1, D=300))) == 0


def test_weight_stream_validation():
    lib, cs, h = _handle(2)
    L = cs.L
    slot = lib.dit_block_weight_bytes(ctypes.byref(cs))
    host = (C.P * (L * 22))(*([FAKE] * (L * 22)))
    assert lib.dit_weight_stream(None, host, FAKE, 2 * slot, 2) == C.DIT_EINVAL
    assert lib.dit_weight_stream(h, host, FAKE, 2 * slot, 0) == C.DIT_EINVAL            # nslot < 1
    assert lib.dit_weight_stream(h, host, FAKE, 9 * slot, L + 1) == C.DIT_EINVAL        # nslot > L
    assert lib.dit_weight_stream(h, host, FAKE + 16, 2 * slot, 2) == C.DIT_EINVAL       # ring alignment
    assert lib.dit_weight_stream(h, host, None, 2 * slot, 2) == C.DIT_EINVAL
    assert lib.dit_weight_stream(h, host, FAKE, 2 * slot - 1, 2) == C.DIT_EWORKSPACE    # ring too small
    host[22 + 2] = None                                                                  # blk1.qkv.w
    assert lib.dit_weight_stream(h, host, FAKE, 2 * slot, 2) == C.DIT_EINVAL
    assert "NULL" in C.last_error()
    assert lib.dit_weight_stream(h, None, FAKE, 0, 0) == C.DIT_EINVAL                   # off, but a ring
    assert lib.dit_weight_stream(h, None, None, 0, 0) == C.DIT_OK                        # off (already)
    lib.dit_destroy(h)


def test_audio_kv_precompute_validation():
    lib, cs, h = _handle(2)
    assert lib.audio_kv_precompute(None, FAKE, 10) == C.DIT_EINVAL
    assert lib.audio_kv_precompute(h, None, 10) == C.DIT_EINVAL
    assert lib.audio_kv_precompute(h, FAKE, 0) == C.DIT_EINVAL                     # audio with M = 0
    assert lib.audio_kv_precompute(h, FAKE, cs.max_audio + 1) == C.DIT_ESHAPE
    assert lib.audio_kv_precompute(h, FAKE, -3) == C.DIT_ESHAPE
    assert lib.audio_kv_precompute(h, None, 0) == C.DIT_OK                         # clear
    g = C.DitGrid(0, 1, 4, 4)
    # held audio requested with nothing held, or together with an audio pointer
    assert lib.dit_chunk_step(h, FAKE, None, FAKE, C.DIT_AUDIO_HELD, g, 1.0, 0.9, None) == C.DIT_EINVAL
    lib.dit_destroy(h)
    lib, cs, h = _handle(4)  # no audio weights (d_a = 0)
    assert lib.audio_kv_precompute(h, FAKE, 4) == C.DIT_EINVAL
    lib.dit_destroy(h)


def test_zero_rows_launch_nothing():
    """A call with zero rows is validated, then returns 0 without a launch; its row
    buffers may be NULL (what an empty tensor hands over), the weights may not."""
    lib = C.lib()
    assert lib.ditk_linear(1, None, FAKE, FAKE, 0, 64, 128, 0, None, None) == C.DIT_OK
    assert lib.ditk_linear(1, None, None, FAKE, 0, 64, 128, 0, None, None) == C.DIT_EINVAL  # W
    assert lib.ditk_linear(1, None, FAKE, FAKE, 0, 64, 100, 0, None, None) == C.DIT_ESHAPE  # K % 64
    assert lib.ditk_linear(1, None, FAKE, FAKE, 0, 64, 128, 9, None, None) == C.DIT_EINVAL  # act
    assert lib.ditk_linear_residual(1, None, FAKE, FAKE, None, 0, 256, 64, None, None, 0, None) == C.DIT_OK
    assert lib.ditk_rmsnorm_modulate(1, None, 0, 256, None, None, 1e-6, None, None) == C.DIT_OK
    assert lib.ditk_rmsnorm_modulate(1, None, 0, 300, None, None, 1e-6, None, None) == C.DIT_ESHAPE
    g = C.DitGrid(0, 1, 2, 2)
    assert lib.ditk_qknorm_rope(1, 128, 2, 0, None, FAKE, None, 256, None, FAKE, 1, g, 1e-6, 1e4,
                                1.0, None, FAKE, None, 64, None) == C.DIT_OK
    assert lib.ditk_attention_probs(2, None, 0, FAKE, 50, 64, 1, None, None) == C.DIT_OK
    assert lib.ditk_attention_probs(2, None, 0, None, 50, 64, 1, None, None) == C.DIT_EINVAL  # keys
    k = (C.P * 2)(FAKE, FAKE)
    n = (ctypes.c_int * 2)(40, 130)
    cap = (ctypes.c_int * 2)(64, 192)
    assert lib.ditk_attention(1, 128, 2, None, 0, 2, k, k, n, cap, 2, None, 0, 0, None, None, 0.0, None,
                              None) == C.DIT_OK
    n[1] = 200  # > cap: still rejected with zero queries
    assert lib.ditk_attention(1, 128, 2, None, 0, 2, k, k, n, cap, 1, None, 0, 0, None, None, 0.0, None,
                              None) == C.DIT_ESHAPE
    assert lib.ditk_patch_input(1, None, 0, 64, None, 0, 0, g, None, None) == C.DIT_OK
    assert lib.ditk_patch_embed(None, 0, 64, None, 0, 0, g, FAKE, FAKE, None, 256, None) == C.DIT_OK
    assert lib.fm_euler_step(None, None, 0.1, 0, None) == C.DIT_OK

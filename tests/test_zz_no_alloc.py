"""The allocation-free attention entry point (ditk_attention_noalloc) against
ditk_attention with a caller-allocated partial buffer: the same kernels on the same
inputs, so the outputs must agree bit for bit, and both must match the oracle's
attention.  Two calls in a row on the device's shared scratch, the second smaller (it
must not read anything the first left behind), plus the size bound of the scratch."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import synth
from chunked_streaming_dit_amd import _lib as C
from chunked_streaming_dit_amd import ops, torch_dtype
from tests.gpu_util import TOL, device, rel_err, to_np

pytestmark = pytest.mark.gpu

Q_SCALE = {64: np.log2(np.e) / 8.0, 128: np.log2(np.e) / np.sqrt(128.0)}


def _pack_vt(v, cap, dtype):
    """V [n, D] -> V^T [D, cap] in the documented key order (bf16: each aligned group of
    16 keys permuted so that key offset o sits at 8((o%8)/4) + 4(o/8) + o%4)."""
    n, D = v.shape
    vp = np.zeros((cap, D), dtype=np.float32)
    vp[:n] = v
    pos = np.arange(cap)
    key = pos.copy()
    if dtype == "bf16":
        g, j = (pos & 15) >> 3, pos & 7
        key = (pos & ~15) + 8 * (j >> 2) + 4 * g + (j & 3)
    return np.ascontiguousarray(vp[key].T)


def _dev(a, dtype, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(torch_dtype(dtype))


def _case(dtype, dh, H, nq, seg_ns, nsplit, unsplit, seed):
    dev = device()
    r = np.random.default_rng(seed)
    D = H * dh
    rnd = (lambda a: synth.round_bf16(a)) if dtype == "bf16" else (lambda a: a)
    q = rnd((r.standard_normal((nq, D)) * 2.0).astype(np.float32))
    segs, ks, vs, keep = [], [], [], []
    for n in seg_ns:
        cap = max(64, (n + 63) // 64 * 64)
        k = rnd((r.standard_normal((n, D)) * 2.0).astype(np.float32))
        v = rnd(r.standard_normal((n, D)).astype(np.float32))
        kp = np.zeros((cap, D), dtype=np.float32)
        kp[:n] = k
        kd, vd = _dev(kp, dtype, dev), _dev(_pack_vt(v, cap, dtype), dtype, dev)
        keep += [kd, vd]
        segs.append((kd, vd, n, cap))
        ks.append(k)
        vs.append(v)
    qd = _dev(q, dtype, dev)
    o_ref = torch.empty((nq, D), device=dev, dtype=torch_dtype(dtype))
    part = torch.empty(nsplit * nq * (D + 2 * H), device=dev)
    ops.attention(dtype, dh, H, qd, segs, o_ref, nsplit, part, q_prescaled=True, unsplit_rows=unsplit)
    o = torch.full((nq, D), float("nan"), device=dev, dtype=torch_dtype(dtype))
    ns = len(segs)
    P = ctypes.c_void_p
    kp_ = (P * ns)(*[s[0].data_ptr() for s in segs])
    vp_ = (P * ns)(*[s[1].data_ptr() for s in segs])
    nn = (ctypes.c_int * ns)(*[s[2] for s in segs])
    cp = (ctypes.c_int * ns)(*[s[3] for s in segs])
    dt = C.DIT_BF16 if dtype == "bf16" else C.DIT_F32
    C.check(C.lib().ditk_attention_noalloc(dt, dh, H, qd.data_ptr(), nq, ns, kp_, vp_, nn, cp, nsplit, unsplit, 1,
                                           None, None, 0.0, o.data_ptr(),
                                           torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref), "noalloc output differs from ditk_attention's"
    K = np.concatenate(ks).astype(np.float64).reshape(-1, H, dh)
    V = np.concatenate(vs).astype(np.float64).reshape(-1, H, dh)
    ref = O.attention((q.astype(np.float64) / Q_SCALE[dh]).reshape(nq, H, dh), K, V).reshape(nq, D)
    err = rel_err(to_np(o), ref)
    print(f"noalloc {dtype} dh {dh} H {H} nq {nq} segs {seg_ns} split {nsplit} unsplit {unsplit}: err {err:.2e}")
    assert err <= TOL[dtype] / 4, err


def test_noalloc_attention_matches_allocating_entry_point():
    # first call: a 3-way split of 2 tail q-tiles over a large key range
    _case("bf16", 128, 12, 3000, [1560, 1560, 3000], 3, 2560, 1)
    # second call, smaller, on the same scratch: must not see the first call's partials
    _case("bf16", 128, 2, 700, [130, 0, 700], 2, 256, 2)
    # fp32, every query split, a split part with no key tiles
    _case("f32", 64, 3, 300, [70, 33], 8, 0, 3)
    # nothing split (unsplit_rows >= nq): no scratch use at all
    _case("bf16", 64, 2, 200, [90], 4, 256, 4)


def test_noalloc_attention_rejects_a_split_beyond_the_scratch():
    """A split needing more than DITK_NOALLOC_SCRATCH_BYTES is DIT_EWORKSPACE, checked
    before any launch (fake, never dereferenced device addresses)."""
    fake = 0x7F0000000000
    P = ctypes.c_void_p
    k = (P * 1)(fake)
    n = (ctypes.c_int * 1)(4096)
    cap = (ctypes.c_int * 1)(4096)
    # 8 x 4096 x (1536 + 24) floats = 204 MB > 64 MiB
    rc = C.lib().ditk_attention_noalloc(C.DIT_BF16, 128, 12, fake, 4096, 1, k, k, n, cap, 8, 0, 1, None, None,
                                        0.0, fake, None)
    assert rc == C.DIT_EWORKSPACE and "allocation-free scratch" in C.last_error()

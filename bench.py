"""Benchmark of the chunked streaming DiT step on one MI355X.

Default workload (the headline): one full denoising step of the large base chunk, the
largest workload that fits one GPU: 21x30x52 = 32760 latent tokens attending to keys
[1560 reference | 1560 boundary | 32760 chunk], 200 audio tokens, 30 DiT blocks, hidden
3072, 24 heads x 128, MLP 4x, resident bf16 weights.  One bench step = the chunk's audio
K/V (audio_kv_precompute) + one dit_chunk_step (patch embed, 30 blocks of
self-attention, audio cross-attention and adaLN MLP, final layer + Euler update 1 ->
0.875); the reference and boundary passes run once before, as they do once per request
and chunk.  Inputs are resident in HBM when the timed region starts.

value = latent tokens per second of the timed steps (32760 per bench step).
roofline = the self-attention kernel (the dominant kernel: 58% of the step): algorithmic
flop 4 N_q N_kv D per launch over its dispatch-stamped HIP-event duration (from the main
kernel's start to the end of the merge of its key-range parts), against the bf16 dense
MFMA peak; traffic = the measured HBM bytes per launch (rocprofv3 FETCH_SIZE and
WRITE_SIZE, scaled by a 256 MiB copy) of profiles/attention_<workload>_traffic.json,
null when that file was taken on another attention source.
After the timed region one more bench step runs with the block GEMMs and the
elementwise kernels timed the same way: GEMM TFLOP/s (2 M N K per launch) and
elementwise GB/s (bytes the RMSNorm passes and the final layer must move).  Then the
board's measured ceilings (the library's dense bf16 MFMA loop with changing operands
and its 1 GiB copy) are taken, and every figure is also given as a fraction of them.
cpu_baseline = the f64 oracle timed on the host on a bounded sample (large chunk: one
DiT block with the K/V of all tokens and the queries of 1 and of 2048 sampled rows,
extrapolated linearly in the rows to the whole block and times 30 blocks; base chunk:
one whole DiT block of one step, times 4).

Other workloads (--workload):
  base     one base low-res chunk job: modulation table, reference K/V, boundary K/V,
           audio K/V, 8 Euler steps 1 -> 0 (7800 tokens, keys 1560 + 1560 + 7800, 4
           blocks, hidden 1536, 12 heads); value = 7800 x 8 latent tokens per job / time
  stream6  the streaming sequence: 6 consecutive base chunks, each chunk's boundary
           from the previous chunk's final latent (the first chunk has none); one bench
           step = one whole session (modulation table and reference K/V once, then per
           chunk boundary K/V, audio K/V and 8 steps); value = generated latent tokens/s
           at the steady-state per-chunk latency (median over chunks 1-5); chunk 0's
           latency is reported as the time to the first chunk
  interp   an interpolation chunk of the base shape (boundary and anchor passes, keys
           [reference | boundary | anchor | chunk])
  iwin     an interpolation chunk of the base shape under the window reading: a window of
           the chunk's frames between its two anchor frames (10920 tokens, keys 1560
           reference + 10920 window), both anchors re-noised to each step's time
           (fm_noise_to) before each of the 8 steps; value = the chunk's 7800 latent
           tokens x 8 per job / time
  reuse    base chunk jobs whose boundary is carried by reuse (no boundary pass)
  sr, sr1  super-resolution chunk jobs (31200 tokens, 2 blocks, no audio): boundary
           pass + 4 Euler steps (sr) or one step 1 -> 0 (sr1)
  tiny     the launch-bound fp32 single-block chunk (128 tokens): one step's latency,
           eager and replayed from a captured HIP graph (value: the graph's rate)
  wstream  the large-chunk step with the block weights streamed from pinned host memory
           through a 2-slot device ring (dit_weight_stream), with the resident step, the
           first (cold) streamed step and the stage hand-over measured in the same process
Measurement modes besides the workloads: --elementwise-sweep (the HBM-bound kernels over
sizes), --copy-probe (the counter calibration copy), --gemm-compare (the block-Linear
GEMMs next to the vendor BLAS on the same shapes, as a reference point for their rate).
The large-chunk weights are drawn on the GPU (seeded N(0, 1/fan_in), gammas
1 + 0.1 N(0, 1)) to keep the 6.7 G parameters' set-up short; the other workloads use the
seeded host catalogue of synth.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "DiT chunk-step latent tokens/sec and attention TFLOP/s (% bf16 MFMA peak), 1 GPU"
METRIC_STREAM6 = ("DiT streaming sequence generated latent tokens/sec (steady-state chunk latency) and "
                  "attention TFLOP/s (% bf16 MFMA peak), 1 GPU")
METRIC_INTERP = ("DiT interpolation-chunk latent tokens/sec and attention TFLOP/s "
                 "(% bf16 MFMA peak), 1 GPU")
METRIC_IWIN = ("DiT interpolation-chunk (anchor window) latent tokens/sec and attention TFLOP/s "
               "(% bf16 MFMA peak), 1 GPU")
METRIC_SR = ("DiT super-resolution chunk latent tokens/sec and attention TFLOP/s "
             "(% bf16 MFMA peak), 1 GPU")
METRIC_SR1 = ("DiT single-step super-resolution chunk latent tokens/sec and attention TFLOP/s "
              "(% bf16 MFMA peak), 1 GPU")
METRIC_WSTREAM = ("DiT large-chunk denoising step latent tokens/sec with block weights streamed "
                  "from pinned host memory, 1 GPU")
METRIC_REUSE = ("DiT chunk-step latent tokens/sec, boundary carried by reuse, and attention "
                "TFLOP/s (% bf16 MFMA peak), 1 GPU")
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
ATTN_SRC = os.path.join(ROOT, "chunked_streaming_dit_amd", "csrc", "attention.hip")
TRAFFIC_FILES = {
    "large": os.path.join(ROOT, "profiles", "attention_large_chunk_traffic.json"),
    "base": os.path.join(ROOT, "profiles", "attention_base_chunk_traffic.json"),
    "sr": os.path.join(ROOT, "profiles", "attention_sr_chunk_traffic.json"),
    "sr1": os.path.join(ROOT, "profiles", "attention_sr1_chunk_traffic.json"),
}
DIT_TIME_ATTN, DIT_TIME_GEMM, DIT_TIME_ELEM = 0, 1, 2

WORKLOAD_LARGE = ("large base chunk: 21x30x52 = 32760 latent tokens, keys 1560 reference + 1560 "
                  "boundary + 32760 chunk, 200 audio tokens of dim 768, 30 DiT blocks, hidden 3072, "
                  "24 heads x 128, MLP 4x, one Euler step 1 -> 0.875; one bench step = audio K/V + "
                  "one denoising step (the reference and boundary passes run before)")
WORKLOAD_BASE = ("base low-res chunk: 5x30x52 = 7800 latent tokens, 1560 reference + 1560 "
                 "boundary tokens, 50 audio tokens of dim 768, 4 DiT blocks, hidden 1536, "
                 "12 heads x 128, MLP 4x, 8 Euler steps 1 -> 0; one bench step = modulation "
                 "table + reference K/V + boundary K/V + audio K/V + 8 denoising steps")


def _src_hash(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def _traffic(workload: str):
    """HBM bytes per self-attention launch from the committed rocprofv3 counter summary of
    the workload, or None if it is missing or was taken on a different attention source."""
    path = TRAFFIC_FILES.get(workload)
    try:
        d = json.load(open(path))
    except (OSError, ValueError, TypeError):
        return None
    if d.get("attention_src_sha256_16") != _src_hash(ATTN_SRC):
        return None
    return d.get("hbm_bytes_per_launch")


COPY_PROBE_BYTES = 256 << 20


def copy_probe(reps: int = 3) -> None:
    """The library's plain copy kernel (ditk_probe_copy) over COPY_PROBE_BYTES: the
    known-size kernel that calibrates the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    from chunked_streaming_dit_amd import _lib as C
    dev = torch.device("cuda", 0)
    a = torch.empty(COPY_PROBE_BYTES // 4, device=dev)
    b = torch.empty_like(a)
    for _ in range(reps):
        C.check(C.lib().ditk_probe_copy(a.data_ptr(), b.data_ptr(), COPY_PROBE_BYTES,
                                        torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()


def elementwise_sweep(reps: int = 20) -> int:
    """HBM-bound kernels of the step swept over sizes up to about 1 GB moved per launch:
    RMSNorm + modulate (hidden 1536 and 3072, bf16 out), the standalone QK-norm + RoPE +
    V^T repack (24 heads x 128), the Euler update, the flow-matching re-noise and the
    plain copy.  Each launch is timed by HIP events over `reps` launches after two
    untimed ones; bytes are the algorithmic ones (every input read once, every output
    written once).  Sizes up to a few hundred MB can be served partly by the 256 MB
    memory-side cache on repeats, so their rates may exceed what HBM alone gives.
    Prints one JSON line per (kernel, size)."""
    import torch

    from chunked_streaming_dit_amd import _lib as C
    from chunked_streaming_dit_amd import fm_euler_step, fm_noise_to, grid, ops
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(5)

    def timed(fn) -> float:
        for _ in range(2):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    def emit(kernel, shape, nbytes, us):
        gbs = nbytes / (us * 1e-6) / 1e9
        print(json.dumps({"kernel": kernel, "shape": shape, "bytes": nbytes, "us": round(us, 2),
                          "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 3)}), flush=True)

    for D in (1536, 3072):
        for n in (1560, 7800, 32760, 65520) if D == 3072 else (1560, 7800, 32760, 109200):
            h = torch.randn(n, D, generator=g, device=dev)
            shift = torch.randn(D, generator=g, device=dev)
            scale = torch.randn(D, generator=g, device=dev)
            out = torch.empty(n, D, device=dev, dtype=torch.bfloat16)
            us = timed(lambda: ops.rmsnorm_modulate(h, shift, scale, 1e-6, out, "bf16"))
            emit("rmsnorm_modulate", f"{n}x{D} fp32 -> bf16", n * D * 6 + 2 * D * 4, us)
            del h, out
    H, dh = 24, 128
    D = H * dh
    for frames in (1, 5, 21, 42):
        n = frames * 1560
        cap = (n + 63) // 64 * 64
        qkv = torch.randn(n, 3 * D, generator=g, device=dev).to(torch.bfloat16)
        gq = torch.ones(dh, device=dev, dtype=torch.bfloat16)
        gk = torch.ones(dh, device=dev, dtype=torch.bfloat16)
        qo = torch.empty(cap, D, device=dev, dtype=torch.bfloat16)
        ko = torch.empty(cap, D, device=dev, dtype=torch.bfloat16)
        vt = torch.empty(D, cap, device=dev, dtype=torch.bfloat16)
        gr = grid(0, frames, 30, 52)
        us = timed(lambda: ops.qknorm_rope("bf16", dh, H, n, qkv, qkv[:, D:], qkv[:, 2 * D:], 3 * D, gq, gk,
                                           True, gr, 1e-6, 10000.0, qo, ko, vt, cap))
        emit("qknorm_rope", f"{n} tokens x 3 x {H}x{dh} bf16", n * 3 * D * 2 * 2 + 2 * dh * 2, us)
        del qkv, qo, ko, vt
    for n in (1 << 20, 8 << 20, 32 << 20, 89 << 20):
        x = torch.randn(n, generator=g, device=dev)
        v = torch.randn(n, generator=g, device=dev)
        e = torch.randn(n, generator=g, device=dev)
        us = timed(lambda: fm_euler_step(x, v, -0.125))
        emit("fm_euler_step", f"{n} fp32", 12 * n, us)
        us = timed(lambda: fm_noise_to(x, v, e, 0.375))
        emit("fm_noise_to", f"{n} fp32", 12 * n, us)
        us = timed(lambda: C.check(C.lib().ditk_probe_copy(v.data_ptr(), x.data_ptr(), 4 * n,
                                                           torch.cuda.current_stream().cuda_stream)))
        emit("probe_copy", f"{4 * n} bytes", 8 * n, us)
        del x, v, e
    return 0


GEMM_COMPARE_SHAPES = (
    # (name, M, N, K, epilogue): the block Linears of the large and of the base chunk
    ("large QKV (bias)", 32760, 9216, 3072, "bias"),
    ("large MLP in (bias + GELU)", 32760, 12288, 3072, "gelu"),
    ("large MLP out (gated residual)", 32760, 3072, 12288, "resid"),
    ("large out-projection (gated residual)", 32760, 3072, 3072, "resid"),
    ("base QKV (bias)", 7800, 4608, 1536, "bias"),
    ("base MLP in (bias + GELU)", 7800, 6144, 1536, "gelu"),
)


def gemm_compare(reps: int = 20, rounds: int = 5) -> int:
    """The library's block-Linear GEMM (ditk_linear / ditk_linear_residual, bf16, fused
    epilogue) next to the vendor BLAS on the same operands (torch.nn.functional.linear,
    which runs hipBLASLt on this stack: bias only, its output written in bf16), timed by
    HIP events over `reps` launches after three untimed ones, the two alternated for
    `rounds` rounds (median).  A reference point for the GEMM's rate on this board, not
    a path of the library.  Prints one JSON line per shape."""
    import torch
    import torch.nn.functional as F

    from chunked_streaming_dit_amd import ops
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(11)

    def timed(fn) -> float:
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    for name, M, N, K, epi in GEMM_COMPARE_SHAPES:
        A = torch.randn(M, K, generator=g, device=dev).to(torch.bfloat16)
        W = (torch.randn(N, K, generator=g, device=dev) / K ** 0.5).to(torch.bfloat16)
        bias = (0.1 * torch.randn(N, generator=g, device=dev)).to(torch.bfloat16)
        if epi == "resid":
            gate = torch.rand(N, generator=g, device=dev)
            h = torch.zeros(M, N, device=dev)
            ours = lambda: ops.linear_residual(A, W, bias, gate, h, "bf16")
        else:
            out = torch.empty(M, N, device=dev, dtype=torch.bfloat16)
            act = 1 if epi == "gelu" else 0
            ours = lambda: ops.linear(A, W, bias, act, out, "bf16")
        vendor = lambda: F.linear(A, W, bias)
        t_ours, t_vendor = [], []
        for _ in range(rounds):
            t_ours.append(timed(ours))
            t_vendor.append(timed(vendor))
        us_o, us_v = sorted(t_ours)[rounds // 2], sorted(t_vendor)[rounds // 2]
        fl = 2.0 * M * N * K
        print(json.dumps({"gemm": name, "M": M, "N": N, "K": K, "epilogue": epi,
                          "library_us": round(us_o, 1), "library_tflops": round(fl / us_o / 1e6, 1),
                          "vendor_us": round(us_v, 1), "vendor_tflops": round(fl / us_v / 1e6, 1),
                          "library_over_vendor": round(us_v / us_o, 3)}), flush=True)
        del A, W, bias
    return 0


def ceilings() -> dict:
    """Measured ceilings on this board, in the same process: the library's dense bf16
    MFMA loop (operands with changing bits, no memory traffic) and its plain copy of
    1 GiB (HBM bandwidth, 2 x bytes moved), each timed with HIP events."""
    import ctypes

    import torch

    from chunked_streaming_dit_amd import _lib as C
    dev = torch.device("cuda", 0)
    st = torch.cuda.current_stream().cuda_stream
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    data = torch.randn(2048, generator=g, device=dev).to(torch.bfloat16)
    sink = torch.empty(C.DITK_PROBE_SINK_FLOATS, device=dev)
    flop = ctypes.c_double()

    def timed(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        return a.elapsed_time(b)

    # about 0.5 s of warm-up, then about 0.5 s timed: long enough for the board's clock
    # and power management to settle, as it does over the bench's timed steps
    C.check(C.lib().ditk_probe_mfma(data.data_ptr(), 2000000, sink.data_ptr(), sink.numel(), ctypes.byref(flop), st))
    ms = timed(lambda: C.check(C.lib().ditk_probe_mfma(data.data_ptr(), 2000000, sink.data_ptr(), sink.numel(),
                                                        ctypes.byref(flop), st)))
    mfma = flop.value / (ms * 1e-3) / 1e12
    nbytes = 1 << 30
    src = torch.empty(nbytes // 4, device=dev)
    dst = torch.empty_like(src)
    copy = lambda: C.check(C.lib().ditk_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, st))  # noqa: E731
    copy()
    ms = timed(lambda: [copy() for _ in range(10)]) / 10
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    del src, dst
    return {"mfma_bf16_ceiling_tflops": mfma, "hbm_copy_ceiling_gbs": gbs}


def _counter_means(path: str, counter: str, match, largest_grid: bool = False, skip_first: bool = False) -> tuple:
    """(mean counter value, dispatches) over the dispatches of a rocprofv3 counter CSV
    whose kernel name satisfies match (largest_grid: only those of the largest grid;
    skip_first: without the first of them in dispatch order)."""
    import csv
    rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter and match(r["Kernel_Name"])]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    if skip_first:
        rows = rows[1:]
    if largest_grid and rows:
        g = max(int(r["Grid_Size"]) for r in rows)
        rows = [r for r in rows if int(r["Grid_Size"]) == g]
    vals = [float(r["Counter_Value"]) for r in rows]
    if not vals:
        raise SystemExit(f"bench.py: no {counter} rows matched in {path}")
    return sum(vals) / len(vals), len(vals)


def _is_self_attention(name: str) -> bool:
    """attn_kernel<T, DH, KIND> with KIND 0 (self-attention; 1 is the audio cross-attention),
    demangled or mangled."""
    import re
    return re.search(r"attn_kernel(<[^<>]*,\s*0>|I\w*Li0EE)", name) is not None


# The timed region's self-attention launches: the large-chunk bench times only the
# denoising step's launches (the largest grid; its context passes run before); the base
# chunk job times all of its launches, reference pass included; a super-resolution job
# times its boundary pass and steps, while the session's one reference pass (the first
# self-attention dispatch of the run) lies outside the timed region.
TRAFFIC_LARGEST_GRID = {"large": True, "base": False, "sr": False, "sr1": False}
TRAFFIC_SKIP_FIRST = {"sr": True, "sr1": True}


def reduce_traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, largest_grid=False,
                   skip_first=False) -> dict:
    """HBM bytes per self-attention launch from four rocprofv3 --pmc runs (FETCH_SIZE and
    WRITE_SIZE, in KiB per dispatch, over the bench and over copy_probe), each counter
    scaled so that the copy reads COPY_PROBE_BYTES and writes COPY_PROBE_BYTES."""
    kib = COPY_PROBE_BYTES / 1024
    cf, _ = _counter_means(copy_fetch_csv, "FETCH_SIZE", lambda n: "copy" in n.lower())
    cw, _ = _counter_means(copy_write_csv, "WRITE_SIZE", lambda n: "copy" in n.lower())
    f, nf = _counter_means(fetch_csv, "FETCH_SIZE", _is_self_attention, largest_grid, skip_first)
    w, nw = _counter_means(write_csv, "WRITE_SIZE", _is_self_attention, largest_grid, skip_first)
    sf, sw = kib / cf, kib / cw
    return {
        "attention_src_sha256_16": _src_hash(ATTN_SRC),
        "hbm_bytes_per_launch": (f * sf + w * sw) * 1024,
        "fetch_bytes_per_launch": f * sf * 1024,
        "write_bytes_per_launch": w * sw * 1024,
        "fetch_scale": sf,
        "write_scale": sw,
        "dispatches": [nf, nw],
        "largest_grid_only": bool(largest_grid),
        "first_dispatch_skipped": bool(skip_first),
    }


# ---------------------------------------------------------------------------- CPU baseline


def _cpu_info() -> tuple:
    """(BLAS threads in use, CPU model name)."""
    from threadpoolctl import threadpool_info
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return threads, model


def cpu_baseline_block(cfg, P, inp, budget_s: float = 12.0):
    """The oracle on one DiT block of one denoising step at the full chunk shape (repeated
    up to L times while under the budget), scaled to the L-block step."""
    import dataclasses

    import numpy as np

    import oracle as O

    one = dataclasses.replace(cfg, L=1)
    ref_kv = O.ref_context(P, one, inp["ref"], one.ref)
    bkv = O.bnd_context(P, one, ref_kv, inp["bnd"], one.bnd.h, one.bnd.w)
    ctx = [[ref_kv[0], bkv[0]]]
    pos = O.grid_positions(0, cfg.chunk.frames, cfg.chunk.h, cfg.chunk.w)
    times = []
    while len(times) < cfg.L and sum(times) < budget_s:
        t0 = time.perf_counter()
        O.dit_velocity(P, one, inp["x_init"], 1.0, pos, ctx, inp["audio"])
        times.append(time.perf_counter() - t0)
    t_block = float(np.median(times))
    threads, model = _cpu_info()
    return {
        "value": cfg.N / (t_block * cfg.L),
        "unit": "latent tokens/s",
        "cores": threads,
        "cpu": model,
        "kind": "oracle",
        "sample": (f"{len(times)} x one DiT block of one denoising step at the full chunk shape "
                   f"({cfg.N} tokens, {cfg.N_ref}+{cfg.N_bnd}+{cfg.N} keys, audio {cfg.M}), "
                   f"median {t_block:.2f} s x {cfg.L} blocks; context passes excluded"),
    }


def cpu_baseline_rows(cfg, inp, rows=(1, 2048)):
    """The oracle on one DiT block of the workload (its block 0 weights from the seeded
    catalogue) with the keys and values of every token and the queries of sampled rows,
    timed for one row (almost only the keys and values of all tokens) and for many rows;
    the block's time is extrapolated linearly in the rows to all N rows, times L blocks."""
    import dataclasses

    import numpy as np

    import oracle as O
    import synth

    one = dataclasses.replace(cfg, L=1)
    P = synth.make_weights(one, threads=16, compact=True)
    ref_kv = O.ref_context(P, one, inp["ref"], one.ref)
    bkv = O.bnd_context(P, one, ref_kv, inp["bnd"], one.bnd.h, one.bnd.w)
    ctx = [[ref_kv[0], bkv[0]]]
    g = cfg.chunk
    pos = O.grid_positions(0, g.frames, g.h, g.w)
    ts = []
    for r in rows:
        sel = np.linspace(0, cfg.N - 1, r).astype(np.int64)
        t0 = time.perf_counter()
        O.velocity_rows(P, one, inp["x_init"], cfg.t_start, pos, ctx, inp["audio"], sel)
        ts.append(time.perf_counter() - t0)
    t_row = max(ts[1] - ts[0], 0.0) / (rows[1] - rows[0])
    t_block = ts[0] + t_row * (cfg.N - rows[0])
    threads, model = _cpu_info()
    return {
        "value": cfg.N / (t_block * cfg.L),
        "unit": "latent tokens/s",
        "cores": threads,
        "cpu": model,
        "kind": "oracle",
        "sample": (f"one DiT block of the large chunk ({cfg.N} tokens, keys {cfg.N_ref}+{cfg.N_bnd}+{cfg.N}, "
                   f"audio {cfg.M}): K/V of every token with the queries of {rows[0]} row in {ts[0]:.1f} s "
                   f"and of {rows[1]} sampled rows in {ts[1]:.1f} s; block extrapolated linearly in the "
                   f"rows to {t_block:.0f} s ({t_row * 1e3:.2f} ms per row), x {cfg.L} blocks; "
                   f"context passes excluded"),
    }


# ---------------------------------------------------------------------------- shared


def _device_weights(cfg, dev, seed: int = 5):
    """Random-init weights of the workload's shapes drawn on the GPU: N(0, 1/fan_in),
    QK-norm gammas 1 + 0.1 N(0, 1), in the compute dtype."""
    import torch

    import synth
    from chunked_streaming_dit_amd import torch_dtype
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    td = torch_dtype(cfg.dtype)
    out = {}
    for name, (shape, fan_in, kind) in synth.weight_catalogue(cfg).items():
        z = torch.randn(shape, generator=g, device=dev, dtype=torch.float32)
        z = z * (fan_in ** -0.5) if kind == "w" else 1.0 + 0.1 * z
        out[name] = z.to(td)
    return out


def _attn_fields(h):
    """(attention TFLOP/s, config fields) from the handle's self-attention timing window."""
    n, ms, flop = h.timing_read(DIT_TIME_ATTN)
    tf = flop / (ms * 1e-3) / 1e12 if ms > 0 else 0.0
    return tf, {"attention_tflops": tf, "attention_frac_bf16_peak": tf / PEAK_BF16_TFLOPS,
                "attention_launches": n, "attention_avg_launch_ms": ms / max(n, 1)}


def _breakdown(h, one_step) -> dict:
    """One more bench step with the block GEMMs and the elementwise kernels timed by
    dispatch-stamped events (outside the timed region)."""
    import torch
    h.timing_enable((1 << DIT_TIME_GEMM) | (1 << DIT_TIME_ELEM))
    one_step()
    torch.cuda.synchronize()
    ng, msg, fg = h.timing_read(DIT_TIME_GEMM)
    ne, mse, be = h.timing_read(DIT_TIME_ELEM)
    h.timing_enable(False)
    gtf = fg / (msg * 1e-3) / 1e12 if msg > 0 else 0.0
    egb = be / (mse * 1e-3) / 1e9 if mse > 0 else 0.0
    return {"gemm_tflops": gtf, "gemm_frac_bf16_peak": gtf / PEAK_BF16_TFLOPS, "gemm_launches": ng,
            "gemm_ms_per_step": msg, "elementwise_gbs": egb, "elementwise_frac_hbm": egb / PEAK_HBM_GBS,
            "elementwise_launches": ne, "elementwise_ms_per_step": mse}


def _with_ceilings(extra: dict) -> dict:
    """The measured ceilings and each figure's fraction of them."""
    c = ceilings()
    extra.update(c)
    m, h = c["mfma_bf16_ceiling_tflops"], c["hbm_copy_ceiling_gbs"]
    if "attention_tflops" in extra:
        extra["attention_frac_mfma_ceiling"] = extra["attention_tflops"] / m
    if "gemm_tflops" in extra:
        extra["gemm_frac_mfma_ceiling"] = extra["gemm_tflops"] / m
    if "elementwise_gbs" in extra:
        extra["elementwise_frac_copy_ceiling"] = extra["elementwise_gbs"] / h
    return extra


def _line(metric, value, args, ms, workload, extra, achieved, traffic, data=None):
    return {
        "metric": metric,
        "value": value,
        "unit": "latent tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": data or "synthetic (seeded N(0,1) latents/audio, N(0,1/fan_in) random-init weights)",
        "config": dict({"workload": workload}, **extra),
        "roofline": {
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": traffic,
        },
    }


# ---------------------------------------------------------------------------- workloads


def large_main(args) -> int:
    """large (default) / wstream: one denoising step of the large base chunk."""
    import torch

    import synth
    from chunked_streaming_dit_amd import AUDIO_HELD, DitChunk
    from chunked_streaming_dit_amd.workload import chunk_config, f32, grid_of

    dev = torch.device("cuda", 0)
    cfg = synth.LARGE_CHUNK
    W = _device_weights(cfg, dev)
    inp = synth.make_inputs(cfg, 0)
    h = DitChunk(chunk_config(cfg), W, dev)
    x0 = f32(inp["x_init"], dev)
    audio = f32(inp["audio"], dev)
    x = torch.empty_like(x0)
    t0, t1 = cfg.t_start, cfg.t_end
    g_chunk = grid_of(cfg.chunk)
    wstream = args.workload == "wstream"

    def context():
        h.ref_kv_precompute(f32(inp["ref"], dev), grid_of(cfg.ref))
        h.boundary_kv_carry(f32(inp["bnd"], dev), grid_of(synth.Grid(0, 1, cfg.bnd.h, cfg.bnd.w)))

    def step():
        x.copy_(x0)
        h.audio_kv_precompute(audio)
        h.step(x, t0, t1, g_chunk, audio=AUDIO_HELD)

    def timed(k):
        torch.cuda.synchronize()
        a = time.perf_counter()
        for _ in range(k):
            step()
        torch.cuda.synchronize()
        return (time.perf_counter() - a) * 1e3 / k

    context()
    extra = {"tokens_per_step": cfg.N}
    host = None
    if wstream:
        for _ in range(args.warmup):
            step()
        resident_ms = timed(args.steps)
        host = {}
        for name, t in W.items():
            if name.startswith("blk"):
                p = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
                p.copy_(t)
                host[name] = p
        # cold: nothing runs while the first blocks are copied
        torch.cuda.synchronize()
        a = time.perf_counter()
        h.weight_stream(host, nslot=2)
        step()
        torch.cuda.synchronize()
        cold_ms = (time.perf_counter() - a) * 1e3
        extra.update({"resident_ms_per_step": resident_ms, "cold_first_step_ms": cold_ms,
                      "block_weight_bytes": h.cfg.block_weight_bytes(), "ring_slots": 2})
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    h.timing_enable(1 << DIT_TIME_ATTN)
    ms = timed(args.steps)
    achieved, af = _attn_fields(h)
    h.timing_enable(False)
    extra.update(af)
    if wstream:
        extra["exposed_ms_per_step"] = ms - resident_ms
        extra["cold_exposed_ms"] = cold_ms - ms
        # switch: streaming is enabled while a resident step still runs, so the first
        # blocks' transfer overlaps it (the hand-over between two models' stages);
        # exposed = pair - resident step - streamed step, median of 3
        sw = []
        for _ in range(3):
            h.weight_stream(None)
            torch.cuda.synchronize()
            a = time.perf_counter()
            step()
            h.weight_stream(host, nslot=2)
            step()
            torch.cuda.synchronize()
            sw.append((time.perf_counter() - a) * 1e3 - resident_ms - ms)
        extra["switch_exposed_ms"] = sorted(sw)[1]
    else:
        extra.update(_breakdown(h, step))
        _with_ceilings(extra)
    if not torch.isfinite(x).all():
        print("bench.py: non-finite output", file=sys.stderr)
        return 1
    workload = WORKLOAD_LARGE
    if wstream:
        workload += ("; block weights (387.0 MB each) streamed from pinned host memory "
                     "through a 2-slot device ring")
    line = _line(METRIC_WSTREAM if wstream else METRIC, cfg.N / (ms * 1e-3), args, ms, workload, extra,
                 achieved, None if wstream else _traffic("large"),
                 data="synthetic (seeded N(0,1) latents/audio, random-init weights drawn on the GPU)")
    # Teardown before the baseline and the exit: the handle first (streaming off, device
    # synchronised), then the ring and the pinned host blocks.
    h.close()
    host = None
    torch.cuda.synchronize()
    if not args.no_cpu_baseline and not wstream:
        line["cpu_baseline"] = cpu_baseline_rows(cfg, inp)
    print(json.dumps(line), flush=True)
    return 0


def tiny_main(args) -> int:
    """tiny: the launch-bound fp32 single-block workload (128 tokens, hidden 256): one
    denoising step's latency run eagerly and as a captured HIP graph replayed."""
    import numpy as np
    import torch

    import synth
    from chunked_streaming_dit_amd import DitChunk
    from chunked_streaming_dit_amd.workload import chunk_config, f32, grid_of, upload_weights

    dev = torch.device("cuda", 0)
    cfg = synth.TINY_FP32
    P = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg, 0)
    s = torch.cuda.Stream(device=dev)
    reps = max(args.steps, 1) * 20
    with torch.cuda.stream(s):
        h = DitChunk(chunk_config(cfg), upload_weights(P, cfg.dtype, dev), dev)
        h.ref_kv_precompute(f32(inp["ref"], dev), grid_of(cfg.ref))
        h.boundary_kv_carry(f32(inp["bnd"], dev), grid_of(synth.Grid(0, 1, cfg.bnd.h, cfg.bnd.w)))
        audio = f32(inp["audio"], dev)
        x = f32(inp["x_init"], dev)
        g_chunk = grid_of(cfg.chunk)
        t0, t1 = cfg.t_start, cfg.t_end

        def timed(fn):
            out = []
            for _ in range(reps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(s)
                fn()
                b.record(s)
                out.append((a, b))
            s.synchronize()
            return float(np.median([a.elapsed_time(b) for a, b in out])) * 1e3

        step = lambda: h.step(x, t0, t1, g_chunk, audio=audio)  # noqa: E731
        for _ in range(args.warmup * 20 + 1):
            step()
        eager_us = timed(step)
    s.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step()
    with torch.cuda.stream(s):
        for _ in range(args.warmup * 20 + 1):
            graph.replay()
        graph_us = timed(graph.replay)
    s.synchronize()
    if not torch.isfinite(x).all():
        print("bench.py: non-finite output", file=sys.stderr)
        return 1
    workload = ("tiny single-block chunk, fp32: 2x8x8 = 128 latent tokens, keys 64 reference + 32 boundary + "
                "128 chunk, 16 audio tokens of dim 64, 1 DiT block, hidden 256, 4 heads x 64, MLP 4x, one Euler "
                "step 0.5 -> 0.45; one bench step = one denoising step (median of "
                f"{reps} event-timed steps), replayed from a captured HIP graph; the eager latency alongside")
    line = _line("DiT tiny chunk-step latent tokens/sec (fp32, launch-bound; HIP-graph replay), 1 GPU",
                 cfg.N / (graph_us * 1e-6), args, graph_us * 1e-3, workload,
                 {"tokens_per_step": cfg.N, "graph_us_per_step": graph_us, "eager_us_per_step": eager_us,
                  "graph_speedup": eager_us / graph_us}, 0.0, None)
    line["dtype"] = "f32"
    line["roofline"] = None
    print(json.dumps(line), flush=True)
    h.close()
    return 0


def stream6_main(args) -> int:
    """stream6: whole 6-chunk streaming sessions of the base chunk shape."""
    import numpy as np
    import torch

    import synth
    from chunked_streaming_dit_amd import AUDIO_HELD, DitChunk
    from chunked_streaming_dit_amd.workload import chunk_config, f32, grid_of, upload_weights

    dev = torch.device("cuda", 0)
    cfg = synth.STREAM_6_CHUNKS
    P = synth.make_weights(cfg)
    chunks = [synth.make_inputs(cfg, c) for c in range(cfg.n_chunks)]
    h = DitChunk(chunk_config(cfg), upload_weights(P, cfg.dtype, dev), dev)
    ref = f32(chunks[0]["ref"], dev)
    x0 = [f32(c["x_init"], dev) for c in chunks]
    aud = [f32(c["audio"], dev) for c in chunks]
    xs = [torch.empty_like(a) for a in x0]
    S = cfg.steps
    ts = [cfg.t_start + (cfg.t_end - cfg.t_start) * k / S for k in range(S + 1)]
    g_chunk, g_ref, g_none = grid_of(cfg.chunk), grid_of(cfg.ref), grid_of(synth.Grid(0, 0, 0, 0))

    def session():
        """One request: per-chunk latencies (ms), chunk 0 including the request's set-up."""
        lat = []
        torch.cuda.synchronize()
        a = time.perf_counter()
        h.modulation_table(ts[:-1] + [0.0])
        h.ref_kv_precompute(ref, g_ref)
        for c in range(cfg.n_chunks):
            h.boundary_kv_carry(xs[c - 1] if c else None, g_chunk if c else g_none)
            xs[c].copy_(x0[c])
            h.audio_kv_precompute(aud[c])
            for k in range(S):
                h.step(xs[c], ts[k], ts[k + 1], g_chunk, audio=AUDIO_HELD)
            torch.cuda.synchronize()
            b = time.perf_counter()
            lat.append((b - a) * 1e3)
            a = b
        return lat

    for _ in range(args.warmup):
        session()
    h.timing_enable(1 << DIT_TIME_ATTN)
    lats = [session() for _ in range(args.steps)]
    achieved, af = _attn_fields(h)
    h.timing_enable(False)
    steady = float(np.median([l for s in lats for l in s[1:]]))
    first = float(np.median([s[0] for s in lats]))
    ms = float(np.mean([sum(s) for s in lats]))
    if not all(torch.isfinite(x).all() for x in xs):
        print("bench.py: non-finite output", file=sys.stderr)
        return 1
    extra = {"chunks": cfg.n_chunks, "tokens_per_chunk": cfg.N, "steady_chunk_ms": steady,
             "first_chunk_ms": first,
             "chunk_ms_median_by_index": [float(np.median([s[c] for s in lats])) for c in range(cfg.n_chunks)]}
    extra.update(af)
    workload = ("streaming sequence: 6 consecutive base low-res chunks (7800 latent tokens each, keys "
                "1560 reference + 1560 boundary (none for chunk 0) + 7800 chunk, 50 audio tokens, 4 DiT "
                "blocks, hidden 1536, 12 heads x 128, 8 Euler steps 1 -> 0 per chunk), each boundary the "
                "last latent frame of the previous chunk's final latent; one bench step = one session "
                "(modulation table + reference K/V once, then per chunk boundary K/V + audio K/V + 8 "
                "steps); value = 7800 / steady-state chunk latency (median over chunks 1-5)")
    print(json.dumps(_line(METRIC_STREAM6, cfg.N / (steady * 1e-3), args, ms, workload, extra, achieved, None)),
          flush=True)
    h.close()
    return 0


def chunk_main(args) -> int:
    """base / interp / iwin / reuse / sr / sr1: chunk jobs of the base or super-resolution shape."""
    import torch

    import synth
    from chunked_streaming_dit_amd import AUDIO_HELD, DitChunk, fm_noise_to
    from chunked_streaming_dit_amd.workload import chunk_config, f32, grid_of, upload_weights

    dev = torch.device("cuda", 0)
    sr = args.workload in ("sr", "sr1")
    cfg = synth.SUPER_RES if sr else synth.BASE_CHUNK
    P = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg, 0)
    W = upload_weights(P, cfg.dtype, dev)
    iwin = args.workload == "iwin"
    gc = cfg.chunk
    hw = gc.h * gc.w
    F = gc.frames
    h = DitChunk(chunk_config(cfg, max_tokens=(F + 2) * hw if iwin else None), W, dev)
    ref = f32(inp["ref"], dev)
    bnd = f32(inp["bnd"], dev)
    x0 = f32(inp["x_init"], dev)
    audio = f32(inp["audio"], dev) if cfg.M else None
    cond = f32(inp["cond_lr"], dev) if sr else None
    x = torch.empty(((F + 2) * hw, cfg.C_p), device=dev) if iwin else torch.empty_like(x0)
    S = 1 if args.workload == "sr1" else cfg.steps
    ts = [cfg.t_start + (cfg.t_end - cfg.t_start) * k / S for k in range(S + 1)]
    g_chunk = grid_of(cfg.chunk)
    g_ref = grid_of(cfg.ref)
    g_prev = grid_of(synth.Grid(0, 1, cfg.bnd.h, cfg.bnd.w))
    interp = args.workload == "interp"
    reuse = args.workload == "reuse"
    if sr or reuse or interp or iwin:
        h.ref_kv_precompute(ref, g_ref)  # once per request, outside the timed region
    if reuse:
        h.boundary_kv_carry(bnd, g_prev)  # the first job's boundary; later ones are carried
    if interp:
        # the neighbouring N-chunks' final latents (seeded stand-ins of the chunk shape)
        x_before = f32(synth.make_inputs(cfg, 1)["x_init"], dev)
        x_after = f32(synth.make_inputs(cfg, 2)["x_init"], dev)
    if iwin:
        # the window sees the reference only; the anchors are the neighbouring N-chunks'
        # last and first frames (seeded stand-ins), their noise drawn once per chunk
        h.boundary_kv_carry(None, grid_of(synth.Grid(0, 0, 0, 0)))
        z0 = f32(synth.make_inputs(cfg, 1)["x_init"][(F - 1) * hw:], dev)
        z1 = f32(synth.make_inputs(cfg, 2)["x_init"][:hw], dev)
        e = f32(synth.anchor_noise(cfg, 0), dev)
        g_win = grid_of(synth.Grid(-1, F + 2, gc.h, gc.w))
        xc = x[hw:(F + 1) * hw]

    table = ts[:-1] + [0.0]  # the schedule's timesteps and t = 0 of the context passes

    def step():
        h.modulation_table(table)
        if interp:
            h.boundary_kv_carry(x_before, g_chunk)
            h.interp_anchor_kv(x_after, g_chunk, cfg.chunk.frames)
        elif sr:
            h.boundary_kv_carry(bnd, g_prev)
        elif not reuse:
            h.ref_kv_precompute(ref, g_ref)
            h.boundary_kv_carry(bnd, g_prev)
        (xc if iwin else x).copy_(x0)
        if audio is not None:  # the chunk's audio K/V, once per chunk
            h.audio_kv_precompute(audio)
        for k in range(S):
            if iwin:
                fm_noise_to(x[:hw], z0, e[:hw], ts[k])
                fm_noise_to(x[(F + 1) * hw:], z1, e[hw:], ts[k])
            h.step(x, ts[k], ts[k + 1], g_win if iwin else g_chunk, cond=cond,
                   audio=AUDIO_HELD if audio is not None else None, carry_boundary=reuse and k == S - 1)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    h.timing_enable(1 << DIT_TIME_ATTN)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    achieved, af = _attn_fields(h)
    h.timing_enable(False)
    if not torch.isfinite(x).all():
        print("bench.py: non-finite output", file=sys.stderr)
        return 1
    extra = {"tokens_per_step": cfg.N * S}
    extra.update(af)
    extra.update(_breakdown(h, step))
    _with_ceilings(extra)
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    workload = WORKLOAD_BASE
    if reuse:
        workload = ("base low-res chunk, boundary carried by reuse: 7800 latent tokens, keys 1560 "
                    "reference + 1560 boundary + 7800 chunk, 50 audio tokens, 4 blocks, hidden 1536, "
                    "12 heads x 128, 8 Euler steps 1 -> 0; one bench step = modulation table + audio K/V + "
                    "8 denoising steps, the last one leaving its last frame's K/V as the next boundary")
    if interp:
        workload = ("interpolation chunk of the base low-res shape: 7800 latent tokens, keys "
                    "1560 reference + 1560 boundary + 1560 anchor + 7800 chunk, 50 audio tokens, "
                    "4 blocks, hidden 1536, 12 heads x 128, 8 Euler steps 1 -> 0; one bench step = "
                    "modulation table + boundary K/V + anchor K/V + audio K/V + 8 denoising steps")
    if iwin:
        workload = ("interpolation chunk of the base low-res shape, anchor-window reading: a window "
                    "of 7 frames (2 anchor + 5 chunk frames, 10920 tokens), keys 1560 reference + 10920 "
                    "window, 50 audio tokens, 4 blocks, hidden 1536, 12 heads x 128, 8 Euler steps 1 -> 0 "
                    "with both anchors re-noised to each step's time; one bench step = modulation table "
                    "+ audio K/V + 8 x (2 anchor re-noisings + denoising step); value counts the 7800 "
                    "chunk tokens")
    if sr:
        workload = ("super-resolution chunk: 5x60x104 = 31200 latent tokens conditioned on the "
                    "nearest-2x upsample of a 5x30x52 latent (64 + 64 input channels), keys 6240 "
                    "reference + 6240 boundary + 31200 chunk, no audio, 2 DiT blocks, hidden 1536, "
                    f"12 heads x 128, MLP 4x, {S} Euler step{'s' if S > 1 else ''} 1 -> 0; one bench "
                    f"step = modulation table + boundary K/V + {S} denoising step{'s' if S > 1 else ''}")
    metric = {"interp": METRIC_INTERP, "iwin": METRIC_IWIN, "reuse": METRIC_REUSE, "sr": METRIC_SR,
              "sr1": METRIC_SR1}.get(args.workload, METRIC)
    line = _line(metric, cfg.N * S / ((t1 - t0) / args.steps), args, ms_per_step, workload, extra, achieved,
                 _traffic(args.workload))
    h.close()
    if not args.no_cpu_baseline and args.workload == "base":
        line["cpu_baseline"] = cpu_baseline_block(cfg, P, inp)
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="large",
                    choices=["large", "base", "stream6", "tiny", "interp", "iwin", "reuse", "sr", "sr1", "wstream"],
                    help="large: one large-chunk denoising step (default, the headline); base: one base "
                         "chunk job; stream6: whole 6-chunk streaming sessions; see the module docstring")
    ap.add_argument("--elementwise-sweep", action="store_true",
                    help="only sweep the HBM-bound kernels over sizes (one JSON line per size)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run the 256 MiB calibration copy (for the traffic counters)")
    ap.add_argument("--gemm-compare", action="store_true",
                    help="only time the block-Linear GEMMs next to the vendor BLAS on the same shapes")
    ap.add_argument("--reduce-traffic", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="write the workload's attention traffic file from rocprofv3 counter CSVs")
    args = ap.parse_args()
    if args.copy_probe:
        copy_probe()
        return 0
    if args.elementwise_sweep:
        return elementwise_sweep()
    if args.gemm_compare:
        return gemm_compare()
    if args.reduce_traffic:
        if args.workload not in TRAFFIC_FILES:
            raise SystemExit(f"bench.py: no traffic file for workload {args.workload}")
        d = reduce_traffic(*args.reduce_traffic, largest_grid=TRAFFIC_LARGEST_GRID[args.workload],
                           skip_first=TRAFFIC_SKIP_FIRST.get(args.workload, False))
        with open(TRAFFIC_FILES[args.workload], "w") as fh:
            json.dump(d, fh, indent=1)
            fh.write("\n")
        print(json.dumps(d))
        return 0
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (--gpus {args.gpus} requested); "
              "the multi-GPU sharding is a design, not a measured path", file=sys.stderr)
        return 2
    if args.workload in ("large", "wstream"):
        return large_main(args)
    if args.workload == "stream6":
        return stream6_main(args)
    if args.workload == "tiny":
        return tiny_main(args)
    return chunk_main(args)


if __name__ == "__main__":
    sys.exit(main())

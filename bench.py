"""Benchmark of the chunked streaming DiT step on one MI355X.

One bench step = one whole base low-res chunk job through the C ABI: the adaLN
modulation table of the job's timesteps (dit_modulation_table), the reference
K/V pass (ref_kv_precompute), the boundary K/V pass from the previous chunk's last
latent frame (boundary_kv_carry), the chunk's audio K/V (audio_kv_precompute, once per
chunk: the audio is the same at every step), then the 8 Euler denoising steps
(dit_chunk_step: patch embed, 4 DiT blocks of self-attention over
[reference | boundary | chunk] keys, audio cross-attention and adaLN MLP, final
layer + Euler update).  Inputs are seeded synthetic tensors already resident in HBM.

value = latent tokens x denoising steps / second (7800 x 8 per bench step; the
context passes are included in the time).
roofline = the self-attention kernel (the dominant kernel): algorithmic flop
4 * N_q * N_kv * D per launch over its HIP-event-timed duration, against the
bf16 dense MFMA peak.
cpu_baseline = the f64 oracle timed on the host on a bounded sample (one DiT block of
one denoising step at the full chunk shape, scaled to the 4-block step).

--workload interp times an interpolation chunk of the same shape instead (the
boundary from one neighbouring chunk's last frame, the anchor from the other's first
frame, then 8 steps whose keys are [reference | boundary | anchor | chunk]); the
reference pass runs once, outside the timed region, as it does once per request.
--workload reuse times N-chunk jobs whose boundary is carried by reuse: 8 steps, the
last of which leaves its last frame's K/V as the next job's boundary (no boundary
pass); the reference pass again runs once, outside the timed region.
--workload sr / sr1 time super-resolution chunk jobs (5x60x104 = 31200 latent tokens
conditioned on the nearest-2x upsample of a 5x30x52 latent, keys 6240 reference + 6240
boundary + 31200 chunk, 2 blocks, no audio): the boundary pass and 4 Euler steps (sr) or
a single step 1 -> 0 (sr1); the reference pass runs once, outside the timed region.
--workload large times one denoising step of the large base chunk (21x30x52 = 32760
tokens, keys 1560 reference + 1560 boundary + 32760 chunk, 200 audio tokens, 30 blocks,
hidden 3072, 24 heads x 128) with resident weights; --workload stream times the same
step with the block weights streamed from pinned host memory through a 2-slot device
ring (dit_weight_stream) and also reports, from the same process, the resident step,
the first (cold) streamed step after the switch, and the difference.  Their weights are
drawn on the GPU (seeded N(0, 1/fan_in), gammas 1 + 0.1 N(0, 1)) to keep the 6.7 G
parameters' set-up short.
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
METRIC_INTERP = ("DiT interpolation-chunk latent tokens/sec and attention TFLOP/s "
                 "(% bf16 MFMA peak), 1 GPU")
METRIC_SR = ("DiT super-resolution chunk latent tokens/sec and attention TFLOP/s "
             "(% bf16 MFMA peak), 1 GPU")
METRIC_SR1 = ("DiT single-step super-resolution chunk latent tokens/sec and attention TFLOP/s "
              "(% bf16 MFMA peak), 1 GPU")
METRIC_LARGE = ("DiT large-chunk denoising step latent tokens/sec and attention TFLOP/s "
                "(% bf16 MFMA peak), 1 GPU")
METRIC_STREAM = ("DiT large-chunk denoising step latent tokens/sec with block weights streamed "
                 "from pinned host memory, 1 GPU")
METRIC_REUSE = ("DiT chunk-step latent tokens/sec, boundary carried by reuse, and attention "
                "TFLOP/s (% bf16 MFMA peak), 1 GPU")
PEAK_BF16_TFLOPS = 2500.0
ATTN_SRC = os.path.join(ROOT, "chunked_streaming_dit_amd", "csrc", "attention.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_base_chunk_traffic.json")


def _src_hash(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def _traffic():
    """HBM bytes per attention launch from the committed rocprofv3 counter summary, or
    None if it is missing or was taken on a different attention source."""
    try:
        d = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if d.get("attention_src_sha256_16") != _src_hash(ATTN_SRC):
        return None
    return d.get("hbm_bytes_per_launch")


COPY_PROBE_BYTES = 256 << 20


def copy_probe(reps: int = 3) -> None:
    """A plain device copy of COPY_PROBE_BYTES, the known-size kernel that calibrates
    the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    dev = torch.device("cuda", 0)
    a = torch.empty(COPY_PROBE_BYTES // 4, device=dev)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()


def _counter_means(path: str, counter: str, match) -> tuple:
    """(mean counter value, dispatches) over the dispatches of a rocprofv3 counter CSV
    whose kernel name satisfies match."""
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
            if r["Counter_Name"] == counter and match(r["Kernel_Name"])]
    if not vals:
        raise SystemExit(f"bench.py: no {counter} rows matched in {path}")
    return sum(vals) / len(vals), len(vals)


def _is_self_attention(name: str) -> bool:
    """attn_kernel<T, DH, KIND> with KIND 0 (self-attention; 1 is the audio cross-attention),
    demangled or mangled."""
    import re
    return re.search(r"attn_kernel(<[^<>]*,\s*0>|I\w*Li0EE)", name) is not None


def reduce_traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv) -> dict:
    """HBM bytes per self-attention launch from four rocprofv3 --pmc runs (FETCH_SIZE and
    WRITE_SIZE, in KiB per dispatch, over the bench and over copy_probe), each counter
    scaled so that the copy reads COPY_PROBE_BYTES and writes COPY_PROBE_BYTES."""
    kib = COPY_PROBE_BYTES / 1024
    cf, _ = _counter_means(copy_fetch_csv, "FETCH_SIZE", lambda n: "copy" in n.lower())
    cw, _ = _counter_means(copy_write_csv, "WRITE_SIZE", lambda n: "copy" in n.lower())
    f, nf = _counter_means(fetch_csv, "FETCH_SIZE", _is_self_attention)
    w, nw = _counter_means(write_csv, "WRITE_SIZE", _is_self_attention)
    sf, sw = kib / cf, kib / cw
    return {
        "attention_src_sha256_16": _src_hash(ATTN_SRC),
        "hbm_bytes_per_launch": (f * sf + w * sw) * 1024,
        "fetch_bytes_per_launch": f * sf * 1024,
        "write_bytes_per_launch": w * sw * 1024,
        "fetch_scale": sf,
        "write_scale": sw,
        "dispatches": [nf, nw],
    }


def cpu_baseline(cfg, P, inp, budget_s: float = 12.0):
    """Time the oracle on one DiT block of one denoising step at the full chunk shape
    (repeated up to L times while under the budget) and scale to the L-block step."""
    import dataclasses

    import numpy as np
    from threadpoolctl import threadpool_info

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
    t_step = t_block * cfg.L
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {
        "value": cfg.N / t_step,
        "unit": "latent tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{len(times)} x one DiT block of one denoising step at the full chunk shape "
                   f"({cfg.N} tokens, {cfg.N_ref}+{cfg.N_bnd}+{cfg.N} keys, audio {cfg.M}), "
                   f"median {t_block:.2f} s x {cfg.L} blocks; context passes excluded"),
    }


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


def large_main(args) -> int:
    """--workload large / stream: one denoising step of the large base chunk."""
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
    stream = args.workload == "stream"

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
    extra = {}
    host = None
    if stream:
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
        extra = {"resident_ms_per_step": resident_ms, "cold_first_step_ms": cold_ms,
                 "block_weight_bytes": h.cfg.block_weight_bytes(), "ring_slots": 2}
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    h.timing_enable(True)
    ms = timed(args.steps)
    n_attn, attn_ms, attn_flop = h.timing_read()
    h.timing_enable(False)
    if stream:
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
    if not torch.isfinite(x).all():
        print("bench.py: non-finite output", file=sys.stderr)
        return 1
    achieved = attn_flop / (attn_ms * 1e-3) / 1e12
    workload = ("large base chunk: 21x30x52 = 32760 latent tokens, keys 1560 reference + 1560 "
                "boundary + 32760 chunk, 200 audio tokens of dim 768, 30 DiT blocks, hidden 3072, "
                "24 heads x 128, MLP 4x, one Euler step 1 -> 0.875; one bench step = audio K/V + "
                "one denoising step (the context passes run before)")
    if stream:
        workload += ("; block weights (387.0 MB each) streamed from pinned host memory "
                     "through a 2-slot device ring")
    line = {
        "metric": METRIC_STREAM if stream else METRIC_LARGE,
        "value": cfg.N / (ms * 1e-3),
        "unit": "latent tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) latents/audio, random-init weights drawn on the GPU)",
        "config": dict({
            "workload": workload,
            "tokens_per_step": cfg.N,
            "attention_tflops": achieved,
            "attention_frac_bf16_peak": achieved / PEAK_BF16_TFLOPS,
            "attention_launches": n_attn,
            "attention_avg_launch_ms": attn_ms / max(n_attn, 1),
        }, **extra),
        "roofline": {
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": None,
        },
    }
    print(json.dumps(line), flush=True)
    h.close()
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", choices=["base", "interp", "reuse", "sr", "sr1", "large", "stream"], default="base",
                    help="base: one N-chunk job (default); interp: one interpolation-chunk job; "
                         "reuse: one N-chunk job with the boundary carried by reuse")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run the 256 MiB calibration copy (for the traffic counters)")
    ap.add_argument("--reduce-traffic", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="write the attention traffic file from rocprofv3 counter CSVs")
    args = ap.parse_args()
    if args.copy_probe:
        copy_probe()
        return 0
    if args.reduce_traffic:
        d = reduce_traffic(*args.reduce_traffic)
        with open(TRAFFIC_FILE, "w") as fh:
            json.dump(d, fh, indent=1)
            fh.write("\n")
        print(json.dumps(d))
        return 0
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (--gpus {args.gpus} requested); "
              "the multi-GPU sharding is a design, not a measured path", file=sys.stderr)
        return 2

    if args.workload in ("large", "stream"):
        return large_main(args)

    import torch

    import synth
    from chunked_streaming_dit_amd import AUDIO_HELD, DitChunk
    from chunked_streaming_dit_amd.workload import chunk_config, f32, grid_of, upload_weights

    dev = torch.device("cuda", 0)
    sr = args.workload in ("sr", "sr1")
    cfg = synth.SUPER_RES if sr else synth.BASE_CHUNK
    P = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg, 0)
    W = upload_weights(P, cfg.dtype, dev)
    h = DitChunk(chunk_config(cfg), W, dev)
    ref = f32(inp["ref"], dev)
    bnd = f32(inp["bnd"], dev)
    x0 = f32(inp["x_init"], dev)
    audio = f32(inp["audio"], dev) if cfg.M else None
    cond = f32(inp["cond_lr"], dev) if sr else None
    x = torch.empty_like(x0)
    S = 1 if args.workload == "sr1" else cfg.steps
    ts = [cfg.t_start + (cfg.t_end - cfg.t_start) * k / S for k in range(S + 1)]
    g_chunk = grid_of(cfg.chunk)
    g_ref = grid_of(cfg.ref)
    g_prev = grid_of(synth.Grid(0, 1, cfg.bnd.h, cfg.bnd.w))
    interp = args.workload == "interp"
    reuse = args.workload == "reuse"
    if sr:
        h.ref_kv_precompute(ref, g_ref)
    if reuse:
        h.ref_kv_precompute(ref, g_ref)
        h.boundary_kv_carry(bnd, g_prev)  # the first job's boundary; later ones are carried
    if interp:
        # the neighbouring N-chunks' final latents (seeded stand-ins of the chunk shape)
        x_before = f32(synth.make_inputs(cfg, 1)["x_init"], dev)
        x_after = f32(synth.make_inputs(cfg, 2)["x_init"], dev)
        h.ref_kv_precompute(ref, g_ref)

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
        x.copy_(x0)
        if audio is not None:  # the chunk's audio K/V, once per chunk
            h.audio_kv_precompute(audio)
        for k in range(S):
            h.step(x, ts[k], ts[k + 1], g_chunk, cond=cond, audio=AUDIO_HELD if audio is not None else None,
                   carry_boundary=reuse and k == S - 1)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    h.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    n_attn, attn_ms, attn_flop = h.timing_read()
    h.timing_enable(False)
    if not torch.isfinite(x).all():
        print("bench.py: non-finite output", file=sys.stderr)
        return 1

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = cfg.N * S / ((t1 - t0) / args.steps)
    achieved = attn_flop / (attn_ms * 1e-3) / 1e12
    traffic = _traffic()
    workload = ("base low-res chunk: 5x30x52 = 7800 latent tokens, 1560 reference + 1560 "
                "boundary tokens, 50 audio tokens of dim 768, 4 DiT blocks, hidden 1536, "
                "12 heads x 128, MLP 4x, 8 Euler steps 1 -> 0; one bench step = modulation "
                "table + reference K/V + boundary K/V + audio K/V + 8 denoising steps")
    if reuse:
        workload = ("base low-res chunk, boundary carried by reuse: 7800 latent tokens, keys 1560 "
                    "reference + 1560 boundary + 7800 chunk, 50 audio tokens, 4 blocks, hidden 1536, "
                    "12 heads x 128, 8 Euler steps 1 -> 0; one bench step = modulation table + audio K/V + 8 denoising steps, the "
                    "last one leaving its last frame's K/V as the next boundary")
    if interp:
        workload = ("interpolation chunk of the base low-res shape: 7800 latent tokens, keys "
                    "1560 reference + 1560 boundary + 1560 anchor + 7800 chunk, 50 audio tokens, "
                    "4 blocks, hidden 1536, 12 heads x 128, 8 Euler steps 1 -> 0; one bench step = "
                    "modulation table + boundary K/V + anchor K/V + audio K/V + 8 denoising steps")
    if sr:
        workload = ("super-resolution chunk: 5x60x104 = 31200 latent tokens conditioned on the "
                    "nearest-2x upsample of a 5x30x52 latent (64 + 64 input channels), keys 6240 "
                    "reference + 6240 boundary + 31200 chunk, no audio, 2 DiT blocks, hidden 1536, "
                    f"12 heads x 128, MLP 4x, {S} Euler step{'s' if S > 1 else ''} 1 -> 0; one bench "
                    f"step = modulation table + boundary K/V + {S} denoising step{'s' if S > 1 else ''}")
    metric = METRIC
    if interp:
        metric = METRIC_INTERP
    elif reuse:
        metric = METRIC_REUSE
    elif sr:
        metric = METRIC_SR1 if S == 1 else METRIC_SR
    line = {
        "metric": metric,
        "value": value,
        "unit": "latent tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) latents/audio, N(0,1/fan_in) random-init weights)",
        "config": {
            "workload": workload,
            "tokens_per_step": cfg.N * S,
            "attention_tflops": achieved,
            "attention_frac_bf16_peak": achieved / PEAK_BF16_TFLOPS,
            "attention_launches": n_attn,
            "attention_avg_launch_ms": attn_ms / max(n_attn, 1),
        },
        "roofline": {
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": traffic,
        },
    }
    if not args.no_cpu_baseline and args.workload == "base":
        line["cpu_baseline"] = cpu_baseline(cfg, P, inp)
    print(json.dumps(line), flush=True)
    h.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Write the oracle's expected values for the full-size workloads into tests/golden/.

Every value written here comes from the float64 oracle (``oracle/``) on the seeded
synthetic inputs (``synth/``); nothing is read from the GPU path.  The GPU tests then
run the same workloads through the C ABI and compare.

What is stored (float32, ``<workload>.npz``), on a fixed set of sampled token rows (the
first 64 rows, the last 64 rows, i.e. the ragged tail of the last 256-query tile, and
256 rows drawn with the seed below):
  base    base low-res chunk, 8 Euler steps 1 -> 0: v of every step and dx = x_8 - x_0
  stream  6 chunks of the base shape, the boundary of chunk c the last frame of chunk
          c-1's final latent: per chunk the first step's v, the last step's v and dx
  sr      super-resolution chunk, 4 Euler steps 1 -> 0: v of every step and dx
  large   large base chunk, one Euler step 1 -> 0.875: v
The chunk's schedule, sizes and the reading of each workload are the oracle's (the
pages: HeyGen, "Avatar inference at scale", sections "The underlying model
architecture" and "The streaming framework and pipeline loop").

Usage:  python tests/golden/make_goldens.py {base,stream,sr,large} [--threads N] [--head-threads N]
The large chunk takes about an hour of CPU time on 8 cores with --head-threads 8 (30
blocks of 32760 tokens in float64, about 40 GB of memory); run with MALLOC_MMAP_MAX_=0
MALLOC_TRIM_THRESHOLD_=<large> where first-touch page faults are expensive.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import synth  # noqa: E402

WORKLOADS = {"base": 2, "stream": 3, "sr": 4, "large": 5}
ROW_SEED = 9001
N_RANDOM_ROWS = 256


def sample_rows(cfg) -> np.ndarray:
    """The sampled token rows of a workload (sorted, unique)."""
    n = cfg.N
    r = np.random.default_rng(np.random.SeedSequence([cfg.cid, ROW_SEED]))
    pick = r.choice(n, N_RANDOM_ROWS, replace=False)
    return np.unique(np.concatenate([np.arange(64), np.arange(n - 64, n), pick])).astype(np.int64)


class _Progress:
    """Weight mapping that reports when a pass reaches a block (first access of the
    block's QKV weight): progress lines for the hours-long runs."""

    def __init__(self, P, t0):
        self.P, self.t0 = P, t0

    def __getitem__(self, name):
        if name.endswith(".qkv.w"):
            print(f"  {time.time() - self.t0:8.0f} s  {name[:name.index('.')]}", flush=True)
        return self.P[name]

    def __contains__(self, name):
        return name in self.P


def _f32(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float32)


def run(name: str) -> dict:
    cfg = synth.CONFIGS[WORKLOADS[name]]
    t0 = time.time()
    P = synth.make_weights(cfg, threads=8, compact=cfg.dtype == "bf16")
    print(f"{name}: weights in {time.time() - t0:.0f} s", flush=True)
    Pp = _Progress(P, t0)
    rows = sample_rows(cfg)
    out = {"rows": rows}
    if name == "stream":
        chunks = [synth.make_inputs(cfg, c) for c in range(cfg.n_chunks)]
        finals, vels = O.stream(Pp, cfg, chunks, chunks[0]["ref"], record=True)
        out["v_first"] = np.stack([_f32(v[0][rows]) for v in vels])
        out["v_last"] = np.stack([_f32(v[-1][rows]) for v in vels])
        out["dx"] = np.stack([_f32((x - c["x_init"])[rows]) for x, c in zip(finals, chunks)])
    else:
        inp = synth.make_inputs(cfg, 0)
        x, vs, _, _ = O.standalone(Pp, cfg, inp)
        out["v"] = np.stack([_f32(v[rows]) for v in vs])
        out["dx"] = _f32((x - inp["x_init"])[rows])
    meta = {
        "workload": cfg.name, "cid": cfg.cid, "N": cfg.N, "steps": cfg.steps,
        "schedule": O.schedule(cfg.steps, cfg.t_start, cfg.t_end).tolist(),
        "rows": f"first 64, last 64, {N_RANDOM_ROWS} drawn with SeedSequence([cid, {ROW_SEED}])",
        "oracle_sha256_16": hashlib.sha256(open(os.path.join(ROOT, "oracle", "dit.py"), "rb").read()).hexdigest()[:16],
        "script": "tests/golden/make_goldens.py",
        "seconds": round(time.time() - t0, 1),
    }
    out["meta"] = np.array(json.dumps(meta))
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("workload", choices=sorted(WORKLOADS))
    ap.add_argument("--threads", type=int, default=0, help="BLAS threads (0: the library default)")
    ap.add_argument("--head-threads", type=int, default=1,
                    help="attention heads computed concurrently by the oracle (same arithmetic)")
    ap.add_argument("--query-group", type=int, default=0,
                    help="query rows per score matrix in the oracle's attention (0: its default)")
    args = ap.parse_args()
    if args.threads:
        from threadpoolctl import threadpool_limits
        threadpool_limits(args.threads)
    import oracle.dit
    oracle.dit.HEAD_THREADS = args.head_threads
    if args.query_group:
        oracle.dit.QUERY_GROUP = args.query_group
    out = run(args.workload)
    path = os.path.join(HERE, f"{args.workload}.npz")
    np.savez_compressed(path + ".tmp.npz", **out)
    os.replace(path + ".tmp.npz", path)
    print(f"wrote {path}: {json.loads(str(out['meta']))}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

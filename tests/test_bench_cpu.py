"""Host-side behaviour of bench.py that needs no GPU: it measures one GPU only and says so
for any other count, and its metric is the one the benchmark is reported under."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_gemm_compare_shapes_are_the_block_linears():
    sys.path.insert(0, ROOT)
    import bench
    names = {s[0] for s in bench.GEMM_COMPARE_SHAPES}
    assert len(names) == len(bench.GEMM_COMPARE_SHAPES)
    for name, M, N, K, epi in bench.GEMM_COMPARE_SHAPES:
        assert epi in ("bias", "gelu", "resid")
        assert K % 64 == 0 and N % 256 == 0 and M > 0
    # the large chunk's QKV, MLP in / out and out-projection at hidden 3072, MLP 4x
    large = {(M, N, K) for _, M, N, K, _ in bench.GEMM_COMPARE_SHAPES if M == 32760}
    assert large == {(32760, 9216, 3072), (32760, 12288, 3072), (32760, 3072, 12288), (32760, 3072, 3072)}


def test_traffic_files_are_present_and_complete():
    """Every workload with an attention traffic file has it committed, with the per-launch
    bytes and the source hash it was taken on, and a rule for which launches it averages."""
    import json
    sys.path.insert(0, ROOT)
    import bench
    assert set(bench.TRAFFIC_FILES) == set(bench.TRAFFIC_LARGEST_GRID)
    for w, path in bench.TRAFFIC_FILES.items():
        d = json.load(open(path))
        assert d["hbm_bytes_per_launch"] > 0
        assert abs(d["hbm_bytes_per_launch"] - d["fetch_bytes_per_launch"] - d["write_bytes_per_launch"]) < 1.0
        assert len(d["attention_src_sha256_16"]) == 16
        assert d["largest_grid_only"] == bench.TRAFFIC_LARGEST_GRID[w]
        assert d.get("first_dispatch_skipped", False) == bench.TRAFFIC_SKIP_FIRST.get(w, False)

"""The stored oracle values of the full-size workloads (tests/golden/*.npz): their rows,
shapes and metadata match what tests/golden/make_goldens.py writes for the workload
(CPU only; the values themselves come from the oracle and are compared with the GPU by
tests/test_gpu_full_size.py)."""
import importlib.util
import json
import os

import numpy as np
import pytest

import oracle as O
import synth

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")


def _script():
    spec = importlib.util.spec_from_file_location("make_goldens", os.path.join(GOLDEN, "make_goldens.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


@pytest.mark.parametrize("name", ["base", "stream", "sr", "large"])
def test_golden_file_matches_its_workload(name):
    path = os.path.join(GOLDEN, name + ".npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated yet")
    mg = _script()
    cfg = synth.CONFIGS[mg.WORKLOADS[name]]
    d = np.load(path)
    meta = json.loads(str(d["meta"]))
    rows = d["rows"]
    assert np.array_equal(rows, mg.sample_rows(cfg))
    assert rows[0] == 0 and rows[-1] == cfg.N - 1 and np.all(np.diff(rows) > 0)
    assert meta["cid"] == cfg.cid and meta["N"] == cfg.N and meta["steps"] == cfg.steps
    assert np.allclose(meta["schedule"], O.schedule(cfg.steps, cfg.t_start, cfg.t_end), rtol=0, atol=0)
    R = len(rows)
    if name == "stream":
        for k in ("v_first", "v_last", "dx"):
            assert d[k].shape == (cfg.n_chunks, R, cfg.C_p), k
    else:
        assert d["v"].shape == (cfg.steps, R, cfg.C_p)
        assert d["dx"].shape == (R, cfg.C_p)
    for k in d.files:
        if k not in ("meta", "rows"):
            assert d[k].dtype == np.float32 and np.isfinite(d[k]).all(), k
    if name != "stream":
        # the Euler update: dx is the schedule's dt-weighted sum of the stored velocities
        ts = meta["schedule"]
        dx = sum((ts[k + 1] - ts[k]) * d["v"][k].astype(np.float64) for k in range(cfg.steps))
        assert np.abs(dx - d["dx"]).max() <= 1e-5 * np.abs(d["dx"]).max()

"""Host-side logic of bench.py (no GPU): the algorithmic FLOPs and bytes its
rooflines divide by, the lookup of committed HBM counter readings, which
workload may be timed as a secondary line, and the one-GPU exit.

The FLOP and byte figures are pinned to reference values worked out by hand
from the workload shapes (not to bench.py's own formulas):
  Base-1, T = 4,096: 6.55e12 FLOPs, 96.9 GB (the 512 experts' weights once,
  x in, fp32 out, the latent projections and the fp32 router weights);
  Base-1, T = 32,768: 5.24e13 FLOPs, 98.0 GB; Base-2, T = 16,384: 3.61e13
  FLOPs, 104.7 GB; the Base-1 gate/up GEMM at T = 4,096: 4.12e12 FLOPs.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from moe_synth import CONFIGS  # noqa: E402


@pytest.mark.parametrize("name, flops, gbytes", [
    ("base1_small_batch", 6.55e12, 96.9),
    ("base1_compute", 5.24e13, 98.0),
    ("base2", 3.61e13, 104.7),
])
def test_layer_flops_and_bytes(name, flops, gbytes):
    cfg = CONFIGS[name]
    assert cfg.flops() == pytest.approx(flops, rel=2e-3)
    assert bench.layer_bytes(cfg, cfg.E) / 1e9 == pytest.approx(gbytes, rel=1e-3)


def test_gate_up_work_counts_each_latent_row_once():
    cfg = CONFIGS["base1_small_batch"]
    counts = np.full(cfg.E, cfg.T * cfg.k // cfg.E)
    flops, nbytes, touched = bench.dominant_work(cfg, counts)
    assert touched == 512
    assert flops == pytest.approx(4.12e12, rel=2e-3)
    # gate and up weights of 512 experts (64.42 GB), z once (25.2 MB: not the
    # 201 MB of its k-fold gather), H out (671 MB), bf16
    w = 512 * 2 * 10240 * 3072 * 2
    z = 4096 * 3072 * 2
    h = 4096 * 8 * 10240 * 2
    assert nbytes == w + z + h
    # FP8: one byte per value; experts without rows are not counted
    counts[::2] = 0
    _, nb8, touched8 = bench.dominant_work(cfg, counts, esize=1)
    assert touched8 == 256 and nb8 == 256 * 2 * 10240 * 3072 + 4096 * 3072 + 4096 * 8 * 10240


def test_backward_flops_twice_the_forward_plus_recompute():
    for name in ("base1_ep8", "base2_ep8"):
        cfg = CONFIGS[name]
        model, executed = bench.backward_flops(cfg)
        assert model == pytest.approx(2 * cfg.flops())
        T, d, L, k, F, Fs = cfg.T, cfg.d, cfg.L, cfg.k, cfg.F, cfg.Fs
        assert executed - model == pytest.approx(2 * T * d * L + 4 * T * k * L * F + 4 * T * d * Fs)


def test_stored_traffic_only_for_the_current_sources(monkeypatch):
    path = os.path.join(ROOT, "profiles", f"{bench.DOMINANT}_base1_compute_traffic.json")
    if os.path.exists(path):
        import json
        with open(path) as f:
            rec = json.load(f)
        if rec["sources_sha256_16"] == bench.sources_digest():
            assert bench.stored_traffic("base1_compute") == rec["traffic_bytes_per_launch"]
    monkeypatch.setattr(bench, "sources_digest", lambda: "0" * 16)
    assert bench.stored_traffic("base1_compute") is None
    assert bench.stored_traffic("no_such_workload") is None


def test_secondary_workload_shares_the_weights():
    small, big = CONFIGS["base1_small_batch"], CONFIGS["base1_compute"]
    assert bench.same_weights(small, big)
    assert not bench.same_weights(small, CONFIGS["base1_imbalanced"])   # router bias differs
    assert not bench.same_weights(small, CONFIGS["base1_f5120"])        # expert width differs
    assert not bench.same_weights(small, CONFIGS["base2"])


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""

"""Host-side checks of bench.py's contract (no GPU)."""

import json
import os
import subprocess
import sys

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_counts():
    # 60-layer gate projection, 16 tokens, rank 256 (bf16).
    O, I, R, M = 21504, 5376, 256, 16
    assert bench.call_bytes(M, O, I, R) == 2 * (O * I + R * (O + I) + O + M * (I + O))
    assert bench.call_flops(M, O, I, R) == 2 * M * (O * I + R * (O + I))
    # Per-layer W0 bytes of the 60-layer stack: 913,833,984.
    from rank_factored_linear_amd import inputs
    assert sum(2 * o * i for o, i in inputs.SHAPES_60.values()) == 913_833_984
    assert sum(2 * o * i for o, i in inputs.SHAPES_26.values()) == 53_673_984


def test_traffic_record_requires_current_kernel_source(tmp_path, monkeypatch):
    assert len(bench.kernel_source_digest()) == 16


def test_reconstruct_and_error_bytes_per_stack():
    # The 60-layer stack's 420 weights: rebuild in fp32 from bf16 bundles (rank 256 and 0), then read the
    # rebuilt and the original fp32 matrices once for the error.
    from rank_factored_linear_amd import inputs
    shapes = inputs.SHAPES_60.values()
    assert 60 * sum(bench.reconstruct_bytes(o, i, 256) for o, i in shapes) == 168_265_052_160
    assert 60 * sum(bench.reconstruct_bytes(o, i, 0) for o, i in shapes) == 164_498_042_880
    assert 60 * sum(bench.frobenius_bytes(o, i) for o, i in shapes) == 219_320_156_160


def test_spread_of_trials():
    assert bench.spread([3.0, 1.0, 2.0]) == {"median_ms": 2.0, "min_ms": 1.0, "max_ms": 3.0, "trials": 3}
    assert bench.spread([4.0, 1.0, 2.0, 3.0])["median_ms"] == 2.5


def test_fused_error_bytes():
    # The error without the rebuilt weight reads the bf16 bundle and the fp32 original once: 6 bytes per element
    # plus the factors, against 14 for rebuilding in fp32 and then comparing.
    O, I, R = 21504, 5376, 256
    assert bench.fused_error_bytes(O, I, R) == 2 * (O * I + R * (O + I) + O) + 4 * O * I
    ratio = (bench.reconstruct_bytes(O, I, R) + bench.frobenius_bytes(O, I)) / bench.fused_error_bytes(O, I, R)
    assert 2.2 < ratio < 2.35


def test_dense_call_bytes():
    # A materialised weight streams O x I alone: the bundle's extra bytes are U, V and s.
    M, O, I, R = 16, 8192, 5376, 256
    assert bench.dense_call_bytes(M, O, I) == 2 * (O * I + M * (I + O))
    assert bench.call_bytes(M, O, I, R) - bench.dense_call_bytes(M, O, I) == 2 * (R * (O + I) + O)
    assert bench.call_flops(M, O, I, 0) == 2 * M * O * I


def test_decompose_workloads_are_declared():
    for name in ("decompose26", "decompose60"):
        wl = bench.WORKLOADS[name]
        assert wl["rank"] > 0 and 1 <= wl["bands"] <= wl["layers"]


def test_reconstruct_kernel_names_follow_the_k_tiles_of_32():
    assert bench.reconstruct_kernel_names(256) == ("rp::reconstruct_persistent_kernel<float, false, 8>",
                                                  "rp::reconstruct_persistent_kernel<float, true, 8>")
    assert bench.reconstruct_kernel_names(128) == ("rp::reconstruct_persistent_kernel<float, false, 4>",
                                                  "rp::reconstruct_persistent_kernel<float, true, 4>")
    assert bench.reconstruct_kernel_names(64) == ("rp::reconstruct_persistent_kernel<float, false, 2>",
                                                 "rp::reconstruct_persistent_kernel<float, true, 4>")
    assert bench.reconstruct_kernel_names(0) == ("reconstruct_rank0_kernel", "rerr_rank0_kernel")
    assert bench.reconstruct_kernel_names(264) == ("mm::reconstruct_mfma_kernel", "rerr_t128_kernel")
    assert bench.reconstruct_kernel_names(12) == ("reconstruct_lowrank_kernel", "rerr_t64_kernel")


def test_committed_rebuild_traffic_names_the_benched_kernel():
    # The rebuild's HBM record is looked up by kernel name: it must name the kernel bench.py reports.
    rec = json.load(open(os.path.join(ROOT, "profiles", "hbm_traffic.json"))).get("reconstruct60_R256_G6")
    assert rec is not None and rec["kernel"] == bench.reconstruct_kernel_names(256)[0]

"""The measurement script's host logic (no GPU): the one-GPU contract, the
roofline choice, and its byte model against the library's panel layout and the
traffic counters recorded in profiles/."""

import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

KERNELS = ["fwd_prep", "fwd_scan", "fwd_out", "bwd_scan", "bwd_intra"]
CHUNK_HEADS = 16384 * 64 / 64      # 1doc and 4doc: T * H / 64


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _panel_constants():
    """Element offsets of the operand panel layout, read from the library's header."""
    src = open(os.path.join(ROOT, "kda_chunked_amd", "csrc", "kda_internal.h")).read()
    body = src[src.index("namespace fwd_panel {"):src.index("}  // namespace fwd_panel")]
    env = {}
    for name, expr in re.findall(r"constexpr int (\w+) = ([^;]+);", body):
        env[name] = eval(expr, {}, dict(env))
    return env


def test_byte_model_matches_panel_layout():
    p = _panel_constants()
    assert bench._PANEL_B == 2 * p["ELEMS"]
    assert bench._FWD_CHAIN_B == 2 * p["CHAIN"]


@pytest.mark.parametrize("raw", [False, True])
def test_every_kernel_is_hbm_bound(raw):
    # the path's intensity is far below the MI355X ridge (2.5 PFLOP/s / 8 TB/s)
    for k in KERNELS:
        r = bench.kernel_roofline(k, 1.0, CHUNK_HEADS, raw)
        assert r["bound"] == "hbm", k
        flop = 2.0 * bench.MAC_PER_CHUNK_HEAD[k]
        assert flop / bench.algo_bytes_per_chunk_head(k, raw) < 312 / 4
        assert r["achieved"] == pytest.approx(r["algorithmic_bytes_per_launch"] / 1e-3 / 1e9, rel=1e-3)
        assert r["frac"] == pytest.approx(r["achieved"] / bench.PEAK_HBM_GBS, abs=1e-4)


@pytest.mark.parametrize("workload,raw", [("1doc", False), ("4doc", True)])
def test_recorded_traffic_is_close_to_the_byte_model(workload, raw):
    fig = bench.profile_figures(workload, "bwd_intra", bench.fingerprint())
    if fig is None:
        pytest.skip("profiles/ were taken on other kernel sources")
    model = bench.algo_bytes_per_chunk_head("bwd_intra", raw) * CHUNK_HEADS
    # measured HBM traffic within 15 % above the model and never far below it
    assert 0.97 * model <= fig["traffic_bytes"] <= 1.15 * model

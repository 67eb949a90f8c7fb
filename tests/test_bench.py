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


def test_method_work_and_compulsory_bytes():
    """The method's own figures per token-head: 4.51 M + 11.17 M multiply-adds
    per 64-token chunk-head (141 k + 349 k FLOP per token-head), and every
    input read and output written once (g form 1538 + 2820 B, raw 1282 +
    2308 B). 1doc fwd+bwd is then 5.14e11 FLOP and 4.57 GB."""
    f = bench.FLOP_PER_TOKEN_HEAD
    assert f["fwd"] == pytest.approx(141e3, rel=1e-3)
    assert f["bwd"] == pytest.approx(349e3, rel=1e-3)
    fwd_mac = 258048 + 266240 + 64 ** 3 / 6 + 3 * 266240 + 2 * 64 * 128 * 128 + 64 * 128 * 128
    assert fwd_mac == pytest.approx(4.51e6, rel=1e-3)
    cb = bench.COMPULSORY_BYTES_PER_TOKEN_HEAD
    assert (cb[False]["fwd"], cb[False]["bwd"]) == (1538, 2820)
    assert (cb[True]["fwd"], cb[True]["bwd"]) == (1282, 2308)
    e = bench.end_to_end(1.0, 16384, 64, False)
    assert e["algorithmic_flop"] == pytest.approx(5.14e11, rel=2e-3)
    assert e["compulsory_bytes"] == pytest.approx(4.57e9, rel=2e-3)
    assert e["mfma_frac"] == pytest.approx(e["algorithmic_flop"] / 1e-3 / 2.5e15, rel=1e-3)
    assert e["hbm_frac"] == pytest.approx(e["compulsory_bytes"] / 1e-3 / 8e12, rel=1e-3)
    # the per-chunk backward's own I/O: q, k, g, beta, dO in; dq, dk, dbeta, dg out
    assert bench.BWD_INTRA_COMPULSORY_BYTES_PER_TOKEN_HEAD[False] * 16384 * 64 == \
        pytest.approx(2.42e9, rel=2e-3)


@pytest.mark.parametrize("raw", [False, True])
def test_contraction_kernels_report_against_the_mfma_peak(raw):
    for k in KERNELS:
        r = bench.kernel_roofline(k, 2.0, CHUNK_HEADS, raw)
        assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
        flop = 2.0 * bench.MAC_PER_CHUNK_HEAD[k] * CHUNK_HEADS
        assert r["achieved"] == pytest.approx(flop / 2e-3 / 1e12, rel=1e-3)
        assert r["frac"] == pytest.approx(r["achieved"] / 2500.0, abs=1e-4)
    # the per-chunk backward at 1doc: 1.766e11 FLOP, here timed at 2.2273 ms
    r = bench.kernel_roofline("bwd_intra", 2.2273, CHUNK_HEADS, raw)
    assert r["algorithmic_flop_per_launch"] == pytest.approx(1.766e11, rel=1e-3)
    assert r["frac"] == pytest.approx(0.0317, abs=2e-4)


@pytest.mark.parametrize("workload,raw", [("1doc", False), ("4doc", True)])
def test_recorded_traffic_is_close_to_the_byte_model(workload, raw):
    fig = bench.profile_figures(workload, "bwd_intra", bench.fingerprint())
    if fig is None:
        pytest.skip("profiles/ were taken on other kernel sources")
    model = bench.algo_bytes_per_chunk_head("bwd_intra", raw) * CHUNK_HEADS
    # measured HBM traffic within 15 % above the model and never far below it
    assert 0.97 * model <= fig["traffic_bytes"] <= 1.15 * model

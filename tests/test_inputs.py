"""The seeded input generator: determinism, bf16 rounding, workload shapes."""

import numpy as np
import torch

from kda_chunked_amd import inputs


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(1000) * 1e-30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 65504.0, 3.3895314e38, 1.00390625, 1.01171875], np.float32),
    ])
    # ties: mantissas ending exactly in 0x8000
    ties = (np.arange(1000, dtype=np.uint32) << 16 | 0x8000 | 0x3F800000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ours = inputs.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(inputs.bf16_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generator_is_deterministic_and_shaped():
    w = inputs.WORKLOADS[0]
    a = inputs.make_inputs(w)
    b = inputs.make_inputs(w)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    assert a["q"].shape == (256, 2, 128) and a["q"].dtype == np.uint16
    assert a["gate"].dtype == np.float32
    assert list(a["cu_seqlens"]) == [0, 200, 256]
    c = inputs.make_inputs(w, seed=99)
    assert not np.array_equal(a["q"], c["q"])


def test_workload_table():
    names = [w.name for w in inputs.WORKLOADS]
    assert names == ["tiny", "m2", "R2", "1doc", "4doc"]
    assert [w.T for w in inputs.WORKLOADS] == [256, 3548, 16384, 16384, 16384]
    assert [w.H for w in inputs.WORKLOADS] == [2, 4, 4, 64, 64]
    assert inputs.BY_NAME["4doc"].backward == ("saved", "replay")


def test_prenormalised_keys_and_gate_ranges():
    w = inputs.custom([300, 50], 2, gate="raw", alog_range=(np.log(4), np.log(32)), seed=5)
    x = inputs.make_inputs(w)
    k = inputs.bf16_to_f32(x["k"]).astype(np.float64)
    n = np.linalg.norm(k, axis=-1)
    assert np.all(np.abs(n - 1) < 1e-2)
    assert np.all((x["A_log"] >= np.log(4)) & (x["A_log"] <= np.log(32)))
    w = inputs.custom([64], 1, gate="g")
    g = inputs.make_inputs(w)["gate"]
    assert g.dtype == np.float32 and np.all(g < 0)
    w = inputs.custom([64], 1, gate="g", l2norm=True)
    q = inputs.bf16_to_f32(inputs.make_inputs(w)["q"])
    assert np.linalg.norm(q, axis=-1).mean() > 5      # raw N(0,1) keys, not normalised

"""Seeded input generators: reproducible, per-head, bf16 rounding correct."""
import numpy as np
import torch

from bayesian_memory_scan_amd import synth


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 3.0e38, 1e-40, -2.5], np.float32)])
    # ties: values exactly halfway between two bf16 numbers
    ties = (np.arange(0, 4096, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.f32_to_bf16_bits(x), ref)


def test_diag_inputs_reproducible_and_per_head():
    spec = synth.workload("diag_b1h2t64d16_f32").with_(B=2, H=3, T=20)
    a = synth.diag_inputs(spec)
    b = synth.diag_inputs(spec)
    for n in ("q", "k", "v", "beta", "d"):
        np.testing.assert_array_equal(a[n], b[n])
    one = synth.diag_head(spec, 1, 2)
    np.testing.assert_array_equal(a["q"][1, 2], one["q"])
    assert np.allclose(np.linalg.norm(a["k"], axis=-1), 1.0, atol=1e-6)
    assert np.all((a["beta"] > 0) & (a["beta"] < 1)) and np.all(a["d"] > 0)
    np.testing.assert_array_equal(a["A"], np.ones(3, np.float32))


def test_bf16_workload_dtype_and_A_range():
    spec = synth.workload("diag_b8h16t2048d128_bf16").with_(B=1, H=4, T=8)
    x = synth.diag_inputs(spec)
    assert x["q"].dtype == np.uint16 and x["q"].shape == (1, 4, 8, 128)
    assert np.all((x["A"] >= 0.5) & (x["A"] <= 2.0))


def test_iso_inputs_ranges():
    spec = synth.workload("iso_b1h32t65536d64_f32").with_(H=2, T=50)
    x = synth.iso_inputs(spec)
    assert np.all((x["a"] > 0) & (x["a"] < 1))
    assert np.all(x["p"] > 0) and np.all(x["Lambda"] > 0)
    assert x["q"].shape == (1, 2, 50, 64)


def test_decode_workload_has_prefix():
    spec = synth.workload("decode_b256h16d128_bf16").with_(B=1, H=1)
    x = synth.diag_inputs(spec)
    assert x["q"].shape == (1, 1, 513, 128)

"""The seeded input generator: bf16 quantisation and the named workloads (CPU only)."""
import numpy as np
import pytest
import torch

import workloads
from workloads import bf16_bits_to_f64, f32_to_bf16_bits, make_workload, quantise


def test_bf16_rounding_ties_to_even():
    x = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 1 + 2**-7, 3.0e38], dtype=np.float32)
    got = bf16_bits_to_f64(f32_to_bf16_bits(x))
    assert got.tolist()[:5] == [1.0, 1.0, 1 + 2**-6, -1.0, 1 + 2**-7]


def test_bf16_rounding_matches_torch():
    x = np.random.Generator(np.random.PCG64(0)).standard_normal(100000).astype(np.float32) * 37
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)


def test_quantised_values_are_exact():
    q = quantise(np.array([0.1, -2.5, 1e-3]), "bf16")
    assert np.array_equal(bf16_bits_to_f64(q.raw), q.f64)
    q = quantise(np.array([0.1, -2.5, 1e-3]), "f32")
    assert np.array_equal(q.raw.astype(np.float64), q.f64)


@pytest.mark.parametrize("name", [n for n in workloads.WORKLOADS if "4096" not in n])
def test_workloads_deterministic_and_shaped(name):
    w = workloads.WORKLOADS[name]
    a, b = make_workload(name), make_workload(name)
    for key in a:
        assert np.array_equal(a[key].f64, b[key].f64)
    if w["kind"] == "sdpa":
        assert a["Q"].shape == (w["B"], w["h"], w["n_q"], w["d_k"])
        assert a["K"].shape == (w["B"], w["h"], w["n_k"], w["d_k"])
        assert a["V"].shape == (w["B"], w["h"], w["n_k"], w["d_v"])
    elif w["kind"] == "encoder":
        assert a["X"].shape == (w["B"], w["n_q"], w["d_model"])
        assert a["W1"].shape == (w["d_model"], w["d_ff"]) and a["W2"].shape == (w["d_ff"], w["d_model"])
        assert a["b1"].shape == (w["d_ff"],) and a["ln2_beta"].shape == (w["d_model"],)
        assert abs(a["W1"].f64.std() - (1 / w["d_model"]) ** 0.5) < 2e-3
        assert abs(a["W2"].f64.std() - (1 / w["d_ff"]) ** 0.5) < 1e-3
        assert abs(a["ln1_gamma"].f64.mean() - 1.0) < 0.02
    else:
        assert a["Xq"].shape == (w["B"], w["n_q"], w["d_model"])
        assert a["Wo"].shape == (w["h"] * w["d_v"], w["d_model"])
        # W ~ N(0, 1/d_model)
        assert abs(a["Wq"].f64.std() - (1 / w["d_model"]) ** 0.5) < 2e-3

"""Parity of restricted (windowed) self-attention (sdpa_forward_window) with the float64 oracle.

Radii cover the tile boundaries (0, 1, 31, 32, 63, 64, 65) and wide bands, with and without the causal mask, in both
dtypes. Bars as for sdpa_forward: bf16 max-abs <= 2e-2, mean-abs <= 2e-3, normalised rms <= 1e-2; fp32 1e-5
relative. Radius 0 is exact: each row sees only itself, its weight is exactly 1, and the output is its own value row.
"""
import numpy as np
import pytest
import torch

import transformer_head_scaled_02_amd as m
import workloads
from oracle import sdpa_lse_ref, sdpa_ref
from tests._helpers import assert_bf16_parity, assert_f32_parity, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")
    m.load_library()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n,w,causal", [
    (1, 0, False), (77, 0, True), (77, 5, False), (256, 31, False), (256, 32, True), (256, 63, False),
    (256, 64, False), (300, 65, True), (700, 100, False), (700, 200, True), (520, 1000, False), (129, 128, True)])
def test_window_parity(dtype, n, w, causal):
    x = workloads.make_sdpa_inputs(2, 2, n, n, 64, 64, dtype, 9500 + n + w, scale_q=1.5)
    q, k, v = (to_dev(x[nm]) for nm in "QKV")
    out, lse = m.sdpa_forward_window(q, k, v, w, mask="causal" if causal else "none", return_lse=True)
    torch.cuda.synchronize()
    ref = sdpa_ref(x["Q"].f64, x["K"].f64, x["V"].f64, causal, window=w)
    got = to_f64(out)
    if dtype == "f32":
        assert_f32_parity(got, ref, f"window f32 n={n} w={w}")
    else:
        assert_bf16_parity(got, ref, f"window bf16 n={n} w={w}")
    lref = sdpa_lse_ref(x["Q"].f64, x["K"].f64, causal, window=w)
    d = np.abs(to_f64(lse) - lref)
    assert d.max() <= (1e-2 if dtype == "bf16" else 1e-5 * max(1.0, np.abs(lref).max())), d.max()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_radius_zero_returns_values(dtype):
    # bf16: the single weight is exactly 1 and the output is bitwise the value row. fp32 forms the weight as
    # exp2(s c - m) with m the fp32 product s c, whose rounding leaves exp2 of a residue of order 1e-7: within an ulp.
    x = workloads.make_sdpa_inputs(2, 3, 150, 150, 64, 64, dtype, 9600)
    q, k, v = (to_dev(x[nm]) for nm in "QKV")
    for mask in ("none", "causal"):
        out = m.sdpa_forward_window(q, k, v, 0, mask=mask)
        torch.cuda.synchronize()
        if dtype == "bf16":
            assert torch.equal(out, v)
        else:
            torch.testing.assert_close(out, v, rtol=1e-6, atol=1e-7)


def test_window_n4096_sampled_rows():
    # the long-sequence tensors with a band of radius 256 (513 keys per row)
    x = workloads.make_workload("sdpa_bf16_b4_h8_n4096")
    q, k, v = (to_dev(x[nm]) for nm in "QKV")
    got = to_f64(m.sdpa_forward_window(q, k, v, 256))
    rows = np.array([0, 1, 255, 256, 257, 1000, 2047, 3839, 3840, 4095])
    for b, hh in ((0, 0), (3, 7)):
        ref = sdpa_ref(x["Q"].f64[b, hh, rows], x["K"].f64[b, hh], x["V"].f64[b, hh], q_index=rows, window=256)
        assert_bf16_parity(got[b, hh, rows], ref, f"window n4096 head {b},{hh}")


def test_window_rejects_bad_arguments():
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.AttnError):
        m.sdpa_forward_window(q, q, q, -1)
    k = torch.zeros(1, 1, 9, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.AttnError):
        m.sdpa_forward_window(q, k, k, 2)

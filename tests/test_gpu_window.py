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


def test_window_n4096_every_head():
    # the long-sequence tensors with a band of radius 256 (513 keys per row): sampled rows of every head, and two
    # heads in full
    x = workloads.make_workload("sdpa_bf16_b4_h8_n4096")
    q, k, v = (to_dev(x[nm]) for nm in "QKV")
    got = to_f64(m.sdpa_forward_window(q, k, v, 256))
    rng = np.random.Generator(np.random.PCG64(11))
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 257, 1000, 2047, 3839, 3840, 4095],
                                     rng.choice(4096, 54, replace=False)]))
    for b in range(4):
        for hh in range(8):
            ref = sdpa_ref(x["Q"].f64[b, hh, rows], x["K"].f64[b, hh], x["V"].f64[b, hh], q_index=rows, window=256)
            assert_bf16_parity(got[b, hh, rows], ref, f"window n4096 head {b},{hh} sampled rows")
    for b, hh in ((0, 0), (3, 7)):
        ref = sdpa_ref(x["Q"].f64[b, hh], x["K"].f64[b, hh], x["V"].f64[b, hh], window=256)
        assert_bf16_parity(got[b, hh], ref, f"window n4096 head {b},{hh} in full")


def test_window_rejects_bad_arguments():
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.AttnError):
        m.sdpa_forward_window(q, q, q, -1)
    k = torch.zeros(1, 1, 9, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.AttnError):
        m.sdpa_forward_window(q, k, k, 2)


def _check_grads(got, ref, dtype, what):
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        g = to_f64(g)
        assert np.all(np.isfinite(g)), f"{what} {name}: non-finite"
        if not np.any(r):
            # radius 0: one key per row, so dS = P (dP - D) = 0 exactly and dQ = dK = 0; the kernels return the
            # rounding residue of dP - D (terms of order 10, rounded in fp32 or fed from bf16 operands)
            assert np.abs(g).max() <= (1e-4 if dtype == "f32" else 2e-2), f"{what} {name}: {np.abs(g).max():.3g}"
            continue
        d = np.abs(g - r)
        rel = float(d.max()) / max(float(np.abs(r).max()), 0.05)
        if dtype == "f32":
            assert rel <= 1e-5, f"{what} {name}: max rel {rel:.3g}"
        else:
            nrms = float(np.sqrt(np.mean(d * d)) / max(np.sqrt(np.mean(r * r)), 0.05))
            assert nrms <= 1e-2 and rel <= 1.5e-2, f"{what} {name}: nrms {nrms:.3g} max rel {rel:.3g}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n,w,causal", [(77, 0, False), (256, 31, False), (256, 64, True), (300, 65, False),
                                        (700, 200, True), (520, 1000, False), (129, 1, False)])
def test_window_backward_parity(dtype, n, w, causal):
    # bars as for the unpadded backward (normalised rms <= 1e-2, max-rel <= 1.5e-2 in bf16; 1e-5 in fp32)
    from oracle import sdpa_backward_ref
    x = workloads.make_sdpa_inputs(2, 2, n, n, 64, 64, dtype, 9700 + n + w, dout=True)
    q, k, v, do = (to_dev(x[nm]) for nm in ("Q", "K", "V", "dO"))
    mask = "causal" if causal else "none"
    out, lse = m.sdpa_forward_window(q, k, v, w, mask=mask, return_lse=True)
    grads = m.sdpa_backward(q, k, v, out, do, lse, mask=mask, window=w)
    torch.cuda.synchronize()
    ref = sdpa_backward_ref(x["Q"].f64, x["K"].f64, x["V"].f64, x["dO"].f64, causal, window=w)
    _check_grads(grads, ref, dtype, f"window backward {dtype} n={n} w={w} causal={causal}")


def test_autograd_wrapper_with_window():
    x = workloads.make_sdpa_inputs(2, 2, 200, 200, 64, 64, "bf16", 9800, dout=True)
    q, k, v, do = (to_dev(x[nm]) for nm in ("Q", "K", "V", "dO"))
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    m.attention(qa, ka, va, window=40).backward(do)
    out, out32, lse = m.sdpa_forward_train(q, k, v, window=40)  # the wrapper keeps the float32 output for D
    dq, dk, dv = m.sdpa_backward(q, k, v, out32, do, lse, window=40)
    torch.cuda.synchronize()
    assert torch.equal(qa.grad, dq) and torch.equal(ka.grad, dk) and torch.equal(va.grad, dv)

"""Long sequences: the forward at n = 65536 and the backward at n = 32768 (one head each), checked against the
float64 oracle on sampled query rows (a row of the output, or of dQ, depends on that row alone), and through the
sum rules of the gradient over all keys. These sizes exercise 64-bit offsets and thousands of key tiles per row.
Bars as for the n = 4096 workloads.
"""
import numpy as np
import pytest
import torch

import transformer_head_scaled_02_amd as m
import workloads
from oracle import sdpa_backward_head, sdpa_ref
from tests._helpers import assert_bf16_parity, to_dev, to_f64

pytestmark = pytest.mark.gpu

ROWS = np.array([0, 1, 63, 64, 1000, 4095, 4096, 20000, 32767])


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")
    m.load_library()


@pytest.mark.parametrize("causal", [False, True])
def test_forward_n65536(causal):
    n = 65536
    x = workloads.make_sdpa_inputs(1, 1, n, n, 64, 64, "bf16", 9900)
    q, k, v = (to_dev(x[nm]) for nm in "QKV")
    out, lse = m.sdpa_forward_lse(q, k, v, mask="causal" if causal else "none")
    torch.cuda.synchronize()
    rows = np.concatenate([ROWS, [65535]])
    ref = sdpa_ref(x["Q"].f64[0, 0, rows], x["K"].f64[0, 0], x["V"].f64[0, 0], causal, q_index=rows)
    assert_bf16_parity(to_f64(out)[0, 0, rows], ref, f"n65536 causal={causal}")
    assert torch.all(torch.isfinite(lse))


def test_backward_n32768():
    n = 32768
    x = workloads.make_sdpa_inputs(1, 1, n, n, 64, 64, "bf16", 9901, dout=True)
    q, k, v, do = (to_dev(x[nm]) for nm in ("Q", "K", "V", "dO"))
    out, lse = m.sdpa_forward_lse(q, k, v)
    dq, dk, dv = m.sdpa_backward(q, k, v, out, do, lse)
    torch.cuda.synchronize()
    Q, K, V, dO = (x[nm].f64[0, 0] for nm in ("Q", "K", "V", "dO"))
    ref_dq = sdpa_backward_head(Q[ROWS], K, V, dO[ROWS], q_index=ROWS)[0]
    got = to_f64(dq)[0, 0, ROWS]
    d = np.abs(got - ref_dq)
    nrms = np.sqrt(np.mean(d * d)) / np.sqrt(np.mean(ref_dq * ref_dq))
    assert nrms <= 1e-2 and d.max() <= 1.5e-2 * np.abs(ref_dq).max(), (nrms, d.max())
    # over all keys: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i, up to the rounding of n bf16 rows
    gk, gv = to_f64(dk)[0, 0], to_f64(dv)[0, 0]
    assert np.all(np.isfinite(gk)) and np.all(np.isfinite(gv))
    assert np.abs(gk.sum(axis=0)).max() <= 0.05 * np.abs(gk).max() * np.sqrt(n)
    assert np.abs(gv.sum(axis=0) - dO.sum(axis=0)).max() <= 0.02 * np.abs(dO.sum(axis=0)).max()

"""Parity of the key padding mask (sdpa_forward_padded, sdpa_backward with kv_len) with the float64 oracle.

Lengths cover the degenerate and tile-boundary cases: 0 (a row with no key: output 0, lse -inf, no gradient), 1, 63,
64, 65, full, and out-of-range values (clamped to [0, n_k]). Bars as for the unpadded paths: bf16 outputs max-abs
<= 2e-2, mean-abs <= 2e-3, normalised rms <= 1e-2; bf16 gradients normalised rms <= 1e-2 and max-rel <= 1.5e-2; fp32
1e-5 relative. Padding contents must not matter at all: NaN in every padding row changes no bit of any result.
"""
import numpy as np
import pytest
import torch

import transformer_head_scaled_02_amd as m
import workloads
from oracle import sdpa_backward_ref, sdpa_lse_ref, sdpa_ref
from tests._helpers import assert_bf16_parity, assert_f32_parity, to_dev, to_f64

pytestmark = pytest.mark.gpu

SCALE_FLOOR = 0.05  # as in the backward tests: the scale of a gradient that vanishes identically


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")
    m.load_library()


def _mask(causal):
    return "causal" if causal else "none"


def _lens(lengths):
    return torch.tensor(lengths, dtype=torch.int32, device="cuda")


def _clamped(lengths, n_k):
    return np.clip(np.asarray(lengths), 0, n_k)


def _check_grads(got, ref, dtype, what):
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        g = to_f64(g) if isinstance(g, torch.Tensor) else g
        assert np.all(np.isfinite(g)), f"{what} {name}: non-finite"
        d = np.abs(g - r)
        rel = float(d.max()) / max(float(np.abs(r).max()), SCALE_FLOOR)
        if dtype == "f32":
            assert rel <= 1e-5, f"{what} {name}: max rel {rel:.3g}"
        else:
            nrms = float(np.sqrt(np.mean(d * d)) / max(np.sqrt(np.mean(r * r)), SCALE_FLOOR))
            assert nrms <= 1e-2 and rel <= 1.5e-2, f"{what} {name}: nrms {nrms:.3g} max rel {rel:.3g}"


CASES = [  # (n_q, n_k, lengths per batch entry, causal)
    (256, 256, [0, 1, 65, 200, 256], False),
    (256, 256, [256, 64, 63, 1, 0], True),
    (100, 300, [300, 129, 128, 7, 500], False),
    (77, 77, [-3, 77, 40], True),
    (1, 130, [130, 64, 0], False),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n_q,n_k,lengths,causal", CASES)
def test_padded_forward_and_lse(dtype, n_q, n_k, lengths, causal):
    B = len(lengths)
    x = workloads.make_sdpa_inputs(B, 2, n_q, n_k, 64, 64, dtype, 9000 + n_q + n_k, scale_q=1.5)
    q, k, v = (to_dev(x[n]) for n in "QKV")
    out, lse = m.sdpa_forward_padded(q, k, v, _lens(lengths), mask=_mask(causal), return_lse=True)
    torch.cuda.synchronize()
    kv = _clamped(lengths, n_k)
    ref = sdpa_ref(x["Q"].f64, x["K"].f64, x["V"].f64, causal, kv_len=kv)
    got = to_f64(out)
    if dtype == "f32":
        assert_f32_parity(got, ref, "padded f32")
    else:
        assert_bf16_parity(got, ref, "padded bf16")
    for b, L in enumerate(kv):
        if L == 0:
            assert torch.count_nonzero(out[b]) == 0
            assert torch.all(torch.isneginf(lse[b]))
    lref = sdpa_lse_ref(x["Q"].f64, x["K"].f64, causal, kv_len=kv)
    finite = np.isfinite(lref)
    assert np.array_equal(np.isfinite(to_f64(lse)), finite)
    d = np.abs(to_f64(lse)[finite] - lref[finite])
    assert d.max() <= (1e-2 if dtype == "bf16" else 1e-5 * max(1.0, np.abs(lref[finite]).max())), d.max()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n_q,n_k,lengths,causal", CASES)
def test_padded_backward(dtype, n_q, n_k, lengths, causal):
    B = len(lengths)
    x = workloads.make_sdpa_inputs(B, 2, n_q, n_k, 64, 64, dtype, 9100 + n_q + n_k, dout=True)
    q, k, v, do = (to_dev(x[n]) for n in ("Q", "K", "V", "dO"))
    lens = _lens(lengths)
    out, lse = m.sdpa_forward_padded(q, k, v, lens, mask=_mask(causal), return_lse=True)
    grads = m.sdpa_backward(q, k, v, out, do, lse, mask=_mask(causal), kv_len=lens)
    torch.cuda.synchronize()
    kv = _clamped(lengths, n_k)
    ref = sdpa_backward_ref(x["Q"].f64, x["K"].f64, x["V"].f64, x["dO"].f64, causal, kv_len=kv)
    _check_grads(grads, ref, dtype, f"padded backward {dtype} {n_q}x{n_k} {lengths} causal={causal}")
    for b, L in enumerate(kv):
        assert torch.count_nonzero(grads[1][b, :, L:]) == 0 and torch.count_nonzero(grads[2][b, :, L:]) == 0
        if L == 0:
            assert torch.count_nonzero(grads[0][b]) == 0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_padding_contents_never_matter(dtype, causal):
    # NaN in every padding row of K and V: no bit of the output, lse or gradients may change
    n, lengths = 200, [200, 70, 1, 0]
    B = len(lengths)
    x = workloads.make_sdpa_inputs(B, 2, n, n, 64, 64, dtype, 9200, dout=True)
    q, k, v, do = (to_dev(x[nm]) for nm in ("Q", "K", "V", "dO"))
    lens = _lens(lengths)

    def run(k_, v_):
        out, lse = m.sdpa_forward_padded(q, k_, v_, lens, mask=_mask(causal), return_lse=True)
        return (out, lse) + m.sdpa_backward(q, k_, v_, out, do, lse, mask=_mask(causal), kv_len=lens)

    base = run(k, v)
    k2, v2 = k.clone(), v.clone()
    for b, L in enumerate(lengths):
        k2[b, :, L:] = float("nan")
        v2[b, :, L:] = float("nan")
    other = run(k2, v2)
    torch.cuda.synchronize()
    for a, b_ in zip(base, other):
        assert torch.equal(a, b_)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_full_lengths_equal_no_padding(dtype, causal):
    n = 130
    x = workloads.make_sdpa_inputs(3, 2, n, n, 64, 64, dtype, 9300, dout=True)
    q, k, v, do = (to_dev(x[nm]) for nm in ("Q", "K", "V", "dO"))
    lens = _lens([n, n, n])
    out_p, lse_p = m.sdpa_forward_padded(q, k, v, lens, mask=_mask(causal), return_lse=True)
    out, lse = m.sdpa_forward_lse(q, k, v, mask=_mask(causal))
    g_p = m.sdpa_backward(q, k, v, out, do, lse, mask=_mask(causal), kv_len=lens)
    g = m.sdpa_backward(q, k, v, out, do, lse, mask=_mask(causal))
    torch.cuda.synchronize()
    assert torch.equal(out_p, out) and torch.equal(lse_p, lse)
    for a, b in zip(g_p, g):
        assert torch.equal(a, b)


def test_padded_n4096_sampled_heads():
    # the long-sequence tensors with a length mix of a length-bucketed batch; the oracle checks one head per entry
    w = workloads.WORKLOADS["sdpa_bwd_bf16_b4_h8_n4096"]
    x = workloads.make_workload("sdpa_bwd_bf16_b4_h8_n4096")
    lengths = [4096, 3000, 1025, 64]
    q, k, v, do = (to_dev(x[nm]) for nm in ("Q", "K", "V", "dO"))
    lens = _lens(lengths)
    out, lse = m.sdpa_forward_padded(q, k, v, lens, return_lse=True)
    grads = m.sdpa_backward(q, k, v, out, do, lse, kv_len=lens)
    torch.cuda.synchronize()
    got = to_f64(out)
    gg = [to_f64(t) for t in grads]
    for b, L in enumerate(lengths):
        hh = (3 * b + 1) % w["h"]
        ins = [x[nm].f64[b:b + 1, hh:hh + 1] for nm in ("Q", "K", "V", "dO")]
        ref = sdpa_ref(*ins[:3], kv_len=np.array([L]))[0, 0]
        assert_bf16_parity(got[b, hh], ref, f"padded n4096 entry {b}")
        gref = sdpa_backward_ref(*ins, kv_len=np.array([L]))
        _check_grads([g[b, hh] for g in gg], [r[0, 0] for r in gref], "bf16",
                     f"padded n4096 backward entry {b}")


def test_autograd_wrapper_with_padding():
    x = workloads.make_sdpa_inputs(3, 2, 96, 96, 64, 64, "bf16", 9400, dout=True)
    q, k, v, do = (to_dev(x[nm]) for nm in ("Q", "K", "V", "dO"))
    lens = _lens([96, 40, 0])
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    m.attention(qa, ka, va, mask="causal", kv_len=lens).backward(do)
    # the wrapper keeps the float32 output for D (sdpa_forward_train's out_f32)
    out, out32, lse = m.sdpa_forward_train(q, k, v, "causal", kv_len=lens)
    dq, dk, dv = m.sdpa_backward(q, k, v, out32, do, lse, mask="causal", kv_len=lens)
    torch.cuda.synchronize()
    assert torch.equal(qa.grad, dq) and torch.equal(ka.grad, dk) and torch.equal(va.grad, dv)

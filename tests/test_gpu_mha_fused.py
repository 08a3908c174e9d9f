"""Parity of the one-launch projection + attention path of short self-attention (n <= 128, head width 64) with the
float64 oracle, through mha_forward and encoder_layer_forward.

That path computes, per (batch entry, head), the head's Q/K/V projections and its attention in one workgroup (every
key in LDS, the plain softmax over all of them). Swept here: sequence lengths around its 32-key blocks and its limit
(1 .. 128, with 129 falling back to the separate kernels), d_model from one to thirty-two heads and projections of
h * 64 columns narrower or wider than d_model, the causal mask, key
padding down to zero keys (encoder layer), and the same call twice (no state). Bars as everywhere for bf16:
max-abs <= 2e-2, mean-abs <= 2e-3, normalised rms <= 1e-2 (the encoder layer's LayerNorm outputs are order 1 and use
the encoder tests' bars).
"""
import pytest
import torch

import transformer_head_scaled_02_amd as m
import workloads
from oracle import mha_ref
from tests._helpers import assert_bf16_parity, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")
    m.load_library()


@pytest.mark.parametrize("n", [1, 2, 17, 31, 32, 33, 63, 64, 65, 96, 127, 128, 129])
@pytest.mark.parametrize("causal", [False, True])
def test_fused_mha_lengths(n, causal):
    B, d_model, h = 3, 512, 8
    x = workloads.make_mha_inputs(B, n, n, d_model, h, 64, 64, "bf16", 7000 + n)
    xq = to_dev(x["Xq"])
    ws = [to_dev(x[k]) for k in ("Wq", "Wk", "Wv", "Wo")]
    got = to_f64(m.mha_forward(xq, xq, *ws, h=h, mask="causal" if causal else "none"))
    ref = mha_ref(x["Xq"].f64, x["Xq"].f64, x["Wq"].f64, x["Wk"].f64, x["Wv"].f64, x["Wo"].f64, h=h, causal=causal)
    assert_bf16_parity(got, ref, f"mha n={n} causal={causal}")


@pytest.mark.parametrize("B,n,d_model,h", [(1, 128, 64, 1), (2, 77, 128, 2), (5, 40, 256, 4), (2, 128, 1024, 16),
                                           (1, 3, 2048, 32),
                                           # h * 64 != d_model: projections narrower or wider than the model
                                           (2, 100, 512, 4), (3, 50, 192, 8), (1, 128, 64, 3)])
def test_fused_mha_widths(B, n, d_model, h):
    x = workloads.make_mha_inputs(B, n, n, d_model, h, 64, 64, "bf16", 7100 + d_model + n)
    xq = to_dev(x["Xq"])
    ws = [to_dev(x[k]) for k in ("Wq", "Wk", "Wv", "Wo")]
    got = to_f64(m.mha_forward(xq, xq, *ws, h=h))
    ref = mha_ref(x["Xq"].f64, x["Xq"].f64, x["Wq"].f64, x["Wk"].f64, x["Wv"].f64, x["Wo"].f64, h=h)
    assert_bf16_parity(got, ref, f"mha B={B} n={n} d_model={d_model} h={h}")


def test_fused_mha_repeatable_and_noalloc_equal():
    B, n, d_model, h = 32, 128, 512, 8
    x = workloads.make_mha_inputs(B, n, n, d_model, h, 64, 64, "bf16", 1002)
    xq = to_dev(x["Xq"])
    ws = [to_dev(x[k]) for k in ("Wq", "Wk", "Wv", "Wo")]
    a = m.mha_forward(xq, xq, *ws, h=h).clone()
    b = m.mha_forward(xq, xq, *ws, h=h)
    c = m.mha_forward_noalloc(xq, xq, *ws, h=h, out=torch.empty_like(a))
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


@pytest.mark.parametrize("n,causal,kv_len", [(128, False, [128, 0, 1, 64]), (100, True, [100, 33, 99, 2]),
                                             (33, False, [0, 0, 33, 32])])
def test_fused_encoder_layer_padding(n, causal, kv_len):
    # the encoder layer takes the same path for its attention step (with key padding); bars of the encoder tests
    from tests.test_gpu_encoder import _check, _ref, _run
    B, d_model, h, d_ff = 4, 512, 8, 2048
    x = workloads.make_encoder_inputs(B, n, d_model, h, d_ff, "bf16", 7200 + n)
    got = to_f64(_run(x, h, 1e-5, causal, kv_len))
    _check(got, _ref(x, h, 1e-5, causal, kv_len), f"encoder n={n} causal={causal} kv={kv_len}")

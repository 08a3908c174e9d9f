"""The allocation-free multi-head attention entry point (mha_forward_noalloc) against mha_forward through the C ABI.

mha_forward_noalloc runs the same three launches as mha_forward with its intermediates in the library's own device
scratch instead of a caller workspace. On the same inputs the two entry points must give identical bits. Two calls in
a row, the second smaller than the first, check that what the first left in the scratch does not leak into the
second (every scratch byte a call reads is written earlier in that call). Sizes beyond the scratch are rejected with
ATTN_ERR_INVALID before any HIP call.
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


def _inputs(B, n, d_model, h, seed, causal=False):
    x = workloads.make_mha_inputs(B, n, n, d_model, h, d_model // h, d_model // h, "bf16", seed)
    return x, [to_dev(x[k]) for k in ("Xq", "Wq", "Wk", "Wv", "Wo")]


def _both(B, n, d_model, h, seed, mask="none"):
    x, (xq, wq, wk, wv, wo) = _inputs(B, n, d_model, h, seed)
    ref_out = m.mha_forward(xq, xq, wq, wk, wv, wo, h=h, mask=mask)
    out = torch.full_like(ref_out, float("nan"))
    m.mha_forward_noalloc(xq, xq, wq, wk, wv, wo, h=h, mask=mask, out=out)
    torch.cuda.synchronize()
    return x, ref_out, out


def test_noalloc_matches_mha_forward_two_calls_second_smaller():
    # the base model's encoder self-attention (16 MiB of scratch), then a smaller, ragged, causal call
    x1, ref1, out1 = _both(32, 128, 512, 8, 1002)
    assert torch.equal(out1, ref1), "noalloc output differs from mha_forward (first call)"
    x2, ref2, out2 = _both(2, 33, 512, 8, 43, mask="causal")
    assert torch.equal(out2, ref2), "noalloc output differs from mha_forward (second, smaller call)"
    # and the smaller call against the oracle, to the usual bf16 bars
    want = mha_ref(x2["Xq"].f64, x2["Xq"].f64, x2["Wq"].f64, x2["Wk"].f64, x2["Wv"].f64, x2["Wo"].f64, h=8,
                   causal=True)
    assert_bf16_parity(to_f64(out2), want, "noalloc second call vs oracle")


def test_noalloc_other_head_width():
    x, ref, out = _both(4, 200, 512, 4, 1008)
    assert torch.equal(out, ref)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    B, n, d_model, h = 64, 512, 512, 8  # needs 128 MiB of scratch
    assert m.mha_workspace_size(B, n, n, h) > m._binding.NOALLOC_SCRATCH_BYTES
    xq = torch.zeros(B, n, d_model, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(d_model, d_model, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(xq)
    with pytest.raises(m.AttnError) as e:
        m.mha_forward_noalloc(xq, xq, w, w, w, w, h=h, out=out)
    assert e.value.status == m.ATTN_ERR_INVALID and "scratch" in str(e.value)

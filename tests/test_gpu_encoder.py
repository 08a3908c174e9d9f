"""Parity of encoder_layer_forward (the post-norm encoder layer: self-attention + residual + LayerNorm, FFN + residual
+ LayerNorm) with the float64 oracle on the same seeded bf16 inputs.

Bars. The layer's output is LayerNorm-scaled (rms 1, |values| up to about 6), and every intermediate is stored in
bf16 (Q/K/V, the heads, both residual sums, H1, the FFN hidden layer); an emulation of those roundings against the
float64 oracle gives max-abs 0.038-0.040, mean-abs 2.5e-3 and normalised rms 3.5e-3 on these shapes. Bars: normalised
rms <= 1e-2, mean-abs <= 6e-3, max-abs <= 0.1.
"""
import numpy as np
import pytest
import torch

import transformer_head_scaled_02_amd as m
import workloads
from oracle import encoder_layer_ref
from tests._helpers import to_dev, to_f64

pytestmark = pytest.mark.gpu

NAMES = ("Wq", "Wk", "Wv", "Wo", "ln1_gamma", "ln1_beta", "W1", "b1", "W2", "b2", "ln2_gamma", "ln2_beta")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")
    m.load_library()


def _check(got, ref, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    d = np.abs(got - ref)
    nrms = float(np.sqrt(np.mean(d * d)) / np.sqrt(np.mean(ref * ref)))
    assert nrms <= 1e-2 and d.mean() <= 6e-3 and d.max() <= 0.1, \
        f"{what}: max_abs {d.max():.3g} mean_abs {d.mean():.3g} nrms {nrms:.3g}"


def _run(x, h, eps, causal=False, kv_len=None, **kw):
    ts = [to_dev(x[nm]) for nm in NAMES]
    lens = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32, device="cuda")
    out = m.encoder_layer_forward(to_dev(x["X"]), *ts, h=h, eps=eps, mask="causal" if causal else "none",
                                  kv_len=lens, **kw)
    torch.cuda.synchronize()
    return out


def _ref(x, h, eps, causal=False, kv_len=None):
    return encoder_layer_ref(x["X"].f64, *(x[nm].f64 for nm in NAMES), h, eps, causal,
                             None if kv_len is None else np.asarray(kv_len))


def test_encoder_layer_workload():
    w = workloads.WORKLOADS["encoder_layer_bf16_b32_n128_dm512"]
    x = workloads.make_workload("encoder_layer_bf16_b32_n128_dm512")
    got = to_f64(_run(x, w["h"], w["eps"]))
    _check(got, _ref(x, w["h"], w["eps"]), "encoder layer b32 n128")


@pytest.mark.parametrize("B,n,d_model,h,d_ff,causal,kv_len", [
    (2, 1, 512, 8, 2048, False, None), (3, 77, 512, 8, 2048, True, None), (2, 130, 256, 4, 1024, False, None),
    (4, 65, 512, 8, 2048, False, [65, 30, 1, 0]), (2, 200, 1024, 16, 4096, True, [200, 100]),
    (1, 64, 64, 1, 64, False, None),
    # d_model = 320: three column tiles per row, the last one half wide, and 150 rows (a ragged last row tile)
    (3, 50, 320, 5, 640, False, None),
    # 8192 rows x 1024 columns: the W^O and W2 products take 128-row tiles (the LayerNorm covers 128 rows per tile)
    (64, 128, 1024, 16, 1024, False, None)])
def test_encoder_layer_shapes(B, n, d_model, h, d_ff, causal, kv_len):
    x = workloads.make_encoder_inputs(B, n, d_model, h, d_ff, "bf16", 1100 + n + d_model)
    got = to_f64(_run(x, h, 1e-5, causal, kv_len))
    _check(got, _ref(x, h, 1e-5, causal, kv_len), f"encoder {B}x{n} d_model={d_model} causal={causal} kv={kv_len}")


def test_encoder_layer_eps_and_constant_rows():
    # X = 0 and W^O = 0: R1 = 0 in every row, so LayerNorm 1 returns its shift exactly (with any eps > 0)
    x = workloads.make_encoder_inputs(2, 40, 512, 8, 2048, "bf16", 1200)
    for nm in ("X", "Wo"):
        x[nm] = workloads.quantise(np.zeros(x[nm].shape), "bf16")
    for eps in (1e-5, 1e-2):
        got = to_f64(_run(x, 8, eps))
        _check(got, _ref(x, 8, eps), f"constant rows eps={eps}")


def test_encoder_layer_workspace_reuse_and_no_writes_outside():
    B, n, d_model, h, d_ff = 2, 96, 512, 8, 2048
    ws = torch.empty(m.encoder_layer_workspace_size(B, n, d_model, h, d_ff), dtype=torch.uint8, device="cuda")
    for n_i in (96, 33):
        x = workloads.make_encoder_inputs(B, n_i, d_model, h, d_ff, "bf16", 1300 + n_i)
        numel = B * n_i * d_model
        big = torch.full((numel + 2048,), 5.0, dtype=torch.bfloat16, device="cuda")
        out = big[1024:1024 + numel].view(B, n_i, d_model)
        _run(x, h, 1e-5, out=out, workspace=ws)
        assert torch.all(big[:1024] == 5.0) and torch.all(big[-1024:] == 5.0)
        _check(to_f64(out), _ref(x, h, 1e-5), f"reuse n={n_i}")


@pytest.mark.parametrize("n", [128, 200])
def test_encoder_layer_workspace_contents_do_not_matter(n):
    # Every workspace region is written before it is read within a call: the result must not depend on what the
    # workspace held before (here: all bits set, random bytes, the previous call's intermediates).
    B, d_model, h, d_ff = 8, 512, 8, 2048
    x = workloads.make_encoder_inputs(B, n, d_model, h, d_ff, "bf16", 1400 + n)
    ws = torch.empty(m.encoder_layer_workspace_size(B, n, d_model, h, d_ff), dtype=torch.uint8, device="cuda")
    outs = []
    for fill in ("ones", "random", "previous"):
        if fill == "ones":
            ws.fill_(255)
        elif fill == "random":
            ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device="cuda"))
        outs.append(_run(x, h, 1e-5, workspace=ws).clone())
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    _check(to_f64(outs[0]), _ref(x, h, 1e-5), f"workspace contents n={n}")

"""Pins of the oracle's encoder layer (LayerNorm(x + Sublayer(x)) around multi-head self-attention and the
position-wise FFN: "Transformer：抛弃循环与卷积的序列建模", sections "FFN" and "Residual Connection 与 LayerNorm";
lettle.cn translation, section 3.1) to facts other than its own formulas:
  * LayerNorm closed forms (zero mean, variance var/(var + eps), constant rows, invariance to shift and positive scale
    with eps = 0) and torch's float64 layer_norm;
  * FFN closed forms (zero first weight, ReLU clipping);
  * the whole layer against torch's float64 nn.TransformerEncoderLayer in its post-norm form with ReLU and no dropout
    (its attention biases set to zero, since the pages' attention has none), also with the causal mask and key padding;
  * degenerate layers that reduce to LayerNorm alone.
"""
import numpy as np
import pytest
import torch

from oracle import encoder_layer_ref, ffn_ref, layer_norm_ref


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def test_layer_norm_closed_forms():
    r = _rng(1)
    x = r.standard_normal((5, 7, 64)) * 3 + 2
    eps = 1e-5
    y = layer_norm_ref(x, np.ones(64), np.zeros(64), eps)
    np.testing.assert_allclose(y.mean(axis=-1), 0.0, atol=1e-14)
    var = x.var(axis=-1)
    np.testing.assert_allclose(np.square(y).mean(axis=-1), var / (var + eps), rtol=1e-12)
    # a constant row normalises to beta; gamma and beta act per feature
    c = np.full((1, 64), 3.5)
    beta = r.standard_normal(64)
    np.testing.assert_allclose(layer_norm_ref(c, r.standard_normal(64), beta, eps)[0], beta, atol=1e-12)
    gamma = r.standard_normal(64)
    np.testing.assert_allclose(layer_norm_ref(x, gamma, beta, eps), y * gamma + beta, atol=1e-12)
    # with eps = 0 a shift and a positive scale of the row change nothing
    np.testing.assert_allclose(layer_norm_ref(4.0 * x - 7.0, np.ones(64), np.zeros(64), 0.0),
                               layer_norm_ref(x, np.ones(64), np.zeros(64), 0.0), atol=1e-12)


def test_layer_norm_matches_torch_float64():
    r = _rng(2)
    x, g, b = r.standard_normal((3, 9, 512)), r.standard_normal(512), r.standard_normal(512)
    want = torch.nn.functional.layer_norm(torch.tensor(x), (512,), torch.tensor(g), torch.tensor(b), eps=1e-6)
    np.testing.assert_allclose(layer_norm_ref(x, g, b, 1e-6), want.numpy(), atol=1e-12)


def test_ffn_closed_forms():
    r = _rng(3)
    x = r.standard_normal((4, 16))
    W2, b2 = r.standard_normal((32, 16)), r.standard_normal(16)
    b1 = r.standard_normal(32)
    # zero first weight: every row is relu(b1) W2 + b2
    np.testing.assert_allclose(ffn_ref(x, np.zeros((16, 32)), b1, W2, b2),
                               np.tile(np.maximum(b1, 0) @ W2 + b2, (4, 1)), atol=1e-12)
    # identity-like first layer on a crafted input: negative pre-activations are clipped to zero
    W1 = np.eye(16, 32)
    xs = np.array([[1.0, -2.0] + [0.0] * 14])
    got = ffn_ref(xs, W1, np.zeros(32), np.eye(32, 16), np.zeros(16))
    np.testing.assert_allclose(got, [[1.0, 0.0] + [0.0] * 14], atol=1e-15)


def _torch_layer(d_model, h, d_ff, eps, P):
    layer = torch.nn.TransformerEncoderLayer(d_model, h, d_ff, dropout=0.0, activation="relu", batch_first=True,
                                             norm_first=False, layer_norm_eps=eps, dtype=torch.float64)
    with torch.no_grad():
        a = layer.self_attn
        a.in_proj_weight.copy_(torch.tensor(np.concatenate([P["Wq"].T, P["Wk"].T, P["Wv"].T])))
        a.in_proj_bias.zero_()
        a.out_proj.weight.copy_(torch.tensor(P["Wo"].T))
        a.out_proj.bias.zero_()
        layer.linear1.weight.copy_(torch.tensor(P["W1"].T))
        layer.linear1.bias.copy_(torch.tensor(P["b1"]))
        layer.linear2.weight.copy_(torch.tensor(P["W2"].T))
        layer.linear2.bias.copy_(torch.tensor(P["b2"]))
        layer.norm1.weight.copy_(torch.tensor(P["g1"]))
        layer.norm1.bias.copy_(torch.tensor(P["be1"]))
        layer.norm2.weight.copy_(torch.tensor(P["g2"]))
        layer.norm2.bias.copy_(torch.tensor(P["be2"]))
    return layer.eval()


def _params(seed, d_model, d_ff):
    r = _rng(seed)
    s = 1 / np.sqrt(d_model)
    P = {n: r.standard_normal((d_model, d_model)) * s for n in ("Wq", "Wk", "Wv", "Wo")}
    P.update(W1=r.standard_normal((d_model, d_ff)) * s, b1=r.standard_normal(d_ff) * 0.1,
             W2=r.standard_normal((d_ff, d_model)) / np.sqrt(d_ff), b2=r.standard_normal(d_model) * 0.1,
             g1=1 + 0.1 * r.standard_normal(d_model), be1=0.1 * r.standard_normal(d_model),
             g2=1 + 0.1 * r.standard_normal(d_model), be2=0.1 * r.standard_normal(d_model))
    return P


def _ref(X, P, h, eps, causal=False, kv_len=None):
    return encoder_layer_ref(X, P["Wq"], P["Wk"], P["Wv"], P["Wo"], P["g1"], P["be1"], P["W1"], P["b1"], P["W2"],
                             P["b2"], P["g2"], P["be2"], h, eps, causal, kv_len)


@pytest.mark.parametrize("causal,padded", [(False, False), (True, False), (False, True)])
def test_encoder_layer_matches_torch_float64(causal, padded):
    B, n, d_model, h, d_ff, eps = 3, 10, 64, 4, 128, 1e-5
    P = _params(4, d_model, d_ff)
    X = _rng(5).standard_normal((B, n, d_model))
    kv_len = np.array([10, 6, 3]) if padded else None
    layer = _torch_layer(d_model, h, d_ff, eps, P)
    kw = {}
    if causal:
        kw["src_mask"] = torch.nn.Transformer.generate_square_subsequent_mask(n, dtype=torch.float64)
        kw["is_causal"] = True
    if padded:
        kw["src_key_padding_mask"] = torch.tensor(np.arange(n)[None, :] >= kv_len[:, None])
    with torch.no_grad():
        want = layer(torch.tensor(X), **kw).numpy()
    np.testing.assert_allclose(_ref(X, P, h, eps, causal, kv_len), want, atol=1e-10)


def test_layer_without_sublayers_is_layer_norm_twice():
    # zero W^O and zero FFN output weights: H1 = LN(X), Y = LN(H1 + b2)
    d_model, d_ff, eps = 64, 128, 1e-5
    P = _params(6, d_model, d_ff)
    P["Wo"] = np.zeros_like(P["Wo"])
    P["W2"] = np.zeros_like(P["W2"])
    X = _rng(7).standard_normal((2, 5, d_model))
    h1 = layer_norm_ref(X, P["g1"], P["be1"], eps)
    np.testing.assert_allclose(_ref(X, P, 4, eps), layer_norm_ref(h1 + P["b2"], P["g2"], P["be2"], eps), atol=1e-12)

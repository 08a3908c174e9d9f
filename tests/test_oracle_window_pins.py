"""Pins of the oracle's restricted (windowed) self-attention ("Transformer：抛弃循环与卷积的序列建模", section
"Self-Attention的优势": each position attends to a neighbourhood of size r; read as radius w, |i - j| <= w) to facts
other than its own code: the pure-Python literal definition over each query's neighbourhood, the closed form of
radius 0 (each row sees only itself: output = its own value row), a radius covering the sequence equals unmasked
attention, the window combined with the causal mask, and torch's float64 attention with a banded boolean mask.
"""
import numpy as np
import pytest
import torch

from oracle import sdpa_brute, sdpa_lse_ref, sdpa_ref, sdpa_weights_ref


def _case(seed, B, h, n, d=8, dv=5):
    r = np.random.Generator(np.random.PCG64(seed))
    return r.standard_normal((B, h, n, d)), r.standard_normal((B, h, n, d)), r.standard_normal((B, h, n, dv))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("w", [0, 1, 3])
def test_window_equals_brute_force_over_each_neighbourhood(w, causal):
    n = 9
    Q, K, V = _case(1, 1, 2, n)
    got = sdpa_ref(Q, K, V, causal, window=w)
    for hh in range(2):
        for i in range(n):
            lo, hi = max(0, i - w), (i if causal else min(n - 1, i + w))
            want = sdpa_brute([Q[0, hh, i]], K[0, hh, lo:hi + 1], V[0, hh, lo:hi + 1])[0]
            np.testing.assert_allclose(got[0, hh, i], want, rtol=0, atol=1e-13)


def test_radius_zero_gives_own_value():
    Q, K, V = _case(2, 2, 2, 7)
    for causal in (False, True):
        np.testing.assert_allclose(sdpa_ref(Q, K, V, causal, window=0), V, rtol=0, atol=1e-15)


def test_wide_window_is_no_window():
    Q, K, V = _case(3, 2, 2, 10)
    for causal in (False, True):
        assert np.array_equal(sdpa_ref(Q, K, V, causal, window=9), sdpa_ref(Q, K, V, causal))
        assert np.array_equal(sdpa_ref(Q, K, V, causal, window=1000), sdpa_ref(Q, K, V, causal))


def test_window_weights_are_banded_and_normalised():
    Q, K, _ = _case(4, 1, 3, 12)
    w = sdpa_weights_ref(Q, K, window=2)
    band = np.abs(np.arange(12)[None, :] - np.arange(12)[:, None]) <= 2
    assert np.all(w[..., ~band] == 0.0) and np.all(w[..., band] > 0.0)
    np.testing.assert_allclose(w.sum(axis=-1), 1.0, atol=1e-14)
    assert np.all(np.isfinite(sdpa_lse_ref(Q, K, window=2)))


def test_window_needs_self_attention():
    Q, K, V = _case(5, 1, 1, 4)
    with pytest.raises(ValueError):
        sdpa_ref(Q, K[:, :, :3], V[:, :, :3], window=1)


@pytest.mark.parametrize("causal", [False, True])
def test_window_matches_torch_banded_mask(causal):
    n, w = 13, 3
    Q, K, V = _case(6, 2, 2, n, d=16, dv=8)
    i, j = np.arange(n)[:, None], np.arange(n)[None, :]
    mask = np.abs(i - j) <= w
    if causal:
        mask &= j <= i
    want = torch.nn.functional.scaled_dot_product_attention(torch.tensor(Q), torch.tensor(K), torch.tensor(V),
                                                            attn_mask=torch.tensor(mask)).numpy()
    np.testing.assert_allclose(sdpa_ref(Q, K, V, causal, window=w), want, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_window_backward_equals_central_differences(causal):
    from oracle import sdpa_backward_ref
    n, w = 6, 1
    Q, K, V = _case(7, 1, 1, n, d=4, dv=3)
    dO = np.random.Generator(np.random.PCG64(8)).standard_normal((1, 1, n, 3))
    grads = sdpa_backward_ref(Q, K, V, dO, causal, window=w)

    def loss():
        return float(np.sum(dO * sdpa_ref(Q, K, V, causal, window=w)))

    eps = 1e-5
    for got, x in zip(grads, (Q, K, V)):
        num = np.empty_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + eps
            fp = loss()
            x[idx] = old - eps
            fm = loss()
            x[idx] = old
            num[idx] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(got, num, rtol=0, atol=1e-8)

"""Pins of the oracle's key-padding mask ("Transformer：抛弃循环与卷积的序列建模", section "训练样本": <PAD> positions
that fill a batch are excluded by a padding mask) to facts other than the oracle's own code:
  * a padded batch entry equals attention over its real keys only, computed by the pure-Python literal definition on
    the truncated tensors (and, under the causal mask, rows past the length see exactly the real keys);
  * padding contents never matter (bitwise);
  * the reading for a row with no real key: output 0, log-sum-exp -inf, no gradient;
  * gradients with padding equal central finite differences, padding rows of dK/dV are exactly 0;
  * torch's CPU float64 attention with a boolean key mask agrees.
"""
import math

import numpy as np
import pytest
import torch

from oracle import sdpa_backward_ref, sdpa_brute, sdpa_lse_ref, sdpa_ref, sdpa_weights_ref


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _case(seed, B, h, n_q, n_k, d=8, dv=5):
    r = _rng(seed)
    return (r.standard_normal((B, h, n_q, d)), r.standard_normal((B, h, n_k, d)), r.standard_normal((B, h, n_k, dv)),
            r.standard_normal((B, h, n_q, dv)))


@pytest.mark.parametrize("causal", [False, True])
def test_padding_equals_truncated_brute_force(causal):
    n = 7
    Q, K, V, _ = _case(1, 3, 2, n, n)
    kv_len = np.array([7, 3, 1])
    got = sdpa_ref(Q, K, V, causal, kv_len=kv_len)
    for b, L in enumerate(kv_len):
        for hh in range(2):
            if not causal:
                want = sdpa_brute(Q[b, hh], K[b, hh, :L], V[b, hh, :L])
            else:
                # row i sees keys j <= i with j < L: the causal prefix for i < L, all L real keys for i >= L
                want = [sdpa_brute([Q[b, hh, i]], K[b, hh, :min(i + 1, L)], V[b, hh, :min(i + 1, L)])[0]
                        for i in range(n)]
            np.testing.assert_allclose(got[b, hh], want, rtol=0, atol=1e-13)


def test_padding_contents_do_not_matter():
    Q, K, V, _ = _case(2, 2, 3, 9, 12)
    kv_len = np.array([5, 12])
    K2, V2 = K.copy(), V.copy()
    r = _rng(3)
    K2[0, :, 5:] = r.standard_normal(K2[0, :, 5:].shape) * 1e3
    V2[0, :, 5:] = r.standard_normal(V2[0, :, 5:].shape) * 1e3
    for causal in (False,):
        assert np.array_equal(sdpa_ref(Q, K, V, causal, kv_len=kv_len), sdpa_ref(Q, K2, V2, causal, kv_len=kv_len))
    assert np.array_equal(sdpa_lse_ref(Q, K, kv_len=kv_len), sdpa_lse_ref(Q, K2, kv_len=kv_len))


def test_full_length_is_no_padding():
    Q, K, V, dO = _case(4, 2, 2, 6, 6)
    full = np.array([6, 6])
    for causal in (False, True):
        assert np.array_equal(sdpa_ref(Q, K, V, causal, kv_len=full), sdpa_ref(Q, K, V, causal))
        for a, b in zip(sdpa_backward_ref(Q, K, V, dO, causal, kv_len=full), sdpa_backward_ref(Q, K, V, dO, causal)):
            assert np.array_equal(a, b)


def test_empty_rows_reading():
    Q, K, V, dO = _case(5, 2, 2, 4, 6)
    kv_len = np.array([0, 3])
    out = sdpa_ref(Q, K, V, kv_len=kv_len)
    assert np.all(out[0] == 0.0) and np.all(np.isfinite(out))
    assert np.all(sdpa_weights_ref(Q, K, kv_len=kv_len)[0] == 0.0)
    assert np.all(np.isneginf(sdpa_lse_ref(Q, K, kv_len=kv_len)[0]))
    dQ, dK, dV = sdpa_backward_ref(Q, K, V, dO, kv_len=kv_len)
    assert np.all(dQ[0] == 0.0) and np.all(dK[0] == 0.0) and np.all(dV[0] == 0.0)


def test_weights_rows_sum_to_one_over_real_keys():
    Q, K, _, _ = _case(6, 3, 2, 5, 10)
    kv_len = np.array([10, 4, 1])
    w = sdpa_weights_ref(Q, K, kv_len=kv_len)
    for b, L in enumerate(kv_len):
        np.testing.assert_allclose(w[b].sum(axis=-1), 1.0, atol=1e-14)
        assert np.all(w[b, :, :, L:] == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_padded_backward_equals_central_differences(causal):
    Q, K, V, dO = _case(7, 2, 1, 5, 5, d=4, dv=3)
    kv_len = np.array([3, 5])
    dQ, dK, dV = sdpa_backward_ref(Q, K, V, dO, causal, kv_len=kv_len)

    def loss():
        return float(np.sum(dO * sdpa_ref(Q, K, V, causal, kv_len=kv_len)))

    eps = 1e-5
    for got, x in ((dQ, Q), (dK, K), (dV, V)):
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
    assert np.all(dK[0, :, 3:] == 0.0) and np.all(dV[0, :, 3:] == 0.0)


def test_padded_lse_matches_log_of_real_keys():
    Q, K, _, _ = _case(8, 2, 1, 4, 6, d=16)
    kv_len = np.array([2, 6])
    lse = sdpa_lse_ref(Q, K, kv_len=kv_len)
    for b, L in enumerate(kv_len):
        s = Q[b, 0] @ K[b, 0, :L].T / 4.0
        want = [math.log(math.fsum(math.exp(x) for x in row)) for row in s]
        np.testing.assert_allclose(lse[b, 0], want, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_padding_matches_torch_masked_sdpa(causal):
    n = 11
    Q, K, V, dO = _case(9, 3, 2, n, n, d=16, dv=8)
    kv_len = np.array([11, 6, 2])
    allowed = np.arange(n)[None, :] < kv_len[:, None]                       # [B, n_k]
    mask = np.broadcast_to(allowed[:, None, None, :], (3, 1, n, n)).copy()
    if causal:
        mask &= np.tril(np.ones((n, n), bool))[None, None]
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (Q, K, V))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.tensor(mask))
    out.backward(torch.tensor(dO))
    np.testing.assert_allclose(sdpa_ref(Q, K, V, causal, kv_len=kv_len), out.detach().numpy(), atol=1e-12)
    for got, t in zip(sdpa_backward_ref(Q, K, V, dO, causal, kv_len=kv_len), (tq, tk, tv)):
        np.testing.assert_allclose(got, t.grad.numpy(), atol=1e-12)

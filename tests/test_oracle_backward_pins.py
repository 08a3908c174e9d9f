"""Pins of the oracle's backward pass and row log-sum-exp to facts other than the oracle's own formulas.

The backward pass is the derivative of the forward function ("Transformer：抛弃循环与卷积的序列建模", section
"训练样本", subsection "反向传播": the loss is carried back through attention by the chain rule). What fixes it here:
  * central finite differences of the forward oracle (itself pinned in test_oracle_pins.py): an independent way to
    get the same derivative, which catches any dropped term, wrong sign, wrong scale or transposed operand;
  * identities that follow from the forward definition: a shift of every key leaves the weights unchanged (so the
    key gradients sum to zero), rows of the weights sum to one (so the value gradients sum to the upstream gradient),
    and scaling Q by a while scaling K by 1/a leaves the scores unchanged (so sum_i dQ_i.Q_i = sum_j dK_j.K_j);
  * closed forms (two keys; all queries zero) and the causal mask's dependence structure;
  * torch's CPU float64 autograd of its own attention routine, and scipy's logsumexp, as library cross-checks.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import sdpa_backward_head, sdpa_backward_ref, sdpa_lse_ref, sdpa_ref, sdpa_weights_ref


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _case(seed, B, h, n_q, n_k, d_k, d_v, scale=1.0):
    r = _rng(seed)
    return (r.standard_normal((B, h, n_q, d_k)) * scale, r.standard_normal((B, h, n_k, d_k)),
            r.standard_normal((B, h, n_k, d_v)), r.standard_normal((B, h, n_q, d_v)))


def _numeric_grad(f, x, eps=1e-5):
    """Central differences of the scalar f at x, element by element."""
    g = np.empty_like(x)
    for idx in np.ndindex(*x.shape):
        old = x[idx]
        x[idx] = old + eps
        fp = f()
        x[idx] = old - eps
        fm = f()
        x[idx] = old
        g[idx] = (fp - fm) / (2 * eps)
    return g


@pytest.mark.parametrize("causal,n_q,n_k,d_k,d_v,seed", [
    (False, 3, 5, 4, 3, 1), (False, 4, 2, 6, 5, 2), (True, 4, 4, 4, 3, 3), (True, 6, 6, 3, 2, 4),
    (False, 1, 1, 4, 4, 5)])
def test_backward_equals_central_differences(causal, n_q, n_k, d_k, d_v, seed):
    Q, K, V, dO = _case(seed, 1, 2, n_q, n_k, d_k, d_v)
    dQ, dK, dV = sdpa_backward_ref(Q, K, V, dO, causal)

    def loss():
        return float(np.sum(dO * sdpa_ref(Q, K, V, causal)))

    for got, x in ((dQ, Q), (dK, K), (dV, V)):
        num = _numeric_grad(loss, x)
        np.testing.assert_allclose(got, num, rtol=0, atol=1e-8)


def test_backward_of_large_scores_equals_central_differences():
    # scores of order +-20: the softmax is nearly one-hot and the gradients are tiny but must still be right
    Q, K, V, dO = _case(11, 1, 1, 3, 4, 4, 2, scale=10.0)
    dQ, dK, dV = sdpa_backward_ref(Q, K, V, dO)

    def loss():
        return float(np.sum(dO * sdpa_ref(Q, K, V)))

    for got, x in ((dQ, Q), (dK, K), (dV, V)):
        np.testing.assert_allclose(got, _numeric_grad(loss, x, eps=1e-6), rtol=0, atol=1e-7)


@pytest.mark.parametrize("causal", [False, True])
def test_key_gradients_sum_to_zero(causal):
    # adding u to every key adds q_i.u / sqrt(d_k) to a whole row of scores: the weights do not change
    Q, K, V, dO = _case(21, 2, 3, 9, 9, 8, 5)
    _, dK, _ = sdpa_backward_ref(Q, K, V, dO, causal)
    np.testing.assert_allclose(dK.sum(axis=-2), 0.0, atol=1e-12)


@pytest.mark.parametrize("causal,n_q,n_k", [(False, 7, 11), (True, 9, 9)])
def test_value_gradients_sum_to_upstream_gradient(causal, n_q, n_k):
    # O_i = sum_j W_ij V_j with sum_j W_ij = 1: adding u to every value adds u to every output row
    Q, K, V, dO = _case(22, 2, 2, n_q, n_k, 8, 5)
    _, _, dV = sdpa_backward_ref(Q, K, V, dO, causal)
    np.testing.assert_allclose(dV.sum(axis=-2), dO.sum(axis=-2), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_query_key_rescaling_balance(causal):
    # S depends on Q and K only through Q K^T: scaling Q by a and K by 1/a changes nothing, so
    # d/da [L(aQ, K/a)] at a = 1 is sum_i dQ_i.Q_i - sum_j dK_j.K_j = 0
    Q, K, V, dO = _case(23, 1, 3, 8, 8, 6, 4)
    dQ, dK, _ = sdpa_backward_ref(Q, K, V, dO, causal)
    lhs = np.einsum("bhid,bhid->bh", dQ, Q)
    rhs = np.einsum("bhjd,bhjd->bh", dK, K)
    np.testing.assert_allclose(lhs, rhs, atol=1e-12)
    assert np.abs(lhs).max() > 1e-3  # not trivially zero


def test_two_keys_closed_form():
    # q = (8, 0, ...), k1 = 0, k2 = e1 with d_k = 64: scores (0, 1), weights (1 - s, s) with s = sigmoid(1);
    # dV_j = W_j dO; dS_2 = s(1-s) dO.(v2 - v1) = -dS_1; dq = dS_2 e1 / 8; dk_j = dS_j q / 8
    d = 64
    q = np.zeros((1, d)); q[0, 0] = 8.0
    k = np.zeros((2, d)); k[1, 0] = 1.0
    r = _rng(24)
    v = r.standard_normal((2, 5))
    do = r.standard_normal((1, 5))
    dq, dk, dv = sdpa_backward_head(q, k, v, do)
    s = 1.0 / (1.0 + math.exp(-1.0))
    ds2 = s * (1 - s) * float(do[0] @ (v[1] - v[0]))
    np.testing.assert_allclose(dv, np.array([[1 - s], [s]]) * do, atol=1e-15)
    want_dq = np.zeros((1, d)); want_dq[0, 0] = ds2 / 8.0
    np.testing.assert_allclose(dq, want_dq, atol=1e-15)
    np.testing.assert_allclose(dk, np.stack([-ds2 * q[0] / 8.0, ds2 * q[0] / 8.0]), atol=1e-15)


def test_zero_queries_closed_form():
    # Q = 0: every weight is 1/n_k, so dV_j = mean over... = (1/n_k) sum_i dO_i, dK = 0, and
    # dQ_i = (1 / (n_k sqrt(d_k))) sum_j (dO_i.(v_j - vbar)) k_j
    n_q, n_k, d_k, d_v = 5, 7, 16, 6
    r = _rng(25)
    q = np.zeros((n_q, d_k))
    k = r.standard_normal((n_k, d_k))
    v = r.standard_normal((n_k, d_v))
    do = r.standard_normal((n_q, d_v))
    dq, dk, dv = sdpa_backward_head(q, k, v, do)
    np.testing.assert_allclose(dv, np.tile(do.sum(axis=0) / n_k, (n_k, 1)), atol=1e-14)
    assert np.all(dk == 0.0)
    vc = v - v.mean(axis=0)
    want = np.array([[sum(float(do[i] @ vc[j]) * k[j, t] for j in range(n_k)) for t in range(d_k)]
                     for i in range(n_q)]) / (n_k * math.sqrt(d_k))
    np.testing.assert_allclose(dq, want, atol=1e-14)


def test_causal_gradient_dependence():
    # dQ_i uses keys/values j <= i only; dK_j and dV_j use query rows i >= j only
    n, t = 10, 6
    Q, K, V, dO = _case(26, 1, 2, n, n, 8, 4)
    dQ, dK, dV = sdpa_backward_ref(Q, K, V, dO, True)
    r = _rng(27)
    K2, V2 = K.copy(), V.copy()
    K2[..., t:, :] = r.standard_normal(K2[..., t:, :].shape)
    V2[..., t:, :] = r.standard_normal(V2[..., t:, :].shape)
    dQ2, _, _ = sdpa_backward_ref(Q, K2, V2, dO, True)
    assert np.array_equal(dQ2[..., :t, :], dQ[..., :t, :])
    Q3, dO3 = Q.copy(), dO.copy()
    Q3[..., :t, :] = r.standard_normal(Q3[..., :t, :].shape)
    dO3[..., :t, :] = r.standard_normal(dO3[..., :t, :].shape)
    _, dK3, dV3 = sdpa_backward_ref(Q3, K, V, dO3, True)
    assert np.array_equal(dK3[..., t:, :], dK[..., t:, :])
    assert np.array_equal(dV3[..., t:, :], dV[..., t:, :])
    # and the causal gradients differ from the unmasked ones (negative control)
    dQu, _, _ = sdpa_backward_ref(Q, K, V, dO, False)
    assert np.abs(dQu - dQ).max() > 1e-3


@pytest.mark.parametrize("causal,n_q,n_k", [(False, 9, 13), (True, 12, 12), (False, 1, 5)])
def test_backward_matches_torch_autograd_float64(causal, n_q, n_k):
    Q, K, V, dO = _case(28, 2, 2, n_q, n_k, 16, 8)
    dQ, dK, dV = sdpa_backward_ref(Q, K, V, dO, causal)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (Q, K, V))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
    out.backward(torch.tensor(dO, dtype=torch.float64))
    for got, t in ((dQ, tq), (dK, tk), (dV, tv)):
        np.testing.assert_allclose(got, t.grad.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal,n_q,n_k", [(False, 9, 13), (True, 12, 12)])
def test_lse_matches_scipy_logsumexp(causal, n_q, n_k):
    Q, K, _, _ = _case(29, 2, 3, n_q, n_k, 16, 8, scale=3.0)
    s = np.einsum("bhid,bhjd->bhij", Q, K) / 4.0
    if causal:
        s = np.where(np.arange(n_k)[None, :] > np.arange(n_q)[:, None], -np.inf, s)
    np.testing.assert_allclose(sdpa_lse_ref(Q, K, causal), scipy.special.logsumexp(s, axis=-1), rtol=0,
                               atol=1e-12)
    # the weights are exp(s - lse)
    w = np.exp(s - sdpa_lse_ref(Q, K, causal)[..., None])
    np.testing.assert_allclose(w, sdpa_weights_ref(Q, K, causal), rtol=0, atol=1e-14)


def test_lse_closed_forms():
    # one key: lse = its score; n equal scores s: lse = s + log n; causal row 0 sees key 0 only
    q = np.full((1, 1, 1, 4), 2.0)
    k = np.ones((1, 1, 1, 4))
    assert sdpa_lse_ref(q, k)[0, 0, 0] == pytest.approx(4.0, abs=1e-15)  # 2*4 / sqrt(4)
    k5 = np.ones((1, 1, 5, 4))
    assert sdpa_lse_ref(q, k5)[0, 0, 0] == pytest.approx(4.0 + math.log(5.0), abs=1e-14)
    qc = np.zeros((1, 1, 5, 4))
    lse = sdpa_lse_ref(qc, np.zeros((1, 1, 5, 4)), causal=True)[0, 0]
    np.testing.assert_allclose(lse, np.log(np.arange(1, 6)), atol=1e-15)

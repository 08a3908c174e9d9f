"""Pins of the float64 oracle against facts the pages and the mathematics fix (CPU only).

Each test names the passage it follows. Together they are chosen so that a plausible slip in the oracle (a missing
or wrong 1/sqrt(d_k), a softmax over the wrong axis, a mask in the wrong direction or without the diagonal, a missing
max shift, a wrong head column block, a wrong concat order, a missing W^O, Xq and Xkv swapped) fails at least one.
"""
import math
from pathlib import Path

import numpy as np
import pytest
import torch

from oracle import mha_ref, sdpa_brute, sdpa_ref, sdpa_weights_ref

GOLDEN = Path(__file__).parent / "golden"


def _golden(name):
    rows = [ln.split() for ln in (GOLDEN / name).read_text().splitlines() if ln.strip() and not ln.startswith("#")]
    return rows


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# --- softmax weights are a normalised distribution over the keys --------------------------------------------------
# "Transformer：抛弃循环与卷积的序列建模", section "Scaled Dot-Product Attention": after the softmax every query has a
# set of normalised weights, and the output is the weighted sum of the values.

# causal is defined only for n_q == n_k, so the rectangular shape runs unmasked only
@pytest.mark.parametrize("causal,n_q,n_k,d", [(c, n, n, d) for c in (False, True)
                                              for n, d in ((1, 64), (7, 16), (33, 64))] + [(False, 5, 19, 8)])
def test_rows_sum_to_one(causal, n_q, n_k, d):
    r = _rng(1)
    w = sdpa_weights_ref(r.standard_normal((2, 3, n_q, d)), r.standard_normal((2, 3, n_k, d)), causal=causal)
    assert np.all(w >= 0)
    np.testing.assert_allclose(w.sum(-1), 1.0, rtol=0, atol=1e-14)


# --- causal mask --------------------------------------------------------------------------------------------------
# Same page, section "Transformer 中的三种 Attention": future scores are set to -inf before the softmax, so their
# weight is 0; the training example's matrix M (section "训练样本") lets position i read positions <= i, itself
# included.

def test_causal_pattern_equals_printed_mask():
    m = np.array(_golden("causal_mask_n4.txt"), dtype=int)
    r = _rng(2)
    w = sdpa_weights_ref(r.standard_normal((4, 64)), r.standard_normal((4, 64)), causal=True)
    assert np.array_equal((w > 0).astype(int), m)
    assert np.all(w[m == 0] == 0.0)


@pytest.mark.parametrize("n", [1, 2, 37, 130])
def test_causal_future_weights_exactly_zero(n):
    r = _rng(3)
    w = sdpa_weights_ref(r.standard_normal((2, n, 64)), r.standard_normal((2, n, 64)), causal=True)
    j, i = np.meshgrid(np.arange(n), np.arange(n))
    assert np.all(w[:, j > i] == 0.0)
    assert np.all(w[:, j <= i] > 0.0)


def test_causal_output_ignores_future_rows():
    r = _rng(4)
    q, k, v = (r.standard_normal((40, 64)) for _ in range(3))
    o = sdpa_ref(q, k, v, causal=True)
    k2, v2 = k.copy(), v.copy()
    k2[25:] = r.standard_normal((15, 64)) * 5
    v2[25:] = r.standard_normal((15, 64)) * 5
    o2 = sdpa_ref(q, k2, v2, causal=True)
    assert np.array_equal(o[:25], o2[:25])
    assert not np.allclose(o[25:], o2[25:])


def test_causal_requires_equal_lengths():
    with pytest.raises(ValueError):
        sdpa_ref(np.zeros((3, 8)), np.zeros((4, 8)), np.zeros((4, 8)), causal=True)


def test_q_index_selects_true_positions():
    r = _rng(5)
    q, k, v = (r.standard_normal((2, 50, 64)) for _ in range(3))
    rows = np.array([0, 7, 31, 49])
    full = sdpa_ref(q, k, v, causal=True)
    part = sdpa_ref(q[:, rows], k, v, causal=True, q_index=rows)
    np.testing.assert_allclose(part, full[:, rows], rtol=0, atol=1e-15)


# --- closed forms -----------------------------------------------------------------------------------------------

def test_identical_keys_give_mean_of_values():
    # all scores of a row are equal -> uniform weights -> the plain mean of V (prefix mean under the causal mask)
    r = _rng(6)
    q = r.standard_normal((9, 64))
    k = np.tile(r.standard_normal((1, 64)), (9, 1))
    v = r.standard_normal((9, 64))
    np.testing.assert_allclose(sdpa_ref(q, k, v), np.tile(v.mean(0), (9, 1)), rtol=0, atol=1e-14)
    prefix = np.cumsum(v, 0) / np.arange(1, 10)[:, None]
    np.testing.assert_allclose(sdpa_ref(q, k, v, causal=True), prefix, rtol=0, atol=1e-14)


def test_single_key_returns_its_value():
    r = _rng(7)
    q = r.standard_normal((5, 64)) * 10
    k = r.standard_normal((1, 64))
    v = r.standard_normal((1, 64))
    assert np.array_equal(sdpa_ref(q, k, v), np.tile(v, (5, 1)))


def test_two_keys_closed_form_pins_the_scale():
    # q = 8 e_0 with d_k = 64: scores are q.k / sqrt(64) = (0, 1) -> weights (1/(1+e), e/(1+e)).
    # Dividing by d_k instead of sqrt(d_k) would give scores (0, 1/8) and fail.
    q = np.zeros((1, 64)); q[0, 0] = 8.0
    k = np.zeros((2, 64)); k[1, 0] = 1.0
    w = sdpa_weights_ref(q, k)[0]
    np.testing.assert_allclose(w, [1 / (1 + math.e), math.e / (1 + math.e)], rtol=0, atol=1e-16)
    np.testing.assert_allclose(w, [0.2689414213699951, 0.7310585786300049], rtol=0, atol=1e-16)


def test_printed_three_token_weights():
    # Scores ln(0.30), ln(0.20), ln(0.50) give exactly the weights of the page's encoder example, and the output is
    # 0.30 v1 + 0.20 v2 + 0.50 v3.
    w_gold = np.array(_golden("weights_example_3tok.txt")[0], dtype=np.float64)
    q = np.zeros((1, 64)); q[0, 0] = 8.0                # sqrt(64) = 8 cancels the scale
    k = np.zeros((3, 64)); k[:, 0] = np.log(w_gold)
    v = _rng(8).standard_normal((3, 64))
    np.testing.assert_allclose(sdpa_weights_ref(q, k)[0], w_gold, rtol=0, atol=1e-15)
    np.testing.assert_allclose(sdpa_ref(q, k, v)[0], w_gold @ v, rtol=0, atol=1e-14)


def test_causal_zero_scores_give_prefix_means():
    # Q = K = 0 with the mask: W = [[1,0,0,0],[1/2,1/2,0,0],[1/3,1/3,1/3,0],[1/4,1/4,1/4,1/4]]
    w = sdpa_weights_ref(np.zeros((4, 64)), np.zeros((4, 64)), causal=True)
    expect = np.tril(np.ones((4, 4))) / np.arange(1, 5)[:, None]
    np.testing.assert_allclose(w, expect, rtol=0, atol=1e-16)


def test_large_scores_stay_finite():
    # scores (1000, 1001): e^1000 overflows float64, so only the max-shifted softmax gets (1/(1+e), e/(1+e))
    q = np.zeros((1, 64)); q[0, 0] = 8.0
    k = np.zeros((2, 64)); k[0, 0] = 1000.0; k[1, 0] = 1001.0
    w = sdpa_weights_ref(q, k)[0]
    np.testing.assert_allclose(w, [1 / (1 + math.e), math.e / (1 + math.e)], rtol=0, atol=1e-15)


# --- brute force on tiny inputs ------------------------------------------------------------------------------------

@pytest.mark.parametrize("causal,n_q,n_k,d_k,d_v,scale",
                         [(c,) + shape for c in (False, True)
                          for shape in ((1, 1, 4, 4, 1.0), (3, 3, 8, 5, 1.0), (6, 6, 16, 16, 3.0), (8, 8, 8, 8, 10.0))]
                         + [(False, 4, 7, 4, 6, 1.0)])
def test_against_pure_python_brute_force(causal, n_q, n_k, d_k, d_v, scale):
    r = _rng(9)
    q = r.standard_normal((n_q, d_k)) * scale
    k = r.standard_normal((n_k, d_k)) * scale
    v = r.standard_normal((n_k, d_v))
    np.testing.assert_allclose(sdpa_ref(q, k, v, causal=causal), np.array(sdpa_brute(q, k, v, causal)),
                               rtol=1e-12, atol=1e-13)


# --- invariances ---------------------------------------------------------------------------------------------------
# "Transformer 为什么抛弃循环网络", section "没有循环，顺序从哪里来": self-attention does not see word order; swapping
# inputs without position information is invisible to it.

def test_self_attention_is_permutation_equivariant():
    r = _rng(10)
    x = r.standard_normal((2, 3, 20, 64))
    perm = r.permutation(20)
    o = sdpa_ref(x, x * 0.5, x[..., ::-1])
    xp = x[:, :, perm]
    op = sdpa_ref(xp, xp * 0.5, xp[..., ::-1])
    np.testing.assert_allclose(op, o[:, :, perm], rtol=0, atol=1e-13)


def test_key_value_permutation_invariance():
    r = _rng(11)
    q, k, v = r.standard_normal((12, 64)), r.standard_normal((17, 64)), r.standard_normal((17, 64))
    perm = r.permutation(17)
    np.testing.assert_allclose(sdpa_ref(q, k[perm], v[perm]), sdpa_ref(q, k, v), rtol=0, atol=1e-13)


def test_causal_breaks_permutation_equivariance():
    # negative control: the mask ties outputs to positions
    r = _rng(12)
    x = r.standard_normal((10, 64))
    perm = np.roll(np.arange(10), 3)
    o = sdpa_ref(x, x, x, causal=True)
    assert not np.allclose(sdpa_ref(x[perm], x[perm], x[perm], causal=True), o[perm])


def test_mha_self_attention_permutation_equivariant():
    r = _rng(13)
    d_model, h = 64, 8
    x = r.standard_normal((2, 11, d_model))
    ws = [r.standard_normal((d_model, d_model)) / 8 for _ in range(4)]
    perm = r.permutation(11)
    o = mha_ref(x, x, *ws, h=h)
    np.testing.assert_allclose(mha_ref(x[:, perm], x[:, perm], *ws, h=h), o[:, perm], rtol=0, atol=1e-13)


def test_shift_of_all_keys_leaves_output_unchanged():
    # adding the same u to every key adds q.u/sqrt(d_k) to a whole row of scores, which the softmax cancels
    r = _rng(14)
    q, k, v = r.standard_normal((9, 64)), r.standard_normal((13, 64)), r.standard_normal((13, 64))
    u = r.standard_normal(64) * 3
    np.testing.assert_allclose(sdpa_ref(q, k + u, v), sdpa_ref(q, k, v), rtol=0, atol=1e-12)


def test_output_is_affine_in_values():
    r = _rng(15)
    q, k, v = r.standard_normal((9, 64)), r.standard_normal((13, 64)), r.standard_normal((13, 64))
    for causal in (False,):
        o = sdpa_ref(q, k, v, causal)
        np.testing.assert_allclose(sdpa_ref(q, k, 2.5 * v - 0.75, causal), 2.5 * o - 0.75, rtol=0, atol=1e-13)


# --- library routines (float64 on the CPU) ------------------------------------------------------------------------

@pytest.mark.parametrize("causal,n_q,n_k", [(c, n, n) for c in (False, True) for n in (16, 65)] + [(False, 20, 37)])
def test_sdpa_matches_torch_cpu_float64(causal, n_q, n_k):
    r = _rng(16)
    q, k, v = r.standard_normal((2, 4, n_q, 64)), r.standard_normal((2, 4, n_k, 64)), r.standard_normal((2, 4, n_k, 64))
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k),
                                                           torch.from_numpy(v), is_causal=causal).numpy()
    np.testing.assert_allclose(sdpa_ref(q, k, v, causal), ref, rtol=0, atol=1e-12)


def _torch_mha(xq, xkv, wq, wk, wv, wo, h, causal):
    # torch's weights are [out, in] and its sequences come first: q = x @ Wq^T, so pass the transposes.
    tq, tkv = torch.from_numpy(xq).transpose(0, 1), torch.from_numpy(xkv).transpose(0, 1)
    mask = None
    if causal:
        n = xq.shape[1]
        mask = torch.triu(torch.full((n, n), float("-inf"), dtype=torch.float64), diagonal=1)
    d_model = xq.shape[-1]
    out, _ = torch.nn.functional.multi_head_attention_forward(
        tq, tkv, tkv, d_model, h, None, None, None, None, False, 0.0,
        torch.from_numpy(wo.T.copy()), None, training=False, need_weights=False, attn_mask=mask,
        use_separate_proj_weight=True, q_proj_weight=torch.from_numpy(wq.T.copy()),
        k_proj_weight=torch.from_numpy(wk.T.copy()), v_proj_weight=torch.from_numpy(wv.T.copy()))
    return out.transpose(0, 1).numpy()


@pytest.mark.parametrize("causal,cross", [(False, False), (True, False), (False, True)])
@pytest.mark.parametrize("d_model,h,n_q,n_k", [(64, 8, 9, 9), (512, 8, 12, 12), (128, 2, 5, 13)])
def test_mha_matches_torch_cpu_float64(causal, cross, d_model, h, n_q, n_k):
    if not cross:
        n_k = n_q
    r = _rng(17)
    xq = r.standard_normal((3, n_q, d_model))
    xkv = r.standard_normal((3, n_k, d_model)) if cross else xq
    ws = [r.standard_normal((d_model, d_model)) / math.sqrt(d_model) for _ in range(4)]
    np.testing.assert_allclose(mha_ref(xq, xkv, *ws, h=h, causal=causal), _torch_mha(xq, xkv, *ws, h, causal),
                               rtol=0, atol=1e-12)


def test_mha_concat_order_closed_form():
    # Wq = Wk = 0 makes every weight uniform, so head i = mean_j (X Wv)_j restricted to its columns. With Wv = I the
    # in-order concat is mean_j X_j itself, and the output is mean_j X_j Wo; a permuted head order would not be.
    r = _rng(18)
    d_model, h = 512, 8
    x = r.standard_normal((2, 6, d_model))
    wo = r.standard_normal((d_model, d_model))
    z = np.zeros((d_model, d_model))
    out = mha_ref(x, x, z, z, np.eye(d_model), wo, h=h)
    np.testing.assert_allclose(out, np.broadcast_to(x.mean(1, keepdims=True) @ wo, out.shape), rtol=0, atol=1e-11)


def test_mha_single_full_width_head_is_plain_attention():
    # h = 1, d_k = d_model: MultiHead reduces to one attention over the projected inputs followed by W^O
    r = _rng(19)
    x = r.standard_normal((1, 7, 32))
    wq, wk, wv, wo = (r.standard_normal((32, 32)) / 6 for _ in range(4))
    brute = np.array(sdpa_brute(x[0] @ wq, x[0] @ wk, x[0] @ wv)) @ wo
    np.testing.assert_allclose(mha_ref(x, x, wq, wk, wv, wo, h=1)[0], brute, rtol=0, atol=1e-12)


def test_base_model_head_sizing():
    dims = {k: int(v) for k, v in _golden("base_model_dims.txt")}
    assert dims["d_k"] == dims["d_model"] // dims["h"] == dims["d_v"]

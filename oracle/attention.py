"""Plain float64 CPU oracle for scaled dot-product attention (forward and backward) and multi-head attention.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench's CPU-baseline leg may import this module.
The library's GPU path never imports, links or calls anything here, and this module imports nothing from it.

Every function is the plain definition written out in float64 with NumPy (matmul, exp, max and sum are the only
library primitives). No blocking, no streaming softmax, no fusion: one head at a time, the full score matrix, then
the row softmax, then the weighted sum of the values.

Sources (web pages about "Attention Is All You Need"):
  * "Attention Is All You Need" (lettle.cn translation), section 3.2.1 Scaled Dot-Product Attention, equation
    Attention(Q,K,V) = softmax(QK^T / sqrt(d_k)) V; section 3.2.2 Multi-Head Attention.
  * "Transformer：抛弃循环与卷积的序列建模" (jiashun-ye.github.io), sections "Scaled Dot-Product Attention",
    "Multi-Head Attention" (head_i = Attention(QW_i^Q, KW_i^K, VW_i^V), MultiHead = Concat(head_1..head_h) W^O),
    "Transformer 中的三种 Attention" (future scores set to -inf before the softmax in decoder self-attention), and
    the training example's mask matrix M (section "训练样本").
  * "Transformer 为什么抛弃循环网络" (treecat.cn), sections "一次注意力计算在做什么" and "为什么需要多头注意力".
  * Backward pass: "Transformer：抛弃循环与卷积的序列建模", section "训练样本", subsection "反向传播": training
    carries the loss back through the attention computation by the chain rule to reach the gradients of W^Q, W^K and
    W^V; the gradients with respect to Q, K and V are the step of that chain that passes through attention.

Readings where the pages leave a step open:
  * The causal mask sets the score of key j for query i to -inf when j > i (the diagonal is allowed), so those
    weights are exactly 0. It is defined only for self-attention, where n_q == n_k; `q_index` lets a caller ask for a
    subset of query rows and still get the mask of their true positions.
  * Subtracting the row max before exp is an exact identity of the softmax, used only to avoid overflow.
  * The backward pass of attention is the exact derivative of the forward function: given an upstream gradient dO
    (the derivative of some loss L with respect to O), it returns dL/dQ, dL/dK and dL/dV, i.e. the gradient of
    L = sum(dO * O) with the forward outputs O treated as a function of Q, K and V.
  * Key padding ("Transformer：抛弃循环与卷积的序列建模", section "训练样本", subsection "反向传播": <PAD> positions
    added to fill a batch of different-length sequences are excluded by a padding mask; section "训练配置",
    "训练数据与 Batching": batches group sequences of similar length). With per-sequence valid key counts kv_len[b],
    keys j >= kv_len[b] of batch b get score -inf (weight exactly 0), like masked future keys. A row left with no key
    it may see (kv_len[b] = 0) has no softmax; its output is read as 0, its log-sum-exp as -inf, and it passes no
    gradient.
  * Restricted self-attention ("Transformer：抛弃循环与卷积的序列建模", section "Self-Attention的优势": each position
    attends only to a neighbourhood of size r, cost O(rnd); section "总结": proposed for very long sequences). Read as
    a band centred on the query: with radius w, query i sees keys j with |i - j| <= w (r = 2w + 1), positions shared
    between queries and keys as in self-attention; with the causal mask as well, keys i - w .. i.
  * The row log-sum-exp of the scaled scores, lse_i = log sum_j exp(s_ij) over the keys the row may see, is the
    statistic a forward pass hands to the backward pass: the weights are then exp(s_ij - lse_i).
  * Projections carry no bias (the attention formulas on the pages have none). The row-vector convention X W is used:
    W_i^Q is the column block i of Wq [d_model, h*d_k]; Concat orders the heads 1..h along the last axis; W^O is
    [h*d_v, d_model].
"""
from __future__ import annotations

import math

import numpy as np


def _as_f64(x):
    return np.asarray(x, dtype=np.float64)


def _causal_disallowed(n_q, n_k, q_index):
    """Boolean [n_q, n_k]: True where key j comes after query position i (j > i)."""
    if q_index is None:
        if n_q != n_k:
            raise ValueError("the causal mask is defined for self-attention only (n_q == n_k)")
        q_index = np.arange(n_q)
    q_index = np.asarray(q_index)
    if q_index.shape != (n_q,):
        raise ValueError("q_index must give one position per query row")
    return np.arange(n_k)[None, :] > q_index[:, None]


def _window_disallowed(n_q, n_k, q_index, window):
    """Boolean [n_q, n_k]: True where key j lies farther than `window` positions from query position i."""
    if q_index is None:
        if n_q != n_k:
            raise ValueError("the restricted (windowed) mask is defined for self-attention only (n_q == n_k)")
        q_index = np.arange(n_q)
    return np.abs(np.arange(n_k)[None, :] - np.asarray(q_index)[:, None]) > window


def _masked_scores(q, k, causal, q_index, n_valid, window=None):
    """Scaled scores q k^T / sqrt(d_k) of one head with -inf where the key may not be seen (after the query under the
    causal mask, at or past n_valid, or farther than `window` positions from the query)."""
    q = _as_f64(q)
    k = _as_f64(k)
    if q.ndim != 2 or k.ndim != 2 or q.shape[1] != k.shape[1]:
        raise ValueError("q [n_q, d_k] and k [n_k, d_k] expected")
    s = (q @ k.T) / math.sqrt(q.shape[1])                # dot products divided by sqrt(d_k)
    if causal:
        s = np.where(_causal_disallowed(s.shape[0], s.shape[1], q_index), -np.inf, s)
    if n_valid is not None:
        s[:, max(int(n_valid), 0):] = -np.inf            # padding keys
    if window is not None:
        s = np.where(_window_disallowed(s.shape[0], s.shape[1], q_index, window), -np.inf, s)
    return s


def sdpa_weights_head(q, k, causal=False, q_index=None, n_valid=None, window=None):
    """Attention weights softmax(q k^T / sqrt(d_k)) of one head. q [n_q, d_k], k [n_k, d_k] -> [n_q, n_k].
    `n_valid`: only keys 0 .. n_valid-1 are real (the rest are padding); a row with no key to see gets weights 0.
    `window`: radius of the restricted self-attention (keys farther from the query are not seen)."""
    s = _masked_scores(q, k, causal, q_index, n_valid, window)
    empty = np.isneginf(s).all(axis=1, keepdims=True)    # only possible with padding
    m = np.where(empty, 0.0, s.max(axis=1, keepdims=True))
    e = np.exp(s - m)
    return np.where(empty, 0.0, e / np.where(empty, 1.0, e.sum(axis=1, keepdims=True)))


def sdpa_head(q, k, v, causal=False, q_index=None, n_valid=None, window=None):
    """Output softmax(q k^T / sqrt(d_k)) v of one head. v [n_k, d_v] -> [n_q, d_v]."""
    v = _as_f64(v)
    w = sdpa_weights_head(q, k, causal, q_index, n_valid, window)
    if v.ndim != 2 or v.shape[0] != w.shape[1]:
        raise ValueError("v [n_k, d_v] expected")
    return w @ v


def _per_head(fn, Q, *rest, **kw):
    Q = _as_f64(Q)
    lead = Q.shape[:-2]
    rest = [_as_f64(r) for r in rest]
    for r in rest:
        if r.shape[:-2] != lead:
            raise ValueError("leading (batch, head) dimensions differ")
    outs = None
    for idx in np.ndindex(*lead):
        o = fn(Q[idx], *[r[idx] for r in rest], **kw)
        if outs is None:
            outs = np.empty(lead + o.shape, dtype=np.float64)
        outs[idx] = o
    return outs


def _per_batch_head(fn, kv_len, Q, *rest, **kw):
    """fn over [B, h, ...] tensors with the padding length of batch b passed as n_valid."""
    Q = _as_f64(Q)
    if Q.ndim != 4:
        raise ValueError("kv_len needs [B, h, n, d] tensors")
    kv_len = np.asarray(kv_len)
    if kv_len.shape != (Q.shape[0],):
        raise ValueError("kv_len must give one length per batch entry")
    rest = [_as_f64(r) for r in rest]
    outs = None
    for b in range(Q.shape[0]):
        for hh in range(Q.shape[1]):
            o = fn(Q[b, hh], *[r[b, hh] for r in rest], n_valid=int(kv_len[b]), **kw)
            if outs is None:
                outs = np.empty(Q.shape[:2] + np.shape(o), dtype=np.float64)
            outs[b, hh] = o
    return outs


def sdpa_weights_ref(Q, K, causal=False, q_index=None, kv_len=None, window=None):
    """Attention weights for every leading (batch, head) index. Q [..., n_q, d_k], K [..., n_k, d_k].
    `kv_len` [B] (with [B, h, n, d] tensors): keys j >= kv_len[b] of batch b are padding; `window`: radius of the
    restricted self-attention."""
    if kv_len is not None:
        return _per_batch_head(sdpa_weights_head, kv_len, Q, K, causal=causal, q_index=q_index, window=window)
    return _per_head(sdpa_weights_head, Q, K, causal=causal, q_index=q_index, window=window)


def sdpa_ref(Q, K, V, causal=False, q_index=None, kv_len=None, window=None):
    """Scaled dot-product attention, head by head. Q [..., n_q, d_k], K [..., n_k, d_k], V [..., n_k, d_v].
    `kv_len` [B] (with [B, h, n, d] tensors): keys j >= kv_len[b] of batch b are padding. `window`: radius of the
    restricted self-attention."""
    if kv_len is not None:
        return _per_batch_head(sdpa_head, kv_len, Q, K, V, causal=causal, q_index=q_index, window=window)
    return _per_head(sdpa_head, Q, K, V, causal=causal, q_index=q_index, window=window)


def mha_ref(Xq, Xkv, Wq, Wk, Wv, Wo, h, causal=False, kv_len=None):
    """Multi-head attention: Concat(head_1..head_h) W^O with head_i = Attention(Xq W_i^Q, Xkv W_i^K, Xkv W_i^V).

    Xq [B, n_q, d_model], Xkv [B, n_k, d_model]; Wq, Wk [d_model, h*d_k]; Wv [d_model, h*d_v]; Wo [h*d_v, d_model].
    Each head projects from the full d_model-wide input with its own column block of the weight matrices.
    `kv_len` [B]: keys (positions of Xkv) at or past kv_len[b] are padding.
    """
    Xq, Xkv, Wq, Wk, Wv, Wo = (_as_f64(a) for a in (Xq, Xkv, Wq, Wk, Wv, Wo))
    if Wq.shape[1] % h or Wv.shape[1] % h:
        raise ValueError("projection widths must be multiples of h")
    d_k = Wq.shape[1] // h
    d_v = Wv.shape[1] // h
    heads = []
    for i in range(h):
        qi = Xq @ Wq[:, i * d_k:(i + 1) * d_k]
        ki = Xkv @ Wk[:, i * d_k:(i + 1) * d_k]
        vi = Xkv @ Wv[:, i * d_v:(i + 1) * d_v]
        heads.append(sdpa_ref(qi[:, None], ki[:, None], vi[:, None], causal=causal, kv_len=kv_len)[:, 0])
    concat = np.concatenate(heads, axis=-1)              # head 1 first, along the feature axis
    return concat @ Wo


def sdpa_brute(q, k, v, causal=False):
    """Pure-Python literal definition for one small head, with no max shift: weight_ij = e^{s_ij} / sum_j e^{s_ij}.

    q, k, v are nested lists (or arrays) [n][d]. Only for tiny cases with moderate scores (e^s must not overflow).
    Masked positions (j > i under the causal mask) get weight exactly 0 (e^{-inf} = 0).
    """
    q = [[float(x) for x in row] for row in q]
    k = [[float(x) for x in row] for row in k]
    v = [[float(x) for x in row] for row in v]
    d_k = len(q[0])
    n_k = len(k)
    if causal and len(q) != n_k:
        raise ValueError("the causal mask is defined for self-attention only (n_q == n_k)")
    out = []
    for i, qi in enumerate(q):
        e = []
        for j in range(n_k):
            if causal and j > i:
                e.append(0.0)
                continue
            s = math.fsum(qi[t] * k[j][t] for t in range(d_k)) / math.sqrt(d_k)
            e.append(math.exp(s))
        total = math.fsum(e)
        out.append([math.fsum(e[j] * v[j][c] for j in range(n_k)) / total for c in range(len(v[0]))])
    return out


def sdpa_lse_head(q, k, causal=False, q_index=None, n_valid=None, window=None):
    """Row log-sum-exp of the scaled scores of one head: lse_i = log sum_j exp(q_i . k_j / sqrt(d_k)) over the keys
    query i may see (natural log; -inf for a row with none). q [n_q, d_k], k [n_k, d_k] -> [n_q]."""
    s = _masked_scores(q, k, causal, q_index, n_valid, window)
    empty = np.isneginf(s).all(axis=1)
    m = np.where(empty, 0.0, s.max(axis=1))              # the max shift again only avoids overflow
    with np.errstate(divide="ignore"):
        return np.where(empty, -np.inf, m + np.log(np.exp(s - m[:, None]).sum(axis=1)))


def sdpa_lse_ref(Q, K, causal=False, q_index=None, kv_len=None, window=None):
    """Row log-sum-exp for every leading (batch, head) index. Q [..., n_q, d_k], K [..., n_k, d_k] -> [..., n_q]."""
    fn = lambda q, k, **kw: sdpa_lse_head(q, k, **kw)[:, None]  # noqa: E731
    if kv_len is not None:
        return _per_batch_head(fn, kv_len, Q, K, causal=causal, q_index=q_index, window=window)[..., 0]
    return _per_head(fn, Q, K, causal=causal, q_index=q_index, window=window)[..., 0]


def sdpa_backward_head(q, k, v, dout, causal=False, q_index=None, n_valid=None, window=None):
    """Gradients (dq, dk, dv) of L = sum(dout * O) for one head, O = softmax(q k^T / sqrt(d_k)) v.

    The chain rule through the three steps of the forward pass, from the output back:
      * O = W v:        dL/dv = W^T dout and dL/dW = dout v^T;
      * W_i = softmax(S_i) row by row: the Jacobian of a softmax row is diag(W_i) - W_i^T W_i, so
                        dL/dS_ij = W_ij (dL/dW_ij - sum_t W_it dL/dW_it);
      * S = q k^T / sqrt(d_k): dL/dq = (dL/dS) k / sqrt(d_k) and dL/dk = (dL/dS)^T q / sqrt(d_k).
    Masked scores have W_ij = 0, so their dL/dS_ij is 0 and they pass no gradient.
    q [n_q, d_k], k [n_k, d_k], v [n_k, d_v], dout [n_q, d_v].
    """
    v = _as_f64(v)
    dout = _as_f64(dout)
    w = sdpa_weights_head(q, k, causal, q_index, n_valid, window)
    if v.ndim != 2 or v.shape[0] != w.shape[1] or dout.shape != (w.shape[0], v.shape[1]):
        raise ValueError("v [n_k, d_v] and dout [n_q, d_v] expected")
    q = _as_f64(q)
    k = _as_f64(k)
    d_k = q.shape[1]
    dv = w.T @ dout
    dw = dout @ v.T
    ds = w * (dw - (w * dw).sum(axis=1, keepdims=True))
    dq = ds @ k / math.sqrt(d_k)
    dk = ds.T @ q / math.sqrt(d_k)
    return dq, dk, dv


def sdpa_backward_ref(Q, K, V, dO, causal=False, kv_len=None, window=None):
    """(dQ, dK, dV) of attention for every leading (batch, head) index, head by head.

    Q [..., n_q, d_k], K [..., n_k, d_k], V [..., n_k, d_v], dO [..., n_q, d_v] -> arrays shaped like Q, K, V.
    `kv_len` [B] (with [B, h, n, d] tensors): keys j >= kv_len[b] of batch b are padding (their gradients are 0).
    `window`: radius of the restricted self-attention.
    """
    Q, K, V, dO = (_as_f64(a) for a in (Q, K, V, dO))
    lead = Q.shape[:-2]
    if K.shape[:-2] != lead or V.shape[:-2] != lead or dO.shape[:-2] != lead:
        raise ValueError("leading (batch, head) dimensions differ")
    if kv_len is not None and (len(lead) != 2 or np.shape(kv_len) != (lead[0],)):
        raise ValueError("kv_len needs [B, h, n, d] tensors and one length per batch entry")
    dQ, dK, dV = np.empty_like(Q), np.empty_like(K), np.empty_like(V)
    for idx in np.ndindex(*lead):
        n_valid = None if kv_len is None else int(kv_len[idx[0]])
        dQ[idx], dK[idx], dV[idx] = sdpa_backward_head(Q[idx], K[idx], V[idx], dO[idx], causal, n_valid=n_valid,
                                                       window=window)
    return dQ, dK, dV


def layer_norm_ref(x, gamma, beta, eps):
    """LayerNorm over the last axis: (x - mean) / sqrt(var + eps) * gamma + beta, with the biased variance (the mean of
    the squared deviations). The pages name the operation; its form, the learnable gamma/beta and eps are the usual
    definition (eps is an argument)."""
    x = _as_f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = np.square(x - mu).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * _as_f64(gamma) + _as_f64(beta)


def ffn_ref(x, W1, b1, W2, b2):
    """Position-wise feed-forward network FFN(x) = max(0, x W1 + b1) W2 + b2, the same weights at every position
    ("Transformer：抛弃循环与卷积的序列建模", section "FFN")."""
    return np.maximum(0.0, _as_f64(x) @ _as_f64(W1) + _as_f64(b1)) @ _as_f64(W2) + _as_f64(b2)


def encoder_layer_ref(X, Wq, Wk, Wv, Wo, g1, be1, W1, b1, W2, b2, g2, be2, h, eps, causal=False, kv_len=None):
    """One encoder layer in the pages' post-norm form: each sub-layer's output is LayerNorm(x + Sublayer(x))
    ("Transformer：抛弃循环与卷积的序列建模", section "Residual Connection 与 LayerNorm"; lettle.cn translation,
    section 3.1): H1 = LayerNorm(X + MultiHead(X, X, X)), Y = LayerNorm(H1 + FFN(H1)).

    X [B, n, d_model]; attention weights as mha_ref (no bias); W1 [d_model, d_ff], b1 [d_ff], W2 [d_ff, d_model],
    b2 [d_model]; g1/be1, g2/be2 [d_model] the two LayerNorms' scale and shift. `causal` turns the self-attention
    into the decoder's masked self-attention; `kv_len` [B] marks padding keys.
    """
    X = _as_f64(X)
    h1 = layer_norm_ref(X + mha_ref(X, X, Wq, Wk, Wv, Wo, h, causal, kv_len), g1, be1, eps)
    return layer_norm_ref(h1 + ffn_ref(h1, W1, b1, W2, b2), g2, be2, eps)

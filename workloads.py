"""Seeded synthetic inputs shared by the parity tests, the smoke check and the bench.

This module holds no attention arithmetic. It only draws seeded normal samples, quantises them to the storage
dtype the GPU path consumes (fp32 or bf16, round-to-nearest-even), and hands both sides the same numbers: the raw
storage (float32 array or bf16 bit patterns as uint16) for the device, and the exact same values widened to float64
for the oracle. bf16 and fp32 values are exactly representable in float64, so the comparison measures kernel error,
not input quantisation.

Shapes follow the base model of "Attention Is All You Need": d_model = 512, h = 8, d_k = d_v = 64 (the
"Multi-Head Attention" section and the "模型变体与消融实验" base-configuration table of the page
"Transformer：抛弃循环与卷积的序列建模"). The datasets the pages train on are not used: these seeded normal inputs
stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# Named workloads. Seeds are fixed so that every run (tests, smoke, bench) sees the same numbers.
WORKLOADS = {
    # single-head fp32 attention, Q/K/V ~ N(0,1)
    "sdpa_f32_b1_h1_n16": dict(kind="sdpa", dtype="f32", B=1, h=1, n_q=16, n_k=16, d_k=64, d_v=64,
                               causal=False, seed=1001),
    # encoder self-attention MHA: X ~ N(0,1), W ~ N(0, 1/512)
    "mha_self_bf16_b32_n128_dm512": dict(kind="mha", dtype="bf16", B=32, h=8, n_q=128, n_k=128, d_model=512,
                                         d_k=64, d_v=64, causal=False, seed=1002),
    # the same MHA with 16 heads of 32 and 4 heads of 128 (the head-count variants at d_model = 512)
    "mha_self_bf16_b32_n128_dm512_h16": dict(kind="mha", dtype="bf16", B=32, h=16, n_q=128, n_k=128, d_model=512,
                                             d_k=32, d_v=32, causal=False, seed=1002),
    "mha_self_bf16_b32_n128_dm512_h4": dict(kind="mha", dtype="bf16", B=32, h=4, n_q=128, n_k=128, d_model=512,
                                            d_k=128, d_v=128, causal=False, seed=1002),
    # the attention step of the MHA workload above on its own: per-head Q/K/V [32, 8, 128, 64] ~ N(0,1) (the
    # projections of X ~ N(0,1) by W ~ N(0, 1/512) have unit variance)
    "sdpa_bf16_b32_h8_n128": dict(kind="sdpa", dtype="bf16", B=32, h=8, n_q=128, n_k=128, d_k=64, d_v=64,
                                  causal=False, seed=1002),
    # decoder masked self-attention
    "sdpa_causal_bf16_b32_h8_n256": dict(kind="sdpa", dtype="bf16", B=32, h=8, n_q=256, n_k=256, d_k=64, d_v=64,
                                         causal=True, seed=1003),
    # encoder-decoder cross-attention, 200 decoder positions against 256 encoder positions
    "sdpa_cross_bf16_b16_h8_nq200_nk256": dict(kind="sdpa", dtype="bf16", B=16, h=8, n_q=200, n_k=256, d_k=64,
                                               d_v=64, causal=False, seed=1004),
    # long-sequence self-attention, unmasked and causal over the same tensors
    "sdpa_bf16_b4_h8_n4096": dict(kind="sdpa", dtype="bf16", B=4, h=8, n_q=4096, n_k=4096, d_k=64, d_v=64,
                                  causal=False, seed=1005),
    "sdpa_causal_bf16_b4_h8_n4096": dict(kind="sdpa", dtype="bf16", B=4, h=8, n_q=4096, n_k=4096, d_k=64, d_v=64,
                                         causal=True, seed=1005),
    # the head-count variants at d_model = 512: 16 heads of width 32 and 4 heads of width 128 over the same sequence
    # length (the same attention FLOPs as 8 heads of 64)
    "sdpa_bf16_b4_h16_n4096_d32": dict(kind="sdpa", dtype="bf16", B=4, h=16, n_q=4096, n_k=4096, d_k=32, d_v=32,
                                       causal=False, seed=1007),
    "sdpa_causal_bf16_b4_h16_n4096_d32": dict(kind="sdpa", dtype="bf16", B=4, h=16, n_q=4096, n_k=4096, d_k=32,
                                              d_v=32, causal=True, seed=1007),
    "sdpa_bf16_b4_h4_n4096_d128": dict(kind="sdpa", dtype="bf16", B=4, h=4, n_q=4096, n_k=4096, d_k=128, d_v=128,
                                       causal=False, seed=1008),
    "sdpa_causal_bf16_b4_h4_n4096_d128": dict(kind="sdpa", dtype="bf16", B=4, h=4, n_q=4096, n_k=4096, d_k=128,
                                              d_v=128, causal=True, seed=1008),
    # key padding: the long-sequence tensors as one length bucket of a length-grouped batch, each entry padded to 4096
    # (real key counts per entry in kv_len)
    "sdpa_padded_bf16_b4_h8_n4096": dict(kind="sdpa_padded", dtype="bf16", B=4, h=8, n_q=4096, n_k=4096, d_k=64,
                                         d_v=64, causal=False, seed=1005, kv_len=[4096, 3700, 3300, 3100]),
    # restricted self-attention of radius 256 (a band of 513 keys per query) over the long-sequence tensors
    "sdpa_window_bf16_b4_h8_n4096_w256": dict(kind="sdpa_window", dtype="bf16", B=4, h=8, n_q=4096, n_k=4096, d_k=64,
                                              d_v=64, causal=False, seed=1005, window=256),
    # one encoder layer (self-attention, FFN 512 -> 2048 -> 512, two post-norm LayerNorms) at the MHA shape above
    "encoder_layer_bf16_b32_n128_dm512": dict(kind="encoder", dtype="bf16", B=32, h=8, n_q=128, n_k=128, d_model=512,
                                              d_ff=2048, d_k=64, d_v=64, causal=False, seed=1006, eps=1e-5),
    # backward pass (dQ, dK, dV) of the long-sequence attention: the same Q, K, V and an upstream gradient ~ N(0,1)
    "sdpa_bwd_bf16_b4_h8_n4096": dict(kind="sdpa_bwd", dtype="bf16", B=4, h=8, n_q=4096, n_k=4096, d_k=64, d_v=64,
                                      causal=False, seed=1005),
    "sdpa_bwd_causal_bf16_b4_h8_n4096": dict(kind="sdpa_bwd", dtype="bf16", B=4, h=8, n_q=4096, n_k=4096, d_k=64,
                                             d_v=64, causal=True, seed=1005),
    # the backward at 16 heads of 32 (the d = 32 forward workload's tensors and an upstream gradient)
    "sdpa_bwd_bf16_b4_h16_n4096_d32": dict(kind="sdpa_bwd", dtype="bf16", B=4, h=16, n_q=4096, n_k=4096, d_k=32,
                                           d_v=32, causal=False, seed=1007),
    # and at 4 heads of 128
    "sdpa_bwd_bf16_b4_h4_n4096_d128": dict(kind="sdpa_bwd", dtype="bf16", B=4, h=4, n_q=4096, n_k=4096, d_k=128,
                                           d_v=128, causal=False, seed=1008),
}


@dataclass
class Quantised:
    """One tensor: `raw` is what the device gets, `f64` is the same values for the oracle."""
    raw: np.ndarray      # float32 array (dtype "f32") or uint16 bf16 bit patterns (dtype "bf16")
    f64: np.ndarray      # float64 array of exactly the same values
    dtype: str

    @property
    def shape(self):
        return self.f64.shape


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even) and return the 16-bit patterns."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if not np.all(np.isfinite(x32)):
        raise ValueError("inputs must be finite")
    u = x32.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float64 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def quantise(x: np.ndarray, dtype: str) -> Quantised:
    """Quantise float64 samples to the storage dtype: float64 -> float32 (RNE) [-> bf16 (RNE)]."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return Quantised(raw=x32, f64=x32.astype(np.float64), dtype="f32")
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x32)
        return Quantised(raw=bits, f64=bf16_bits_to_f64(bits), dtype="bf16")
    raise ValueError(f"unknown dtype {dtype!r}")


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def make_sdpa_inputs(B, h, n_q, n_k, d_k, d_v, dtype, seed, scale_q=1.0, dout=False):
    """Q [B,h,n_q,d_k], K [B,h,n_k,d_k], V [B,h,n_k,d_v], each ~ N(0,1), drawn in the order Q, K, V; with `dout`
    also an upstream gradient dO [B,h,n_q,d_v] ~ N(0,1), drawn after V (Q, K, V are the same with or without it)."""
    rng = _rng(seed)
    q = rng.standard_normal((B, h, n_q, d_k)) * scale_q
    k = rng.standard_normal((B, h, n_k, d_k))
    v = rng.standard_normal((B, h, n_k, d_v))
    out = {"Q": quantise(q, dtype), "K": quantise(k, dtype), "V": quantise(v, dtype)}
    if dout:
        out["dO"] = quantise(rng.standard_normal((B, h, n_q, d_v)), dtype)
    return out


def make_mha_inputs(B, n_q, n_k, d_model, h, d_k, d_v, dtype, seed, cross=False):
    """X ~ N(0,1) [B,n,d_model]; Wq, Wk [d_model, h*d_k], Wv [d_model, h*d_v], Wo [h*d_v, d_model] ~ N(0, 1/d_model).

    Drawn in the order X (then Xkv when `cross`), Wq, Wk, Wv, Wo. For self-attention Xkv is Xq itself.
    """
    rng = _rng(seed)
    xq = rng.standard_normal((B, n_q, d_model))
    xkv = rng.standard_normal((B, n_k, d_model)) if cross else None
    sd = np.sqrt(1.0 / d_model)
    wq = rng.standard_normal((d_model, h * d_k)) * sd
    wk = rng.standard_normal((d_model, h * d_k)) * sd
    wv = rng.standard_normal((d_model, h * d_v)) * sd
    wo = rng.standard_normal((h * d_v, d_model)) * sd
    out = {"Xq": quantise(xq, dtype)}
    out["Xkv"] = quantise(xkv, dtype) if cross else out["Xq"]
    out.update(Wq=quantise(wq, dtype), Wk=quantise(wk, dtype), Wv=quantise(wv, dtype), Wo=quantise(wo, dtype))
    return out


def make_encoder_inputs(B, n, d_model, h, d_ff, dtype, seed):
    """One encoder layer's inputs, drawn in this order: X ~ N(0,1) [B,n,d_model]; Wq, Wk, Wv, Wo ~ N(0, 1/d_model)
    [d_model,d_model]; W1 ~ N(0, 1/d_model) [d_model,d_ff]; b1 ~ N(0, 0.1^2) [d_ff]; W2 ~ N(0, 1/d_ff) [d_ff,d_model];
    b2 ~ N(0, 0.1^2); LayerNorm scales 1 + N(0, 0.1^2) and shifts N(0, 0.1^2) [d_model] (ln1_gamma, ln1_beta,
    ln2_gamma, ln2_beta). The pages give no initialisation; these keep every sub-layer's output of order 1."""
    rng = _rng(seed)
    out = {"X": quantise(rng.standard_normal((B, n, d_model)), dtype)}
    sd = np.sqrt(1.0 / d_model)
    for name in ("Wq", "Wk", "Wv", "Wo"):
        out[name] = quantise(rng.standard_normal((d_model, d_model)) * sd, dtype)
    out["W1"] = quantise(rng.standard_normal((d_model, d_ff)) * sd, dtype)
    out["b1"] = quantise(rng.standard_normal(d_ff) * 0.1, dtype)
    out["W2"] = quantise(rng.standard_normal((d_ff, d_model)) * np.sqrt(1.0 / d_ff), dtype)
    out["b2"] = quantise(rng.standard_normal(d_model) * 0.1, dtype)
    for name in ("ln1_gamma", "ln1_beta", "ln2_gamma", "ln2_beta"):
        base = 1.0 if name.endswith("gamma") else 0.0
        out[name] = quantise(base + rng.standard_normal(d_model) * 0.1, dtype)
    return out


def make_workload(name: str):
    """Inputs of a named workload (see WORKLOADS)."""
    w = WORKLOADS[name]
    if w["kind"] in ("sdpa", "sdpa_bwd", "sdpa_padded", "sdpa_window"):
        return make_sdpa_inputs(w["B"], w["h"], w["n_q"], w["n_k"], w["d_k"], w["d_v"], w["dtype"], w["seed"],
                                dout=w["kind"] == "sdpa_bwd")
    if w["kind"] == "encoder":
        return make_encoder_inputs(w["B"], w["n_q"], w["d_model"], w["h"], w["d_ff"], w["dtype"], w["seed"])
    return make_mha_inputs(w["B"], w["n_q"], w["n_k"], w["d_model"], w["h"], w["d_k"], w["d_v"], w["dtype"],
                           w["seed"], cross=w["n_q"] != w["n_k"])

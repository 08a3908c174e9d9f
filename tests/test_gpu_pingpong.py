"""Parity of the eight-wave ping-pong attention kernel (unmasked, width 64, n_q >= 512) with the float64 oracle.

That kernel serves every unmasked width-64 call with at least 512 queries: sdpa_forward, sdpa_forward_lse,
sdpa_forward_padded and the attention step of mha_forward. Its own edge cases are swept here: query counts that
leave some waves of the last 512-query workgroup without a query, key counts that stop the four-tile ring after one,
two, three, four or five tiles (with and without a ragged last tile), key padding down to zero keys, scores large
enough to take the offset slow path, outputs written through the strides of the concatenated-heads layout, and the
row log-sum-exp. Bars as everywhere for bf16: max-abs <= 2e-2, mean-abs <= 2e-3, normalised rms <= 1e-2.
"""
import numpy as np
import pytest
import torch

import transformer_head_scaled_02_amd as m
import workloads
from oracle import mha_ref, sdpa_lse_ref, sdpa_ref
from tests._helpers import assert_bf16_parity, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")
    m.load_library()


def _case(B, h, n_q, n_k, seed, scale_q=1.0):
    x = workloads.make_sdpa_inputs(B, h, n_q, n_k, 64, 64, "bf16", seed, scale_q=scale_q)
    return x, tuple(to_dev(x[n]) for n in "QKV")


# n_q: a full workgroup, one query over, waves 1..7 of the last workgroup empty or partly filled, several blocks.
# n_k: 1..5 tiles of the ring, full and ragged last tiles.
SHAPES = [(1, 1, 512, 64), (1, 1, 512, 1), (1, 2, 513, 63), (1, 1, 520, 65), (2, 1, 600, 128), (1, 1, 700, 129),
          (1, 2, 1023, 192), (1, 1, 1024, 200), (1, 1, 1025, 256), (1, 1, 1100, 257), (1, 1, 1536, 320),
          (2, 1, 777, 1000), (1, 1, 2048, 2048)]


@pytest.mark.parametrize("B,h,n_q,n_k", SHAPES)
def test_pingpong_shapes(B, h, n_q, n_k):
    x, (q, k, v) = _case(B, h, n_q, n_k, 4000 + n_q + 3 * n_k)
    out = m.sdpa_forward(q, k, v)
    torch.cuda.synchronize()
    assert_bf16_parity(to_f64(out), sdpa_ref(x["Q"].f64, x["K"].f64, x["V"].f64), f"{(B, h, n_q, n_k)}")


@pytest.mark.parametrize("n_k", [64, 130, 520])
def test_pingpong_large_scores(n_k):
    # Q x 30: scores of order +-100 in exponent units, far past where an unshifted fp32 exp2 overflows; later tiles
    # raise the offset through the slow path many times
    x, (q, k, v) = _case(1, 2, 640, n_k, 4100 + n_k, scale_q=30.0)
    out = m.sdpa_forward(q, k, v)
    torch.cuda.synchronize()
    assert_bf16_parity(to_f64(out), sdpa_ref(x["Q"].f64, x["K"].f64, x["V"].f64), f"large scores n_k={n_k}")


def test_pingpong_increasing_scores_take_the_slow_path_every_tile():
    # every key tile has larger scores than all earlier ones (keys scaled up along the sequence), so each tile's row
    # sums exceed the limit and the offset is raised on every tile
    B, h, n_q, n_k = 1, 1, 512, 384
    x = workloads.make_sdpa_inputs(B, h, n_q, n_k, 64, 64, "bf16", 4200)
    q = torch.ones(B, h, n_q, 64, dtype=torch.bfloat16, device="cuda") * 0.5
    ramp = torch.linspace(0.0, 8.0, n_k, dtype=torch.float32, device="cuda").view(1, 1, n_k, 1)
    k = (torch.ones(B, h, n_k, 64, device="cuda") * ramp).to(torch.bfloat16)
    v = to_dev(x["V"])
    out = m.sdpa_forward(q, k, v)
    torch.cuda.synchronize()
    ref = sdpa_ref(to_f64(q), to_f64(k), to_f64(v))
    assert_bf16_parity(to_f64(out), ref, "increasing scores")


def test_pingpong_all_ones_values_give_ones():
    x, (q, k, v) = _case(1, 2, 1030, 321, 4300)
    out = m.sdpa_forward(q, k, torch.ones_like(v))
    torch.cuda.synchronize()
    assert torch.all(out == 1.0), "rows of the weights must sum to 1 exactly in the output of an all-ones V"


def test_pingpong_lse():
    x, (q, k, v) = _case(2, 1, 700, 333, 4400)
    out, lse = m.sdpa_forward_lse(q, k, v)
    torch.cuda.synchronize()
    assert_bf16_parity(to_f64(out), sdpa_ref(x["Q"].f64, x["K"].f64, x["V"].f64), "lse call output")
    ref = sdpa_lse_ref(x["Q"].f64, x["K"].f64)
    got = lse.double().cpu().numpy()
    err = np.abs(got - ref).max()
    assert err <= 1e-2, f"lse max error {err:.3g}"
    # asking for the lse changes no bit of the output
    assert torch.equal(out, m.sdpa_forward(q, k, v))


@pytest.mark.parametrize("lengths", [[0, 1, 64, 65], [333, 200, 129, 63], [-5, 600, 1, 128]])
def test_pingpong_key_padding(lengths):
    n_q, n_k = 600, 333
    x, (q, k, v) = _case(4, 2, n_q, n_k, 4500 + sum(max(L, 0) for L in lengths))
    lens = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    # padding rows hold NaN: they must never be read
    kk, vv = k.clone(), v.clone()
    for b, L in enumerate(np.clip(lengths, 0, n_k)):
        kk[b, :, L:] = float("nan")
        vv[b, :, L:] = float("nan")
    out = m.sdpa_forward_padded(q, kk, vv, lens)
    torch.cuda.synchronize()
    got = to_f64(out)
    for b, L in enumerate(np.clip(lengths, 0, n_k)):
        if L == 0:
            assert np.all(got[b] == 0.0), "a row with no key gives 0"
            continue
        ref = sdpa_ref(x["Q"].f64[b:b + 1], x["K"].f64[b:b + 1, :, :L], x["V"].f64[b:b + 1, :, :L])
        assert_bf16_parity(got[b:b + 1], ref, f"batch entry {b}, {L} keys")


def test_pingpong_mha_concat_strides():
    # mha_forward at n = 512 runs its attention step on this kernel, writing the concatenated [B, n, h*64] layout
    B, n, d_model, h = 2, 512, 512, 8
    x = workloads.make_mha_inputs(B, n, n, d_model, h, 64, 64, "bf16", 4600)
    xq = to_dev(x["Xq"])
    out = m.mha_forward(xq, xq, to_dev(x["Wq"]), to_dev(x["Wk"]), to_dev(x["Wv"]), to_dev(x["Wo"]), h=h)
    torch.cuda.synchronize()
    ref = mha_ref(x["Xq"].f64, x["Xq"].f64, x["Wq"].f64, x["Wk"].f64, x["Wv"].f64, x["Wo"].f64, h=h)
    assert_bf16_parity(to_f64(out), ref, "mha n=512")


def test_pingpong_matches_across_block_boundaries():
    # the same query rows computed in different workgroup positions give the same bits: rows 0..511 of a 1024-query
    # call and of a 512-query call over the same keys
    x, (q, k, v) = _case(1, 1, 1024, 300, 4700)
    full = m.sdpa_forward(q, k, v)
    head = m.sdpa_forward(q[:, :, :512].contiguous(), k, v)
    torch.cuda.synchronize()
    assert torch.equal(full[:, :, :512], head)


def test_pingpong_train_forward_float32_output():
    # the training forward also writes the output before its bf16 rounding, [B, h, n_q, 64] float32: rounding it gives
    # the bf16 output bit for bit, and it meets the oracle at least as closely
    x, (q, k, v) = _case(2, 2, 700, 333, 4800)
    out, o32, lse = m.sdpa_forward_train(q, k, v)
    torch.cuda.synchronize()
    assert o32.dtype == torch.float32 and o32.shape == out.shape
    assert torch.equal(o32.to(torch.bfloat16), out)
    ref = sdpa_ref(x["Q"].f64, x["K"].f64, x["V"].f64)
    assert_bf16_parity(o32.double().cpu().numpy(), ref, "float32 output")

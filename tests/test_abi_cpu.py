"""The C-ABI library without a GPU: it loads, exports every symbol the header declares, and rejects bad arguments
before any HIP call (so these calls are safe with no device present)."""
import ctypes
import re
from pathlib import Path

import pytest

import transformer_head_scaled_02_amd as m

HEADERS = sorted((Path(__file__).resolve().parents[1] / "include").glob("*.h"))
INVALID, UNSUPPORTED = m.ATTN_ERR_INVALID, m.ATTN_ERR_UNSUPPORTED
F32, BF16 = m.ATTN_F32, m.ATTN_BF16

pytestmark = pytest.mark.skipif(not m.LIB_PATH.exists(), reason="library not built")


def header_functions():
    names = set()
    for header in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", header.read_text(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_header_declares_the_binding_names():
    assert header_functions() == sorted(m.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(str(m.LIB_PATH))
    for name in header_functions():
        assert hasattr(lib, name), name


@pytest.fixture(scope="module")
def lib():
    return m.load_library()


A = 4096  # a fake, 16-byte aligned "device" address: validation must fail before anything dereferences it


def sdpa(lib, Q=A, K=A * 2, V=A * 3, mask=0, out=A * 1000, dtype=BF16, B=1, h=1, n_q=16, n_k=16, d_k=64, d_v=64):
    return lib.sdpa_forward(Q, K, V, mask, out, dtype, B, h, n_q, n_k, d_k, d_v, None)


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), INVALID), (dict(out=None), INVALID), (dict(B=0), INVALID), (dict(n_q=-1), INVALID),
    (dict(n_k=0), INVALID), (dict(mask=7), INVALID), (dict(dtype=5), UNSUPPORTED), (dict(d_k=32), UNSUPPORTED),
    (dict(d_v=128), UNSUPPORTED), (dict(mask=1, n_q=16, n_k=17), UNSUPPORTED), (dict(Q=A + 2), INVALID),
    (dict(out=A + 8), INVALID), (dict(n_q=1 << 25), UNSUPPORTED), (dict(B=1 << 17), UNSUPPORTED),
    # out [1,1,16,64] bf16 = 2 KiB starting inside K
    (dict(out=A * 2 + 1024), INVALID), (dict(out=A * 3 - 1024), INVALID),
    # head widths: d_k = d_v in {32, 64, 128} only; the overlap checks use the width (out [1,1,16,128] = 4 KiB)
    (dict(d_k=48, d_v=48), UNSUPPORTED), (dict(d_k=16, d_v=16), UNSUPPORTED), (dict(d_k=256, d_v=256), UNSUPPORTED),
    (dict(d_k=32, d_v=64), UNSUPPORTED), (dict(d_k=128, d_v=128, out=A * 3 + 2048), INVALID),
])
def test_sdpa_rejects_bad_arguments(lib, kw, code):
    assert sdpa(lib, **kw) == code
    assert lib.attn_last_error().decode().startswith("sdpa_forward")


def mha(lib, Xq=A, Xkv=A, Wq=A * 100, Wk=A * 200, Wv=A * 300, Wo=A * 400, mask=0, out=A * 1000, ws=A * 2000,
        ws_bytes=1 << 30, dtype=BF16, B=2, n_q=8, n_k=8, d_model=64, h=1, d_k=64, d_v=64):
    return lib.mha_forward(Xq, Xkv, Wq, Wk, Wv, Wo, mask, out, ws, ws_bytes, dtype, B, n_q, n_k, d_model, h, d_k, d_v,
                           None)


@pytest.mark.parametrize("kw,code", [
    (dict(Wo=None), INVALID), (dict(ws=None), INVALID), (dict(dtype=F32), UNSUPPORTED), (dict(h=0), INVALID),
    (dict(d_model=96), UNSUPPORTED), (dict(d_k=32), UNSUPPORTED), (dict(mask=1, n_k=9), UNSUPPORTED),
    (dict(d_k=32, d_v=32), UNSUPPORTED), (dict(d_k=48, d_v=48, h=4), UNSUPPORTED), (dict(d_k=256, d_v=256), UNSUPPORTED),
    (dict(mask=3), INVALID), (dict(ws_bytes=100), INVALID), (dict(Wq=A * 100 + 4), INVALID),
    (dict(out=A * 100), INVALID), (dict(ws=A * 300), INVALID), (dict(out=A * 2000 + 4096), INVALID),
])
def test_mha_rejects_bad_arguments(lib, kw, code):
    assert mha(lib, **kw) == code
    assert lib.attn_last_error().decode().startswith("mha_forward")


def test_workspace_size(lib):
    # Q, K, V per head and the concat, bf16, each rounded up to 256 bytes
    B, n_q, n_k, h = 32, 128, 128, 8
    assert lib.mha_workspace_size(BF16, B, n_q, n_k, h, 64, 64) == 4 * B * h * 128 * 64 * 2
    got = lib.mha_workspace_size(BF16, 1, 3, 5, 1, 64, 64)
    assert got >= (3 + 5 + 5 + 3) * 64 * 2 and got % 256 == 0
    assert lib.mha_workspace_size(F32, 1, 3, 5, 1, 64, 64) == 0
    assert lib.mha_workspace_size(BF16, 1, 3, 5, 1, 32, 64) == 0
    # other head widths: [B, h, n, d] regions for d in {32, 128}; h * d must be a multiple of 64
    assert lib.mha_workspace_size(BF16, 2, 10, 12, 16, 32, 32) == 90112  # 20480 + 24576 + 24576 + 20480
    assert lib.mha_workspace_size(BF16, 2, 10, 12, 4, 128, 128) == 90112
    assert lib.mha_workspace_size(BF16, 1, 3, 5, 1, 32, 32) == 0
    assert lib.mha_workspace_size(BF16, 1, 3, 5, 2, 48, 48) == 0


def sdpa_lse(lib, Q=A, K=A * 2, V=A * 3, mask=0, out=A * 1000, lse=A * 1100, dtype=BF16, B=1, h=1, n_q=16, n_k=16,
             d_k=64, d_v=64):
    return lib.sdpa_forward_lse(Q, K, V, mask, out, lse, dtype, B, h, n_q, n_k, d_k, d_v, None)


@pytest.mark.parametrize("kw,code", [
    (dict(lse=None), INVALID), (dict(Q=None), INVALID), (dict(lse=A * 1100 + 4), INVALID), (dict(dtype=5), UNSUPPORTED),
    (dict(mask=1, n_k=17), UNSUPPORTED), (dict(d_k=128), UNSUPPORTED),
    # lse [1,1,16] float32 = 64 bytes, placed inside out (2 KiB at A*1000) or inside Q
    (dict(lse=A * 1000 + 256), INVALID), (dict(lse=A + 16), INVALID),
])
def test_sdpa_forward_lse_rejects_bad_arguments(lib, kw, code):
    assert sdpa_lse(lib, **kw) == code
    assert lib.attn_last_error().decode().startswith("sdpa_forward_lse")


def bwd(lib, Q=A, K=A * 2, V=A * 3, O=A * 4, dO=A * 5, lse=A * 6, kv_len=None, window=-1, mask=0, dQ=A * 100,
        dK=A * 200, dV=A * 300, ws=A * 400, ws_bytes=1 << 20, dtype=BF16, B=1, h=1, n_q=16, n_k=16, d_k=64, d_v=64):
    return lib.sdpa_backward(Q, K, V, O, dO, lse, kv_len, window, mask, dQ, dK, dV, ws, ws_bytes, dtype, B, h, n_q,
                             n_k, d_k, d_v, None)


@pytest.mark.parametrize("kw,code", [
    (dict(O=None), INVALID), (dict(dO=None), INVALID), (dict(lse=None), INVALID), (dict(dQ=None), INVALID),
    (dict(dK=None), INVALID), (dict(dV=None), INVALID), (dict(ws=None), INVALID), (dict(ws_bytes=1023), INVALID),
    (dict(B=0), INVALID), (dict(mask=3), INVALID), (dict(dtype=7), UNSUPPORTED), (dict(d_v=32), UNSUPPORTED),
    (dict(mask=1, n_q=16, n_k=32), UNSUPPORTED), (dict(n_k=1 << 25), UNSUPPORTED), (dict(dK=A * 200 + 8), INVALID),
    (dict(lse=A * 6 + 4), INVALID),
    # outputs over inputs, outputs over each other, workspace over an input
    (dict(dQ=A * 4), INVALID), (dict(dV=A * 200 + 1024), INVALID), (dict(ws=A * 6), INVALID),
    (dict(dK=A * 400), INVALID), (dict(kv_len=A * 7 + 4), INVALID), (dict(kv_len=A * 100 + 64), INVALID),
    (dict(window=3, n_k=32), UNSUPPORTED), (dict(window=3, kv_len=A * 7), UNSUPPORTED),
    # the backward kernels take d_k = d_v in {32, 64, 128}
    (dict(d_k=256, d_v=256), UNSUPPORTED), (dict(d_k=48, d_v=48), UNSUPPORTED), (dict(d_k=32, d_v=64), UNSUPPORTED),
    (dict(d_k=128, d_v=128, dQ=A * 4 + 2048 + 16), INVALID),
])
def test_sdpa_backward_rejects_bad_arguments(lib, kw, code):
    assert bwd(lib, **kw) == code
    assert lib.attn_last_error().decode().startswith("sdpa_backward")


def padded(lib, Q=A, K=A * 2, V=A * 3, kv_len=A * 4, mask=0, out=A * 1000, lse=None, dtype=BF16, B=1, h=1, n_q=16,
           n_k=16, d_k=64, d_v=64):
    return lib.sdpa_forward_padded(Q, K, V, kv_len, mask, out, lse, dtype, B, h, n_q, n_k, d_k, d_v, None)


@pytest.mark.parametrize("kw,code", [
    (dict(kv_len=None), INVALID), (dict(out=None), INVALID), (dict(kv_len=A * 4 + 4), INVALID),
    (dict(kv_len=A * 1000 + 16), INVALID), (dict(lse=A * 1100, kv_len=A * 1100 + 32), INVALID),
    (dict(dtype=9), UNSUPPORTED), (dict(mask=1, n_k=20), UNSUPPORTED), (dict(d_v=16), UNSUPPORTED),
    (dict(B=-1), INVALID), (dict(lse=A * 1000 + 256), INVALID),
])
def test_sdpa_forward_padded_rejects_bad_arguments(lib, kw, code):
    assert padded(lib, **kw) == code
    assert lib.attn_last_error().decode().startswith("sdpa_forward_padded")


def enc(lib, X=A, kv_len=None, W=A * 10, ln=A * 20, W1=A * 30, b1=A * 40, W2=A * 50, b2=A * 60, eps=1e-5, mask=0,
        out=A * 1000, ws=A * 2000, ws_bytes=1 << 30, dtype=BF16, B=1, n=16, d_model=512, h=8, d_ff=2048):
    return lib.encoder_layer_forward(X, kv_len, W, W + 1 << 20, W + 2 << 20, W + 3 << 20, ln, ln + 4096, W1, b1, W2,
                                     b2, ln + 8192, ln + 12288, eps, mask, out, ws, ws_bytes, dtype, B, n, d_model, h,
                                     d_ff, None)


@pytest.mark.parametrize("kw,code", [
    (dict(X=None), INVALID), (dict(W1=None), INVALID), (dict(out=None), INVALID), (dict(ws=None), INVALID),
    (dict(dtype=F32), UNSUPPORTED), (dict(mask=4), INVALID), (dict(eps=-1.0), INVALID),
    (dict(eps=float("nan")), INVALID), (dict(d_model=512, h=32), UNSUPPORTED), (dict(d_ff=100), UNSUPPORTED),
    # head width d_model / h in {32, 64, 128} with d_model a multiple of 64
    (dict(d_model=512, h=3), UNSUPPORTED), (dict(d_model=96, h=3), UNSUPPORTED), (dict(d_model=1024, h=4), UNSUPPORTED),
    (dict(d_model=2048, h=32), UNSUPPORTED), (dict(n=0), INVALID), (dict(ws_bytes=1000), INVALID),
    (dict(b1=A * 40 + 2), INVALID), (dict(kv_len=A * 70 + 4), INVALID),
    # out [1,16,512] bf16 = 16 KiB over X; the workspace over W1
    (dict(out=A + 4096), INVALID), (dict(ws=A * 30), INVALID),
])
def test_encoder_layer_rejects_bad_arguments(lib, kw, code):
    assert enc(lib, **kw) == code
    assert lib.attn_last_error().decode().startswith("encoder_layer_forward")


def test_encoder_layer_workspace_size(lib):
    B, n, dm, h, ff = 32, 128, 512, 8, 2048
    act = B * n * dm * 2
    # Q, K, V, the concat, the residual sums and H1 (six [B, n, d_model] regions) plus the FFN hidden [B, n, d_ff]
    assert lib.encoder_layer_workspace_size(BF16, B, n, dm, h, ff) == 6 * act + B * n * ff * 2
    assert lib.encoder_layer_workspace_size(F32, B, n, dm, h, ff) == 0
    # 4 heads of 128 and 16 of 32 need the same regions; 32 heads of 16 are not implemented
    assert lib.encoder_layer_workspace_size(BF16, B, n, dm, 4, ff) == 6 * act + B * n * ff * 2
    assert lib.encoder_layer_workspace_size(BF16, B, n, dm, 16, ff) == 6 * act + B * n * ff * 2
    assert lib.encoder_layer_workspace_size(BF16, B, n, dm, 32, ff) == 0
    assert lib.encoder_layer_workspace_size(BF16, B, n, dm, h, 100) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(window=-1), INVALID), (dict(Q=None), INVALID), (dict(n_k=17), UNSUPPORTED), (dict(dtype=4), UNSUPPORTED),
    (dict(d_k=32), UNSUPPORTED), (dict(out=A + 8), INVALID), (dict(lse=A * 1100 + 4), INVALID),
])
def test_sdpa_forward_window_rejects_bad_arguments(lib, kw, code):
    a = dict(Q=A, K=A * 2, V=A * 3, window=4, mask=0, out=A * 1000, lse=None, dtype=BF16, B=1, h=1, n_q=16, n_k=16,
             d_k=64, d_v=64)
    a.update(kw)
    assert lib.sdpa_forward_window(a["Q"], a["K"], a["V"], a["window"], a["mask"], a["out"], a["lse"], a["dtype"],
                                   a["B"], a["h"], a["n_q"], a["n_k"], a["d_k"], a["d_v"], None) == code
    assert lib.attn_last_error().decode().startswith("sdpa_forward_window")


def test_backward_workspace_size(lib):
    # 1 KiB per (batch, head) and 64-row query tile: lse and D of the tile's rows
    assert lib.sdpa_backward_workspace_size(BF16, 4, 8, 4096, 4096, 64, 64) == 4 * 8 * 64 * 1024
    assert lib.sdpa_backward_workspace_size(F32, 1, 1, 65, 3, 64, 64) == 2 * 1024
    assert lib.sdpa_backward_workspace_size(BF16, 1, 1, 16, 16, 32, 64) == 0
    assert lib.sdpa_backward_workspace_size(5, 1, 1, 16, 16, 64, 64) == 0
    assert lib.sdpa_backward_workspace_size(BF16, 0, 1, 16, 16, 64, 64) == 0


def test_status_strings(lib):
    assert lib.attn_status_string(0) == b"ATTN_OK"
    assert lib.attn_status_string(2) == b"ATTN_ERR_UNSUPPORTED"
    assert lib.attn_status_string(99) == b"ATTN_UNKNOWN_STATUS"


def test_python_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        m.sdpa_forward(q, q, q)


def test_probe_scratch_size_is_positive(lib):
    assert lib.probe_scratch_size() > 0


@pytest.mark.parametrize("case", ["null", "small", "iters0", "iters_big", "misaligned"])
def test_probes_reject_bad_scratch_before_any_hip_call(lib, case):
    import ctypes
    need = lib.probe_scratch_size()
    scratch, nbytes, iters = A, need, 10
    if case == "null":
        scratch = 0
    elif case == "small":
        nbytes = need - 1
    elif case == "iters0":
        iters = 0
    elif case == "iters_big":
        iters = 10**7
    else:
        scratch = A + 4
    x, y = ctypes.c_double(), ctypes.c_double()
    assert lib.probe_mfma_bf16(scratch, nbytes, iters, None, ctypes.byref(x), ctypes.byref(y)) == INVALID
    assert lib.probe_exp_f32(scratch, nbytes, iters, None, ctypes.byref(x), ctypes.byref(y)) == INVALID
    for tr in (0, 1):
        assert lib.probe_lds_read(scratch, nbytes, iters, tr, None, ctypes.byref(x), ctypes.byref(y)) == INVALID


def test_probe_lds_read_rejects_bad_form(lib):
    import ctypes
    x, y = ctypes.c_double(), ctypes.c_double()
    assert lib.probe_lds_read(A, lib.probe_scratch_size(), 10, 2, None, ctypes.byref(x), ctypes.byref(y)) == INVALID
    assert lib.probe_lds_read(A, lib.probe_scratch_size(), 10, 0, None, None, ctypes.byref(y)) == INVALID


@pytest.mark.parametrize("kw", [dict(src=0), dict(nbytes=0), dict(nbytes=24), dict(reps=0), dict(reps=1001),
                                dict(dst=A + 16)])
def test_probe_copy_rejects_bad_arguments(lib, kw):
    import ctypes
    args = dict(src=A, dst=A * 1000, nbytes=1 << 20, reps=2)
    args.update(kw)
    g = ctypes.c_double()
    assert lib.probe_hbm_copy(args["src"], args["dst"], args["nbytes"], args["reps"], None, ctypes.byref(g)) == INVALID


def mha_noalloc(lib, Xq=A, Xkv=A, W=A * 2, out=A * 1000, mask=0, dtype=BF16, B=2, n_q=16, n_k=16, d_model=512, h=8,
                d_k=64, d_v=64):
    return lib.mha_forward_noalloc(Xq, Xkv, W, W + 0x100000, W + 0x200000, W + 0x300000, mask, out, dtype, B, n_q, n_k,
                                   d_model, h, d_k, d_v, None)


@pytest.mark.parametrize("kw,code", [
    (dict(Xq=None), INVALID), (dict(out=None), INVALID), (dict(B=0), INVALID), (dict(dtype=F32), UNSUPPORTED),
    (dict(mask=1, n_k=17), UNSUPPORTED), (dict(d_k=48, d_v=48), UNSUPPORTED),
    # sizes whose intermediates need more than the library's 32 MiB scratch: rejected before any HIP call
    (dict(B=64, n_q=512, n_k=512), INVALID), (dict(B=1, n_q=1 << 16, n_k=1 << 16), INVALID),
])
def test_mha_noalloc_rejects_bad_arguments(lib, kw, code):
    assert mha_noalloc(lib, **kw) == code
    if kw.get("B") == 64:
        assert b"scratch" in lib.attn_last_error()


def train(lib, Q=A, K=A * 2, V=A * 3, kv_len=None, window=-1, mask=0, out=A * 1000, out32=None, lse=A * 1100,
          dtype=BF16, B=1, h=1, n_q=16, n_k=16, d_k=64, d_v=64):
    return lib.sdpa_forward_train(Q, K, V, kv_len, window, mask, out, out32, lse, dtype, B, h, n_q, n_k, d_k, d_v,
                                  None)


@pytest.mark.parametrize("kw,code", [
    (dict(lse=None), INVALID), (dict(Q=None), INVALID), (dict(out=None), INVALID),
    # out_f32 is for bf16 only; aligned; [1,1,16,64] float32 = 4 KiB must not overlap out, Q or lse
    (dict(out32=A * 1200, dtype=F32), INVALID), (dict(out32=A * 1200 + 4), INVALID),
    (dict(out32=A * 1000 + 512), INVALID), (dict(out32=A + 64), INVALID), (dict(out32=A * 1100 - 2048), INVALID),
    (dict(window=3, n_k=32), UNSUPPORTED), (dict(window=3, kv_len=A * 7), UNSUPPORTED),
    (dict(dtype=m.ATTN_BF16_F32O), UNSUPPORTED), (dict(d_k=48, d_v=48), UNSUPPORTED),
    (dict(mask=1, n_k=17), UNSUPPORTED), (dict(kv_len=A * 7 + 4), INVALID), (dict(mask=2), INVALID),
])
def test_sdpa_forward_train_rejects_bad_arguments(lib, kw, code):
    assert train(lib, **kw) == code
    assert lib.attn_last_error().decode().startswith("sdpa_forward_train")


def test_backward_with_f32_output_checks_its_size(lib):
    # O float32 [1,1,16,64] = 4 KiB at A*4: dQ 2 KiB + 16 bytes in overlaps it only when O is counted as float32
    assert bwd(lib, dtype=m.ATTN_BF16_F32O, dQ=A * 4 + 2048 + 16) == INVALID
    assert "overlaps" in lib.attn_last_error().decode()
    assert bwd(lib, dtype=m.ATTN_BF16_F32O, O=None) == INVALID
    assert bwd(lib, dtype=m.ATTN_BF16_F32O, d_k=256, d_v=256) == UNSUPPORTED
    assert lib.sdpa_backward_workspace_size(m.ATTN_BF16_F32O, 4, 8, 4096, 4096, 64, 64) == 4 * 8 * 64 * 1024

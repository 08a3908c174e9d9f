"""ctypes binding over libmi355_attn.so: argument marshalling only.

Every step of the computation runs in the library's HIP kernels. torch provides the device buffers and the current
stream; this module checks shapes, dtypes and devices, passes raw pointers, and raises on a non-OK status. If the
library has not been built, loading fails loudly: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path

import torch

# The library this package loads: the in-tree build, or another build of the same sources named by MI355_ATTN_LIB
# (the host-sanitized copy the CPU argument-checking tests run against).
LIB_PATH = Path(os.environ.get("MI355_ATTN_LIB") or Path(__file__).resolve().parent / "libmi355_attn.so")

ATTN_OK, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP = 0, 1, 2, 3
ATTN_MASK_NONE, ATTN_MASK_CAUSAL = 0, 1
ATTN_F32, ATTN_BF16, ATTN_BF16_F32O = 0, 1, 2

# every symbol include/mi355_attn.h declares
EXPORTED = ("sdpa_forward", "sdpa_forward_lse", "sdpa_forward_padded", "sdpa_forward_window", "sdpa_forward_train",
            "sdpa_backward", "sdpa_backward_workspace_size", "mha_forward", "mha_forward_noalloc",
            "encoder_layer_forward", "encoder_layer_workspace_size",
            "mha_workspace_size", "attn_status_string", "attn_last_error", "probe_scratch_size", "probe_mfma_bf16", "probe_exp_f32", "probe_lds_read", "probe_hbm_copy")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def load_library(path: Path | str | None = None) -> ctypes.CDLL:
    """Load libmi355_attn.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path is not None else LIB_PATH
    if not p.exists():
        raise ImportError(f"{p} is missing: build it with `python -m transformer_head_scaled_02_amd.build` "
                          "(or __graft_entry__.build()); there is no non-HIP fallback")
    lib = ctypes.CDLL(str(p))
    i64, vp, ci, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.sdpa_forward.argtypes = [vp, vp, vp, ci, vp, ci, i64, i64, i64, i64, i64, i64, vp]
    lib.sdpa_forward.restype = ci
    lib.sdpa_forward_lse.argtypes = [vp, vp, vp, ci, vp, vp, ci, i64, i64, i64, i64, i64, i64, vp]
    lib.sdpa_forward_lse.restype = ci
    lib.sdpa_forward_padded.argtypes = [vp, vp, vp, vp, ci, vp, vp, ci, i64, i64, i64, i64, i64, i64, vp]
    lib.sdpa_forward_padded.restype = ci
    lib.sdpa_forward_window.argtypes = [vp, vp, vp, i64, ci, vp, vp, ci, i64, i64, i64, i64, i64, i64, vp]
    lib.sdpa_forward_window.restype = ci
    lib.sdpa_forward_train.argtypes = [vp, vp, vp, vp, i64, ci, vp, vp, vp, ci, i64, i64, i64, i64, i64, i64, vp]
    lib.sdpa_forward_train.restype = ci
    lib.sdpa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, ci, vp, vp, vp, vp, sz, ci, i64, i64, i64, i64, i64,
                                  i64, vp]
    lib.sdpa_backward.restype = ci
    lib.sdpa_backward_workspace_size.argtypes = [ci, i64, i64, i64, i64, i64, i64]
    lib.sdpa_backward_workspace_size.restype = sz
    lib.mha_forward.argtypes = [vp, vp, vp, vp, vp, vp, ci, vp, vp, sz, ci, i64, i64, i64, i64, i64, i64, i64, vp]
    lib.mha_forward.restype = ci
    lib.mha_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, ci, vp, ci, i64, i64, i64, i64, i64, i64, i64, vp]
    lib.mha_forward_noalloc.restype = ci
    lib.mha_workspace_size.argtypes = [ci, i64, i64, i64, i64, i64, i64]
    lib.mha_workspace_size.restype = sz
    lib.encoder_layer_forward.argtypes = [vp] * 14 + [ctypes.c_float, ci, vp, vp, sz, ci, i64, i64, i64, i64, i64, vp]
    lib.encoder_layer_forward.restype = ci
    lib.encoder_layer_workspace_size.argtypes = [ci, i64, i64, i64, i64, i64]
    lib.encoder_layer_workspace_size.restype = sz
    lib.attn_status_string.argtypes = [ci]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    dp = ctypes.POINTER(ctypes.c_double)
    lib.probe_scratch_size.argtypes = []
    lib.probe_scratch_size.restype = sz
    lib.probe_mfma_bf16.argtypes = [vp, sz, i64, vp, dp, dp]
    lib.probe_mfma_bf16.restype = ci
    lib.probe_exp_f32.argtypes = [vp, sz, i64, vp, dp, dp]
    lib.probe_exp_f32.restype = ci
    lib.probe_lds_read.argtypes = [vp, sz, i64, ci, vp, dp, dp]
    lib.probe_lds_read.restype = ci
    lib.probe_hbm_copy.argtypes = [vp, vp, sz, ci, vp, dp]
    lib.probe_hbm_copy.restype = ci
    if path is None:
        _lib = lib
    return lib


def _check(status: int):
    if status != ATTN_OK:
        lib = load_library()
        raise AttnError(status, f"{lib.attn_status_string(status).decode()}: {lib.attn_last_error().decode()}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _mask_code(mask) -> int:
    if mask in (None, "none", ATTN_MASK_NONE, False):
        return ATTN_MASK_NONE
    if mask in ("causal", ATTN_MASK_CAUSAL, True):
        return ATTN_MASK_CAUSAL
    raise ValueError(f"mask must be 'none' or 'causal', got {mask!r}")


def _dev_tensor(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def sdpa_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask="none",
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """softmax(q k^T / sqrt(d_k)) v per (batch, head). q [B,h,n_q,d], k/v [B,h,n_k,d] -> [B,h,n_q,d], d in
    {32, 64, 128}."""
    lib = load_library()
    q, k, v = _dev_tensor(q, "q"), _dev_tensor(k, "k"), _dev_tensor(v, "v")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, h, n, d]")
    if not (q.dtype == k.dtype == v.dtype) or not (q.device == k.device == v.device):
        raise ValueError("q, k, v must share dtype and device")
    B, h, n_q, d_k = q.shape
    n_k, d_v = k.shape[2], v.shape[3]
    if k.shape != (B, h, n_k, d_k) or v.shape[:3] != (B, h, n_k):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if out is None:
        out = torch.empty((B, h, n_q, d_v), dtype=q.dtype, device=q.device)
    else:
        out = _dev_tensor(out, "out")
        if out.shape != (B, h, n_q, d_v) or out.dtype != q.dtype or out.device != q.device:
            raise ValueError("out has the wrong shape, dtype or device")
    _check(lib.sdpa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), _mask_code(mask), out.data_ptr(),
                            _dtype_code(q), B, h, n_q, n_k, d_k, d_v, _stream_handle(q.device)))
    return out


def _sdpa_shapes(q, k, v):
    q, k, v = _dev_tensor(q, "q"), _dev_tensor(k, "k"), _dev_tensor(v, "v")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, h, n, d]")
    if not (q.dtype == k.dtype == v.dtype) or not (q.device == k.device == v.device):
        raise ValueError("q, k, v must share dtype and device")
    B, h, n_q, d_k = q.shape
    n_k, d_v = k.shape[2], v.shape[3]
    if k.shape != (B, h, n_k, d_k) or v.shape[:3] != (B, h, n_k):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    return q, k, v, (B, h, n_q, n_k, d_k, d_v)


def _out_tensor(t, name, shape, dtype, device):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    t = _dev_tensor(t, name)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device:
        raise ValueError(f"{name} has the wrong shape, dtype or device")
    return t


def sdpa_forward_lse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask="none", out: torch.Tensor | None = None,
                     lse: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """sdpa_forward that also returns the row log-sum-exp of the scaled scores, lse [B,h,n_q] float32 (natural log),
    the statistic sdpa_backward needs."""
    lib = load_library()
    q, k, v, (B, h, n_q, n_k, d_k, d_v) = _sdpa_shapes(q, k, v)
    out = _out_tensor(out, "out", (B, h, n_q, d_v), q.dtype, q.device)
    lse = _out_tensor(lse, "lse", (B, h, n_q), torch.float32, q.device)
    _check(lib.sdpa_forward_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), _mask_code(mask), out.data_ptr(),
                                lse.data_ptr(), _dtype_code(q), B, h, n_q, n_k, d_k, d_v, _stream_handle(q.device)))
    return out, lse


def _kv_len_tensor(kv_len, B, device):
    kv_len = _dev_tensor(kv_len, "kv_len")
    if tuple(kv_len.shape) != (B,) or kv_len.dtype != torch.int32 or kv_len.device != device:
        raise ValueError("kv_len must be an int32 GPU tensor [B] on the inputs' device")
    return kv_len


def sdpa_forward_padded(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_len: torch.Tensor, mask="none",
                        out: torch.Tensor | None = None, lse: torch.Tensor | None = None, return_lse: bool = False):
    """Attention with a key padding mask: keys j >= kv_len[b] of batch entry b (int32 [B] on the GPU) get weight 0;
    rows with no real key give 0. Returns out, or (out, lse) with return_lse (or when `lse` is passed)."""
    lib = load_library()
    q, k, v, (B, h, n_q, n_k, d_k, d_v) = _sdpa_shapes(q, k, v)
    kv_len = _kv_len_tensor(kv_len, B, q.device)
    out = _out_tensor(out, "out", (B, h, n_q, d_v), q.dtype, q.device)
    want_lse = return_lse or lse is not None
    if want_lse:
        lse = _out_tensor(lse, "lse", (B, h, n_q), torch.float32, q.device)
    _check(lib.sdpa_forward_padded(q.data_ptr(), k.data_ptr(), v.data_ptr(), kv_len.data_ptr(), _mask_code(mask),
                                   out.data_ptr(), lse.data_ptr() if want_lse else None, _dtype_code(q), B, h, n_q,
                                   n_k, d_k, d_v, _stream_handle(q.device)))
    return (out, lse) if want_lse else out


def sdpa_forward_window(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, window: int, mask="none",
                        out: torch.Tensor | None = None, lse: torch.Tensor | None = None, return_lse: bool = False):
    """Restricted self-attention: query i sees keys j with |i - j| <= window (and j <= i with mask="causal").
    Returns out, or (out, lse) with return_lse (or when `lse` is passed)."""
    lib = load_library()
    q, k, v, (B, h, n_q, n_k, d_k, d_v) = _sdpa_shapes(q, k, v)
    out = _out_tensor(out, "out", (B, h, n_q, d_v), q.dtype, q.device)
    want_lse = return_lse or lse is not None
    if want_lse:
        lse = _out_tensor(lse, "lse", (B, h, n_q), torch.float32, q.device)
    _check(lib.sdpa_forward_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), int(window), _mask_code(mask),
                                   out.data_ptr(), lse.data_ptr() if want_lse else None, _dtype_code(q), B, h, n_q,
                                   n_k, d_k, d_v, _stream_handle(q.device)))
    return (out, lse) if want_lse else out


def sdpa_forward_train(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask="none", kv_len=None, window=None,
                       keep_f32: bool = True, out: torch.Tensor | None = None, out_f32: torch.Tensor | None = None,
                       lse: torch.Tensor | None = None):
    """The training forward pass for every mask (key padding with `kv_len`, restricted attention with `window`):
    returns (out, out_f32, lse). For bf16 inputs with keep_f32 (or when `out_f32` is passed), out_f32 [B,h,n_q,d]
    float32 is the output before its rounding to bf16, from which sdpa_backward forms D = dO . O; otherwise None."""
    lib = load_library()
    q, k, v, (B, h, n_q, n_k, d_k, d_v) = _sdpa_shapes(q, k, v)
    out = _out_tensor(out, "out", (B, h, n_q, d_v), q.dtype, q.device)
    lse = _out_tensor(lse, "lse", (B, h, n_q), torch.float32, q.device)
    want32 = q.dtype == torch.bfloat16 and (keep_f32 or out_f32 is not None)
    if want32:
        out_f32 = _out_tensor(out_f32, "out_f32", (B, h, n_q, d_v), torch.float32, q.device)
    kv_ptr = _kv_len_tensor(kv_len, B, q.device).data_ptr() if kv_len is not None else None
    _check(lib.sdpa_forward_train(q.data_ptr(), k.data_ptr(), v.data_ptr(), kv_ptr, -1 if window is None else int(window),
                                  _mask_code(mask), out.data_ptr(), out_f32.data_ptr() if want32 else None,
                                  lse.data_ptr(), _dtype_code(q), B, h, n_q, n_k, d_k, d_v, _stream_handle(q.device)))
    return out, (out_f32 if want32 else None), lse


def sdpa_backward_workspace_size(B: int, h: int, n_q: int, n_k: int, d_k: int = 64, d_v: int = 64,
                                 dtype: torch.dtype = torch.bfloat16) -> int:
    lib = load_library()
    code = ATTN_BF16 if dtype == torch.bfloat16 else ATTN_F32
    return int(lib.sdpa_backward_workspace_size(code, B, h, n_q, n_k, d_k, d_v))


def sdpa_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, dout: torch.Tensor,
                  lse: torch.Tensor, mask="none", dq: torch.Tensor | None = None, dk: torch.Tensor | None = None,
                  dv: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                  kv_len: torch.Tensor | None = None, window: int | None = None):
    """Gradients (dq, dk, dv) of attention given the forward's output `out`, its `lse` (from sdpa_forward_lse, or
    sdpa_forward_padded with the same `kv_len`) and the upstream gradient `dout` [B,h,n_q,d], d in {32, 64, 128}.
    For bf16 inputs `out` may be the float32 out_f32 of sdpa_forward_train (D = dO . O is then formed from the
    unrounded output). `workspace` (uint8, at least sdpa_backward_workspace_size bytes) may be passed in to avoid an
    allocation."""
    lib = load_library()
    q, k, v, (B, h, n_q, n_k, d_k, d_v) = _sdpa_shapes(q, k, v)
    out, dout, lse = _dev_tensor(out, "out"), _dev_tensor(dout, "dout"), _dev_tensor(lse, "lse")
    o32 = q.dtype == torch.bfloat16 and out.dtype == torch.float32
    for t, name, dt in ((out, "out", torch.float32 if o32 else q.dtype), (dout, "dout", q.dtype)):
        if tuple(t.shape) != (B, h, n_q, d_v) or t.dtype != dt or t.device != q.device:
            raise ValueError(f"{name} must be [B, h, n_q, d_v] like the forward output")
    if tuple(lse.shape) != (B, h, n_q) or lse.dtype != torch.float32 or lse.device != q.device:
        raise ValueError("lse must be float32 [B, h, n_q]")
    dq = _out_tensor(dq, "dq", q.shape, q.dtype, q.device)
    dk = _out_tensor(dk, "dk", k.shape, q.dtype, q.device)
    dv = _out_tensor(dv, "dv", v.shape, q.dtype, q.device)
    need = sdpa_backward_workspace_size(B, h, n_q, n_k, d_k, d_v, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    else:
        workspace = _dev_tensor(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size()
    kv_ptr = _kv_len_tensor(kv_len, B, q.device).data_ptr() if kv_len is not None else None
    _check(lib.sdpa_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                             lse.data_ptr(), kv_ptr, -1 if window is None else int(window), _mask_code(mask),
                             dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                             workspace.data_ptr(), ws_bytes, ATTN_BF16_F32O if o32 else _dtype_code(q), B, h, n_q,
                             n_k, d_k, d_v, _stream_handle(q.device)))
    return dq, dk, dv


class SDPAFunction(torch.autograd.Function):
    """torch.autograd wrapper: forward = sdpa_forward_train, backward = sdpa_backward (all in the HIP library). For
    bf16 the float32 output before rounding is kept for the backward pass (D = dO . O from the unrounded output)."""

    @staticmethod
    def forward(ctx, q, k, v, mask="none", kv_len=None, window=None):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        if window is not None and kv_len is not None:
            raise ValueError("a window with key padding is not supported")
        out, out32, lse = sdpa_forward_train(q, k, v, mask, kv_len=kv_len, window=window)
        ctx.save_for_backward(q, k, v, out if out32 is None else out32, lse)
        ctx.mask, ctx.kv_len, ctx.window = mask, kv_len, window
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, lse = ctx.saved_tensors
        dq, dk, dv = sdpa_backward(q, k, v, out, dout.contiguous(), lse, ctx.mask, kv_len=ctx.kv_len,
                                   window=ctx.window)
        return dq, dk, dv, None, None, None


def attention(q, k, v, mask="none", kv_len=None, window=None):
    """Differentiable attention on the HIP library: softmax(q k^T / sqrt(d_k)) v with gradients for q, k and v;
    `kv_len` (int32 [B] on the GPU) adds the key padding mask, `window` restricts each query to keys within that
    distance."""
    return SDPAFunction.apply(q, k, v, mask, kv_len, window)


def mha_workspace_size(B: int, n_q: int, n_k: int, h: int, d_k: int = 64, d_v: int = 64,
                       dtype: torch.dtype = torch.bfloat16) -> int:
    lib = load_library()
    code = ATTN_BF16 if dtype == torch.bfloat16 else ATTN_F32
    return int(lib.mha_workspace_size(code, B, n_q, n_k, h, d_k, d_v))


def mha_forward(xq: torch.Tensor, xkv: torch.Tensor, wq: torch.Tensor, wk: torch.Tensor, wv: torch.Tensor,
                wo: torch.Tensor, h: int, mask="none", out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Concat(head_1..head_h) W^O with head_i = Attention(xq W_i^Q, xkv W_i^K, xkv W_i^V); no biases.

    xq [B,n_q,d_model], xkv [B,n_k,d_model] (pass xq again for self-attention), wq/wk [d_model, h*d_k],
    wv [d_model, h*d_v], wo [h*d_v, d_model] -> [B, n_q, d_model]. `workspace` (uint8, at least
    mha_workspace_size bytes) may be passed in to avoid an allocation.
    """
    lib = load_library()
    ts = [_dev_tensor(t, n) for t, n in ((xq, "xq"), (xkv, "xkv"), (wq, "wq"), (wk, "wk"), (wv, "wv"), (wo, "wo"))]
    xq, xkv, wq, wk, wv, wo = ts
    if len({t.dtype for t in ts}) != 1 or len({t.device for t in ts}) != 1:
        raise ValueError("all inputs must share dtype and device")
    if xq.dim() != 3 or xkv.dim() != 3:
        raise ValueError("xq and xkv must be [B, n, d_model]")
    B, n_q, d_model = xq.shape
    n_k = xkv.shape[1]
    if xkv.shape != (B, n_k, d_model) or wq.shape[0] != d_model or wq.shape[1] % h or wv.shape[1] % h:
        raise ValueError("shape mismatch")
    d_k, d_v = wq.shape[1] // h, wv.shape[1] // h
    if wk.shape != wq.shape or wv.shape[0] != d_model or wo.shape != (h * d_v, d_model):
        raise ValueError("weight shape mismatch")
    need = mha_workspace_size(B, n_q, n_k, h, d_k, d_v, xq.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=xq.device)
    else:
        workspace = _dev_tensor(workspace, "workspace")
    if out is None:
        out = torch.empty((B, n_q, d_model), dtype=xq.dtype, device=xq.device)
    else:
        out = _dev_tensor(out, "out")
        if out.shape != (B, n_q, d_model) or out.dtype != xq.dtype:
            raise ValueError("out has the wrong shape or dtype")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.mha_forward(xq.data_ptr(), xkv.data_ptr(), wq.data_ptr(), wk.data_ptr(), wv.data_ptr(), wo.data_ptr(),
                           _mask_code(mask), out.data_ptr(), workspace.data_ptr(), ws_bytes, _dtype_code(xq),
                           B, n_q, n_k, d_model, h, d_k, d_v, _stream_handle(xq.device)))
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20  # ATTN_NOALLOC_SCRATCH_BYTES of the header


def mha_forward_noalloc(xq: torch.Tensor, xkv: torch.Tensor, wq: torch.Tensor, wk: torch.Tensor, wv: torch.Tensor,
                        wo: torch.Tensor, h: int, *, out: torch.Tensor, mask="none") -> torch.Tensor:
    """mha_forward with its intermediates in the library's own device scratch (no workspace argument, no allocation
    by the library; `out` must be passed in). Calls that overlap in time on one GPU race on that scratch."""
    lib = load_library()
    ts = [_dev_tensor(t, n) for t, n in ((xq, "xq"), (xkv, "xkv"), (wq, "wq"), (wk, "wk"), (wv, "wv"), (wo, "wo"))]
    xq, xkv, wq, wk, wv, wo = ts
    if len({t.dtype for t in ts}) != 1 or len({t.device for t in ts}) != 1:
        raise ValueError("all inputs must share dtype and device")
    if xq.dim() != 3 or xkv.dim() != 3:
        raise ValueError("xq and xkv must be [B, n, d_model]")
    B, n_q, d_model = xq.shape
    n_k = xkv.shape[1]
    if xkv.shape != (B, n_k, d_model) or wq.shape[0] != d_model or wq.shape[1] % h or wv.shape[1] % h:
        raise ValueError("shape mismatch")
    d_k, d_v = wq.shape[1] // h, wv.shape[1] // h
    if wk.shape != wq.shape or wv.shape[0] != d_model or wo.shape != (h * d_v, d_model):
        raise ValueError("weight shape mismatch")
    out = _dev_tensor(out, "out")
    if out.shape != (B, n_q, d_model) or out.dtype != xq.dtype:
        raise ValueError("out has the wrong shape or dtype")
    _check(lib.mha_forward_noalloc(xq.data_ptr(), xkv.data_ptr(), wq.data_ptr(), wk.data_ptr(), wv.data_ptr(),
                                   wo.data_ptr(), _mask_code(mask), out.data_ptr(), _dtype_code(xq),
                                   B, n_q, n_k, d_model, h, d_k, d_v, _stream_handle(xq.device)))
    return out


def encoder_layer_workspace_size(B: int, n: int, d_model: int, h: int, d_ff: int) -> int:
    return int(load_library().encoder_layer_workspace_size(ATTN_BF16, B, n, d_model, h, d_ff))


def encoder_layer_forward(x, wq, wk, wv, wo, ln1_gamma, ln1_beta, w1, b1, w2, b2, ln2_gamma, ln2_beta, h: int,
                          eps: float = 1e-5, mask="none", kv_len=None, out=None, workspace=None) -> torch.Tensor:
    """LayerNorm_2(H1 + FFN(H1)) with H1 = LayerNorm_1(x + MultiHead(x, x, x)); bf16 tensors (see
    include/mi355_attn.h): x [B,n,d_model], wq..wo [d_model,d_model], w1 [d_model,d_ff], b1 [d_ff],
    w2 [d_ff,d_model], b2 and the LayerNorm parameters [d_model]; kv_len (int32 [B]) adds key padding."""
    lib = load_library()
    named = (("x", x), ("wq", wq), ("wk", wk), ("wv", wv), ("wo", wo), ("ln1_gamma", ln1_gamma),
             ("ln1_beta", ln1_beta), ("w1", w1), ("b1", b1), ("w2", w2), ("b2", b2), ("ln2_gamma", ln2_gamma),
             ("ln2_beta", ln2_beta))
    ts = [_dev_tensor(t, nm) for nm, t in named]
    if any(t.dtype != torch.bfloat16 for t in ts) or len({t.device for t in ts}) != 1:
        raise ValueError("all tensors must be bfloat16 on one device")
    x = ts[0]
    if x.dim() != 3:
        raise ValueError("x must be [B, n, d_model]")
    B, n, d_model = x.shape
    d_ff = w1.shape[1] if w1.dim() == 2 else -1
    shapes = [(d_model, d_model)] * 4 + [(d_model,)] * 2 + [(d_model, d_ff), (d_ff,), (d_ff, d_model), (d_model,),
                                                            (d_model,), (d_model,)]
    for (nm, _), t, shp in zip(named[1:], ts[1:], shapes):
        if tuple(t.shape) != shp:
            raise ValueError(f"{nm} must be {shp}, got {tuple(t.shape)}")
    kv_ptr = _kv_len_tensor(kv_len, B, x.device).data_ptr() if kv_len is not None else None
    out = _out_tensor(out, "out", (B, n, d_model), x.dtype, x.device)
    need = encoder_layer_workspace_size(B, n, d_model, h, d_ff)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    else:
        workspace = _dev_tensor(workspace, "workspace")
    p = [t.data_ptr() for t in ts]
    _check(lib.encoder_layer_forward(p[0], kv_ptr, *p[1:], float(eps), _mask_code(mask), out.data_ptr(),
                                     workspace.data_ptr(), workspace.numel() * workspace.element_size(), ATTN_BF16,
                                     B, n, d_model, h, d_ff, _stream_handle(x.device)))
    return out


def _probe_scratch(device) -> torch.Tensor:
    lib = load_library()
    return torch.empty(int(lib.probe_scratch_size()), dtype=torch.uint8, device=device)


def probe_mfma_bf16(iters: int = 20000, device="cuda") -> tuple[float, float]:
    """Dense bf16 MFMA throughput with every CU busy: (TFLOP/s, shader clock in GHz). Synchronises the stream."""
    lib = load_library()
    dev = torch.device(device)
    scratch = _probe_scratch(dev)
    tf, ghz = ctypes.c_double(), ctypes.c_double()
    _check(lib.probe_mfma_bf16(scratch.data_ptr(), scratch.numel(), iters, _stream_handle(dev), ctypes.byref(tf),
                               ctypes.byref(ghz)))
    return tf.value, ghz.value


def probe_exp_f32(iters: int = 4000, device="cuda") -> tuple[float, float]:
    """v_exp_f32 throughput with every CU busy: (lane results per clock per CU, shader clock in GHz)."""
    lib = load_library()
    dev = torch.device(device)
    scratch = _probe_scratch(dev)
    rate, ghz = ctypes.c_double(), ctypes.c_double()
    _check(lib.probe_exp_f32(scratch.data_ptr(), scratch.numel(), iters, _stream_handle(dev), ctypes.byref(rate),
                             ctypes.byref(ghz)))
    return rate.value, ghz.value


def probe_lds_read(transposed: bool, iters: int = 20000, device="cuda") -> tuple[float, float]:
    """LDS read throughput with every CU busy, ds_read_b128 (transposed=False) or ds_read_b64_tr_b16 (True):
    (bytes per clock per CU, shader clock in GHz). Synchronises the stream."""
    lib = load_library()
    dev = torch.device(device)
    scratch = _probe_scratch(dev)
    rate, ghz = ctypes.c_double(), ctypes.c_double()
    _check(lib.probe_lds_read(scratch.data_ptr(), scratch.numel(), iters, 1 if transposed else 0, _stream_handle(dev),
                              ctypes.byref(rate), ctypes.byref(ghz)))
    return rate.value, ghz.value


def probe_hbm_copy(nbytes: int = 1 << 30, reps: int = 5, device="cuda") -> float:
    """Device-to-device copy bandwidth in GB/s (bytes read + written per second). Synchronises the stream."""
    lib = load_library()
    dev = torch.device(device)
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    gbps = ctypes.c_double()
    _check(lib.probe_hbm_copy(src.data_ptr(), dst.data_ptr(), nbytes, reps, _stream_handle(dev), ctypes.byref(gbps)))
    return gbps.value

"""MI355X (gfx950) scaled dot-product attention (forward and backward), multi-head attention and the encoder layer.

The computation lives in libmi355_attn.so (hand-written HIP kernels behind a C ABI, see include/mi355_attn.h, and
the measurement kernels of include/mi355_probe.h); this package is a thin ctypes binding with the same entry-point
names.
"""
from ._binding import (ATTN_BF16, ATTN_BF16_F32O, ATTN_ERR_HIP, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED,  # noqa: F401
                       ATTN_F32, ATTN_MASK_CAUSAL, ATTN_MASK_NONE, ATTN_OK, EXPORTED, LIB_PATH, AttnError,
                       SDPAFunction, attention, encoder_layer_forward, encoder_layer_workspace_size, load_library, mha_forward, mha_forward_noalloc, mha_workspace_size, probe_exp_f32, probe_lds_read,
                       probe_hbm_copy, probe_mfma_bf16, sdpa_backward, sdpa_backward_workspace_size, sdpa_forward,
                       sdpa_forward_lse, sdpa_forward_padded, sdpa_forward_train, sdpa_forward_window)

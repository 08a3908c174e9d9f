"""Float64 CPU oracle of the attention forward and backward passes and of the encoder layer around them.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the bench's CPU-baseline leg, never by
the library. It shares no code with the GPU path.
"""
from .attention import (encoder_layer_ref, ffn_ref, layer_norm_ref, mha_ref, sdpa_backward_head, sdpa_backward_ref, sdpa_brute, sdpa_head,  # noqa: F401
                        sdpa_lse_head, sdpa_lse_ref, sdpa_ref, sdpa_weights_head, sdpa_weights_ref)

"""CPU oracle for the frame-wise Gated DeltaNet forward and its backward pass.

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's CPU
baseline may import this package.  It shares no code with the GPU library.
"""
from .gdn_ref import (as_f64, frame_maps, transition, gdn_head, gdn_head_residual,
                      build_maps_head, state_pass_head, output_head, compose,
                      state_pass_chunked, tokenwise_gated_delta, flops_per_head_frame)
from .gdn_bwd import gdn_head_backward, scalar_loss
from .gate_ref import frame_gates, gdn_head_gated
from .attn_ref import Layout as AttnLayout, attn_head

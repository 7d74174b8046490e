"""Seeded synthetic inputs shared by the GPU tests and the oracle tests."""
from .configs import (Workload, WORKLOADS, TINY_F32, CLIP_5S, SEQ_60S, STREAM_60S,
                      STRESS_B4, BENCH_WORKLOAD, AttnWorkload, ATTN_60S, ATTN_WORKLOADS)
from .generate import (head_inputs, iter_heads, full_inputs, f32_to_bf16_bits,
                       bf16_bits_to_f32, default_workers, head_list, attn_head_inputs)

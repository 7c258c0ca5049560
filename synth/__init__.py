"""Seeded synthetic inputs shared by the CPU oracle, the tests and the benchmark.

This module only *draws* inputs; it holds none of the denoising step's arithmetic.
Every tensor comes from its own keyed numpy stream, so any slice (one layer, one
sequence, one chunk of rows) can be regenerated on its own and the result does not
depend on how the work was split.  Values are drawn in float32 and, for bfloat16
workloads, stored as bfloat16 bit patterns (round to nearest even); both the oracle
and the HIP path read those stored values, never a re-draw.

Workload shapes follow the block-diffusion denoiser of the pages: a
block of B [MASK] tokens refined by a denoiser tower that attends over a frozen
context tower's prefix K/V (poko-everyday.com Nemotron-TwoTower news item, section
技術/ビジネス面; dzen.guru "NVIDIA Nemotron 70B генерирует текст в 2,4 раза быстрее…",
section "Что нового": blocks of 16, confidence threshold gamma).
"""
from .workloads import WORKLOADS, Workload, get_workload  # noqa: F401
from .gen import (  # noqa: F401
    TowerInputs,
    MoeInputs,
    draw_tower,
    draw_moe,
    draw_prefix_lengths,
    draw_inv_temp,
    draw_prefix_kv,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
)

"""CPU oracle of the block-diffusion denoising step.  TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct numpy implementation in float64 of what the
denoising step computes.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import it; the product path (the HIP library
and its Python binding) never does, and shares no code with it.

Parity pins: every function here is pinned by `-m "not gpu"` tests against
library routines, closed forms, invariants and brute force (tests/test_oracle_*.py).
The whole-step composition has no worked example on the pages to compare with;
it is pinned only through the invariants of the loop (gamma=0 / gamma>1 closed
forms, monotone commits, equivariance, zero-head case) and is otherwise
"parity unpinned" against published numbers.
"""
from .denoise import (  # noqa: F401
    round_bf16,
    rmsnorm,
    gelu,
    moe_route,
    moe_ffn,
    joint_attention,
    OracleTower,
    vocab_reduce,
    commit_rule,
    RULE_THRESHOLD,
    RULE_LEFT_TO_RIGHT,
    StepResult,
    oracle_step,
    oracle_generate,
    OracleContextTower,
    oracle_generate_blocks,
    oracle_ar_decode,
)

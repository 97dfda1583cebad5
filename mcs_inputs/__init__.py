"""Seeded synthetic inputs for MC-Sparse (Meta-Cached Sparse Attention).

This package only draws and shapes data: DiT-like Q/K/V with 3D positional
locality, per-step drift, the hash projection matrix and the per-head keep
budgets of each workload. It contains none of the method's arithmetic (no
attention, no hashing, no selection), so both the GPU path and the CPU oracle
can take their inputs from it without sharing any of the method.
"""

from .generator import (  # noqa: F401
    STREAM_W, STREAM_EQ, STREAM_EK, STREAM_EV, STREAM_DQ, STREAM_DK, STREAM_DV,
    STREAM_PROJ, STREAM_KEEP, STREAM_TEXT,
    position_embedding, text_embedding, token_embedding, head_rotation, head_base, head_step, hash_projections,
    keep_draw, round_bf16, bf16_bits, rng,
)
from .configs import Workload, WORKLOADS, keep_count, workload  # noqa: F401

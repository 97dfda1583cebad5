"""The five synthetic workloads (sizes, keep budgets, drift schedules).

Workload 1 is the tiny fp32 case an exact CPU implementation finishes in
seconds; 2 and 3 are single video-DiT attention layers; 4 is a 3D-asset DiT
layer with a per-head keep budget; 5 is a full denoising-loop sweep; 6 is the
joint attention of an MM-DiT block, workload 2's video tokens followed by text
tokens in one sequence.  The
pages name the two model families (a video DiT and a 3D asset generator) but
none of their shapes, so the shapes here are DiT-typical stand-ins.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from .generator import keep_draw


def keep_count(frac: float, n: int) -> int:
    """Integer keep budget for a keep fraction.

    A fraction below 1 keeps max(64, floor(frac * n / 64) * 64) tokens (a whole
    number of 64-token tiles); a fraction of 1 keeps all n tokens.
    """
    if frac >= 1.0:
        return n
    return max(64, int(math.floor(frac * n / 64.0)) * 64)


@dataclass(frozen=True)
class Workload:
    wid: int                      # workload id (also a seed-stream key)
    name: str
    grid: tuple                   # (T, Y, X)
    heads: int
    head_dim: int
    dtype: str                    # "fp32" | "bf16"
    group: int                    # query group size G
    keep_frac: tuple              # per-head keep fractions (or one shared value)
    reuse_steps: int              # reuse steps after each selection
    drift: float                  # delta in X_t = X_0 + delta * t * E_t
    reselect: int = 0             # re-selection interval (0 = select once)
    keep_override: int | None = None
    sweep: dict = field(default_factory=dict)
    text: int = 0                 # text tokens after the grid tokens (joint attention)

    @property
    def seq_len(self) -> int:
        return int(np.prod(self.grid)) + self.text

    @property
    def num_groups(self) -> int:
        return -(-self.seq_len // self.group)

    def keeps(self, seed: int = 0) -> np.ndarray:
        """Per-head integer keep budgets (int32 [heads])."""
        n = self.seq_len
        if self.keep_override is not None:
            return np.full(self.heads, self.keep_override, dtype=np.int32)
        if len(self.keep_frac) == 1:
            return np.full(self.heads, keep_count(self.keep_frac[0], n), dtype=np.int32)
        fr = keep_draw(seed, self.wid, self.heads, self.keep_frac)
        return np.array([keep_count(f, n) for f in fr], dtype=np.int32)

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    1: Workload(1, "tiny fp32, 1 head, 8x8x16", (8, 8, 16), 1, 64, "fp32", 64, (0.125,), 3, 0.02,
                keep_override=128),
    2: Workload(2, "video-DiT layer, 24 heads, 16x30x52", (16, 30, 52), 24, 128, "bf16", 64, (0.10,), 10, 0.02),
    3: Workload(3, "long video-DiT layer, 24 heads, 21x45x80", (21, 45, 80), 24, 128, "bf16", 64, (0.05,), 20,
                0.01),
    4: Workload(4, "3D-asset-DiT layer, 16 heads, 32^3", (32, 32, 32), 16, 64, "bf16", 128,
                (0.0625, 0.125, 0.25), 15, 0.02),
    5: Workload(5, "denoising-loop sweep, 40 heads, 21x30x52", (21, 30, 52), 40, 128, "bf16", 64, (0.10,), 9,
                0.02, reselect=10,
                sweep={"keep": (0.02, 0.05, 0.10, 0.25, 1.0), "group": (64, 128), "steps": 30}),
    6: Workload(6, "joint video+text DiT layer, 24 heads, 16x30x52 + 226 text", (16, 30, 52), 24, 128, "bf16", 64,
                (0.10,), 10, 0.02, text=226),
}


def workload(wid: int) -> Workload:
    return WORKLOADS[wid]

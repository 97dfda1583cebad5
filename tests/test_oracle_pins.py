"""The oracle against its pins (no GPU)."""

import numpy as np
import pytest

import oracle.mcs_oracle as orc
from oracle_checks import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(orc)


def test_group_ranges_ragged():
    assert orc.group_ranges(10, 4) == [(0, 4), (4, 8), (8, 10)]
    assert orc.group_ranges(8, 4) == [(0, 4), (4, 8)]
    assert orc.group_ranges(0, 4) == []


def test_topk_rejects_bad_keep():
    with pytest.raises(ValueError):
        orc.topk_select(np.ones(4), 0)
    with pytest.raises(ValueError):
        orc.topk_select(np.ones(4), 5)


def test_reuse_zero_drift_equals_dense():
    """With no drift every reuse step sees the selection inputs, so every
    step reproduces dense attention (residual identity, step by step)."""
    r = np.random.default_rng(0)
    n, d, g = 96, 8, 16
    q = (r.standard_normal((n, d)) * 2).astype(np.float32)
    k, v = r.standard_normal((n, d)) * 2, r.standard_normal((n, d))
    proj = r.standard_normal((8, d)).astype(np.float32)
    meta = orc.select_head(q, k, v, proj, g, 12, 0.3)
    dense = orc.dense_attention(q, k, v, 0.3)
    for _ in range(3):
        out = orc.reuse_head(q, k, v, meta, 0.3)
        assert np.max(np.abs(out - dense)) < 1e-12

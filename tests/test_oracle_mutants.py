"""Plant plausible mistakes in the oracle (on the CPU) and check that the
pins catch every one of them."""

import math

import numpy as np
import pytest

import oracle.mcs_oracle as orc
from oracle_checks import ALL_CHECKS


def _hash_ge(q, proj):
    acc = np.asarray(q, np.float64) @ np.asarray(proj, np.float64).T
    return sum(((acc[:, b] >= 0).astype(np.int64) << b) for b in range(acc.shape[1])).astype(np.uint8)


def _hash_msb_first(q, proj):
    acc = np.asarray(q, np.float64) @ np.asarray(proj, np.float64).T
    nb = acc.shape[1]
    return sum(((acc[:, b] > 0).astype(np.int64) << (nb - 1 - b)) for b in range(nb)).astype(np.uint8)


def _perm_unstable(keys):
    n = len(keys)
    return np.lexsort((-np.arange(n), np.asarray(keys, np.int64))).astype(np.int32)


def _attention_noscale(q, k, v, scale):
    return orc.softmax_rows(np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)[0] @ np.asarray(v, np.float64), \
        orc.softmax_rows(np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)[0]


def _attention_vlogits(q, k, v, scale):
    p = orc.softmax_rows(scale * (np.asarray(q, np.float64) @ np.asarray(v, np.float64).T))[0]
    return p @ np.asarray(v, np.float64), p


def _scores_max(p_rows):
    return np.asarray(p_rows, np.float64).max(axis=0)


def _topk_ties_high(c, k):
    c32 = np.asarray(c, np.float64).astype(np.float32).astype(np.float64)
    n = len(c32)
    order = np.lexsort((-np.arange(n), -c32))
    gap = math.inf if k == n else float(c32[order[k - 1]] - c32[order[k]])
    return np.sort(order[:k]).astype(np.int32), gap


def _topk_smallest(c, k):
    order = np.argsort(np.asarray(c), kind="stable")
    return np.sort(order[:k]).astype(np.int32), 0.0


def _sparse_unnormalised(q, k, v, idx, scale):
    _, p = orc.attention(q, k, v, scale)
    idx = np.asarray(idx, np.int64)
    return p[:, idx] @ np.asarray(v, np.float64)[idx]


def _select_residual_flipped(q, k, v, rows, keep, scale, kv_block=1, residual=True, **kw):
    s = orig_select(q, k, v, rows, keep, scale, kv_block, residual, **kw)
    s.residual = -s.residual
    return s


def _select_ignores_no_residual(q, k, v, rows, keep, scale, kv_block=1, residual=True, **kw):
    return orig_select(q, k, v, rows, keep, scale, kv_block, True, **kw)


def _block_scores_max(c, block):
    return np.asarray(c, np.float64).reshape(-1, block).max(axis=1)


def _topk_blocks_first_key(c, k, block):
    # ranks blocks by their first key only
    bidx, gap = orc.topk_select(np.asarray(c, np.float64)[::block], k // block)
    idx = (bidx.astype(np.int64)[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    return idx.astype(np.int32), gap, bidx


def _centred_hash_uncentred(q, proj):
    return orc.hash_keys(q, proj)


def _mean_first_half(q):
    q64 = np.asarray(q, np.float64)
    return q64[: q64.shape[0] // 2].mean(axis=0)


def _morton_xy_swapped(grid):
    tt, yy, xx = np.meshgrid(*(np.arange(n) for n in grid), indexing="ij")
    code = orc.morton_code(tt.ravel(), xx.ravel(), yy.ravel())
    return np.argsort(code, kind="stable").astype(np.int32)


def _morton_code_t_low(t, y, x):
    return orig_morton_code(y, x, t)


def _raster_reversed(n):
    return np.arange(n - 1, -1, -1, dtype=np.int32)


def _reuse_no_residual(q_t, k_t, v_t, rows, idx, residual, scale):
    qg = np.asarray(q_t)[np.asarray(rows, np.int64)]
    return orc.sparse_attention(qg, k_t, v_t, idx, scale)


def _mass_no_cap(c, mass, group_len, cap):
    return orig_mass_count(c, mass, group_len, len(c))


def _mass_from_smallest(c, mass, group_len, cap):
    c32 = np.asarray(c, np.float64).astype(np.float32).astype(np.float64)
    target = mass * group_len
    prefix = np.cumsum(np.sort(c32))
    hit = np.nonzero(prefix >= target)[0]
    return max(1, min(int(hit[0]) + 1 if hit.size else len(c), cap))


def _mass_one_more(c, mass, group_len, cap):
    return min(orig_mass_count(c, mass, group_len, cap) + 1, cap)


def _mass_over_n(c, mass, group_len, cap):
    return orig_mass_count(c, mass * len(c) / group_len, group_len, cap)


def _bf16_truncate(x):
    f = np.ascontiguousarray(np.asarray(x, np.float64).astype(np.float32))
    return (f.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)


orig_select = orc.select_group
orig_mass_count = orc.mass_keep_count
orig_morton_code = orc.morton_code

MUTANTS = {
    "hash >= 0": ("hash_keys", _hash_ge),
    "hash bit order": ("hash_keys", _hash_msb_first),
    "unstable sort": ("group_permutation", _perm_unstable),
    "scale dropped": ("attention", _attention_noscale),
    "logits against V": ("attention", _attention_vlogits),
    "group score = max": ("group_scores", _scores_max),
    "ties to higher index": ("topk_select", _topk_ties_high),
    "keeps smallest scores": ("topk_select", _topk_smallest),
    "no renormalisation": ("sparse_attention", _sparse_unnormalised),
    "residual sign": ("select_group", _select_residual_flipped),
    "reuse drops residual": ("reuse_group", _reuse_no_residual),
    "no-residual option ignored": ("select_group", _select_ignores_no_residual),
    "block score = max": ("block_scores", _block_scores_max),
    "block ranked by first key": ("topk_blocks", _topk_blocks_first_key),
    "raster order reversed": ("raster_permutation", _raster_reversed),
    "centred hash not centred": ("centred_hash_keys", _centred_hash_uncentred),
    "mean over half the queries": ("query_mean", _mean_first_half),
    "morton x and y swapped": ("morton_permutation", _morton_xy_swapped),
    "morton t in the low bit": ("morton_code", _morton_code_t_low),
    "mass budget ignores the cap": ("mass_keep_count", _mass_no_cap),
    "mass counted from the smallest scores": ("mass_keep_count", _mass_from_smallest),
    "mass budget one key too many": ("mass_keep_count", _mass_one_more),
    "mass target relative to N": ("mass_keep_count", _mass_over_n),
    "bf16 residual truncated": ("round_bf16", _bf16_truncate),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    failed = []
    for check in ALL_CHECKS:
        try:
            check(orc)
        except (AssertionError, ValueError, IndexError):
            failed.append(check.__name__)
    assert failed, f"mutant '{name}' passed every pin"

"""CPU oracle for Meta-Cached Sparse Attention (MC-Sparse).

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and
the CPU-baseline leg of the benchmark may import or run this module.  The GPU
library never calls it and shares no code with it.

It is a plain, slow, obviously-correct statement of what the method computes,
in float64 with numpy, one (head, query-group) unit at a time.  Sources (page
titles as given by the pages):

* [ABS]  "MC-Sparse: Deconstructing and Closing the Dense-Sparse Attention Gap
  in Diffusion Transformers", arXiv abstract: individual KV tokens are chosen
  with exact attention probabilities; similar queries are organised into
  tile-aligned groups; the cache holds the query groups, the kept KV indices
  and the difference of the dense and sparse outputs, and later denoising
  steps reuse it.
* [BLOG] "The quality cliff nobody admits to", section "MC-Sparse: three
  failure modes, one fix" (same three cached items, computed once and reused)
  and section "What Trips People Up" (renormalising over the kept tokens moves
  probability mass; the residual is the correction).
* [NARROW] "MC-Sparse Narrows the Dense-Sparse Attention Gap in Diffusion
  Transformers", the list of three design choices (individual KV selection,
  hardware-aware query organisation, metadata and residual reuse).

The pages give no formula, so the readings taken where they are silent are:

* grouping: an 8-bit sign hash of the queries against 8 random projections,
  a stable sort of the tokens by that key, then consecutive runs of G sorted
  tokens form the groups (the last group may be short);
* a group's score for key j is the sum over the group's queries of the exact
  softmax probability P_ij (the probability mass the group keeps on j);
* top-k by that score, ties to the lower key index, indices stored ascending;
  the comparison is made on the scores rounded to float32, the precision in
  which the GPU kernel decides;
* sparse attention is softmax attention restricted to the kept keys
  (renormalised over them); the residual O_dense - O_sparse is kept per query
  (in sorted order) and added back unchanged on every reuse step.

The ablations of the three failure modes the pages name ([ABS] and [BLOG]
"MC-Sparse: three failure modes, one fix": groups that force one pattern on
unlike queries, a selection that misjudges which interactions matter, and the
attention mass of the dropped tokens) swap
one choice each: raster-order query groups instead of hash groups, whole
64-token KV blocks ranked by their summed score instead of individual tokens,
and no residual (the renormalised sparse output alone).  A fourth variant
changes the grouping the other way: the sign hash of the queries centred on
their per-head mean, so that a component shared by all queries does not fix
most of the bits.  A fifth groups the tokens of a (T, Y, X) latent grid in
Morton (Z-curve) order, so that a group of G = 64 tokens is a 4 x 4 x 4
block of the grid: spatially compact queries, the similar queries of a
position-driven DiT.

Two extensions beyond the pages: a per-group keep budget from a retained
probability-mass target (the fewest keys whose group scores reach a fraction
of the group's mass, capped by the head's budget -- per-head budgets
generalised, as the benchmark's 3D-asset workload draws them per head), and
a residual cached in bfloat16 instead of float32 (half the cache; the
per-step metadata cache is the extra cost the table "Three approaches at a
glance" of "The quality cliff nobody admits to" charges to MC-Sparse).

Parity pins for every function live in tests/test_oracle_pins.py.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

HASH_BITS = 8


# ---------------------------------------------------------------------------
# Query grouping ([ABS]: similar queries share a tile-aligned group;
# [NARROW]: the hardware-aware query organisation among its design choices).
# ---------------------------------------------------------------------------

def hash_keys(q: np.ndarray, proj: np.ndarray) -> np.ndarray:
    """8-bit sign hash of every query row.

    key_i = sum_b [q_i . r_b > 0] * 2^b.  The dot product is accumulated in
    float64 in the order c = 0..d-1; every product of a float32 (or bf16)
    value with a float32 projection is exact in float64, so the sum is one
    well-defined float64 value per (i, b).  A dot product of exactly zero
    gives bit 0.
    """
    q64 = np.asarray(q, dtype=np.float64)
    r64 = np.asarray(proj, dtype=np.float64)
    n, d = q64.shape
    nb = r64.shape[0]
    acc = np.zeros((n, nb), dtype=np.float64)
    for c in range(d):
        acc = acc + q64[:, c:c + 1] * r64[None, :, c]
    keys = np.zeros(n, dtype=np.int64)
    for b in range(nb):
        keys |= (acc[:, b] > 0.0).astype(np.int64) << b
    return keys.astype(np.uint8)


def query_mean(q: np.ndarray) -> np.ndarray:
    """Per-dimension mean of one head's queries: float64 sums accumulated in
    token order (i = 0, 1, ..., N-1), then one division by N."""
    q64 = np.asarray(q, dtype=np.float64)
    return np.cumsum(q64, axis=0)[-1] / q64.shape[0]


def centred_hash_keys(q: np.ndarray, proj: np.ndarray) -> np.ndarray:
    """Sign hash of the centred queries q_i - mean.  Every step is one
    rounded float64 operation: the subtraction, then for c = 0..d-1 the
    product (q_ic - mean_c) * r_bc and its addition to the running sum (no
    fused multiply-add), so the keys are one well-defined value."""
    x = np.asarray(q, dtype=np.float64) - query_mean(q)[None, :]
    r64 = np.asarray(proj, dtype=np.float64)
    n, d = x.shape
    nb = r64.shape[0]
    acc = np.zeros((n, nb), dtype=np.float64)
    for c in range(d):
        acc = acc + x[:, c:c + 1] * r64[None, :, c]
    keys = np.zeros(n, dtype=np.int64)
    for b in range(nb):
        keys |= (acc[:, b] > 0.0).astype(np.int64) << b
    return keys.astype(np.uint8)


def group_permutation(keys: np.ndarray) -> np.ndarray:
    """perm[p] = original token at sorted position p (stable sort by key)."""
    return np.argsort(np.asarray(keys, dtype=np.int64), kind="stable").astype(np.int32)


def raster_permutation(n: int) -> np.ndarray:
    """Ablation of the grouping: groups are runs of G tokens in raster order."""
    return np.arange(n, dtype=np.int32)


def morton_code(t: np.ndarray, y: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Z-curve code of grid cells: bit b of x, y, t goes to bit 3b, 3b + 1,
    3b + 2 of the code (10 bits per axis)."""
    code = np.zeros(np.shape(x), dtype=np.int64)
    for b in range(10):
        code |= (((np.asarray(x) >> b) & 1) << (3 * b)) | (((np.asarray(y) >> b) & 1) << (3 * b + 1)) | \
                (((np.asarray(t) >> b) & 1) << (3 * b + 2))
    return code


def morton_permutation(grid, n: int | None = None) -> np.ndarray:
    """Tokens of a raster-ordered (T, Y, X) grid (token = (t * Y + y) * X + x)
    sorted by their Z-curve code; the tokens from T*Y*X to n - 1 (the text
    tokens of a joint video + text sequence) follow in index order."""
    tt, yy, xx = np.meshgrid(*(np.arange(m) for m in grid), indexing="ij")
    code = morton_code(tt.ravel(), yy.ravel(), xx.ravel())
    grid_perm = np.argsort(code, kind="stable").astype(np.int32)
    n_grid = grid_perm.size
    n = n_grid if n is None else n
    if n < n_grid:
        raise ValueError("the grid holds more tokens than the sequence")
    return np.concatenate([grid_perm, np.arange(n_grid, n, dtype=np.int32)])


def group_ranges(n: int, group: int):
    """Sorted-position ranges [start, end) of the ceil(n/group) query groups."""
    return [(s, min(n, s + group)) for s in range(0, n, group)]


# ---------------------------------------------------------------------------
# Exact attention ([ABS]: the kept KV indices are chosen from the exact
# softmax probabilities).
# ---------------------------------------------------------------------------

def softmax_rows(s: np.ndarray):
    """Row softmax of float64 logits: returns (P, row max m, row sum l)."""
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return e / l, m[:, 0], l[:, 0]


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Softmax attention of rows q over keys k / values v (all float64).

    Returns (O, P) with S = scale * q k^T, P = row softmax of S, O = P v.
    """
    q64 = np.asarray(q, dtype=np.float64)
    k64 = np.asarray(k, dtype=np.float64)
    v64 = np.asarray(v, dtype=np.float64)
    s = scale * (q64 @ k64.T)
    p, _, _ = softmax_rows(s)
    return p @ v64, p


def dense_attention(q, k, v, scale):
    """Dense output O[N, d] of one head (float64)."""
    o, _ = attention(q, k, v, scale)
    return o


# ---------------------------------------------------------------------------
# Selection ([ABS], [NARROW] and [BLOG]: each group keeps individual KV
# tokens, ranked by exact attention probabilities).
# ---------------------------------------------------------------------------

def group_scores(p_rows: np.ndarray) -> np.ndarray:
    """c(j) = sum over the group's query rows i of P_ij (float64 [N])."""
    return np.asarray(p_rows, dtype=np.float64).sum(axis=0)


def topk_select(c: np.ndarray, k: int):
    """Top-k keys of a group's scores.

    The scores are compared as float32 values; order is score descending,
    then key index ascending.  Returns (idx ascending int32 [k], gap) where
    gap = c_(k) - c_(k+1) in the float32 scores (inf when k == N).
    """
    c32 = np.asarray(c, dtype=np.float64).astype(np.float32).astype(np.float64)
    n = c32.shape[0]
    if not 1 <= k <= n:
        raise ValueError(f"keep {k} outside [1, {n}]")
    order = np.lexsort((np.arange(n), -c32))
    idx = np.sort(order[:k]).astype(np.int32)
    gap = math.inf if k == n else float(c32[order[k - 1]] - c32[order[k]])
    return idx, gap


MASS_FRAC_BITS = 48


def mass_keep_count(c: np.ndarray, mass: float, group_len: int, cap: int) -> int:
    """Per-group budget from a retained-mass target (an extension of the
    per-head budgets of the benchmark's 3D-asset workload; the pages fix
    none): the fewest keys, taken in the top-k order of the group's scores,
    whose scores add up to at least `mass` of the group's total probability
    mass |g| (the scores of a group sum to its number of queries), at most
    `cap` and at least 1.  When even all keys fall short, all are needed (then
    the cap).

    The sum is decided exactly: every float32 score is a fixed-point integer
    of 2^-48 units (floor), the target is ceil(mass * |g| * 2^48), and the
    prefix sums in the top-k order (score descending, index ascending) are
    integers, so the count does not depend on a summation order."""
    c32 = np.asarray(c, dtype=np.float64).astype(np.float32).astype(np.float64)
    n = c32.shape[0]
    if not 1 <= cap <= n:
        raise ValueError(f"cap {cap} outside [1, {n}]")
    q = np.floor(np.ldexp(c32, MASS_FRAC_BITS)).astype(np.int64)
    target = math.ceil(float(np.float32(mass)) * group_len * 2.0 ** MASS_FRAC_BITS)
    order = np.lexsort((np.arange(n), -c32))
    prefix = np.cumsum(q[order])
    hit = np.nonzero(prefix >= target)[0]
    m = int(hit[0]) + 1 if hit.size else n
    return max(1, min(m, cap))


def topk_mass_select(c: np.ndarray, mass: float, group_len: int, cap: int):
    """The kept keys under a retained-mass target: the top mass_keep_count
    keys (ascending), with the float32-score gap after the last one."""
    n = mass_keep_count(c, mass, group_len, cap)
    idx, gap = topk_select(c, n)
    return idx, gap, n


def round_bf16(x: np.ndarray) -> np.ndarray:
    """x rounded to float32, then to bfloat16 (round to nearest, ties to
    even), returned as float64: the storage of a bf16 cached residual."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def block_scores(c: np.ndarray, block: int) -> np.ndarray:
    """Score of each run of `block` consecutive keys: the sum of the group's
    key scores over the run (float64 [N / block])."""
    c = np.asarray(c, dtype=np.float64)
    if c.shape[0] % block:
        raise ValueError(f"{c.shape[0]} keys do not split into blocks of {block}")
    return c.reshape(-1, block).sum(axis=1)


def topk_blocks(c: np.ndarray, k: int, block: int):
    """Ablation of the selection granularity ([BLOG]: dropping whole blocks
    evicts tokens one wanted to keep): keep the k / block key blocks with the
    largest block scores (compared as float32, ties to the lower block), and
    with them every key of those blocks.  Returns (idx ascending int32 [k],
    gap between the kept and the first dropped block score, kept block ids)."""
    if k % block:
        raise ValueError(f"keep {k} is not a multiple of the block size {block}")
    bidx, gap = topk_select(block_scores(c, block), k // block)
    idx = (bidx.astype(np.int64)[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    return idx.astype(np.int32), gap, bidx


def sparse_attention(q, k, v, idx, scale):
    """Attention of rows q over the kept keys idx only (renormalised)."""
    idx = np.asarray(idx, dtype=np.int64)
    o, _ = attention(q, np.asarray(k)[idx], np.asarray(v)[idx], scale)
    return o


@dataclass
class GroupSelection:
    rows: np.ndarray        # original token ids of the group's queries (sorted order)
    scores: np.ndarray      # c(j), float64 [N]
    idx: np.ndarray         # kept keys, ascending int32 [k]
    gap: float              # float32-score gap between the k-th and (k+1)-th key
    o_dense: np.ndarray     # float64 [|g|, d]
    o_sparse: np.ndarray    # float64 [|g|, d]
    residual: np.ndarray    # o_dense - o_sparse, float64 [|g|, d]


def select_group(q, k, v, rows, keep, scale, kv_block=1, residual=True, keep_mass=0.0,
                 residual_bf16=False) -> GroupSelection:
    """Selection step for one query group ([ABS], [BLOG] "MC-Sparse: three
    failure modes, one fix"): exact dense rows, group scores, top-k, sparse
    rows over the kept keys and the residual between the two.

    Ablations: kv_block > 1 keeps whole key blocks (topk_blocks); residual
    False caches a zero residual, so reuse returns the renormalised sparse
    output alone.  Extensions: keep_mass > 0 keeps the fewest keys reaching
    that retained mass, at most `keep` (topk_mass_select); residual_bf16
    caches the residual rounded to bfloat16 (round_bf16)."""
    rows = np.asarray(rows, dtype=np.int64)
    qg = np.asarray(q)[rows]
    o_d, p = attention(qg, k, v, scale)
    c = group_scores(p)
    if kv_block == 1 and keep_mass > 0:
        idx, gap, _ = topk_mass_select(c, keep_mass, len(rows), keep)
    elif kv_block == 1:
        idx, gap = topk_select(c, keep)
    else:
        idx, gap, _ = topk_blocks(c, keep, kv_block)
    o_s = sparse_attention(qg, k, v, idx, scale)
    res = o_d - o_s if residual else np.zeros_like(o_d)
    if residual_bf16:
        res = round_bf16(res)
    return GroupSelection(rows.astype(np.int32), c, idx, gap, o_d, o_s, res)


def reuse_group(q_t, k_t, v_t, rows, idx, residual, scale):
    """Reuse step for one group: sparse attention over the cached keys on the
    step-t inputs plus the cached residual ([ABS]: metadata "reuses them
    across subsequent denoising steps"; [BLOG] "What Trips People Up": the
    residual restores what renormalisation loses)."""
    qg = np.asarray(q_t)[np.asarray(rows, dtype=np.int64)]
    return sparse_attention(qg, k_t, v_t, idx, scale) + residual


# ---------------------------------------------------------------------------
# Whole-head drivers (loops over the units above).
# ---------------------------------------------------------------------------

@dataclass
class HeadMeta:
    perm: np.ndarray                 # int32 [N]
    keys: np.ndarray                 # uint8 [N]
    groups: list                     # GroupSelection per group


def select_head(q, k, v, proj, group, keep, scale, groups=None, grouping="hash", kv_block=1,
                residual=True, grid=None, keep_mass=0.0, residual_bf16=False) -> HeadMeta:
    """Selection for one head; `groups` restricts the work to a subset of
    group ids (the permutation always covers the whole head).  `grouping`
    "raster" replaces the hash groups by raster-order runs (keys are then 0);
    "centred" hashes the queries centred on their mean; "morton" orders the
    tokens of the (T, Y, X) `grid` along the Z-curve."""
    n = q.shape[0]
    if grouping == "hash":
        keys = hash_keys(q, proj)
        perm = group_permutation(keys)
    elif grouping == "centred":
        keys = centred_hash_keys(q, proj)
        perm = group_permutation(keys)
    elif grouping == "raster":
        keys = np.zeros(n, dtype=np.uint8)
        perm = raster_permutation(n)
    elif grouping == "morton":
        if grid is None or int(np.prod(grid)) > n:
            raise ValueError("morton grouping needs the (T, Y, X) grid of the tokens")
        keys = np.zeros(n, dtype=np.uint8)
        perm = morton_permutation(grid, n)
    else:
        raise ValueError(f"unknown grouping {grouping!r}")
    ranges = group_ranges(n, group)
    gids = range(len(ranges)) if groups is None else groups
    sel = {g: select_group(q, k, v, perm[ranges[g][0]:ranges[g][1]], keep, scale, kv_block, residual,
                           keep_mass=keep_mass, residual_bf16=residual_bf16)
           for g in gids}
    return HeadMeta(perm, keys, sel)


def reuse_head(q_t, k_t, v_t, meta: HeadMeta, scale, residuals=None, idxs=None):
    """Reuse output in original token order for the selected groups of one
    head (rows of groups not in meta stay NaN).  `residuals`/`idxs` override
    the cached residual / kept keys per group (to evaluate another side's
    metadata)."""
    n, d = q_t.shape
    out = np.full((n, np.asarray(v_t).shape[1]), np.nan)
    for g, s in meta.groups.items():
        r = s.residual if residuals is None else residuals[g]
        ix = s.idx if idxs is None else idxs[g]
        out[s.rows] = reuse_group(q_t, k_t, v_t, s.rows, ix, r, scale)
    return out

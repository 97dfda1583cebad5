"""Checks that pin the CPU oracle to facts outside itself.

Each check takes an object exposing the oracle's functions, so the same
checks run against the real oracle (tests/test_oracle_pins.py) and against
deliberately broken copies of it (tests/test_oracle_mutants.py), which must
fail at least one of them.

What the checks compare against:
* hand-derived values in tests/golden/*.json (each with its derivation);
* exact rational arithmetic (fractions.Fraction) for the hash signs;
* torch.nn.functional.scaled_dot_product_attention in float64 on the CPU
  (a library routine) for dense and masked (sparse) attention;
* brute-force enumeration of every k-subset of keys on tiny inputs for the
  top-k selection (the kept set must maximise the group's retained
  probability mass, computed from torch.softmax, not from the oracle);
* invariants the method fixes: keeping every key reproduces dense attention
  and a zero residual; reuse on unchanged inputs reproduces dense; a group of
  one query is per-query top-k attention;
* for the failure-mode ablations: brute force over every choice of whole key
  blocks (block selection), the identity order together with a hash whose
  keys all agree (raster groups), and library masked attention (no residual);
* for the retained-mass budgets: exact rational brute force over every key
  subset of tiny rows, closed forms, and the retained mass computed from
  library softmax; for the bf16 residual: torch's bfloat16 conversion.
"""

from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _sdpa(q, k, v, scale, mask=None):
    """Library attention in float64 on the CPU; mask: bool [n_q, n_k] (True = keep)."""
    qt = torch.tensor(np.asarray(q, dtype=np.float64))[None, None]
    kt = torch.tensor(np.asarray(k, dtype=np.float64))[None, None]
    vt = torch.tensor(np.asarray(v, dtype=np.float64))[None, None]
    am = None if mask is None else torch.tensor(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=am, scale=scale)
    return o[0, 0].numpy()


def _lib_probs(q, k, scale):
    s = torch.tensor(np.asarray(q, np.float64)) @ torch.tensor(np.asarray(k, np.float64)).T
    return torch.softmax(scale * s, dim=-1).numpy()


# --------------------------------------------------------------------- hash

def check_hash_golden(impl):
    g = load_golden("hash_small.json")
    keys = impl.hash_keys(np.array(g["q"], np.float32), np.array(g["proj"], np.float32))
    assert keys.tolist() == g["keys"], (keys.tolist(), g["keys"])
    perm = impl.group_permutation(keys)
    assert perm.tolist() == g["perm"], (perm.tolist(), g["perm"])


def check_hash_exact_rational(impl, seed=3, n=40, d=16):
    """Every hash bit equals the sign of the exact rational dot product."""
    r = np.random.default_rng(seed)
    q = r.standard_normal((n, d)).astype(np.float32)
    proj = r.standard_normal((8, d)).astype(np.float32)
    keys = impl.hash_keys(q, proj)
    for i in range(n):
        want = 0
        for b in range(8):
            exact = sum(Fraction(float(q[i, c])) * Fraction(float(proj[b, c])) for c in range(d))
            want |= int(exact > 0) << b
        assert int(keys[i]) == want, (i, int(keys[i]), want)


def check_perm_stable_sort(impl, seed=4, n=500):
    """perm is a bijection, keys are non-decreasing along it and equal keys
    keep ascending token order: together these fix a stable sort."""
    r = np.random.default_rng(seed)
    keys = r.integers(0, 7, size=n).astype(np.uint8)
    perm = impl.group_permutation(keys)
    assert sorted(perm.tolist()) == list(range(n))
    ks = keys[perm].astype(int)
    assert np.all(np.diff(ks) >= 0)
    same = np.diff(ks) == 0
    assert np.all(np.diff(perm.astype(int))[same] > 0)


# -------------------------------------------------------------- attention

def check_dense_vs_sdpa(impl, seed=5):
    r = np.random.default_rng(seed)
    for (n, m, d) in [(7, 11, 4), (33, 64, 16), (5, 130, 8)]:
        q = r.standard_normal((n, d)) * 2
        k = r.standard_normal((m, d)) * 2
        v = r.standard_normal((m, d))
        scale = 1.0 / math.sqrt(d)
        o, p = impl.attention(q, k, v, scale)
        ref = _sdpa(q, k, v, scale)
        assert np.max(np.abs(o - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref))), np.max(np.abs(o - ref))
        assert np.allclose(p.sum(axis=1), 1.0, atol=1e-13)
        assert np.allclose(p, _lib_probs(q, k, scale), atol=1e-14)


def check_two_token_golden(impl):
    g = load_golden("two_token.json")
    o, p = impl.attention(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]), g["scale"])
    assert np.allclose(p[0], g["p"], atol=1e-14)
    assert abs(o[0, 0] - g["o_dense"]) < 1e-13
    sel = impl.select_group(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]), [0], 1, g["scale"])
    assert sel.idx.tolist() == g["idx_k1"]
    assert abs(sel.o_sparse[0, 0] - g["o_sparse_k1"]) < 1e-13
    assert abs(sel.residual[0, 0] - g["residual_k1"]) < 1e-13
    sel2 = impl.select_group(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]), [0], 2, g["scale"])
    assert np.all(sel2.residual == 0.0)


def check_closed_forms(impl, seed=6):
    r = np.random.default_rng(seed)
    n, d = 9, 8
    v = r.standard_normal((n, d))
    # all keys equal -> uniform weights -> mean of V, whatever q is
    k = np.tile(r.standard_normal((1, d)), (n, 1))
    q = r.standard_normal((3, d)) * 5
    o, _ = impl.attention(q, k, v, 0.3)
    assert np.allclose(o, v.mean(axis=0)[None, :], atol=1e-13)
    # one key far ahead of the others -> output is its value row
    k2 = r.standard_normal((n, d))
    k2[4] = 0.0
    q2 = np.zeros((1, d))
    q2[0, 0] = 1.0
    k2[4, 0] = 1e4
    o2, _ = impl.attention(q2, k2, v, 1.0)
    assert np.allclose(o2[0], v[4], atol=1e-12)


# -------------------------------------------------------------- selection

def check_uniform_golden(impl):
    g = load_golden("uniform_attention.json")
    q, k, v = (np.array(g[x], np.float64) for x in ("q", "k", "v"))
    for rows in ([0, 1, 2], [3, 4, 5]):
        sel = impl.select_group(q, k, v, rows, g["keep"], g["scale"])
        assert np.allclose(sel.scores, g["scores"], atol=1e-14)
        assert sel.idx.tolist() == g["idx"]
        assert np.allclose(sel.o_dense, g["o_dense"], atol=1e-13)
        assert np.allclose(sel.o_sparse, g["o_sparse"], atol=1e-13)
        assert np.allclose(sel.residual, g["residual"], atol=1e-13)
        re = impl.reuse_group(q, k, v, rows, sel.idx, sel.residual, g["scale"])
        assert np.allclose(re, g["o_dense"], atol=1e-13)


def check_scores_mass(impl, seed=7):
    """Each query's probabilities sum to one, so a group's scores sum to |g|;
    a group of one query scores keys by its own probability row."""
    r = np.random.default_rng(seed)
    n, d = 50, 8
    q, k, v = r.standard_normal((n, d)), r.standard_normal((n, d)), r.standard_normal((n, d))
    for rows in ([0], [3, 9, 11], list(range(20, 37))):
        sel = impl.select_group(q, k, v, rows, 5, 0.7)
        assert abs(sel.scores.sum() - len(rows)) < 1e-12
        lib = _lib_probs(q[rows], k, 0.7).sum(axis=0)
        assert np.allclose(sel.scores, lib, atol=1e-13)


def check_topk_bruteforce(impl, seed=8):
    """The kept set maximises the group's retained probability mass over all
    k-subsets (enumerated), the mass being computed from library softmax."""
    r = np.random.default_rng(seed)
    for trial in range(12):
        n = int(r.integers(4, 11))
        d = 3
        gsize = int(r.integers(1, 5))
        k = int(r.integers(1, min(5, n) + 1))
        q = r.standard_normal((gsize, d)) * 1.5
        kk = r.standard_normal((n, d)) * 1.5
        v = r.standard_normal((n, d))
        p = _lib_probs(q, kk, 1.0)
        best, best_set = -1.0, None
        for sub in itertools.combinations(range(n), k):
            mass = sum(p[i, j] for i in range(gsize) for j in sub)
            if mass > best + 1e-12:
                best, best_set = mass, sub
        sel = impl.select_group(q, kk, v, list(range(gsize)), k, 1.0)
        got = sum(p[i, j] for i in range(gsize) for j in sel.idx)
        assert abs(got - best) < 1e-9, (trial, got, best, sel.idx, best_set)
        assert list(sel.idx) == sorted(sel.idx) and len(set(sel.idx.tolist())) == k


def check_topk_ties_lower_index(impl):
    c = np.array([0.2, 0.5, 0.2, 0.5, 0.1, 0.2])
    idx, gap = impl.topk_select(c, 3)
    assert idx.tolist() == [0, 1, 3] and gap == 0.0
    idx, gap = impl.topk_select(c, 4)
    assert idx.tolist() == [0, 1, 2, 3] and gap == 0.0
    idx, gap = impl.topk_select(c, 5)
    assert idx.tolist() == [0, 1, 2, 3, 5]
    assert abs(gap - (np.float32(0.2) - np.float32(0.1))) < 1e-9
    idx, gap = impl.topk_select(c, 6)
    assert idx.tolist() == list(range(6)) and gap == math.inf


def check_single_query_topk(impl, seed=9):
    """G = 1 reduces to per-query top-k attention (torch.topk on the row)."""
    r = np.random.default_rng(seed)
    n, d, k = 40, 8, 6
    q, kk, v = r.standard_normal((1, d)) * 2, r.standard_normal((n, d)) * 2, r.standard_normal((n, d))
    p = _lib_probs(q, kk, 0.5)[0]
    top = torch.topk(torch.tensor(p), k).indices.sort().values.numpy()
    sel = impl.select_group(q, kk, v, [0], k, 0.5)
    assert sel.idx.tolist() == top.tolist()


# ----------------------------------------------------- sparse and residual

def check_sparse_vs_masked_sdpa(impl, seed=10):
    r = np.random.default_rng(seed)
    n, d = 30, 8
    q, kk, v = r.standard_normal((5, d)), r.standard_normal((n, d)), r.standard_normal((n, d))
    idx = np.sort(r.choice(n, size=7, replace=False))
    mask = np.zeros((5, n), dtype=bool)
    mask[:, idx] = True
    o = impl.sparse_attention(q, kk, v, idx, 0.4)
    assert np.allclose(o, _sdpa(q, kk, v, 0.4, mask), atol=1e-13)


def check_keep_one_and_all(impl, seed=11):
    r = np.random.default_rng(seed)
    n, d = 25, 4
    q, kk, v = r.standard_normal((n, d)), r.standard_normal((n, d)), r.standard_normal((n, d))
    rows = [2, 5, 7, 11]
    one = impl.select_group(q, kk, v, rows, 1, 0.5)
    j = int(np.argmax(_lib_probs(q[rows], kk, 0.5).sum(axis=0)))
    assert one.idx.tolist() == [j]
    assert np.allclose(one.o_sparse, np.tile(v[j], (len(rows), 1)), atol=1e-14)
    full = impl.select_group(q, kk, v, rows, n, 0.5)
    assert full.idx.tolist() == list(range(n))
    assert np.all(full.residual == 0.0)
    assert np.allclose(full.o_dense, _sdpa(q[rows], kk, v, 0.5), atol=1e-13)


def check_reuse_identity(impl, seed=12):
    """Reuse on the selection step's own inputs reproduces dense attention."""
    r = np.random.default_rng(seed)
    n, d = 64, 8
    q, kk, v = r.standard_normal((n, d)) * 2, r.standard_normal((n, d)) * 2, r.standard_normal((n, d))
    rows = list(range(0, 64, 3))
    sel = impl.select_group(q, kk, v, rows, 9, 0.35)
    re = impl.reuse_group(q, kk, v, rows, sel.idx, sel.residual, 0.35)
    assert np.max(np.abs(re - _sdpa(q[rows], kk, v, 0.35))) < 1e-12


# ------------------------------------------------------------- ablations

def check_block_topk_bruteforce(impl, seed=13):
    """Block selection keeps the whole key blocks that retain the most group
    probability mass among every choice of k / B blocks (enumerated; the mass
    comes from library softmax), stored ascending and as complete blocks."""
    r = np.random.default_rng(seed)
    for trial in range(12):
        b = int(r.choice([2, 3, 4]))
        nb = int(r.integers(3, 7))
        n = nb * b
        kb = int(r.integers(1, nb))
        gsize = int(r.integers(1, 4))
        q = r.standard_normal((gsize, 3)) * 1.5
        kk = r.standard_normal((n, 3)) * 1.5
        v = r.standard_normal((n, 3))
        p = _lib_probs(q, kk, 1.0).sum(axis=0)
        best = max(sum(float(p[x * b:(x + 1) * b].sum()) for x in sub)
                   for sub in itertools.combinations(range(nb), kb))
        sel = impl.select_group(q, kk, v, list(range(gsize)), kb * b, 1.0, kv_block=b)
        got = float(p[sel.idx].sum())
        assert abs(got - best) < 1e-9, (trial, got, best, sel.idx)
        ids = sel.idx.tolist()
        assert ids == sorted(ids) and len(set(ids)) == kb * b
        blocks = sorted({i // b for i in ids})
        assert ids == [x * b + t for x in blocks for t in range(b)], (trial, ids)
    # hand-derived: block 0 holds one strong key (0.5), block 1 three moderate
    # ones (0.9 in total); the summed score keeps block 1, ties go to the
    # lower block
    c = np.array([0.5, 0.0, 0.0, 0.0, 0.3, 0.3, 0.3, 0.0, 0.1, 0.1, 0.1, 0.1])
    idx, gap, bidx = impl.topk_blocks(c, 4, 4)
    assert bidx.tolist() == [1] and idx.tolist() == [4, 5, 6, 7]
    assert abs(gap - (np.float32(0.9) - np.float32(0.5))) < 1e-7
    idx, _, bidx = impl.topk_blocks(np.array([0.2, 0.2, 0.1, 0.3, 0.2, 0.2]), 2, 2)
    assert bidx.tolist() == [0] and idx.tolist() == [0, 1]


def check_raster_groups(impl, seed=14):
    """Raster grouping keeps the tokens in raster order.  When every query
    hashes to the same key, the hash grouping's stable sort is the identity
    too, so both groupings must give the same permutation and kept keys."""
    r = np.random.default_rng(seed)
    n, d, g, k = 48, 8, 16, 5
    q = r.standard_normal((n, d))
    q[:, 0] = np.abs(q[:, 0]) + 50.0
    proj = np.zeros((8, d), np.float32)
    proj[:, 0] = 1.0
    proj[:, 1:] = r.standard_normal((8, d - 1)) * 0.01
    kk, v = r.standard_normal((n, d)), r.standard_normal((n, d))
    hm = impl.select_head(q, kk, v, proj, g, k, 0.3, grouping="hash")
    rm = impl.select_head(q, kk, v, proj, g, k, 0.3, grouping="raster")
    assert hm.keys.tolist() == [255] * n
    assert hm.perm.tolist() == list(range(n)) and rm.perm.tolist() == list(range(n))
    for gi in hm.groups:
        assert hm.groups[gi].idx.tolist() == rm.groups[gi].idx.tolist()
    q2 = r.standard_normal((n, d))
    rm2 = impl.select_head(q2, kk, v, r.standard_normal((8, d)), g, k, 0.3, grouping="raster")
    assert rm2.perm.tolist() == list(range(n))
    assert rm2.groups[1].rows.tolist() == list(range(16, 32))


def check_centred_hash(impl, seed=16):
    """Centred hash against exact rational arithmetic.  With small-integer
    queries and projections and N a power of two, every float64 step of the
    centred hash is exact, so its bits must be the signs of the exact
    rational dot products (q_i - mean) . r_b; a hand-derived case pins the
    mean and the bits; a shift of every query by a constant leaves the keys
    unchanged."""
    r = np.random.default_rng(seed)
    for trial in range(6):
        n, d = 16, 6
        q = r.integers(-8, 9, size=(n, d)).astype(np.float32)
        proj = r.integers(-3, 4, size=(8, d)).astype(np.float32)
        keys = impl.centred_hash_keys(q, proj)
        mean = [sum(Fraction(int(q[i, c])) for i in range(n)) / n for c in range(d)]
        for i in range(n):
            want = 0
            for b in range(8):
                dot = sum((Fraction(int(q[i, c])) - mean[c]) * int(proj[b, c]) for c in range(d))
                want |= (1 << b) if dot > 0 else 0
            assert int(keys[i]) == want, (trial, i, int(keys[i]), want)
        shifted = impl.centred_hash_keys(q + np.float32(5.0), proj)
        assert shifted.tolist() == keys.tolist()
    # hand-derived: mean (1, 2); centred rows (-1,-1), (1,1), (1,-1), (-1,1);
    # r_0 = (1, 0) -> bit 0 = [x > 0]; r_1 = (0, 1) -> bit 1 = [y > 0];
    # r_2 = (1, 1) -> only the second row is positive, the sums of 0 give 0
    q = np.array([[0, 1], [2, 3], [2, 1], [0, 3]], np.float32)
    proj = np.zeros((8, 2), np.float32)
    proj[0] = [1, 0]
    proj[1] = [0, 1]
    proj[2] = [1, 1]
    assert impl.query_mean(q).tolist() == [1.0, 2.0]
    assert impl.centred_hash_keys(q, proj).tolist() == [0, 7, 1, 2]


def check_morton_groups(impl):
    """Z-curve order: a hand-derived order on a 1 x 2 x 4 grid; on a 4 x 4 x 8
    grid every run of 8 tokens is a 2 x 2 x 2 cube and every run of 64 a
    4 x 4 x 4 cube; on a 3 x 5 x 6 grid (no power of two) the order is a
    bijection that visits each 2 x 2 x 2 cell of the curve before the next."""
    # (y, x) codes: (0,0)=0 (0,1)=1 (1,0)=2 (1,1)=3 (0,2)=8 (0,3)=9 (1,2)=10 (1,3)=11
    assert impl.morton_permutation((1, 2, 4)).tolist() == [0, 1, 4, 5, 2, 3, 6, 7]
    assert impl.morton_permutation((2, 2, 2)).tolist() == list(range(8))
    T, Y, X = 4, 4, 8
    perm = impl.morton_permutation((T, Y, X))
    t, rem = np.divmod(perm, Y * X)
    y, x = np.divmod(rem, X)
    for size, side in ((8, 2), (64, 4)):
        for s in range(0, T * Y * X, size):
            for a in (t[s:s + size], y[s:s + size], x[s:s + size]):
                assert a.max() - a.min() == side - 1 and a.min() % side == 0, (size, s)
            assert len({(int(i), int(j), int(k)) for i, j, k in zip(t[s:s + size], y[s:s + size], x[s:s + size])}) == size
    perm = impl.morton_permutation((3, 5, 6))
    assert sorted(perm.tolist()) == list(range(90))
    t, rem = np.divmod(perm, 30)
    y, x = np.divmod(rem, 6)
    cell = (t // 2) * 100 + (y // 2) * 10 + (x // 2)
    first = {}
    for i, c in enumerate(cell.tolist()):
        first.setdefault(c, i)
    last = {c: i for i, c in enumerate(cell.tolist())}
    for c in first:
        assert last[c] - first[c] + 1 == int(np.sum(cell == c)), "a 2x2x2 cell is split"
    # a joint sequence: the 5 tokens past a 1 x 2 x 4 grid keep their order after it
    assert impl.morton_permutation((1, 2, 4), 13).tolist() == [0, 1, 4, 5, 2, 3, 6, 7, 8, 9, 10, 11, 12]
    assert impl.morton_permutation((1, 2, 4), 8).tolist() == [0, 1, 4, 5, 2, 3, 6, 7]


def check_no_residual(impl, seed=15):
    """Without the residual the cached correction is zero and reuse returns
    the sparse output renormalised over the kept keys (library masked
    attention) -- not dense attention."""
    r = np.random.default_rng(seed)
    n, d = 40, 8
    q, kk, v = r.standard_normal((n, d)) * 2, r.standard_normal((n, d)) * 2, r.standard_normal((n, d))
    rows = list(range(1, 40, 4))
    sel = impl.select_group(q, kk, v, rows, 7, 0.35, residual=False)
    assert np.all(sel.residual == 0.0)
    mask = np.zeros((len(rows), n), dtype=bool)
    mask[:, sel.idx] = True
    re = impl.reuse_group(q, kk, v, rows, sel.idx, sel.residual, 0.35)
    assert np.allclose(re, _sdpa(q[rows], kk, v, 0.35, mask), atol=1e-13)
    assert np.max(np.abs(re - _sdpa(q[rows], kk, v, 0.35))) > 1e-6


# ------------------------------------------------- retained-mass budgets

def check_mass_count_exact_rational(impl, seed=17):
    """The per-group budget for a retained-mass target is the size of the
    smallest key subset whose exact (rational) score sum reaches
    mass * |g|: brute force over every subset of tiny rows, with scores
    from library softmax; cases whose best subset sums lie within 2^-30 of
    the target are skipped, so the fixed-point decision cannot differ from
    the exact one."""
    r = np.random.default_rng(seed)
    tried = 0
    for trial in range(40):
        n = int(r.integers(3, 10))
        g = int(r.integers(1, 4))
        d = 4
        q = r.standard_normal((g, d)) * 1.5
        kk = r.standard_normal((n, d)) * 1.5
        p = _lib_probs(q, kk, 0.8)
        c = p.sum(axis=0).astype(np.float32)
        for mass in (0.3, 0.5, 0.8, 0.95, 1.0):
            target = Fraction(float(np.float32(mass))) * g
            best = {}
            for m in range(1, n + 1):
                best[m] = max(sum(Fraction(float(c[j])) for j in sub) for sub in itertools.combinations(range(n), m))
            if any(abs(best[m] - target) < Fraction(1, 2 ** 30) for m in best):
                continue
            reach = [m for m in range(1, n + 1) if best[m] >= target]
            m = reach[0] if reach else n
            for cap in (1, max(1, n // 2), n):
                want = max(1, min(m, cap))
                got = impl.mass_keep_count(c, mass, g, cap)
                assert got == want, (trial, mass, cap, got, want, c.tolist())
                tried += 1
    assert tried > 100


def check_mass_closed_forms(impl):
    """Equal scores need ceil(mass * N) keys; one key that holds the target
    alone is enough; the cap bounds the count; the kept keys are the top
    ones under the top-k's order."""
    c = np.full(16, 4.0)                      # 16 keys, a group of 64 queries
    assert impl.mass_keep_count(c, 0.5, 64, 16) == 8
    assert impl.mass_keep_count(c, 0.51, 64, 16) == 9
    assert impl.mass_keep_count(c, 1.0, 64, 16) == 16
    assert impl.mass_keep_count(c, 1.0, 64, 5) == 5
    assert impl.mass_keep_count(c, 1e-9, 64, 16) == 1
    dom = np.array([1.0, 60.0, 2.0, 1.0])
    assert impl.mass_keep_count(dom, 0.9, 64, 4) == 1
    assert impl.mass_keep_count(dom, 0.96, 64, 4) == 2
    idx, _, n = impl.topk_mass_select(np.array([3.0, 1.0, 3.0, 8.0, 1.0, 0.0]), 0.7, 16, 6)
    assert n == 3 and idx.tolist() == [0, 2, 3]   # 8 + 3 + 3 = 14 >= 11.2; ties at 3 both needed


def check_mass_selection(impl, seed=18):
    """A mass-targeted selection keeps a set whose retained probability mass
    (library softmax over the group's rows) reaches the target, and dropping
    its weakest key falls short of it (unless the cap stopped it)."""
    r = np.random.default_rng(seed)
    n, d = 60, 8
    q, kk, v = r.standard_normal((n, d)) * 2, r.standard_normal((n, d)) * 2, r.standard_normal((n, d))
    rows = list(range(0, 60, 5))
    for mass, cap in ((0.6, 60), (0.9, 60), (0.99, 60), (0.9, 4)):
        sel = impl.select_group(q, kk, v, rows, cap, 0.4, keep_mass=mass)
        p = _lib_probs(q[rows], kk, 0.4)
        kept = p[:, sel.idx].sum()
        target = mass * len(rows)
        if len(sel.idx) < cap:
            assert kept >= target - 1e-9, (mass, kept, target)
            weakest = sel.idx[np.argmin(p[:, sel.idx].sum(axis=0))]
            assert kept - p[:, weakest].sum() < target + 1e-9
        else:
            assert len(sel.idx) == cap


# ------------------------------------------------------- bf16 residual

def check_bf16_rounding(impl, seed=19):
    """bf16 storage of the residual rounds like torch's float32 -> bfloat16
    conversion (round to nearest, ties to even), halfway cases included."""
    r = np.random.default_rng(seed)
    x = np.concatenate([r.standard_normal(2000) * 10.0 ** r.integers(-6, 3, 2000),
                        [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0, 3.0]])
    want = torch.tensor(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    got = impl.round_bf16(x)
    assert np.array_equal(got, want)
    assert got[-5] == 1.0 and got[-4] == 1.0 + 2 ** -6


def check_bf16_residual(impl, seed=20):
    """A bf16 residual is the float32 residual rounded to bf16, and reuse on
    the selection inputs then reproduces dense attention to within half a
    bf16 unit of the residual."""
    r = np.random.default_rng(seed)
    n, d = 48, 8
    q, kk, v = r.standard_normal((n, d)) * 2, r.standard_normal((n, d)) * 2, r.standard_normal((n, d))
    rows = list(range(3, 48, 3))
    a = impl.select_group(q, kk, v, rows, 9, 0.35)
    b = impl.select_group(q, kk, v, rows, 9, 0.35, residual_bf16=True)
    assert np.array_equal(a.idx, b.idx)
    tb = torch.tensor(a.residual.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(b.residual, tb)
    re = impl.reuse_group(q, kk, v, rows, b.idx, b.residual, 0.35)
    dense = _sdpa(q[rows], kk, v, 0.35)
    assert np.max(np.abs(re - dense)) <= np.max(np.abs(a.residual)) * 2 ** -8 + 1e-12


ALL_CHECKS = [
    check_hash_golden, check_hash_exact_rational, check_perm_stable_sort,
    check_dense_vs_sdpa, check_two_token_golden, check_closed_forms,
    check_uniform_golden, check_scores_mass, check_topk_bruteforce,
    check_topk_ties_lower_index, check_single_query_topk,
    check_sparse_vs_masked_sdpa, check_keep_one_and_all, check_reuse_identity,
    check_block_topk_bruteforce, check_raster_groups, check_no_residual, check_centred_hash,
    check_morton_groups, check_mass_count_exact_rational, check_mass_closed_forms, check_mass_selection,
    check_bf16_rounding, check_bf16_residual,
]

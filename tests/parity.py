"""Shared helpers of the GPU parity tests: build seeded problems from the
input generator, run the library through its Python binding (which calls the
C ABI), and compare against the CPU oracle.

Acceptance rules:
* perm: bit-exact;
* kept keys per group: same size, distinct, ascending, in range; every key
  whose oracle score (float32) exceeds the (k+1)-th score by more than 1e-6 is
  kept; every kept key scores at least the k-th score minus 1e-6 (so the set
  is bit-exact whenever the oracle's k-th/(k+1)-th gap is 1e-6 or more);
* outputs: bf16 max-abs <= 2e-2 and relative L2 <= 5e-3; float32 max-abs
  <= 2e-4 and relative L2 <= 1e-4 (float32 logits of magnitude ~50 carry an
  absolute error of order sqrt(d) * 2^-24 * 50 ~ 3e-5 at d = 128, which moves
  every probability by that relative amount); the residual's relative L2 is measured
  against the dense output's norm.  Residual and reuse outputs are compared
  with the oracle evaluated on the GPU's own kept keys, so a legitimate
  near-tie swap cannot mask an arithmetic error.
"""

from __future__ import annotations

import concurrent.futures as cf
import math
import os
from dataclasses import dataclass, field

import numpy as np
import torch

import oracle.mcs_oracle as orc
from mcs_inputs import hash_projections, head_base, head_step, token_embedding

THREADS = min(16, os.cpu_count() or 8)
GAP = 1e-6
TOL = {"bf16": (2e-2, 5e-3), "fp32": (2e-4, 1e-4)}


def scale_for(d: int) -> float:
    return float(np.float32(1.0 / math.sqrt(d)))


@dataclass
class Problem:
    grid: tuple
    H: int
    d: int
    dtype: str
    G: int
    keeps: np.ndarray
    drift: float
    steps: list                  # reuse steps that were generated (>= 1)
    seed: int = 0
    wid: int = 100
    heads_np: dict = field(default_factory=dict)   # (head, step) -> (q, k, v) float32
    dev: dict = field(default_factory=dict)        # step -> (q, k, v) device tensors
    text: int = 0                # text tokens after the grid tokens (a joint sequence)

    @property
    def N(self):
        return int(np.prod(self.grid)) + self.text

    @property
    def ng(self):
        return -(-self.N // self.G)

    @property
    def tdtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def proj(self):
        return hash_projections(self.seed, self.wid, self.d)


def build_problem(grid, H, d, dtype, G, keeps, drift, steps, seed=0, wid=100, keep_heads=None, text=0) -> Problem:
    """Generates step 0 and the listed reuse steps for every head, uploads
    them, and keeps the float32 host copies of the heads in keep_heads (all
    heads if None) for the oracle.  `text` text tokens follow the grid's
    tokens (a joint video + text sequence)."""
    p = Problem(tuple(grid), H, d, dtype, G, np.asarray(keeps, np.int32), drift, list(steps), seed, wid, text=text)
    pos = token_embedding(grid, d, text, seed, wid)
    bf = dtype == "bf16"
    bases = [None] * H

    def mk_base(h):
        bases[h] = head_base(seed, wid, h, grid, d, pos)

    with cf.ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(mk_base, range(H)))
    for t in [0] + p.steps:
        host = [np.empty((H, p.N, d), np.float32) for _ in range(3)]

        def mk(h, t=t, host=host):
            xs = head_step(bases[h], seed, wid, h, t, drift, bf)
            for i in range(3):
                host[i][h] = xs[i]
            if keep_heads is None or h in keep_heads:
                p.heads_np[(h, t)] = xs

        with cf.ThreadPoolExecutor(THREADS) as ex:
            list(ex.map(mk, range(H)))
        p.dev[t] = tuple(torch.from_numpy(x).to("cuda").to(p.tdtype).contiguous() for x in host)
        del host
    return p


def rel_l2(x, ref, ref_norm=None):
    den = np.linalg.norm(ref) if ref_norm is None else ref_norm
    return float(np.linalg.norm(np.asarray(x, np.float64) - ref) / max(den, 1e-300))


def assert_close(x, ref, dtype, what, ref_norm=None):
    max_abs, rl2 = TOL[dtype]
    x = np.asarray(x, np.float64)
    err = float(np.max(np.abs(x - ref))) if x.size else 0.0
    r = rel_l2(x, ref, ref_norm)
    assert err <= max_abs and r <= rl2, f"{what}: max-abs {err:.3e} (tol {max_abs}), rel-L2 {r:.3e} (tol {rl2})"
    return err, r


def check_idx(gpu_idx, scores, k, n, what):
    """Returns True when the GPU set equals the oracle's, asserts the rule."""
    gi = np.asarray(gpu_idx, np.int64)
    assert gi.shape == (k,), f"{what}: {gi.shape} != ({k},)"
    assert np.all(np.diff(gi) > 0), f"{what}: not strictly ascending"
    assert gi[0] >= 0 and gi[-1] < n, f"{what}: index out of range"
    c32 = np.asarray(scores, np.float64).astype(np.float32).astype(np.float64)
    srt = np.sort(c32)[::-1]
    ck = srt[k - 1]
    ck1 = srt[k] if k < n else -np.inf
    must = np.nonzero(c32 > ck1 + GAP)[0]
    missing = np.setdiff1d(must, gi)
    assert missing.size == 0, f"{what}: clearly-in keys missing {missing[:8]} (scores {c32[missing[:8]]})"
    low = gi[c32[gi] < ck - GAP]
    assert low.size == 0, f"{what}: clearly-out keys kept {low[:8]} (scores {c32[low[:8]]}, k-th {ck})"
    oidx, _ = orc.topk_select(scores, k)
    return bool(np.array_equal(oidx, gi))


def to_np(t):
    return t.detach().float().cpu().numpy()


def sample_groups(ng, extra=4, seed=0):
    """Groups {0, 1, ng/2, last} plus `extra` seeded random ones."""
    base = {0, min(1, ng - 1), ng // 2, ng - 1}
    pool = np.setdiff1d(np.arange(ng), list(base))
    r = np.random.default_rng(seed)
    pick = r.choice(pool, size=min(extra, pool.size), replace=False) if pool.size else []
    return sorted(base | {int(x) for x in pick})


MASS_EPS = 2e-4   # retained-mass comparisons: allowance per query of the group (score rounding)


def check_mass_group(slot, n, scores, mass, glen, cap, what):
    """A group's kept keys under a retained-mass target: n keys (1 <= n <=
    cap) that are a top-n set by the kept-key rule, and n is where the
    oracle's scores, sorted, first reach mass * glen (within MASS_EPS * glen
    either way: the GPU's float32 scores round differently), or the cap.
    Returns (set equal to the oracle's top-n, n equal to the oracle's)."""
    assert 1 <= n <= cap, f"{what}: count {n} outside [1, {cap}]"
    gi = np.asarray(slot[:n])
    exact = check_idx(gi, scores, n, len(scores), what)
    srt = np.sort(np.asarray(scores, np.float64).astype(np.float32).astype(np.float64))[::-1]
    prefix = np.cumsum(srt)
    target, eps = mass * glen, MASS_EPS * glen
    if n < cap:
        assert prefix[n - 1] >= target - eps, f"{what}: {n} keys hold {prefix[n - 1]:.6f} < {target:.6f}"
    assert n == 1 or prefix[n - 2] < target + eps, f"{what}: {n - 1} keys already hold {prefix[n - 2]:.6f}"
    return exact, n == orc.mass_keep_count(scores, mass, glen, cap)


def check_units(p: Problem, meta, od, outs, sc, heads, groups, label="", grouping="hash", kv_block=1,
                residual=True, keep_mass=0.0):
    """Compares the sampled (head, group) units of a GPU run with the oracle:
    perm of the whole head, kept keys (and their number under a retained-mass
    target), dense rows, residual and the reuse outputs of every generated
    step.  Returns the number of kept-key sets equal to the oracle's and the
    number checked."""
    exact = total = 0
    counts = meta.count.cpu().numpy()
    for h in heads:
        q, k, v = p.heads_np[(h, 0)]
        perm_o = orc.select_head(q, k, v, p.proj(), p.G, int(p.keeps[h]), sc, groups=[], grouping=grouping,
                                 grid=p.grid).perm
        perm_g = meta.perm[h].cpu().numpy()
        assert np.array_equal(perm_g, perm_o), f"{label} head {h}: perm differs"
        kh = int(p.keeps[h])
        gidx = meta.head_idx(h, kh)
        ranges = orc.group_ranges(p.N, p.G)
        if keep_mass == 0:
            assert np.all(counts[h] == kh), f"{label} head {h}: group counts differ from the budget {kh}"
        for g in groups:
            s, e = ranges[g]
            rows = perm_o[s:e]
            rows_t = torch.from_numpy(rows.astype(np.int64)).to("cuda")
            sel = orc.select_group(q, k, v, rows, kh, sc, kv_block=kv_block, residual=residual)
            gi = gidx[g].cpu().numpy()
            if keep_mass > 0:
                n = int(counts[h, g])
                same_set, _ = check_mass_group(gi, n, sel.scores, keep_mass, e - s, kh,
                                               f"{label} head {h} group {g}")
                exact += same_set
                gi = gi[:n]
            elif kv_block == 1:
                exact += check_idx(gi, sel.scores, kh, p.N, f"{label} head {h} group {g}")
            else:
                exact += check_blocks(gi, sel.scores, kh, p.N, kv_block, f"{label} head {h} group {g}")
            total += 1
            if od is not None:
                assert_close(to_np(od[h].index_select(0, rows_t)), sel.o_dense, p.dtype,
                             f"{label} head {h} group {g} dense rows")
            if residual:
                res_c = sel.o_dense - orc.sparse_attention(q[rows], k, v, gi, sc)
                if meta.meta.residual_dtype == 1:   # cached in bf16 (the oracle's rounding of the same difference)
                    res_c = orc.round_bf16(res_c)
                assert_close(to_np(meta.residual[h, s:e]), res_c, p.dtype, f"{label} head {h} group {g} residual",
                             ref_norm=np.linalg.norm(sel.o_dense))
            else:
                res_c = np.zeros_like(sel.o_dense)
                assert float(meta.residual[h, s:e].abs().max()) == 0.0, f"{label} head {h} group {g} residual"
            for t, o in outs.items():
                ref = orc.reuse_group(*p.heads_np[(h, t)], rows, gi, res_c, sc)
                assert_close(to_np(o[h].index_select(0, rows_t)), ref, p.dtype,
                             f"{label} head {h} group {g} reuse step {t}")
    return exact, total


def check_blocks(gpu_idx, scores, k, n, block, what):
    """Block-granular kept set: whole, ascending runs of `block` keys, k / block
    of them, chosen by the oracle's block scores under the gap rule (a block
    score is a float32 sum of 64 float32 key scores on the GPU, so the gap
    allowance scales with the largest block score).  Returns True when the
    kept blocks equal the oracle's."""
    gi = np.asarray(gpu_idx, np.int64)
    assert gi.shape == (k,), f"{what}: {gi.shape} != ({k},)"
    runs = gi.reshape(-1, block)
    assert np.all(runs % block == np.arange(block)[None, :]), f"{what}: not whole blocks"
    assert np.all(np.diff(runs[:, 0]) > 0), f"{what}: blocks not ascending"
    assert runs[0, 0] >= 0 and runs[-1, -1] < n, f"{what}: index out of range"
    bs = orc.block_scores(scores, block).astype(np.float32).astype(np.float64)
    kb, nb = k // block, n // block
    gap = GAP + 4e-6 * float(bs.max())
    srt = np.sort(bs)[::-1]
    ck = srt[kb - 1]
    ck1 = srt[kb] if kb < nb else -np.inf
    kept = runs[:, 0] // block
    missing = np.setdiff1d(np.nonzero(bs > ck1 + gap)[0], kept)
    assert missing.size == 0, f"{what}: clearly-in blocks missing {missing[:8]}"
    low = kept[bs[kept] < ck - gap]
    assert low.size == 0, f"{what}: clearly-out blocks kept {low[:8]}"
    _, _, ob = orc.topk_blocks(scores, k, block)
    return bool(np.array_equal(ob, kept))


def check_every_unit(p: Problem, meta, sc, outs, heads, label="", dense=(), dense_heads=(), grouping="hash"):
    """Compares every (head, group) unit of the listed heads with the oracle,
    on host copies of the GPU's outputs.

    For every head in `heads` (a thread per head): the permutation of the
    whole head (oracle grouping), every group's kept keys (ascending,
    distinct, in range), and every group's reuse output at every step in
    `outs`, against the oracle evaluated on the GPU's own permutation, kept
    keys and residual.

    For every head in `dense_heads` (a subset of `heads`) the dense side is
    checked on every row as well: each group's kept keys against the oracle's
    exact group scores (kept-key rule), the cached residual against the
    oracle's dense minus sparse rows, and the dense output `dense` (original
    token order) against the oracle's dense rows, for each (name, tensor) in
    `dense`.

    Returns the number of kept-key sets equal to the oracle's and the number
    checked (dense_heads only)."""
    import threadpoolctl

    perm_all = meta.perm.cpu().numpy()
    idx_all = meta.idx.cpu().numpy()
    starts = meta.idx_start.cpu().numpy()
    res_all = meta.residual.float().cpu().numpy()
    outs_h = {t: to_np(o) for t, o in outs.items()}
    dense_h = [(name, to_np(x)) for name, x in dense]
    ranges = orc.group_ranges(p.N, p.G)

    counts = meta.count.cpu().numpy()

    def kept(h):
        kh = int(p.keeps[h])
        slots = idx_all[starts[h]:starts[h] + p.ng * kh].reshape(p.ng, kh).astype(np.int64)
        return [slots[g, :counts[h, g]] for g in range(p.ng)]

    def head_job(h):
        kh = int(p.keeps[h])
        q0, k0, v0 = p.heads_np[(h, 0)]
        perm_o = orc.select_head(q0, k0, v0, p.proj(), p.G, kh, sc, groups=[], grouping=grouping, grid=p.grid).perm
        assert np.array_equal(perm_all[h], perm_o), f"{label} head {h}: perm differs"
        gidx = kept(h)
        assert np.all(counts[h] == kh), f"{label} head {h}: group counts differ from the budget {kh}"
        for g, gi in enumerate(gidx):
            assert np.all(np.diff(gi) > 0), f"{label} head {h} group {g}: kept keys not strictly ascending"
            assert gi.min() >= 0 and gi.max() < p.N, f"{label} head {h} group {g}: kept key out of range"
        for t, o in outs_h.items():
            qt, kt, vt = p.heads_np[(h, t)]
            for g, (s, e) in enumerate(ranges):
                rows = perm_all[h, s:e]
                ref = orc.reuse_group(qt, kt, vt, rows, gidx[g], res_all[h, s:e].astype(np.float64), sc)
                assert_close(o[h, rows], ref, p.dtype, f"{label} head {h} group {g} reuse step {t}")

    with threadpoolctl.threadpool_limits(1), cf.ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(head_job, heads))

    exact = total = 0
    for h in dense_heads:
        # whole chunks of groups in sorted order: the exact probabilities of a
        # chunk's rows give each group's scores, dense rows and residual
        kh = int(p.keeps[h])
        q0, k0, v0 = p.heads_np[(h, 0)]
        gidx = kept(h)
        per = max(1, 1024 // p.G)
        for g0 in range(0, p.ng, per):
            gs = range(g0, min(p.ng, g0 + per))
            base = ranges[gs[0]][0]
            rows = perm_all[h, base:ranges[gs[-1]][1]]
            o_d, pr = orc.attention(q0[rows], k0, v0, sc)
            for name, x in dense_h:
                assert_close(x[h, rows], o_d, p.dtype, f"{label} head {h} {name}, rows of groups {g0}..")
            for g in gs:
                a, b = ranges[g][0] - base, ranges[g][1] - base
                exact += check_idx(gidx[g], orc.group_scores(pr[a:b]), kh, p.N, f"{label} head {h} group {g}")
                total += 1
                res_c = o_d[a:b] - orc.sparse_attention(q0[rows[a:b]], k0, v0, gidx[g], sc)
                if meta.meta.residual_dtype == 1:
                    res_c = orc.round_bf16(res_c)
                assert_close(res_all[h, ranges[g][0]:ranges[g][1]], res_c, p.dtype,
                             f"{label} head {h} group {g} residual", ref_norm=np.linalg.norm(o_d[a:b]))
    return exact, total

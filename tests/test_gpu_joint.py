"""GPU parity of the DiT-block integration cases: joint video + text
sequences (the joint attention of MM-DiT blocks, text tokens after the latent
grid's tokens in one sequence) under sign-hash and Z-curve query groups, and
a batch folded into the heads, which must give exactly what separate calls on
each batch element give."""

import numpy as np
import pytest
import torch

import oracle.mcs_oracle as orc
from mcs_inputs import workload
from parity import assert_close, build_problem, check_every_unit, check_idx, scale_for, to_np

pytestmark = pytest.mark.gpu

mcs = pytest.importorskip("sparse_attention_diffusion_mcs_amd")

CASES = {
    # name: (grid, text, H, d, dtype, G, keeps, grouping, wid)
    "hash_bf16_d128": ((4, 8, 20), 50, 2, 128, "bf16", 64, [128, 256], "hash", 141),
    "morton_bf16_d128": ((4, 8, 20), 50, 2, 128, "bf16", 64, [128, 256], "morton", 142),
    "hash_bf16_d64_g128": ((4, 8, 16), 77, 2, 64, "bf16", 128, [96, 320], "hash", 143),
    "morton_fp32_d64": ((2, 8, 16), 30, 1, 64, "fp32", 64, [64], "morton", 144),
}


@pytest.mark.parametrize("name", list(CASES))
def test_joint_sequence_parity(name):
    """Every group of every head against the oracle: perm bit-exact, kept
    keys by the kept-key rule, dense output, residual and reuse output."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    grid, text, H, d, dtype, G, keeps, grouping, wid = CASES[name]
    print(f"[joint] {name} grid={grid}+{text} H={H} d={d} {dtype} G={G} keeps={keeps} {grouping}", flush=True)
    p = build_problem(grid, H, d, dtype, G, keeps, 0.02, [2], wid=wid, text=text)
    sc = scale_for(d)
    gkw = dict(grouping=grouping, grid=grid) if grouping == "morton" else dict(grouping=grouping)
    meta, od = mcs.select(*p.dev[0], G, p.keeps, p.proj(), scale=sc, return_dense=True, **gkw)
    out = mcs.sparse_attn(*p.dev[2], meta, scale=sc)
    torch.cuda.synchronize()
    perm_g = meta.perm.cpu().numpy()
    resid_g, od_g, out_g = to_np(meta.residual), to_np(od), to_np(out)
    n_grid = int(np.prod(grid))
    same = 0
    for h in range(H):
        q, k, v = p.heads_np[(h, 0)]
        hm = orc.select_head(q, k, v, p.proj(), G, int(p.keeps[h]), sc, groups=[], **gkw)
        assert np.array_equal(perm_g[h], hm.perm), f"head {h}: perm differs"
        if grouping == "morton":
            assert np.array_equal(perm_g[h, n_grid:], np.arange(n_grid, p.N)), "text tokens out of order"
        assert_close(od_g[h], orc.dense_attention(q, k, v, sc), p.dtype, f"head {h} dense output")
        kh = int(p.keeps[h])
        gidx_all = meta.head_idx(h, kh).cpu().numpy()
        for g, (s, e) in enumerate(orc.group_ranges(p.N, G)):
            rows = hm.perm[s:e]
            sel = orc.select_group(q, k, v, rows, kh, sc)
            same += check_idx(gidx_all[g], sel.scores, kh, p.N, f"head {h} group {g}")
            res_c = sel.o_dense - orc.sparse_attention(q[rows], k, v, gidx_all[g], sc)
            assert_close(resid_g[h, s:e], res_c, p.dtype, f"head {h} group {g} residual",
                         ref_norm=np.linalg.norm(sel.o_dense))
            ref = orc.reuse_group(*p.heads_np[(h, 2)], rows, gidx_all[g], res_c, sc)
            assert_close(out_g[h, rows], ref, p.dtype, f"head {h} group {g} reuse")
    print(f"[joint] kept sets equal to the oracle's: {same} of {H * p.ng}", flush=True)


def test_joint_workload_full_size():
    """The joint video + text layer at full size (24 heads, 24960 video + 226
    text tokens, ragged last group of 34): every group of two heads against
    the oracle on the GPU's own metadata, and every row of one head's dense
    side, with NaN-prefilled outputs."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = workload(6)
    heads = [0, w.heads - 1]
    print(f"[joint] workload 6: H={w.heads} N={w.seq_len} G={w.group} keep={w.keeps()[0]}", flush=True)
    p = build_problem(w.grid, w.heads, w.head_dim, w.dtype, w.group, w.keeps(), w.drift, [10], wid=w.wid,
                      keep_heads=heads, text=w.text)
    sc = scale_for(w.head_dim)
    od = torch.full_like(p.dev[0][0], float("nan"))
    meta, od = mcs.select(*p.dev[0], w.group, p.keeps, p.proj(), scale=sc, return_dense=True, dense_out=od)
    out = torch.full_like(p.dev[10][0], float("nan"))
    out = mcs.sparse_attn(*p.dev[10], meta, out=out, scale=sc)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(od).all()), "rows left unwritten"
    exact, total = check_every_unit(p, meta, sc, {10: out}, heads, "workload 6", dense=[("dense", od)],
                                    dense_heads=[0])
    print(f"[joint] workload 6: kept sets equal to the oracle's: {exact} of {total}", flush=True)


def test_batch_folded_into_heads():
    """A batch of two elements of two heads each, passed as four heads, gives
    byte for byte the metadata and outputs of one call per element."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B, Hb, G = 2, 2, 64
    keeps = [128, 256, 192, 64]
    print(f"[batch] B={B} heads={Hb}", flush=True)
    p = build_problem((3, 8, 20), B * Hb, 128, "bf16", G, keeps, 0.02, [1], wid=145, text=13)
    sc = scale_for(128)
    q0, k0, v0 = p.dev[0]
    q1, k1, v1 = p.dev[1]
    meta, od = mcs.select(q0, k0, v0, G, p.keeps, p.proj(), scale=sc, return_dense=True)
    out = mcs.sparse_attn(q1, k1, v1, meta, scale=sc)
    dense = mcs.dense_attn(q1, k1, v1, scale=sc)
    torch.cuda.synchronize()
    for b in range(B):
        hs = slice(b * Hb, (b + 1) * Hb)
        part = [x[hs].contiguous() for x in (q0, k0, v0)]
        mb, odb = mcs.select(*part, G, p.keeps[hs], p.proj(), scale=sc, return_dense=True)
        outb = mcs.sparse_attn(*(x[hs].contiguous() for x in (q1, k1, v1)), mb, scale=sc)
        denseb = mcs.dense_attn(*(x[hs].contiguous() for x in (q1, k1, v1)), scale=sc)
        torch.cuda.synchronize()
        assert torch.equal(mb.perm, meta.perm[hs]), f"element {b}: perm"
        assert torch.equal(mb.count, meta.count[hs]), f"element {b}: counts"
        assert torch.equal(mb.order, meta.order[hs]), f"element {b}: launch order"
        for i, h in enumerate(range(b * Hb, (b + 1) * Hb)):
            kh = int(p.keeps[h])
            assert torch.equal(mb.head_idx(i, kh), meta.head_idx(h, kh)), f"element {b} head {i}: kept keys"
        assert torch.equal(mb.residual, meta.residual[hs]), f"element {b}: residual"
        assert torch.equal(odb, od[hs]), f"element {b}: dense output of the selection"
        assert torch.equal(outb, out[hs]), f"element {b}: reuse output"
        assert torch.equal(denseb, dense[hs]), f"element {b}: dense attention"

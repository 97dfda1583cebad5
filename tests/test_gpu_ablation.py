"""GPU parity of the options of mcs_select_ex: raster, centred-hash and
Z-curve query groups, whole 64-key KV blocks, and no residual, each against
the CPU oracle run with the same option on every group of every head (the
permutation bit-exact)."""

import numpy as np
import pytest
import torch

import oracle.mcs_oracle as orc
from parity import assert_close, build_problem, check_blocks, check_idx, scale_for, to_np

pytestmark = pytest.mark.gpu

mcs = pytest.importorskip("sparse_attention_diffusion_mcs_amd")

CASES = {
    # name: (grid, H, d, dtype, G, keeps, grouping, kv_block, residual, wid)
    "raster_bf16_d128": ((4, 8, 16), 2, 128, "bf16", 64, [128, 320], "raster", 1, True, 121),
    "block64_bf16_d128": ((4, 8, 16), 2, 128, "bf16", 64, [128, 256], "hash", 64, True, 122),
    "no_residual_bf16_d64_g128": ((4, 10, 30), 2, 64, "bf16", 128, [100, 600], "hash", 1, False, 123),
    "raster_block64_no_residual_bf16": ((2, 16, 16), 2, 128, "bf16", 64, [64, 192], "raster", 64, False, 124),
    "block64_fp32_d64_g128": ((2, 8, 16), 1, 64, "fp32", 128, [128], "hash", 64, True, 125),
    "centred_bf16_d128_ragged": ((3, 9, 23), 3, 128, "bf16", 64, [96, 160, 300], "centred", 1, True, 127),
    "centred_fp32_d64_g128": ((2, 10, 20), 2, 64, "fp32", 128, [50, 200], "centred", 1, True, 128),
    "morton_bf16_d128": ((4, 8, 16), 2, 128, "bf16", 64, [128, 320], "morton", 1, True, 129),
    "morton_ragged_bf16_d64_g128": ((3, 9, 23), 2, 64, "bf16", 128, [100, 250], "morton", 1, True, 130),
    "morton_block64_fp32": ((2, 8, 16), 1, 128, "fp32", 64, [64], "morton", 64, True, 131),
}


@pytest.mark.parametrize("name", list(CASES))
def test_ablation_parity(name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    grid, H, d, dtype, G, keeps, grouping, kvb, resid, wid = CASES[name]
    print(f"[case] {name} grid={grid} H={H} d={d} {dtype} G={G} keeps={keeps} {grouping} block={kvb} "
          f"residual={resid}", flush=True)
    p = build_problem(grid, H, d, dtype, G, keeps, 0.02, [2], wid=wid)
    sc = scale_for(d)
    grid = grid if grouping == "morton" else None
    meta, od = mcs.select(*p.dev[0], G, p.keeps, p.proj(), scale=sc, return_dense=True, grouping=grouping,
                          kv_block=kvb, residual=resid, grid=grid)
    out = mcs.sparse_attn(*p.dev[2], meta, scale=sc)
    torch.cuda.synchronize()
    perm_g = meta.perm.cpu().numpy()
    resid_g, od_g, out_g = to_np(meta.residual), to_np(od), to_np(out)
    same = 0
    for h in range(H):
        q, k, v = p.heads_np[(h, 0)]
        hm = orc.select_head(q, k, v, p.proj(), G, int(p.keeps[h]), sc, groups=[], grouping=grouping, grid=grid)
        assert np.array_equal(perm_g[h], hm.perm), f"head {h}: perm differs"
        assert_close(od_g[h], orc.dense_attention(q, k, v, sc), p.dtype, f"head {h} dense output")
        kh = int(p.keeps[h])
        gidx_all = meta.head_idx(h, kh).cpu().numpy()
        for g, (s, e) in enumerate(orc.group_ranges(p.N, G)):
            rows = hm.perm[s:e]
            sel = orc.select_group(q, k, v, rows, kh, sc, kv_block=kvb, residual=resid)
            if kvb == 1:
                same += check_idx(gidx_all[g], sel.scores, kh, p.N, f"head {h} group {g}")
            else:
                same += check_blocks(gidx_all[g], sel.scores, kh, p.N, kvb, f"head {h} group {g}")
            if resid:
                res_c = sel.o_dense - orc.sparse_attention(q[rows], k, v, gidx_all[g], sc)
                assert_close(resid_g[h, s:e], res_c, p.dtype, f"head {h} group {g} residual",
                             ref_norm=np.linalg.norm(sel.o_dense))
            else:
                res_c = np.zeros_like(sel.o_dense)
                assert np.all(resid_g[h, s:e] == 0.0), f"head {h} group {g}: residual not zero"
            ref = orc.reuse_group(*p.heads_np[(h, 2)], rows, gidx_all[g], res_c, sc)
            assert_close(out_g[h, rows], ref, p.dtype, f"head {h} group {g} reuse")
    print(f"[case] kept sets equal to the oracle's: {same} of {H * p.ng}", flush=True)


def test_default_options_match_plain_select():
    """mcs_select_ex with MC-Sparse's own options is mcs_select, byte for byte."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    p = build_problem((3, 8, 16), 2, 128, "bf16", 64, [96, 200], 0.0, [1], wid=126)
    sc = scale_for(128)
    import ctypes
    from sparse_attention_diffusion_mcs_amd import _lib as L
    from sparse_attention_diffusion_mcs_amd import api
    q, k, v = p.dev[0]
    m1, _ = mcs.select(q, k, v, 64, p.keeps, p.proj(), scale=sc)
    desc = api.desc_for(q, sc)
    ka = np.ascontiguousarray(p.keeps, np.int32)
    pj = np.ascontiguousarray(p.proj(), np.float32)
    mb = torch.empty_like(m1.buffer)
    ws = torch.empty(mcs.workspace_bytes(q, 64), dtype=torch.uint8, device="cuda")
    m2 = L.Meta()
    opts = L.SelectOptions(L.MCS_GROUPING_HASH, 1, 1, 0)
    L.check(L.lib().mcs_select_ex(ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(), 64,
                                  ka.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                  pj.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), ctypes.byref(opts),
                                  mb.data_ptr(), mb.numel(), ws.data_ptr(), ws.numel(), None, ctypes.byref(m2),
                                  torch.cuda.current_stream().cuda_stream), "mcs_select_ex")
    torch.cuda.synchronize()
    for off, n in ((m1.meta.off_perm, p.H * p.N * 4), (m1.meta.off_idx, int(m1.meta.total_idx) * 4),
                   (m1.meta.off_residual, p.H * p.N * 128 * 4)):
        assert torch.equal(m1.buffer[off:off + n], mb[off:off + n])

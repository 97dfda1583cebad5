"""GPU parity on every unit at full size.

The sampled full-size tests compare a few (head, group) units per layer; these
compare every one.  Every output buffer the library writes starts filled with
NaN (the metadata buffer with 0xFF bytes, a NaN pattern for its float32
residual), so a row that no work item wrote cannot pass.  The launches are
the ones the benchmark times, and at these sizes every attention launch has
more than 1024 work items, so the blocks go through the XCD-locality remap's
chunked branch.

* Workload 2 (24 heads, N = 24960, d = 128, G = 64, keep 2496, sign-hash
  groups): the reuse output of all 9360 units at steps 1 and 10 against the
  oracle on the GPU's own permutation, kept keys and residual; the whole-head
  permutation and the kept-key lists of every head; for one head every dense
  row of the selection's dense output and of the dense baseline, every
  group's kept keys against the oracle's exact scores and every group's
  residual.
* Workload 3 (24 heads, N = 75600, G = 64, keep 3776, ragged last group):
  the reuse output of every group of two heads, and every row of every head
  written.
* A mid-size problem (16 heads, N = 8192, d = 128, G = 64, 2048 groups and
  1024 dense row tiles): every unit of every head, selection included.
"""

import numpy as np
import pytest
import torch

from mcs_inputs import WORKLOADS
from parity import build_problem, check_every_unit, scale_for

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

mcs = pytest.importorskip("sparse_attention_diffusion_mcs_amd")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _nan_like(x):
    return torch.full_like(x, float("nan"))


def _run(p, sc, steps, label):
    """Selection on step 0 and reuse on `steps`, every output NaN-prefilled;
    asserts that every element was written."""
    q0 = p.dev[0][0]
    H, N, d = q0.shape
    nbytes = int(mcs.meta_layout(H, N, d, 1, p.G, p.keeps).bytes)
    meta_buf = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    od = _nan_like(q0)
    meta, _ = mcs.select(*p.dev[0], p.G, p.keeps, p.proj(), scale=sc, meta_buf=meta_buf, dense_out=od)
    outs = {}
    for t in steps:
        outs[t] = _nan_like(q0)
        mcs.sparse_attn(*p.dev[t], meta, out=outs[t], scale=sc)
    dense = _nan_like(q0)
    mcs.dense_attn(*p.dev[0], out=dense, scale=sc)
    torch.cuda.synchronize()
    for name, x in [("selection dense output", od), ("residual", meta.residual), ("dense baseline", dense)] + \
            [(f"reuse step {t}", o) for t, o in outs.items()]:
        bad = int((~torch.isfinite(x)).sum())
        assert bad == 0, f"{label}: {name} has {bad} elements unwritten or not finite"
    perm = meta.perm.long()
    assert torch.equal(torch.sort(perm, dim=1).values, torch.arange(N, device="cuda").expand(H, N)), \
        f"{label}: perm is not a permutation of every head"
    return meta, od, outs, dense


def test_workload2_every_unit():
    _need_gpu()
    w = WORKLOADS[2]
    print(f"[exhaustive] workload 2: H={w.heads} N={w.seq_len} G={w.group} keep={w.keeps()[0]}", flush=True)
    p = build_problem(w.grid, w.heads, w.head_dim, w.dtype, w.group, w.keeps(), w.drift, [1, 10], wid=w.wid)
    sc = scale_for(w.head_dim)
    meta, od, outs, dense = _run(p, sc, [1, 10], "workload 2")
    exact, total = check_every_unit(p, meta, sc, outs, range(w.heads), "workload 2",
                                    dense=[("selection dense output", od), ("dense baseline", dense)],
                                    dense_heads=(w.heads - 1,))
    print(f"[exhaustive] workload 2: {w.heads * p.ng} units x 2 reuse steps checked; head {w.heads - 1}: "
          f"{exact}/{total} kept-key sets equal to the oracle's", flush=True)


def test_workload3_every_group_of_two_heads():
    _need_gpu()
    w = WORKLOADS[3]
    heads = (0, w.heads - 1)
    print(f"[exhaustive] workload 3: H={w.heads} N={w.seq_len} G={w.group} keep={w.keeps()[0]}", flush=True)
    p = build_problem(w.grid, w.heads, w.head_dim, w.dtype, w.group, w.keeps(), w.drift, [20], wid=w.wid,
                      keep_heads=set(heads))
    sc = scale_for(w.head_dim)
    meta, _, outs, _ = _run(p, sc, [20], "workload 3")
    check_every_unit(p, meta, sc, outs, heads, "workload 3")
    print(f"[exhaustive] workload 3: every group of heads {heads} checked", flush=True)


def test_midsize_every_unit_with_selection():
    _need_gpu()
    grid, H, d, G = (8, 32, 32), 16, 128, 64
    keeps = np.array([512, 320, 1024, 64] * 4, np.int32)
    print(f"[exhaustive] mid-size: grid={grid} H={H} d={d} G={G}", flush=True)
    p = build_problem(grid, H, d, "bf16", G, keeps, 0.02, [3], wid=111)
    sc = scale_for(d)
    meta, od, outs, dense = _run(p, sc, [3], "mid-size")
    exact, total = check_every_unit(p, meta, sc, outs, range(H), "mid-size",
                                    dense=[("selection dense output", od), ("dense baseline", dense)],
                                    dense_heads=range(H))
    print(f"[exhaustive] mid-size: {exact}/{total} kept-key sets equal to the oracle's", flush=True)

"""mcs_select_noalloc (the selection with the library's own workspace array,
for callers that cannot allocate) against mcs_select_ex with a caller
workspace, through the C ABI: two calls in a row, the second on a smaller
input.  The first is the full workload-2 layer, whose 24 heads do not fit the
array at once and run in head chunks; the metadata, the step's dense output
and the reuse output on the same metadata are byte-identical to the
workspace call (which the other GPU tests compare with the oracle)."""

import numpy as np
import pytest
import torch

from mcs_inputs import WORKLOADS
from parity import build_problem, scale_for

pytestmark = pytest.mark.gpu

mcs = pytest.importorskip("sparse_attention_diffusion_mcs_amd")
from sparse_attention_diffusion_mcs_amd import _lib as L  # noqa: E402


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


REGIONS = ("perm", "keep", "idx_start", "sched", "idx", "residual")


def _compare(p, label):
    sc = scale_for(p.d)
    q = p.dev[0][0]
    H, N, d = q.shape
    need = mcs.workspace_bytes(q, p.G, 1)
    assert need <= L.MCS_NOALLOC_SCRATCH_BYTES
    print(f"[no-alloc] {label}: H={H} N={N} d={d} G={p.G}; workspace for one head {need} bytes of "
          f"{L.MCS_NOALLOC_SCRATCH_BYTES}", flush=True)
    ref, od_ref = mcs.select(*p.dev[0], p.G, p.keeps, p.proj(), scale=sc, return_dense=True)
    nbytes = ref.buffer.numel()
    # a metadata buffer full of 0xFF (a NaN pattern) and a NaN dense output
    buf = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    od = torch.full_like(od_ref, float("nan"))
    meta, _ = mcs.select(*p.dev[0], p.G, p.keeps, p.proj(), scale=sc, meta_buf=buf, dense_out=od, noalloc=True)
    t = p.steps[0]
    out_ref = mcs.sparse_attn(*p.dev[t], ref, scale=sc)
    out = mcs.sparse_attn(*p.dev[t], meta, scale=sc)
    torch.cuda.synchronize()
    for region in REGIONS:
        assert torch.equal(getattr(meta, region), getattr(ref, region)), f"{label}: {region} differs"
    assert torch.equal(od, od_ref), f"{label}: dense output differs"
    assert torch.equal(out, out_ref), f"{label}: reuse output differs"


def test_noalloc_selection_matches_the_workspace_call_twice():
    _need_gpu()
    w = WORKLOADS[2]
    big = build_problem(w.grid, w.heads, w.head_dim, w.dtype, w.group, w.keeps(), w.drift, [1], wid=w.wid)
    _compare(big, "workload 2")
    del big
    torch.cuda.empty_cache()
    small = build_problem((3, 8, 21), 3, 128, "bf16", 64, [64, 300, 503], 0.02, [1], wid=108)
    _compare(small, "small")

"""GPU parity at the largest sizes the library accepts: the reuse and dense
kernels at N = MCS_MAX_SEQ_LEN (one head), and the selection step at
N = 2^20, whose score workspace (ng x N float32, 69 GB) is the memory bound
of a selection.  The reuse and dense inputs are seeded N(0, 1) bf16 tensors
drawn on the GPU; the selection runs on the workload generator's
DiT-shaped inputs (near-uniform attention over a million random keys would
leave outputs of ~1e-3 from a residual that cancels most of the sparse
output).  Outputs are checked against the oracle on sampled groups and
rows."""

import numpy as np
import pytest
import torch

import oracle.mcs_oracle as orc
from parity import assert_close, build_problem, check_units, sample_groups, scale_for, to_np

pytestmark = pytest.mark.gpu

mcs = pytest.importorskip("sparse_attention_diffusion_mcs_amd")
from sparse_attention_diffusion_mcs_amd import _lib  # noqa: E402


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _qkv(N, d, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return [torch.randn((1, N, d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
            for _ in range(3)]


def _host(t, rows=None):
    x = t[0] if rows is None else t[0, torch.as_tensor(rows, device=t.device, dtype=torch.long)]
    return x.float().cpu().numpy()


@pytest.mark.parametrize("d,keep", [(128, 77), (64, 64)])
def test_reuse_at_max_seq_len(d, keep):
    """Reuse on injected metadata (random permutation, stratified ascending
    kept keys, random residual) over 2^22 tokens: 65536 groups."""
    _need_gpu()
    N, G = _lib.MCS_MAX_SEQ_LEN, 64
    print(f"[case] reuse N={N} d={d} keep={keep}", flush=True)
    sc = scale_for(d)
    q, k, v = _qkv(N, d, 11 + d)
    meta = mcs.meta_init(q, G, [keep])
    ng = meta.meta.num_groups
    g = torch.Generator(device="cuda").manual_seed(5)
    perm = torch.randperm(N, generator=g, device="cuda").to(torch.int32)
    stride = N // keep
    idx = (torch.arange(keep, device="cuda", dtype=torch.int64) * stride
           + torch.randint(0, stride, (ng, keep), generator=g, device="cuda")).to(torch.int32)
    resid = 0.1 * torch.randn((1, N, d), generator=g, device="cuda", dtype=torch.float32)
    meta.perm.copy_(perm.view(1, N))
    meta.idx.copy_(idx.reshape(-1))
    meta.residual.copy_(resid)
    out = mcs.sparse_attn(q, k, v, meta, scale=sc)
    torch.cuda.synchronize()
    for gi in sample_groups(ng, extra=4, seed=d):
        rows = perm[gi * G:(gi + 1) * G].cpu().numpy()
        kept = idx[gi].cpu().numpy()
        res_g = resid[0, gi * G:(gi + 1) * G].cpu().numpy().astype(np.float64)
        ref = orc.reuse_group(_host(q, rows), _host(k, kept), _host(v, kept), np.arange(G), np.arange(keep), res_g,
                              sc)
        assert_close(to_np(out[0, torch.as_tensor(rows, device="cuda", dtype=torch.long)]), ref, "bf16",
                     f"reuse N={N} d={d} group {gi}")


def test_dense_at_max_seq_len():
    """The dense kernel over 2^22 tokens (d = 128), on sampled rows."""
    _need_gpu()
    N, d = _lib.MCS_MAX_SEQ_LEN, 128
    print(f"[case] dense N={N} d={d}", flush=True)
    sc = scale_for(d)
    q, k, v = _qkv(N, d, 21)
    out = mcs.dense_attn(q, k, v, scale=sc)
    torch.cuda.synchronize()
    rows = np.array(sample_groups(N, extra=4, seed=1))
    kh, vh = _host(k), _host(v)
    ref, _ = orc.attention(_host(q, rows), kh, vh, sc)
    assert_close(to_np(out[0, torch.as_tensor(rows, device="cuda", dtype=torch.long)]), ref, "bf16",
                 f"dense N={N} rows {rows.tolist()}")


def test_selection_at_one_million_tokens():
    """Selection over 2^20 tokens of a 16 x 256 x 256 latent grid (the
    workload generator, Z-curve groups of 64, keep 5%), then one drifted reuse
    step: permutation, kept keys, dense rows, residual and reuse output of
    sampled groups against the oracle."""
    _need_gpu()
    grid, d, G = (16, 256, 256), 128, 64
    N = int(np.prod(grid))
    keep = N // 20
    print(f"[case] select N={N} grid={grid} d={d} G={G} keep={keep}", flush=True)
    p = build_problem(grid, 1, d, "bf16", G, [keep], 0.02, [1], wid=110)
    sc = scale_for(d)
    meta, od = mcs.select(*p.dev[0], G, p.keeps, p.proj(), scale=sc, return_dense=True, grouping="morton",
                          grid=grid)
    outs = {1: mcs.sparse_attn(*p.dev[1], meta, scale=sc)}
    torch.cuda.synchronize()
    exact, total = check_units(p, meta, od, outs, sc, [0], sample_groups(p.ng, extra=0), f"N={N}", "morton")
    print(f"[case] select N={N}: {exact}/{total} sampled kept-key sets identical to the oracle's", flush=True)

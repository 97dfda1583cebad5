"""Stream plumbing on the GPU: every call runs on the stream it is given, and
the reuse step, which allocates nothing and issues no memset or copy, can be
captured in a graph and replayed."""

import pytest
import torch

from parity import build_problem, scale_for

pytestmark = pytest.mark.gpu

mcs = pytest.importorskip("sparse_attention_diffusion_mcs_amd")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _problem():
    print("[case] streams: grid (4, 6, 25), 2 heads, d 128, G 64, keep [96, 200]", flush=True)
    return build_problem((4, 6, 25), 2, 128, "bf16", 64, [96, 200], 0.02, [1, 2], wid=120)


def test_side_stream_matches_the_current_stream():
    """Selection, reuse and dense attention launched on a side stream give
    the same bytes as on the current stream."""
    _need_gpu()
    p = _problem()
    sc = scale_for(p.d)
    proj = p.proj()
    meta_a, od_a = mcs.select(*p.dev[0], p.G, p.keeps, proj, scale=sc, return_dense=True)
    out_a = mcs.sparse_attn(*p.dev[1], meta_a, scale=sc)
    dense_a = mcs.dense_attn(*p.dev[1], scale=sc)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        meta_b, od_b = mcs.select(*p.dev[0], p.G, p.keeps, proj, scale=sc, return_dense=True, stream=side)
        out_b = mcs.sparse_attn(*p.dev[1], meta_b, scale=sc, stream=side)
        dense_b = mcs.dense_attn(*p.dev[1], scale=sc, stream=side)
    side.synchronize()
    for region in ("perm", "keep", "idx_start", "sched", "idx", "residual"):
        assert torch.equal(getattr(meta_a, region), getattr(meta_b, region)), region
    assert torch.equal(od_a, od_b) and torch.equal(out_a, out_b) and torch.equal(dense_a, dense_b)


def test_reuse_step_replays_from_a_graph():
    """The reuse step captured once and replayed, with eager work and new
    input values between replays: every replay equals the eager call on the
    inputs of that moment."""
    _need_gpu()
    p = _problem()
    sc = scale_for(p.d)
    meta, _ = mcs.select(*p.dev[0], p.G, p.keeps, p.proj(), scale=sc)
    q, k, v = (x.clone() for x in p.dev[1])
    out = torch.empty_like(q)
    mcs.sparse_attn(q, k, v, meta, out=out, scale=sc)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mcs.sparse_attn(q, k, v, meta, out=out, scale=sc)
    for t in (1, 2, 1):
        for dst, src in zip((q, k, v), p.dev[t]):
            dst.copy_(src)
        graph.replay()
        replayed = out.clone()
        eager = mcs.sparse_attn(q, k, v, meta, scale=sc)
        torch.cuda.synchronize()
        assert torch.equal(replayed, eager), f"replay on the step-{t} inputs"
    # the replays read the buffers captured, not copies of them
    assert not torch.equal(mcs.sparse_attn(*p.dev[1], meta, scale=sc), mcs.sparse_attn(*p.dev[2], meta, scale=sc))


def test_selection_replays_from_a_graph():
    """The selection step (grouping, dense pass with key scores, top-k,
    residual: kernel launches only) captured into a graph with caller-owned
    metadata and workspace buffers; replays on new inputs equal eager
    selections on those inputs."""
    _need_gpu()
    p = _problem()
    sc = scale_for(p.d)
    proj = p.proj()
    q, k, v = (x.clone() for x in p.dev[0])
    ref_meta, _ = mcs.select(q, k, v, p.G, p.keeps, proj, scale=sc)
    meta_buf = torch.empty_like(ref_meta.buffer)
    ws = torch.empty(mcs.workspace_bytes(q, p.G), dtype=torch.uint8, device="cuda")
    mcs.select(q, k, v, p.G, p.keeps, proj, scale=sc, meta_buf=meta_buf, workspace=ws)  # warm-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        meta, _ = mcs.select(q, k, v, p.G, p.keeps, proj, scale=sc, meta_buf=meta_buf, workspace=ws)
    for t in (1, 2, 0):
        for dst, src in zip((q, k, v), p.dev[t]):
            dst.copy_(src)
        graph.replay()
        torch.cuda.synchronize()
        eager, _ = mcs.select(*p.dev[t], p.G, p.keeps, proj, scale=sc)
        torch.cuda.synchronize()
        for region in ("perm", "keep", "idx_start", "sched", "idx", "residual"):
            assert torch.equal(getattr(meta, region), getattr(eager, region)), f"step {t} {region}"

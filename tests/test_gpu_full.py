"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: the whole layer runs on the GPU, and sampled (head, group)
units (groups 0, 1, middle, the ragged last one and four seeded others) are
checked one by one against the CPU oracle, together with the whole-head
permutation."""

import numpy as np
import pytest
import torch

from mcs_inputs import WORKLOADS
from parity import build_problem, check_units, sample_groups, scale_for

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

mcs = pytest.importorskip("sparse_attention_diffusion_mcs_amd")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_workload(w, steps, heads, label, select_step=0, grouping="hash", kv_block=1, residual=True):
    print(f"[full] {label}: H={w.heads} N={w.seq_len} d={w.head_dim} G={w.group} keeps={sorted(set(w.keeps()))}",
          flush=True)
    keeps = w.keeps()
    gen_steps = sorted(set(steps) | ({select_step} - {0}))
    p = build_problem(w.grid, w.heads, w.head_dim, w.dtype, w.group, keeps, w.drift, gen_steps, wid=w.wid,
                      keep_heads=set(heads))
    sc = scale_for(w.head_dim)
    if select_step:
        # re-selection on a later step's inputs: treat that step as step 0
        for h in heads:
            p.heads_np[(h, 0)] = p.heads_np[(h, select_step)]
        p.dev[0] = p.dev[select_step]
    meta, od = mcs.select(*p.dev[0], w.group, keeps, p.proj(), scale=sc, return_dense=True, grouping=grouping,
                          grid=w.grid if grouping == "morton" else None, kv_block=kv_block, residual=residual)
    outs = {t: mcs.sparse_attn(*p.dev[t], meta, scale=sc) for t in steps}
    torch.cuda.synchronize()
    exact, total = check_units(p, meta, od, outs, sc, heads, sample_groups(p.ng), label, grouping, kv_block,
                               residual)
    print(f"[full] {label}: kept-key sets equal to the oracle's: {exact}/{total}", flush=True)


def test_workload2_video_layer():
    _need_gpu()
    w = WORKLOADS[2]
    run_workload(w, [1, 5, 10], [0, w.heads - 1], "workload 2")


def test_workload2_zcurve_groups():
    """The secondary grouping the benchmark also times: Z-curve order over the 16 x 30 x 52 grid."""
    _need_gpu()
    w = WORKLOADS[2]
    run_workload(w, [1, 10], [0, w.heads - 1], "workload 2 z-curve", grouping="morton")


def test_workload5_zcurve_groups_g128():
    _need_gpu()
    w = WORKLOADS[5].with_(group=128)
    run_workload(w, [9], [0, w.heads - 1], "workload 5 z-curve G=128", grouping="morton")


def test_workload2_zcurve_64key_blocks():
    """Block-granular selection (whole 64-key blocks) at the full workload-2 size."""
    _need_gpu()
    w = WORKLOADS[2]
    run_workload(w, [1, 10], [0, w.heads - 1], "workload 2 z-curve 64-key blocks", grouping="morton", kv_block=64)


def test_workload4_no_residual():
    """Renormalised sparse output alone (no residual) at the full workload-4 size."""
    _need_gpu()
    w = WORKLOADS[4]
    run_workload(w, [1, 15], [0, w.heads - 1], "workload 4 no residual", residual=False)


def test_workload3_long_video_layer():
    _need_gpu()
    w = WORKLOADS[3]
    run_workload(w, [1, 20], [0, w.heads - 1], "workload 3")


def test_workload4_asset_layer_per_head_keep():
    _need_gpu()
    w = WORKLOADS[4]
    keeps = w.keeps()
    heads = sorted({0, w.heads - 1} | {int(np.nonzero(keeps == k)[0][0]) for k in set(keeps.tolist())})
    run_workload(w, [1, 15], heads, "workload 4")


@pytest.mark.parametrize("keep", [0.02, 0.05, 0.10, 0.25, 1.0])
@pytest.mark.parametrize("group", [64, 128])
def test_workload5_sweep_point(keep, group):
    _need_gpu()
    w = WORKLOADS[5].with_(keep_frac=(keep,), group=group)
    run_workload(w, [9], [0, w.heads - 1], f"workload 5 keep={keep} G={group}")


def test_workload5_reselection():
    """Re-selection at step 10 of the denoising loop, then reuse at step 19."""
    _need_gpu()
    w = WORKLOADS[5]
    run_workload(w, [19], [0, w.heads - 1], "workload 5 reselect@10", select_step=10)

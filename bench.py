#!/usr/bin/env python3
"""MC-Sparse benchmark on one MI355X.

One timed step is one denoising segment of the workload: the selection step
(hash and group permutation, exact dense attention with per-group key scores,
per-group top-k, selection-time sparse pass and residual) on the step-0
inputs, followed by every reuse step on that step's drifted inputs.  All
inputs are generated (seeded, synthetic) and resident in device memory before
the timed region.  The library's own dense attention is timed on the same
inputs as the speedup baseline.  Workload 6 is the joint attention of an
MM-DiT block: workload 2's video tokens followed by 226 text tokens in one
sequence.

Prints one JSON line: `value` is the mean reuse-step time in ms (lower is
better), with the speedup over dense, the selection time, the amortised time
per denoising step, the roofline of the reuse kernel measured with HIP events
on the launch stream, and the CPU oracle timed on a bounded sample of the same
workload on this host.

With --ablation the line also carries the failure-mode ablations: the same
segment with raster query groups, centred-hash groups, whole 64-key KV
blocks, no residual, and the coarse three together, each with its timings
and per-step fidelity.

The line also carries reuse and dense times measured with the L2s and the
MALL flushed (a 512 MiB buffer overwritten) before each call (--no-cold-cache
skips them), the selection's phases timed with events the library records
between them, the achieved HBM rates of the index-gather kernels (top-k,
hash and sort) on algorithmic bytes, and the same segment with Z-curve
query groups as a secondary measurement (--no-zcurve skips it).  Queries are
grouped by MC-Sparse's 8-bit sign hash unless --grouping says otherwise.

With --sweep (workload 5) the line also carries the denoising-loop sweep:
for every keep fraction and group size, a 30-step loop with re-selection every
10 steps, its amortised time against 30 dense steps and the relative L2 error
of every step's output against dense attention on that step.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--seed 0] [--grouping hash]
                    [--sweep] [--ablation] [--no-cold-cache] [--no-zcurve] [--no-cpu-baseline]

Three converters turn rocprofv3 results into the summaries kept in profiles/
(no GPU needed):

    python bench.py --trace-summary RESULTS.db OUT.md "TITLE" "COMMAND"
    python bench.py --traffic-summary FETCH.db WRITE.db OUT.json GROUPING
    python bench.py --counter-summary OUT.md RESULTS.db [RESULTS.db ...] [--kernel NAME]
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from mcs_inputs import WORKLOADS, hash_projections, head_base, head_step, token_embedding  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
METRIC = "reuse-step sparse attn ms + speedup vs dense; % bf16 MFMA peak (1 GPU)"
ATTN_SRC = os.path.join(ROOT, "sparse_attention_diffusion_mcs_amd", "csrc", "attn_bf16.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_reuse_workload2.json")
SELECT_SRC = os.path.join(ROOT, "sparse_attention_diffusion_mcs_amd", "csrc", "select.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5, help="timed denoising segments")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=2, choices=[2, 3, 4, 5, 6])
    ap.add_argument("--keep", type=float, default=None, help="override the keep fraction")
    ap.add_argument("--group", type=int, default=None, help="override the group size")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold-cache", action="store_true",
                    help="skip timing reuse and dense calls with the L2s and the MALL flushed before each call")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one plain 1 GiB device-to-device copy first (a known-size reference for HBM counters)")
    ap.add_argument("--cpu-groups", type=int, default=288, help="oracle groups sampled per sampled head")
    ap.add_argument("--threads", type=int, default=min(16, os.cpu_count() or 8))
    ap.add_argument("--grouping", default="hash", choices=["hash", "morton", "raster", "centred"],
                    help="query grouping: 8-bit sign hash (default, MC-Sparse), Z-curve over the latent grid, "
                         "raster, centred hash")
    ap.add_argument("--seed", type=int, default=0, help="seed of the synthetic inputs and hash projections")
    ap.add_argument("--no-zcurve", action="store_true", help="skip the secondary Z-curve-grouping measurement")
    ap.add_argument("--ablation", action="store_true",
                    help="add the failure-mode ablations (raster groups, 64-key blocks, no residual)")
    ap.add_argument("--sweep", action="store_true",
                    help="workload 5 only: add the keep x group denoising-loop sweep to the result")
    ap.add_argument("--extensions", action="store_true",
                    help="add the extensions: bf16 residual, retained-mass budgets against fixed budgets of the "
                         "same mean size, and (with a re-selection interval, workload 5) the error-triggered "
                         "re-selection policy against the fixed interval")
    return ap.parse_args()


def workload_of(args):
    w = WORKLOADS[args.workload]
    if args.keep is not None:
        w = w.with_(keep_frac=(args.keep,))
    if args.group is not None:
        w = w.with_(group=args.group)
    return w


def describe(w, keeps):
    ks = sorted(set(int(k) for k in keeps))
    kdesc = str(ks[0]) if len(ks) == 1 else "/".join(map(str, ks))
    T, Y, X = w.grid
    toks = f"{T}x{Y}x{X}" + (f" + {w.text} text" if w.text else "")
    return (f"{w.name}: H={w.heads}, N={w.seq_len} ({toks}), d={w.head_dim}, {w.dtype}, G={w.group}, "
            f"k={kdesc} per group, select once + {w.reuse_steps} reuse steps, drift {w.drift}*t")


def generate(w, steps, threads, seed=0):
    """Device tensors per step: {t: (q, k, v)} in [H, N, d] bf16."""
    import torch
    pos = token_embedding(w.grid, w.head_dim, w.text, seed, w.wid)
    H, N, d = w.heads, w.seq_len, w.head_dim
    bases = [None] * H

    def mk_base(h):
        bases[h] = head_base(seed, w.wid, h, w.grid, d, pos)

    with cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(mk_base, range(H)))
    out = {}
    for t in steps:
        host = [np.empty((H, N, d), np.float32) for _ in range(3)]

        def mk(h):
            xs = head_step(bases[h], seed, w.wid, h, t, w.drift, True)
            for i in range(3):
                host[i][h] = xs[i]

        with cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(mk, range(H)))
        out[t] = tuple(torch.from_numpy(x).to("cuda").to(torch.bfloat16) for x in host)
        del host
    return out


def src_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def cpu_baseline(w, keeps, T, scale, n_groups, seed=0):
    """Times the oracle on sampled (head, group) units of the workload and
    extrapolates to the whole layer."""
    import threadpoolctl

    import oracle.mcs_oracle as orc

    H, N, d, G = w.heads, w.seq_len, w.head_dim, w.group
    ng = w.num_groups
    heads = sorted({0, H - 1})
    rng = np.random.default_rng(1234)
    fixed = [0, 1, ng // 2, ng - 1]
    extra = rng.choice(np.arange(2, ng - 1), size=max(0, min(n_groups, ng) - len(set(fixed))), replace=False)
    groups = sorted(set(fixed) | set(int(x) for x in extra))
    tsteps = sorted({1, max(1, T // 2), T})
    pos = token_embedding(w.grid, d, w.text, seed, w.wid)
    proj = hash_projections(seed, w.wid, d)
    info = threadpoolctl.threadpool_info()
    cores = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    t_hash, t_sel, t_reuse = [], [], []
    for h in heads:
        base = head_base(seed, w.wid, h, w.grid, d, pos)
        q, k, v = head_step(base, seed, w.wid, h, 0, w.drift, True)
        later = {t: head_step(base, seed, w.wid, h, t, w.drift, True) for t in tsteps}
        t0 = time.perf_counter()
        perm = orc.group_permutation(orc.hash_keys(q, proj))
        t_hash.append(time.perf_counter() - t0)
        ranges = orc.group_ranges(N, G)
        for g in groups:
            rows = perm[ranges[g][0]:ranges[g][1]]
            t0 = time.perf_counter()
            sel = orc.select_group(q, k, v, rows, int(keeps[h]), scale)
            t_sel.append(time.perf_counter() - t0)
            for t in tsteps:
                t0 = time.perf_counter()
                orc.reuse_group(*later[t], rows, sel.idx, sel.residual, scale)
                t_reuse.append(time.perf_counter() - t0)
    units = H * ng
    sel_ms = 1e3 * (np.mean(t_hash) * H + np.mean(t_sel) * units)
    reuse_ms = 1e3 * np.mean(t_reuse) * units
    work_s = sum(t_hash) + sum(t_sel) + sum(t_reuse)
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(float(reuse_ms), 3), "unit": "ms", "cores": int(cores), "kind": "oracle",
        "sample": (f"float64 numpy oracle on heads {heads} x {len(groups)} of {ng} query groups "
                   f"(reuse steps {tsteps}); per-unit mean times x {units} units = extrapolated full-layer "
                   f"reuse-step ms; {work_s:.1f} s of CPU work; {cpu_model}"),
        "select_ms_extrapolated": round(float(sel_ms), 1),
    }


FLUSH_BYTES = 512 << 20  # more than the 256 MB MALL and every XCD's L2 together


def cold_cache(X, meta, scale, T, steps, stream, mcs):
    """Reuse and dense calls timed with cold caches: before each timed call a
    512 MiB buffer is overwritten, which evicts the K/V rows that the
    previous call left in the L2s and the MALL.  The fill runs outside the
    events; the same treatment is given to both kernels."""
    import torch
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(X[0][0])

    def timed(fn, k):
        flush.fill_(k & 0xFF)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        return a, b

    reuse = [timed(lambda t=t: mcs.sparse_attn(*X[t], meta, out=out, scale=scale), t) for t in range(1, T + 1)]
    dense = [timed(lambda k=k: mcs.dense_attn(*X[1 + k % T], out=out, scale=scale), k) for k in range(steps)]
    torch.cuda.synchronize()
    r = float(np.median([a.elapsed_time(b) for a, b in reuse]))
    dn = float(np.median([a.elapsed_time(b) for a, b in dense]))
    del flush
    return {"flush_bytes": FLUSH_BYTES, "reuse_ms_median": round(r, 4), "dense_ms_median": round(dn, 4),
            "speedup_vs_dense": round(dn / r, 3)}


def rel_l2(a, b):
    import torch
    return float(torch.linalg.vector_norm(a.float() - b.float()) / torch.linalg.vector_norm(b.float()))


def sweep(w, X, threads, scale, grouping, seed=0):
    """Denoising-loop sweep: for each (keep, G), steps 0..S-1 with selection on
    the steps divisible by the re-selection interval and reuse on the others;
    every step's output is compared with dense attention on that step."""
    import torch

    import sparse_attention_diffusion_mcs_amd as mcs

    S, R = w.sweep["steps"], w.reselect
    H, N, d = w.heads, w.seq_len, w.head_dim
    stream = torch.cuda.current_stream()
    proj = hash_projections(seed, w.wid, d)
    dense = {}
    dense_ms = []
    for t in range(S):  # dense outputs of every step (the fidelity reference), each timed
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dense[t] = mcs.dense_attn(*X[t], scale=scale)
        e1.record(stream)
        torch.cuda.synchronize()
        dense_ms.append(e0.elapsed_time(e1))
    dense_med = float(np.median(dense_ms[1:]))
    points = []
    for G in w.sweep["group"]:
        for frac in w.sweep["keep"]:
            wk = w.with_(keep_frac=(frac,), group=G)
            keeps = wk.keeps(seed)
            ws = torch.empty(mcs.workspace_bytes(X[0][0], G), dtype=torch.uint8, device="cuda")
            mb = torch.empty(int(mcs.meta_layout(H, N, d, 1, G, keeps).bytes), dtype=torch.uint8, device="cuda")
            out = torch.empty_like(X[0][0])
            od = torch.empty_like(X[0][0])
            gkw = grouping_kw(wk, grouping)
            mcs.select(*X[0], G, keeps, proj, scale=scale, meta_buf=mb, workspace=ws, **gkw)  # warm-up
            torch.cuda.synchronize()
            sel_ms, reuse_ms, err = [], [], []
            meta = None
            for t in range(S):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                if t % R == 0:
                    e0.record(stream)
                    meta, _ = mcs.select(*X[t], G, keeps, proj, scale=scale, meta_buf=mb, workspace=ws,
                                         dense_out=od, **gkw)
                    e1.record(stream)
                    torch.cuda.synchronize()
                    sel_ms.append(e0.elapsed_time(e1))
                    err.append(rel_l2(od, dense[t]))
                else:
                    e0.record(stream)
                    mcs.sparse_attn(*X[t], meta, out=out, scale=scale)
                    e1.record(stream)
                    torch.cuda.synchronize()
                    reuse_ms.append(e0.elapsed_time(e1))
                    err.append(rel_l2(out, dense[t]))
            total = float(np.sum(sel_ms) + np.sum(reuse_ms))
            reuse_err = [e for t, e in enumerate(err) if t % R != 0]
            points.append({
                "keep_frac": frac, "group": G, "keep": int(keeps[0]),
                "select_ms": round(float(np.median(sel_ms)), 3),
                "reuse_ms": round(float(np.mean(reuse_ms)), 4),
                "amortised_vs_dense": round(total / (S * dense_med), 4),
                "speedup_vs_dense": round(S * dense_med / total, 3),
                "rel_l2_mean_all_steps": round(float(np.mean(err)), 6),
                "rel_l2_mean_reuse_steps": round(float(np.mean(reuse_err)), 6),
                "rel_l2_final": round(float(err[-1]), 6),
                "meta_bytes": int(mb.numel()),
            })
            log(f"sweep G={G} keep={frac}: {points[-1]}")
            del ws, mb, out, meta
            torch.cuda.empty_cache()
    return {"steps": S, "reselect_every": R, "dense_ms": round(dense_med, 4), "points": points}


def _timed(stream, fn):
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    r = fn()
    e1.record(stream)
    return r, (e0, e1)


def extensions(w, X, keeps, scale, grouping, seed):
    """The method's extensions on the workload's inputs:
    * bf16 residual: the segment (selection on step 0, reuse on steps 1..T)
      with the residual cached in bfloat16 against the float32 one;
    * retained-mass budgets: for each mass target (capped at 25% of the keys)
      the segment's reuse time, the mean kept keys per group and the
      per-step fidelity, next to a fixed budget of the same mean size;
    * re-selection policy (a workload with a re-selection interval R over S
      steps): the fixed interval against an error-triggered policy that
      measures, after every reuse step, the relative L2 error of one probe
      head against exact attention (one head's dense pass) and re-selects on
      the next step when it exceeds a threshold.
    Fidelity is the relative L2 error of each step's output against dense
    attention on that step (computed outside the timed calls)."""
    import torch

    import sparse_attention_diffusion_mcs_amd as mcs
    from mcs_inputs import keep_count

    H, N, d, G, T = w.heads, w.seq_len, w.head_dim, w.group, w.reuse_steps
    stream = torch.cuda.current_stream()
    proj = hash_projections(seed, w.wid, d)
    gkw = grouping_kw(w, grouping)
    steps = sorted(X)
    dense = {t: mcs.dense_attn(*X[t], scale=scale) for t in steps}
    torch.cuda.synchronize()
    out = torch.empty_like(X[0][0])
    res = {}

    def segment(keep_arr, **kw):
        """Selection on step 0 and reuse on steps 1..T, each call timed."""
        ws = torch.empty(mcs.workspace_bytes(X[0][0], G, residual_dtype=kw.get("residual_dtype", "fp32")),
                         dtype=torch.uint8, device="cuda")
        meta, _ = mcs.select(*X[0], G, keep_arr, proj, scale=scale, workspace=ws, **gkw, **kw)  # warm-up
        torch.cuda.synchronize()
        meta, sel_ev = _timed(stream, lambda: mcs.select(*X[0], G, keep_arr, proj, scale=scale, meta_buf=meta.buffer,
                                                          workspace=ws, **gkw, **kw)[0])
        ev, err = [], []
        for t in range(1, T + 1):
            _, e = _timed(stream, lambda t=t: mcs.sparse_attn(*X[t], meta, out=out, scale=scale))
            ev.append(e)
            err.append(rel_l2(out, dense[t]))
        torch.cuda.synchronize()
        counts = meta.count.float()
        r = {"select_ms": round(sel_ev[0].elapsed_time(sel_ev[1]), 3),
             "reuse_ms": round(float(np.mean([a.elapsed_time(b) for a, b in ev])), 4),
             "mean_keys_per_group": round(float(counts.mean()), 1),
             "keys_per_group_p10_p90": [int(torch.quantile(counts, 0.1)), int(torch.quantile(counts, 0.9))],
             "meta_bytes": int(meta.nbytes),
             "rel_l2_step1": round(err[0], 6), "rel_l2_mean": round(float(np.mean(err)), 6),
             "rel_l2_final": round(err[-1], 6)}
        del meta, ws
        torch.cuda.empty_cache()
        return r

    log("extensions: float32 vs bf16 residual")
    res["residual"] = {"fp32": segment(keeps), "bf16": segment(keeps, residual_dtype="bf16")}
    log(f"extensions: {res['residual']}")

    cap = np.full(H, keep_count(0.25, N), dtype=np.int32)
    mass_rows = []
    for mass in (0.9, 0.95, 0.98, 0.99):
        r = segment(cap, keep_mass=mass)
        kfix = int(max(64, round(r["mean_keys_per_group"] / 64) * 64))
        f = segment(np.full(H, min(kfix, N), dtype=np.int32))
        mass_rows.append({"mass": mass, "cap": int(cap[0]), "mass_budget": r, "fixed_budget_same_mean": f,
                          "fixed_keep": kfix})
        log(f"extensions: mass {mass}: {mass_rows[-1]}")
    res["retained_mass_budgets"] = mass_rows

    if w.reselect and len(steps) > w.reselect + 1:
        S = len(steps)
        ws = torch.empty(mcs.workspace_bytes(X[0][0], G), dtype=torch.uint8, device="cuda")
        mb = torch.empty(int(mcs.meta_layout(H, N, d, 1, G, keeps).bytes), dtype=torch.uint8, device="cuda")
        od = torch.empty_like(X[0][0])
        probe_out = torch.empty_like(X[0][0][:1])
        mcs.select(*X[0], G, keeps, proj, scale=scale, meta_buf=mb, workspace=ws, **gkw)  # warm-up
        torch.cuda.synchronize()

        def run(policy, arg):
            total_ms, probe_ms, errs, selected = 0.0, 0.0, [], []
            meta, pending = None, True
            for t in range(S):
                if pending or (policy == "interval" and t % arg == 0):
                    meta, e = _timed(stream, lambda t=t: mcs.select(*X[t], G, keeps, proj, scale=scale, meta_buf=mb,
                                                                     workspace=ws, dense_out=od, **gkw)[0])
                    torch.cuda.synchronize()
                    total_ms += e[0].elapsed_time(e[1])
                    errs.append(rel_l2(od, dense[t]))
                    selected.append(t)
                    pending = False
                    continue
                _, e = _timed(stream, lambda t=t: mcs.sparse_attn(*X[t], meta, out=out, scale=scale))
                if policy == "error":
                    # the measured quantity: one probe head's error against exact attention
                    _, e2 = _timed(stream, lambda t=t: mcs.dense_attn(X[t][0][:1], X[t][1][:1], X[t][2][:1],
                                                                      out=probe_out, scale=scale))
                    torch.cuda.synchronize()
                    total_ms += e2[0].elapsed_time(e2[1])
                    probe_ms += e2[0].elapsed_time(e2[1])
                    pending = rel_l2(out[:1], probe_out) > arg
                torch.cuda.synchronize()
                total_ms += e[0].elapsed_time(e[1])
                errs.append(rel_l2(out, dense[t]))
            return {"policy": policy, "parameter": arg, "selections_at": selected, "n_selections": len(selected),
                    "total_ms": round(total_ms, 3), "probe_ms": round(probe_ms, 3),
                    "ms_per_step": round(total_ms / S, 4),
                    "rel_l2_mean": round(float(np.mean(errs)), 6), "rel_l2_max": round(float(np.max(errs)), 6),
                    "rel_l2_final": round(errs[-1], 6), "rel_l2_per_step": [round(x, 4) for x in errs]}

        dense_ms = []
        for t in steps[1:6]:
            _, e = _timed(stream, lambda t=t: mcs.dense_attn(*X[t], out=out, scale=scale))
            torch.cuda.synchronize()
            dense_ms.append(e[0].elapsed_time(e[1]))
        rows = [run("interval", r) for r in (5, w.reselect, 15)]
        rows += [run("error", th) for th in (0.01, 0.02, 0.04)]
        for r in rows:
            r["speedup_vs_dense"] = round(float(np.median(dense_ms)) * S / r["total_ms"], 3)
            log(f"extensions: policy {r}")
        res["reselection_policy"] = {"steps": S, "dense_ms": round(float(np.median(dense_ms)), 4),
                                     "probe": "head 0, relative L2 against its exact attention", "runs": rows}
        del ws, mb
    return res


def ablations(base):
    """Each row changes one choice of the benchmarked configuration (`base`
    grouping, single KV tokens, residual), then the coarse three together."""
    rows = [("benchmarked: %s groups" % base, dict(grouping=base, kv_block=1, residual=True)),
            ("no residual", dict(grouping=base, kv_block=1, residual=False)),
            ("64-key blocks", dict(grouping=base, kv_block=64, residual=True))]
    for g in ("morton", "hash", "centred", "raster"):
        if g != base:
            rows.append(("%s groups" % g, dict(grouping=g, kv_block=1, residual=True)))
    rows.append(("raster groups + 64-key blocks + no residual", dict(grouping="raster", kv_block=64, residual=False)))
    return rows


def grouping_kw(w, grouping):
    return dict(grouping=grouping, grid=w.grid) if grouping == "morton" else dict(grouping=grouping)


def ablation(w, X, keeps, scale, base, seed=0):
    """Each failure-mode ablation on the workload's segment (selection on step
    0, reuse on steps 1..T): timings and the relative L2 of every reuse step
    against dense attention on that step."""
    import torch

    import sparse_attention_diffusion_mcs_amd as mcs

    H, N, d, G, T = w.heads, w.seq_len, w.head_dim, w.group, w.reuse_steps
    stream = torch.cuda.current_stream()
    proj = hash_projections(seed, w.wid, d)
    dense = {t: mcs.dense_attn(*X[t], scale=scale) for t in range(1, T + 1)}
    ws = torch.empty(mcs.workspace_bytes(X[0][0], G), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(X[0][0])
    rows = []
    for name, opt in ablations(base):
        if opt["kv_block"] > 1 and (N % opt["kv_block"] or np.any(keeps % opt["kv_block"])):
            rows.append({"variant": name, "skipped": "N or keep not whole 64-key blocks"})
            continue
        opt = dict(opt, **grouping_kw(w, opt["grouping"]))
        mb = torch.empty(int(mcs.meta_layout(H, N, d, 1, G, keeps).bytes), dtype=torch.uint8, device="cuda")
        mcs.select(*X[0], G, keeps, proj, scale=scale, meta_buf=mb, workspace=ws, **opt)  # warm-up
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2 * T + 2)]
        e[0].record(stream)
        meta, _ = mcs.select(*X[0], G, keeps, proj, scale=scale, meta_buf=mb, workspace=ws, dense_out=out, **opt)
        e[1].record(stream)
        err = []
        for t in range(1, T + 1):
            e[2 * t].record(stream)
            mcs.sparse_attn(*X[t], meta, out=out, scale=scale)
            e[2 * t + 1].record(stream)
            err.append(rel_l2(out, dense[t]))
        torch.cuda.synchronize()
        reuse = [e[2 * t].elapsed_time(e[2 * t + 1]) for t in range(1, T + 1)]
        rows.append({"variant": name, **{k: (list(v) if k == "grid" else v) for k, v in opt.items()},
                     "select_ms": round(e[0].elapsed_time(e[1]), 3),
                     "reuse_ms": round(float(np.mean(reuse)), 4),
                     "rel_l2_step1": round(err[0], 6), "rel_l2_mean": round(float(np.mean(err)), 6),
                     "rel_l2_final": round(err[-1], 6)})
        log(f"ablation {rows[-1]}")
        del meta, mb
    return rows


def trace_summary(db, out, title, command):
    """Kernel-trace statistics of a rocprofv3 results database as markdown."""
    import sqlite3
    cur = sqlite3.connect(db).cursor()
    lines = [f"# {title}", "", f"command: `{command}`", "",
             "Template arguments of `attn_bf16_kernel<d, waves, mode, tile>`: mode 0 = dense baseline, 1 = selection "
             "dense pass, 2 = reuse step, 3 = selection-time sparse pass and residual, 4 = selection key scores. The "
             "reuse-step "
             "average here is the kernel behind the bench's `value`.", "",
             "| kernel | calls | total us | avg us | % |", "|---|---|---|---|---|"]
    for name, calls, tot, avg, pct in cur.execute("select * from top_kernels limit 14"):
        n = name.replace("(anonymous namespace)::", "")
        n = n.split("(")[0] if "at::native" in n else n
        lines.append(f"| `{n[:110]}` | {calls} | {tot:.1f} | {avg:.1f} | {pct:.2f} |")
    lines += ["", "| kernel | vgpr | agpr | sgpr | lds | grid | wg |", "|---|---|---|---|---|---|---|"]
    for r in cur.execute("select name, vgpr_count, accum_vgpr_count, sgpr_count, lds_size, grid_x, workgroup_x "
                         "from kernels group by name"):
        if "mcs::" in r[0]:
            nm = r[0].replace("(anonymous namespace)::", "").split("(mcs")[0][:80]
            lines.append(f"| `{nm}` | " + " | ".join(str(x) for x in r[1:]) + " |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def traffic_summary(fetch_db, write_db, out, grouping):
    """HBM bytes per workload-2 reuse launch from two rocprofv3 --pmc runs
    (FETCH_SIZE, WRITE_SIZE, KiB per dispatch), each scaled by what the same
    counter reads for the plain 1 GiB device copy of --copy-probe."""
    import sqlite3

    def rows_of(db):
        cur = sqlite3.connect(db).cursor()
        cols = [c[1] for c in cur.execute("pragma table_info(counters_collection)")]
        return [dict(zip(cols, r)) for r in cur.execute("select * from counters_collection")]

    def per_kernel(db, name="attn_bf16_kernel<128, 2, 2, 32>"):
        rows = rows_of(db)
        reuse = [r["value"] for r in rows if name in r["kernel_name"]]
        if not reuse:
            reuse = [float("nan")]
        copies = [r for r in rows if "copy" in r["kernel_name"] and "bfloat16" not in r["kernel_name"]]
        cp = max(copies, key=lambda r: r["value"])
        n = sum(1 for x in reuse if np.isfinite(x))
        return float(np.mean(reuse)), n, float(cp["value"]), cp["kernel_name"][:80]

    f_reuse, n1, f_copy, cname = per_kernel(fetch_db)
    w_reuse, n2, w_copy, _ = per_kernel(write_db)
    gib = 1 << 30
    fs, ws = gib / 1024 / f_copy, gib / 1024 / w_copy
    H, N, d, ng, k = 24, 24960, 128, 390, 2496
    compulsory = 3 * H * N * d * 2 + H * N * d * 4 + H * ng * k * 4 + H * N * d * 2 + H * N * 4
    # the selection's index-gather kernels from the same two runs, against
    # their algorithmic bytes (score rows read once + kept indices written;
    # Q read once + keys written; keys read + permutation written)
    others = {}
    for label, name, alg in (("topk", "group_topk_kernel", H * ng * N * 4 + H * ng * k * 4),
                             ("hash", "hash_keys_kernel", H * N * d * 2 + H * N),
                             ("sort", "perm_sort_kernel", H * N + H * N * 4)):
        fk, nk, _, _ = per_kernel(fetch_db, name)
        wk, _, _, _ = per_kernel(write_db, name)
        if nk == 0 or not (np.isfinite(fk) and np.isfinite(wk)):
            continue  # not in these runs (another grouping)
        others[label] = {"kernel": name, "fetch_bytes": int(round(fk * 1024 * fs)),
                         "write_bytes": int(round(wk * 1024 * ws)), "algorithmic_bytes": int(alg),
                         "launches_averaged": nk}
    cmd = ("rocprofv3 --pmc {c} -d {d} -o {o} -- python3 bench.py --steps 1 --warmup 0 "
           "--no-cpu-baseline --copy-probe --no-zcurve --no-cold-cache" +
           ("" if grouping == "hash" else " --grouping " + grouping))
    res = {
        "kernel": "attn_bf16_kernel<128,2,REUSE,32> (reuse step)", "workload": 2, "grouping": grouping,
        "source_sha": src_hash(ATTN_SRC),
        "fetch_size_kib_per_launch": round(f_reuse, 1), "write_size_kib_per_launch": round(w_reuse, 1),
        "copy_probe": {"bytes": gib, "kernel": cname, "fetch_size_kib": f_copy, "write_size_kib": w_copy,
                       "fetch_scale": round(fs, 4), "write_scale": round(ws, 4)},
        "bytes_per_launch": int(round(f_reuse * 1024 * fs + w_reuse * 1024 * ws)),
        "fetch_bytes": int(round(f_reuse * 1024 * fs)), "write_bytes": int(round(w_reuse * 1024 * ws)),
        "launches_averaged": min(n1, n2), "compulsory_bytes": compulsory,
        "selection_kernels": others,
        "commands": [cmd.format(c="FETCH_SIZE", **profiler_out(fetch_db)),
                     cmd.format(c="WRITE_SIZE", **profiler_out(write_db)),
                     f"python3 bench.py --traffic-summary {fetch_db} {write_db} {out} {grouping}"],
        "note": "FETCH_SIZE counts L2 misses served by the fabric (MALL or HBM); each counter is scaled by what it "
                "reads for a plain 1 GiB device copy (--copy-probe). Compulsory = one read of Q, K, V, residual, "
                "idx, perm and the O write.",
    }
    with open(out, "w") as f:
        json.dump(res, f, indent=1)


# Counter passes of --counter-summary: each fits one rocprofv3 --pmc run
# (at most 8 SQ, 4 TCP, 2 TA, 2 TD, 2 GRBM counters).
COUNTER_PASSES = [
    "SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU "
    "SQ_INSTS_VALU SQ_INSTS_MFMA TA_TA_BUSY_sum TA_ADDR_STALLED_BY_TC_CYCLES_sum TD_TD_BUSY_sum TD_TC_STALL_sum "
    "GRBM_GUI_ACTIVE",
    "SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_VMEM SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE TCP_PENDING_STALL_CYCLES_sum "
    "TCP_TCC_READ_REQ_LATENCY_sum TCP_TCC_READ_REQ_sum TCP_TOTAL_CACHE_ACCESSES_sum GRBM_GUI_ACTIVE",
    "TCC_HIT_sum TCC_MISS_sum GRBM_GUI_ACTIVE",
]
REUSE_KERNEL = "attn_bf16_kernel<128, 2, 2, 32>"


def profiler_out(db):
    """The -d directory and -o name of the rocprofv3 run that wrote `db`
    (<dir>/<name>_results.db)."""
    name = os.path.basename(db)
    return {"d": os.path.dirname(db) or ".", "o": name[:-len("_results.db")] if name.endswith("_results.db") else name}


def counter_summary(out, *args):
    """Hardware counters of one kernel of the workload-2 bench (mean over its
    dispatches; by default the reuse launch, else the kernel named after
    --kernel) from rocprofv3 --pmc runs of the bench, with the ratios that
    locate its bottleneck.  GRBM_GUI_ACTIVE is summed over the eight XCDs, so
    the kernel's own clock is GUI / 8 / duration; per-CU and per-SIMD busy
    fractions divide by GUI / 8 and by 256 CUs or 1024 SIMDs; the SQ wave
    counters are in quad-cycles of one wave."""
    import sqlite3
    args = list(args)
    kernel = REUSE_KERNEL
    if "--kernel" in args:
        i = args.index("--kernel")
        kernel = args[i + 1]
        del args[i:i + 2]
    dbs = args
    vals, durs = {}, []
    for db in dbs:
        cur = sqlite3.connect(db).cursor()
        acc = {}
        for name, value, start, end in cur.execute(
                "select counter_name, value, start, end from counters_collection where kernel_name like ?",
                (f"%{kernel}%",)):
            acc.setdefault(name, []).append(float(value))
            if name == "GRBM_GUI_ACTIVE":
                durs.append((end - start) * 1e-9)
        for name, v in acc.items():
            vals[name] = float(np.mean(v))
    xcd_cycles = vals["GRBM_GUI_ACTIVE"] / 8
    dur = float(np.median(durs))

    def frac(name, units):
        return vals[name] / units / xcd_cycles if name in vals else float("nan")

    def wave(name):
        return vals[name] / vals["SQ_WAVE_CYCLES"] if name in vals else float("nan")

    derived = [
        ("kernel clock (GHz): GUI / 8 / duration", xcd_cycles / dur / 1e9),
        ("MFMA pipe busy, per SIMD", frac("SQ_VALU_MFMA_BUSY_CYCLES", 1024)),
        ("TD busy (processing or waiting for data), per CU", frac("TD_TD_BUSY_sum", 256)),
        ("TD stalled waiting for TC data, per CU", frac("TD_TC_STALL_sum", 256)),
        ("TA busy, per CU", frac("TA_TA_BUSY_sum", 256)),
        ("TA address path stalled by TC, per CU", frac("TA_ADDR_STALLED_BY_TC_CYCLES_sum", 256)),
        ("TCP stalled on data pending from L2, per CU", frac("TCP_PENDING_STALL_CYCLES_sum", 256)),
        ("mean TCP->L2 read latency (cycles)",
         vals.get("TCP_TCC_READ_REQ_LATENCY_sum", float("nan")) / vals.get("TCP_TCC_READ_REQ_sum", float("nan"))),
        ("L2 read requests per gathered 128-byte K/V line (1.0: no L1 reuse; Q, residual and index reads add the "
         "rest)", vals.get("TCP_TCC_READ_REQ_sum", float("nan")) / (24 * 390 * 2496 * 2 * 256 / 128)
         if kernel == REUSE_KERNEL else float("nan")),
        ("L2 hit rate: TCC_HIT / (TCC_HIT + TCC_MISS)",
         vals.get("TCC_HIT_sum", float("nan")) / (vals.get("TCC_HIT_sum", 0.0) + vals.get("TCC_MISS_sum", 0.0) or
                                                   float("nan"))),
        ("wave time waiting (waitcnt, barrier): SQ_WAIT_ANY / SQ_WAVE_CYCLES", wave("SQ_WAIT_ANY")),
        ("wave time ready but not issued: SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES", wave("SQ_WAIT_INST_ANY")),
        ("wave time issuing: SQ_ACTIVE_INST_ANY / SQ_WAVE_CYCLES", wave("SQ_ACTIVE_INST_ANY")),
        ("LDS bank-conflict cycles / LDS active cycles",
         vals.get("SQ_LDS_BANK_CONFLICT", float("nan")) / vals.get("SQ_LDS_IDX_ACTIVE", float("nan"))),
    ]
    cmd = ("rocprofv3 --pmc {c} -d {d} -o {o} -- python3 bench.py --steps 1 --warmup 0 "
           "--no-cpu-baseline --no-zcurve --no-cold-cache")
    what = "reuse launch" if kernel == REUSE_KERNEL else "launch"
    src = ATTN_SRC if "attn_bf16" in kernel else SELECT_SRC
    lines = [f"# Counters of the workload-2 {what} (`{kernel}`)", "",
             f"Source hash of `{os.path.basename(src)}`: `{src_hash(src)}`. Mean over the launch's dispatches in each pass; "
             f"median dispatch time under counter collection {dur * 1e3:.3f} ms.", "", "Commands:", ""]
    lines += [f"- `{cmd.format(c=c, **profiler_out(db))}`" for c, db in zip(COUNTER_PASSES, dbs)]
    sel = "" if kernel == REUSE_KERNEL else f' --kernel "{kernel}"'
    lines += [f"- `python3 bench.py --counter-summary {out} {' '.join(dbs)}{sel}`", "",
              "| derived | value |", "|---|---|"]
    lines += [f"| {k} | {v:.3f} |" for k, v in derived]
    lines += ["", "| counter | mean per dispatch |", "|---|---|"]
    lines += [f"| {k} | {vals[k]:.0f} |" for k in sorted(vals)]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


PHASES = ("grouping", "dense_pass", "key_scores", "topk", "residual_pass")


def gather_rates(w, keeps, phase_ms, grouping):
    """Achieved HBM rates of the index-gather kernels of the selection, on
    algorithmic bytes: the top-k reads every score row once and writes the
    kept indices; the sign-hash grouping reads Q once and writes the 8-bit
    keys, and the stable sort reads the keys and writes the permutation."""
    H, N, d, ng = w.heads, w.seq_len, w.head_dim, w.num_groups
    ldc = -(-N // 64) * 64
    topk_bytes = H * ng * N * 4 + int(np.sum(keeps)) * ng * 4
    rows = [("topk", topk_bytes, phase_ms["topk"])]
    if grouping in ("hash", "centred"):
        rows.append(("hash_and_sort", H * N * d * 2 + H * N + H * N + H * N * 4, phase_ms["grouping"]))
    out = {}
    for name, nbytes, ms in rows:
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"bytes": int(nbytes), "us": round(ms * 1e3, 1), "gbs": round(gbs, 1),
                     "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
    out["topk"]["score_row_stride_floats"] = ldc
    return out


def time_segments(mcs, X, w, keeps, proj, scale, grouping, steps, warmup, meta_buf, ws, out):
    """Selection on step 0 (phases marked with events) and T reuse steps,
    `steps` times after `warmup` untimed segments; returns the per-segment
    events, the phase events and the wall time."""
    import torch
    T, G = w.reuse_steps, w.group
    stream = torch.cuda.current_stream()
    gkw = grouping_kw(w, grouping)

    def segment(ev=None, ph=None):
        if ev is not None:
            ev[0].record(stream)
        # the selection step also produces its own attention output (the exact
        # dense one), as it would inside a denoising loop
        meta, _ = mcs.select(*X[0], G, keeps, proj, scale=scale, meta_buf=meta_buf, workspace=ws, dense_out=out,
                             phase_events=ph, **gkw)
        if ev is not None:
            ev[1].record(stream)
        for t in range(1, T + 1):
            if ev is not None:
                ev[2 * t].record(stream)
            mcs.sparse_attn(*X[t], meta, out=out, scale=scale)
            if ev is not None:
                ev[2 * t + 1].record(stream)
        return meta

    for _ in range(warmup):
        segment()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * T + 2)] for _ in range(steps)]
    phs = [[torch.cuda.Event(enable_timing=True) for _ in PHASES] for _ in range(steps)]
    for ph in phs:  # the HIP events exist once recorded; recorded here, outside the timed region
        for e in ph:
            e.record(stream)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(steps):
        meta = segment(evs[k], phs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    sel_ms = [e[0].elapsed_time(e[1]) for e in evs]
    reuse_ms = [e[2 * t].elapsed_time(e[2 * t + 1]) for e in evs for t in range(1, T + 1)]
    phase_ms = {}
    for i, name in enumerate(PHASES):
        phase_ms[name] = float(np.median([(e[0] if i == 0 else ph[i - 1]).elapsed_time(ph[i])
                                          for e, ph in zip(evs, phs)]))
    return meta, sel_ms, reuse_ms, phase_ms, wall


def fidelity(mcs, X, meta, scale, T):
    import torch
    fid = {}
    for t in sorted({1, max(1, T // 2), T}):
        o_s = mcs.sparse_attn(*X[t], meta, scale=scale).float()
        o_d = mcs.dense_attn(*X[t], scale=scale).float()
        fid[str(t)] = round(float(torch.linalg.vector_norm(o_s - o_d) / torch.linalg.vector_norm(o_d)), 6)
    torch.cuda.synchronize()
    return fid


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--counter-summary":
        counter_summary(*sys.argv[2:])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--trace-summary":
        trace_summary(*sys.argv[2:6])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--traffic-summary":
        traffic_summary(*sys.argv[2:6])
        return
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import sparse_attention_diffusion_mcs_amd as mcs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    mcs.lib()  # fail loudly if the library is missing

    w = workload_of(args)
    keeps = w.keeps(args.seed)
    H, N, d, G, T = w.heads, w.seq_len, w.head_dim, w.group, w.reuse_steps
    scale = float(np.float32(1.0 / math.sqrt(d)))
    log(f"workload {args.workload}: {describe(w, keeps)}; grouping {args.grouping}; seed {args.seed}")
    if args.sweep and not w.sweep:
        print("--sweep needs a workload with a sweep (workload 5)", file=sys.stderr)
        sys.exit(2)
    t0 = time.time()
    n_steps = max(T + 1, w.sweep["steps"] if (args.sweep or (args.extensions and w.reselect)) else 0)
    X = generate(w, range(0, n_steps), args.threads, args.seed)
    torch.cuda.synchronize()
    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log(f"inputs generated and resident ({time.time() - t0:.1f} s)")

    proj = hash_projections(args.seed, w.wid, d)
    q0 = X[0][0]
    ws = torch.empty(mcs.workspace_bytes(q0, G), dtype=torch.uint8, device="cuda")
    meta_probe = mcs.meta_layout(H, N, d, 1, G, keeps)
    meta_buf = torch.empty(int(meta_probe.bytes), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q0)
    stream = torch.cuda.current_stream()

    meta, sel_ms, reuse_ms, phase_ms, wall = time_segments(mcs, X, w, keeps, proj, scale, args.grouping, args.steps,
                                                           args.warmup, meta_buf, ws, out)
    log(f"segments: wall {1e3 * wall / args.steps:.3f} ms/segment; select {np.median(sel_ms):.3f} ms; "
        f"reuse mean {np.mean(reuse_ms):.4f} ms; phases {phase_ms}")

    # dense baseline on the same inputs
    dense_out = torch.empty_like(q0)
    for _ in range(args.warmup):
        mcs.dense_attn(*X[0], out=dense_out, scale=scale)
    dev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for k in range(args.steps):
        dev[k][0].record(stream)
        mcs.dense_attn(*X[1 + k % T], out=dense_out, scale=scale)
        dev[k][1].record(stream)
    torch.cuda.synchronize()
    dense_ms = [a.elapsed_time(b) for a, b in dev]

    cold = None if args.no_cold_cache else cold_cache(X, meta, scale, T, args.steps, stream, mcs)
    fid = fidelity(mcs, X, meta, scale, T)

    reuse_mean = float(np.mean(reuse_ms))
    sel_med = float(np.median(sel_ms))
    dense_med = float(np.median(dense_ms))
    flops_reuse = 4.0 * N * float(np.sum(keeps)) * d  # sum over heads of 4 N k_h d
    flops_dense = 4.0 * N * N * d * H
    flops_select = 1.5 * flops_dense + flops_reuse

    zc = None
    if not args.no_zcurve and args.grouping != "morton":
        # the same segment with Z-curve groups over the latent grid (a grouping
        # the pages do not name; secondary to the sign hash)
        _, zsel, zreuse, zphase, _ = time_segments(mcs, X, w, keeps, proj, scale, "morton", args.steps, 1, meta_buf,
                                                   ws, out)
        zmeta, _ = mcs.select(*X[0], G, keeps, proj, scale=scale, meta_buf=meta_buf, workspace=ws,
                              **grouping_kw(w, "morton"))
        zr = float(np.mean(zreuse))
        zc = {"grouping": "z-curve over the %dx%dx%d latent grid" % w.grid, "reuse_ms": round(zr, 4),
              "select_ms": round(float(np.median(zsel)), 3),
              "pct_bf16_peak_reuse": round(100.0 * flops_reuse / (zr * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
              "speedup_vs_dense": round(dense_med / zr, 3),
              "fidelity_rel_l2_vs_dense": fidelity(mcs, X, zmeta, scale, T)}
        del zmeta

    sweep_res = sweep(w, X, args.threads, scale, args.grouping, args.seed) if args.sweep else None
    ablation_res = ablation(w, X, keeps, scale, args.grouping, args.seed) if args.ablation else None
    ext_res = extensions(w, X, keeps, scale, args.grouping, args.seed) if args.extensions else None
    peak_mem = int(torch.cuda.max_memory_allocated())

    achieved = flops_reuse / (reuse_mean * 1e-3) / 1e12
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        try:
            with open(TRAFFIC_FILE) as f:
                tr = json.load(f)
            if (tr.get("source_sha") == src_hash(ATTN_SRC) and tr.get("workload") == args.workload
                    and tr.get("grouping", "hash") == args.grouping and args.keep is None and args.group is None
                    and args.seed == 0):
                traffic = tr.get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None
    result = {
        "metric": METRIC,
        "value": round(reuse_mean, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * wall / args.steps, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded DiT-shaped generator; no model weights)",
        "config": {"workload": describe(w, keeps), "heads": H, "seq_len": N, "head_dim": d, "group": G,
                   "keep": [int(x) for x in sorted(set(keeps.tolist()))], "reuse_steps": T, "seed": args.seed,
                   "grouping": {"morton": "z-curve over the %dx%dx%d latent grid" % w.grid,
                                "hash": "8-bit sign hash", "raster": "raster order",
                                "centred": "centred 8-bit sign hash"}[args.grouping]},
        "reuse_ms_median": round(float(np.median(reuse_ms)), 4),
        "reuse_ms_p10_p90": [round(float(np.percentile(reuse_ms, 10)), 4),
                             round(float(np.percentile(reuse_ms, 90)), 4)],
        "dense_ms": round(dense_med, 4),
        "speedup_vs_dense": round(dense_med / reuse_mean, 3),
        "select_ms": round(sel_med, 3),
        "select_phases_ms": {k: round(v, 4) for k, v in phase_ms.items()},
        "amortised_ms_per_denoising_step": round((sel_med + T * reuse_mean) / (T + 1), 4),
        "amortised_speedup_vs_dense": round(dense_med * (T + 1) / (sel_med + T * reuse_mean), 3),
        "pct_bf16_peak_reuse": round(100.0 * achieved / PEAK_BF16_TFLOPS, 2),
        "pct_bf16_peak_dense": round(100.0 * flops_dense / (dense_med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "select_tflops": round(flops_select / (sel_med * 1e-3) / 1e12, 1),
        "fidelity_rel_l2_vs_dense": fid,
        "gather": gather_rates(w, keeps, phase_ms, args.grouping),
        "meta_bytes": int(meta_buf.numel()),
        "select_workspace_bytes": int(ws.numel()),
        "peak_device_bytes": peak_mem,
        "roofline": {"kernel": f"attn_bf16_kernel<{d},{G // 32},REUSE> (reuse step)", "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "flops_per_launch": flops_reuse},
    }
    if len(set(keeps.tolist())) > 1:
        ks, cnt = np.unique(keeps, return_counts=True)
        result["keep_histogram"] = {str(int(k)): int(c) for k, c in zip(ks, cnt)}
    if cold is not None:
        result["cold_cache"] = cold
    if zc is not None:
        result["zcurve"] = zc
    if sweep_res is not None:
        result["sweep"] = sweep_res
    if ablation_res is not None:
        result["ablation"] = ablation_res
    if ext_res is not None:
        result["extensions"] = ext_res
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(w, keeps, T, scale, args.cpu_groups, args.seed)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

"""CPU checks of the benchmark's command line (no GPU work)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


# The converters that write profiles/ from rocprofv3 databases, run on small
# hand-built databases with the columns they read.

def _bench():
    sys.path.insert(0, ROOT)
    import bench
    return bench


def _counter_db(path, rows):
    import sqlite3
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (kernel_name text, counter_name text, value real, start integer, "
                "end integer)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?, ?)", rows)
    con.commit()
    con.close()


def test_counter_summary_ratios(tmp_path):
    b = _bench()
    reuse = f"void mcs::(anonymous namespace)::{b.REUSE_KERNEL}(mcs::AttnArgs)"
    other = "void mcs::(anonymous namespace)::attn_bf16_kernel<128, 4, 0, 32>(mcs::AttnArgs)"
    cyc = 2_000_000  # per XCD, over a 1 ms dispatch -> 2 GHz
    rows = []
    for disp in range(3):
        t0 = disp * 10_000_000
        for kern, scale in ((reuse, 1.0), (other, 7.0)):
            rows += [(kern, "GRBM_GUI_ACTIVE", 8 * cyc * scale, t0, t0 + 1_000_000),
                     (kern, "SQ_VALU_MFMA_BUSY_CYCLES", 0.4 * 1024 * cyc * scale, t0, t0 + 1_000_000),
                     (kern, "TD_TD_BUSY_sum", 0.9 * 256 * cyc * scale, t0, t0 + 1_000_000),
                     (kern, "TCP_TCC_READ_REQ_LATENCY_sum", 250.0 * 1000, t0, t0 + 1_000_000),
                     (kern, "TCP_TCC_READ_REQ_sum", 1000.0, t0, t0 + 1_000_000)]
    db = str(tmp_path / "c.db")
    _counter_db(db, rows)
    out = tmp_path / "c.md"
    b.counter_summary(str(out), db)
    text = out.read_text()
    assert "| kernel clock (GHz): GUI / 8 / duration | 2.000 |" in text
    assert "| MFMA pipe busy, per SIMD | 0.400 |" in text
    assert "| TD busy (processing or waiting for data), per CU | 0.900 |" in text
    assert "| mean TCP->L2 read latency (cycles) | 250.000 |" in text
    assert "| TD stalled waiting for TC data, per CU | nan |" in text  # not collected
    assert b.src_hash(b.ATTN_SRC) in text
    # --kernel selects another launch of the same run: its GUI cycles are 7x
    # over the same 1 ms, so its clock reads 14 GHz and its busy fractions
    # keep their ratios
    out2 = tmp_path / "c2.md"
    b.counter_summary(str(out2), db, "--kernel", "attn_bf16_kernel<128, 4, 0, 32>")
    text2 = out2.read_text()
    assert "attn_bf16_kernel<128, 4, 0, 32>" in text2.splitlines()[0]
    assert "| kernel clock (GHz): GUI / 8 / duration | 14.000 |" in text2
    assert "| MFMA pipe busy, per SIMD | 0.400 |" in text2
    assert "gathered 128-byte K/V line" in text2 and "line (1.0: no L1 reuse; Q, residual and index reads add the " \
        "rest) | nan |" in text2


def test_traffic_summary_scales_by_the_copy_probe(tmp_path):
    b = _bench()
    reuse = f"void mcs::(anonymous namespace)::{b.REUSE_KERNEL}(mcs::AttnArgs)"
    copy = "__amd_rocclr_copyBuffer"
    topk = "void mcs::(anonymous namespace)::group_topk_kernel<false>(float const*)"
    for name, reuse_kib, copy_kib in (("f.db", 1000.0, 524288.0), ("w.db", 300.0, 1048576.0)):
        _counter_db(str(tmp_path / name), [(reuse, "X", reuse_kib, 0, 1), (reuse, "X", reuse_kib, 2, 3),
                                           (copy, "X", copy_kib, 4, 5), (topk, "X", reuse_kib / 10, 6, 7)])
    out = tmp_path / "t.json"
    b.traffic_summary(str(tmp_path / "f.db"), str(tmp_path / "w.db"), str(out), "morton")
    import json
    res = json.loads(out.read_text())
    assert res["copy_probe"]["fetch_scale"] == 2.0 and res["copy_probe"]["write_scale"] == 1.0
    assert res["fetch_bytes"] == 1000 * 1024 * 2 and res["write_bytes"] == 300 * 1024
    assert res["bytes_per_launch"] == res["fetch_bytes"] + res["write_bytes"]
    assert res["launches_averaged"] == 2 and res["source_sha"] == b.src_hash(b.ATTN_SRC)
    # the selection's index-gather kernels present in the runs, scaled the same way
    assert set(res["selection_kernels"]) == {"topk"}
    assert res["selection_kernels"]["topk"]["fetch_bytes"] == 100 * 1024 * 2
    assert res["selection_kernels"]["topk"]["write_bytes"] == 30 * 1024


def test_trace_summary_tables(tmp_path):
    import sqlite3
    b = _bench()
    db = str(tmp_path / "k.db")
    con = sqlite3.connect(db)
    con.execute("create table top_kernels (name text, calls integer, total real, average real, percentage real)")
    con.execute("insert into top_kernels values ('void mcs::(anonymous namespace)::attn_bf16_kernel<128, 2, 2, 32>"
                "(mcs::AttnArgs)', 10, 9500.0, 950.0, 42.5)")
    con.execute("create table kernels (name text, vgpr_count integer, accum_vgpr_count integer, sgpr_count integer, "
                "lds_size integer, grid_x integer, workgroup_x integer)")
    con.execute("insert into kernels values ('void mcs::(anonymous namespace)::attn_bf16_kernel<128, 2, 2, 32>"
                "(mcs::AttnArgs)', 120, 0, 112, 32768, 1198080, 128)")
    con.commit()
    con.close()
    out = tmp_path / "k.md"
    b.trace_summary(db, str(out), "T", "CMD")
    text = out.read_text()
    assert "| `void mcs::attn_bf16_kernel<128, 2, 2, 32>(mcs::AttnArgs)` | 10 | 9500.0 | 950.0 | 42.50 |" in text
    assert "| 120 | 0 | 112 | 32768 | 1198080 | 128 |" in text and "command: `CMD`" in text


def test_joint_workload_description():
    """Workload 6 names its text tokens and its full sequence length."""
    b = _bench()
    from mcs_inputs import workload
    w = workload(6)
    text = b.describe(w, w.keeps())
    assert "16x30x52 + 226 text" in text and "N=25186" in text and "k=2496" in text

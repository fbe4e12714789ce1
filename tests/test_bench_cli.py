"""bench.py's command line on the host: more than one GPU is refused with a
message (this build measures one GPU), and every row named on the command
line exists."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_rows_are_known():
    sys.path.insert(0, ROOT)
    import bench
    assert set(bench.ROWS) == {"xattn", "window", "bigtree", "paged", "commit", "rope", "shard"}


def _write_trace(path, K, W, reps, partial_us=50.0, merge_us=7.0):
    """A kernel trace in rocprofv3's csv layout with the launch sequence of a
    default bench run, in the order bench.trace_summary states."""
    import csv
    steps = W + 2 * K + K + reps * K + (1 + reps) * K
    rows, t = [], 1000
    for s in range(steps):
        for name, dur in (("void ltree::(anonymous namespace)::partial_mfma_kernel<128, 3, false,"
                           " false, 0, false>(ltree::PartialArgs)", partial_us + s % 3),
                          ("void ltree::(anonymous namespace)::lse_merge_kernel<128, true>(int)",
                           merge_us)):
            rows.append({"Kernel_Name": name, "Start_Timestamp": t,
                         "End_Timestamp": t + int(dur * 1000)})
            t += int(dur * 1000)
    for s in range((1 + reps) * K):
        rows.append({"Kernel_Name": "void ltree::(anonymous namespace)::partial_mfma_kernel<128, 3,"
                                    " false, false, 0, false>(ltree::PartialArgs)",
                     "Start_Timestamp": t, "End_Timestamp": t + int(partial_us * 1000)})
        t += int(partial_us * 1000)
    rows.append({"Kernel_Name": "__amd_rocclr_copyBuffer", "Start_Timestamp": 1,
                 "End_Timestamp": 2})
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        wr.writeheader()
        wr.writerows(rows)


def test_trace_summary_splits_the_phases(tmp_path):
    sys.path.insert(0, ROOT)
    import bench
    p = tmp_path / "trace.csv"
    _write_trace(p, K=4, W=3, reps=bench.REPS)
    out = bench.trace_summary(str(p), K=4, W=3)
    lines = [ln for ln in out.splitlines() if ln.startswith("| ") and "phase" not in ln]
    assert len(lines) == 10  # nine phases and the cold total
    assert "step graph, timed replay" in out and "hot graph" in out
    # the partial-only phases have no merge
    assert lines[8].split("|")[5].strip() == "-"
    # a trace of another run shape is refused
    import pytest
    with pytest.raises(SystemExit):
        bench.trace_summary(str(p), K=5, W=3)


def test_counter_summary_means_per_dispatch(tmp_path):
    import csv
    sys.path.insert(0, ROOT)
    import bench
    p = tmp_path / "counters.csv"
    with open(p, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                           "Counter_Value"])
        wr.writeheader()
        k = "void ltree::(anonymous namespace)::lse_merge_kernel<128, true>(int)"
        # two dispatches; the first reports its value in two pieces
        for d, v in ((1, 10.0), (1, 20.0), (2, 50.0)):
            wr.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": "SQ_WAVES",
                         "Counter_Value": v})
    out = bench.counter_summary([str(p)])
    assert "`lse_merge_kernel<128, true>`" in out
    assert "| SQ_WAVES | 40 (2) |" in out

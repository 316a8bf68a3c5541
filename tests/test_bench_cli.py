"""bench.py's command-line contract that needs no GPU: a run on more than one
GPU is refused with a message (the path runs on one GPU; there is no
multi-GPU leg), and the help text lists the paths and workloads."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def test_help_lists_paths_and_workloads():
    r = run("--help")
    assert r.returncode == 0
    for word in ("deferred", "tree", "fused", "split_neumann", "split_inverse", "multilayer"):
        assert word in r.stdout, word


def test_deferred_schedule_is_a_real_round_sequence():
    """Each input set's rounds in a captured graph form a cycle (the graph is
    replayed): every launch reads the output group its set's previous round
    wrote, and never the group it writes itself."""
    import bench
    for S in (1, 2, 3, 4, 5):
        for R in range(2 * S, 6 * S + 3):
            sched = bench.deferred_schedule(R, S)
            assert [j for j, _, _ in sched] == [i % S for i in range(R)]
            for j in range(S):
                rounds = [(c, p) for jj, c, p in sched if jj == j]
                n = len(rounds)
                assert n >= 2
                for m, (c, p) in enumerate(rounds):
                    assert c != p
                    assert p == rounds[(m - 1) % n][0]
                    assert 0 <= c < bench.InputSet.GROUPS


def test_graph_steps_divides_k():
    import bench
    for k in (1, 20, 1000, 2048, 2049, 4000, 4099):
        r = bench.graph_steps(k)
        assert k % r == 0 and r <= max(k, 1) and (r == k or r <= 2048)


def test_trace_windows_and_marginal(tmp_path):
    """The profile summary's reading of a kernel trace: the stretches between
    marker kernels that hold only the dominant kernel, in order, and the
    marginal time per launch from the 1 024- and 512-dispatch windows' spans
    (8 replays of 128 and of 64 launches, each replay starting with a gap that
    the difference cancels)."""
    import csv
    import bench
    K = bench.DOMINANT_KERNEL
    rows, t = [], 0

    def add(name, dur):
        nonlocal t
        rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur})
        t += dur + 100  # 0.1 us between dispatches

    def region(n_launch, replays, dur_ns, start_gap_ns):
        nonlocal t
        add("spin_kernel(long)", 1000)
        for _ in range(replays):
            t += start_gap_ns
            for _ in range(n_launch):
                add(f"void bole::{K}(args)", dur_ns)
        add("spin_kernel(long)", 1000)

    add("other_kernel", 5000)
    region(20, 1, 31000, 9000)        # the timed K steps
    region(128, 8, 30000, 9000)       # the marginal's two regions
    region(64, 8, 30000, 9000)
    add(f"void bole::{K}(args)", 30000)  # outside any window
    with open(tmp_path / "run_kernel_trace.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(rows)
    wins = bench.marked_windows(str(tmp_path), K)
    assert [len(x) for x in wins] == [20, 1024, 512]
    assert bench.timed_window(str(tmp_path), K) == [31000] * 20
    # per launch: 30 us of kernel plus the 0.1 us between dispatches; the
    # replay-start gaps (8 in each region) cancel
    assert abs(bench.trace_marginal_us(wins) - 30.1) < 1e-9
    assert bench.trace_marginal_us(wins[:2]) is None


def test_input_sets_rule():
    """The deferred step's captured graph of K steps must give each rotated
    set two rounds, so a short run rotates fewer sets; other paths keep them;
    a graph of fewer than four steps is refused."""
    import pytest as _pytest
    import bench
    assert bench.input_sets(8, 1000, "deferred") == 8
    assert bench.input_sets(8, 20, "deferred") == 8
    assert bench.input_sets(8, 10, "deferred") == 5
    assert bench.input_sets(8, 4, "deferred") == 2
    assert bench.input_sets(8, 10, "tree") == 8
    with _pytest.raises(SystemExit):
        bench.input_sets(8, 3, "deferred")
    # every accepted combination yields a valid deferred schedule
    for k in (4, 5, 7, 10, 16, 20, 33, 1000):
        S = bench.input_sets(8, k, "deferred")
        bench.deferred_schedule(bench.graph_steps(k), S)


def test_summarize_profiles_end_to_end(tmp_path, monkeypatch):
    """--summarize-profiles on synthetic rocprofv3 output: the calibration takes
    the copies that run before any library kernel (a later, larger copy is
    ignored), the counters scale by the copy's known size, the record carries
    the current kernel source hash, and the trace summary gives the marginal
    time from the marked windows next to the traced run's own line."""
    import csv
    import json
    import bench
    out = tmp_path / "profiles"
    out.mkdir()
    monkeypatch.setattr(bench, "PROFILES", str(out))
    monkeypatch.setattr(bench, "PROFILE_COUNTERS", str(out / "counters.json"))
    K = bench.DOMINANT_KERNEL
    name = f"void bole::{K}(args)"

    def write_csv(path, fields, rows):
        path.parent.mkdir(parents=True, exist_ok=True)
        with open(path, "w", newline="") as fh:
            w = csv.DictWriter(fh, fieldnames=fields)
            w.writeheader()
            w.writerows(rows)

    # kernel trace: the timed K = 20 steps, then the marginal's 128- and 64-launch regions
    rows, t = [], 0

    def add(n, dur):
        nonlocal t
        rows.append({"Kernel_Name": n, "Start_Timestamp": t, "End_Timestamp": t + dur})
        t += dur

    for n_launch, replays in ((20, 1), (128, 8), (64, 8)):
        add("spin_kernel", 500)
        for _ in range(replays):
            t += 9000
            for _ in range(n_launch):
                add(name, 30000)
        add("spin_kernel", 500)
    write_csv(tmp_path / "trace" / "run_kernel_trace.csv",
              ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    write_csv(tmp_path / "trace" / "run_kernel_stats.csv",
              ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"],
              [{"Name": name, "Calls": 1556, "AverageNs": 30000, "MinNs": 30000, "MaxNs": 30000}])

    def counters(counter, copy_kib, dom_kib):
        rs, i = [], 0
        for _ in range(3):  # the calibration copies, first in the run
            rs.append({"Dispatch_Id": i, "Kernel_Name": "__amd_rocclr_copyBuffer",
                       "Counter_Name": counter, "Counter_Value": copy_kib})
            i += 1
        for _ in range(5):
            rs.append({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                       "Counter_Value": dom_kib})
            i += 1
        rs.append({"Dispatch_Id": i, "Kernel_Name": "__amd_rocclr_copyBuffer",
                   "Counter_Name": counter, "Counter_Value": 10 * copy_kib})  # the bench's own copy
        return rs

    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    write_csv(tmp_path / "fetch" / "run_counter_collection.csv", fields,
              counters("FETCH_SIZE", 131072, 30000))
    write_csv(tmp_path / "write" / "run_counter_collection.csv", fields,
              counters("WRITE_SIZE", 262144, 57000))
    line = tmp_path / "line.json"
    line.write_text(json.dumps({"ms_per_step": 0.0305,
                                "roofline": {"ms_per_launch": 0.030, "frac": 0.4987}}))
    bench.summarize_profiles(str(tmp_path / "trace"), str(tmp_path / "fetch"),
                             str(tmp_path / "write"), 256,
                             {"trace": "T", "fetch": "F", "write": "W"}, 8, str(line))
    rec = json.load(open(out / "counters.json"))
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["hbm_bytes_per_launch"] == (30000 * 2.0 + 57000 * 1.0) * 1024
    assert rec["kernel_source_hash"] == bench.kernel_source_hash()
    assert bench.traffic_from_profile(bench.kernel_source_hash()) == rec["hbm_bytes_per_launch"]
    md = open(out / "bole_kernels_target_trace.md").read()
    assert "| 20 | 30.00 | 30.00 |" in md          # the timed window's dispatches
    assert "| 30.00 |" in md                        # the marginal from the trace
    assert "0.4987" in md                           # the traced run's own line

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

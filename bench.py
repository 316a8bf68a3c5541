"""Throughput of closed-form tree verification for one GDN layer on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
tree preparation (topology + log-space gate products), the G/C factors,
value-tiled verify and the accepted-path commit.  The default path runs all
of it in one launch (bole_commit_tree_verify: this round's preparation,
factors and verify with the previous round's commit inside); --path tree
times bole_tree_verify + bole_commit_path, and --path fused and --path split
the three- and four-launch forms.  Default workload: 16 requests,
64-node random trees (depth <= 12), 32 state heads, d_k = d_v = 128, bf16
q/k/v with float32 gates and states.  Eight independent input sets are
rotated by default, so one rotation touches about 960 MB, several times the
256 MB last-level cache (with four sets, 480 MB, the default step measured
about 20% faster: partly served from that cache).

Prints one JSON line.  `value` = tree nodes x heads verified per second.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

PEAK_HBM_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
PROFILE_COUNTERS = os.path.join(PROFILES, "bole_commit_tree_verify_target_counters.json")
KERNEL_SOURCE_NAMES = ("verify.hip", "verify_tiles.h", "tree_topo.h", "common.h")
KERNEL_SOURCES = [os.path.join(ROOT, "linear_attention_tree_amd", "csrc", f)
                  for f in KERNEL_SOURCE_NAMES]
# the bf16 verify kernel with preparation and the previous round's commit
# inside, which the default step launches (name as rocprofv3 prints it)
DOMINANT_KERNEL = "verify_kernel<1, true, true, true, 0, true, true>"
# the same without the commit (bole_tree_verify)
TREE_VERIFY_KERNEL = "verify_kernel<1, true, true, true, 0, false, true>"


def verify_algorithmic_bytes(sizes, H, d_k, d_v, e):
    """Compulsory HBM bytes of one verify launch: S_pre read once; q, k, v, logP,
    beta read once; O (token dtype) and U (float32) written once."""
    per_node = 2 * e * d_k + e * d_v + 8 + e * d_v + 4 * d_v
    return int(sum(H * (4 * d_k * d_v + T * per_node) for T in sizes))


def tree_verify_algorithmic_bytes(sizes, H, d_k, d_v, e):
    """bole_tree_verify: the verify bytes (its log-gates g take the place of logP
    as the second per-node-head float read) plus the preparation's own: parent
    read, logP written per node and head, depth, anc and order written per node,
    tree_depth per tree."""
    return verify_algorithmic_bytes(sizes, H, d_k, d_v, e) + int(
        sum(T * (4 * H + 4 + 16) + 4 for T in sizes))


def tree_verify_written_bytes(sizes, H, d_k, d_v, e):
    """The written part of bole_tree_verify's algorithmic bytes: O and U per
    node and head, logP per node and head, depth, anc and order per node,
    tree_depth per tree (the rest is read)."""
    return int(sum(T * (H * (e * d_v + 4 * d_v) + 4 * H + 16) + 4 for T in sizes))


def path_lengths(forest):
    """Nodes on each request's accepted path (root to accepted node), for the
    requests that accept one."""
    out = []
    for b, a in enumerate(forest.accept):
        if a < 0:
            continue
        o, n, j = forest.tree_off[b], 1, int(a)
        while forest.parent[o + j] >= 0:
            j, n = int(forest.parent[o + j]), n + 1
        out.append(n)
    return out


def commit_tree_verify_algorithmic_bytes(sizes, prev_forest, H, d_k, d_v, e):
    """bole_commit_tree_verify: bole_tree_verify's bytes plus the commit's own:
    each committed slot written once (it is read once, already counted), the
    accepted path's key, U and logP entries, the accepted node's ancestor set,
    and the previous offsets and accepted nodes."""
    extra = sum(H * (4 * d_k * d_v + la * (e * d_k + 4 * d_v + 4)) + 8
                for la in path_lengths(prev_forest))
    return tree_verify_algorithmic_bytes(sizes, H, d_k, d_v, e) + int(extra) + 12 * len(sizes)


def commit_tree_verify_written_bytes(sizes, prev_forest, H, d_k, d_v, e):
    """The written part of bole_commit_tree_verify's algorithmic bytes:
    bole_tree_verify's, plus every committed slot."""
    return tree_verify_written_bytes(sizes, H, d_k, d_v, e) + \
        H * 4 * d_k * d_v * len(path_lengths(prev_forest))


def stream_ceiling(torch, dev, read_bytes, write_bytes, n_sets):
    """GB/s of the baselines library's streaming kernel moving read_bytes in
    and write_bytes out per launch over n_sets rotated buffer pairs (the
    footprint and read:write mix of the kernel it is set against): the best of
    three launch shapes, each timed as the marginal time per back-to-back
    launch."""
    from linear_attention_tree_amd import baselines
    nr, nw = int(read_bytes) // 16, int(write_bytes) // 16
    src = torch.ones(n_sets * nr * 4, dtype=torch.float32, device=dev)
    dst = torch.empty(n_sets * nw * 4, dtype=torch.float32, device=dev)
    best = 0.0
    for grid, block in ((1024, 256), (2048, 256), (4096, 256)):
        def calls(n):
            return [lambda i=i: baselines.stream_mix(src[(i % n_sets) * nr * 4:],
                                                     dst[(i % n_sets) * nw * 4:], nr, nw,
                                                     grid, block)
                    for i in range(n)]
        ms = marginal_ms(torch, calls, max(64, 2 * n_sets))
        best = max(best, (nr + nw) * 16 / (ms * 1e-3) / 1e9)
    del src, dst
    torch.cuda.empty_cache()
    return best


DOMINANT = {  # path -> (launch name, algorithmic bytes of one launch)
    "deferred": ("commit_tree_verify", None),  # bytes depend on the previous round
    "tree": ("tree_verify", tree_verify_algorithmic_bytes),
    "fused": ("factor_verify", verify_algorithmic_bytes),
    "split": ("verify", verify_algorithmic_bytes),
    "split_neumann": ("verify_neumann", verify_algorithmic_bytes),
    "split_inverse": ("verify_inverse", verify_algorithmic_bytes),
}


def kernel_source_hash():
    """Hash of the dominant kernel's sources with comments and blank lines
    left out (a comment edit does not change the kernel the counters saw)."""
    import re
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        text = re.sub(r"/\*.*?\*/", "", open(p).read(), flags=re.S)
        for line in text.splitlines():
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def traffic_from_profile(expected_hash):
    try:
        d = json.load(open(PROFILE_COUNTERS))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_hash") != expected_hash:
        return None
    return d.get("hbm_bytes_per_launch")


def _csv_rows(d, suffix):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    with open(files[0]) as fh:
        return list(csv.DictReader(fh))


def _short(name):
    return name.split("(")[0].replace("void ", "")


def all_kernel_traffic(fetch_dir, write_dir, f_fetch, f_write, n_sets):
    """Scaled HBM bytes per dispatch of every library kernel in the two counter
    passes, beside the algorithmic bytes where a model exists (target shape)."""
    def means(d, counter):
        acc = {}
        for r in _csv_rows(d, "counter_collection.csv"):
            if r["Counter_Name"] == counter and "bole::" in r["Kernel_Name"]:
                acc.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}
    fe, wr = means(fetch_dir, "FETCH_SIZE"), means(write_dir, "WRITE_SIZE")
    cfg = W.CONFIGS["target"]
    forests = [W.make_forest(cfg, seed) for seed in range(n_sets)]
    algo = {
        "bole::" + DOMINANT_KERNEL: np.mean(
            [commit_tree_verify_algorithmic_bytes(f.sizes(), f, cfg.H, cfg.d_k, cfg.d_v, 2)
             for f in forests]),
        "bole::" + TREE_VERIFY_KERNEL: np.mean(
            [tree_verify_algorithmic_bytes(f.sizes(), cfg.H, cfg.d_k, cfg.d_v, 2) for f in forests]),
        "bole::commit_kernel<1>": np.mean(
            [commit_algorithmic_bytes(f, 1, cfg.H, cfg.d_k, cfg.d_v, 2) for f in forests]),
        "bole::tree_conv_kernel<1>": conv_algorithmic_bytes(
            forests[0].N, cfg.B, W.conv_channels(cfg), W.CONV_WIDTH, 2),
    }
    out = ["## Every library kernel in the same two passes", "",
           "| kernel | dispatches | FETCH KiB | WRITE KiB | HBM MB (scaled) | algorithmic MB | ratio |",
           "|---|---|---|---|---|---|---|"]
    for k in sorted(set(fe) & set(wr)):
        hbm = (fe[k][0] * f_fetch + wr[k][0] * f_write) * 1024.0
        a = algo.get(k)
        out.append(f"| `{k}` | {fe[k][1]} | {fe[k][0]:.0f} | {wr[k][0]:.0f} | {hbm / 1e6:.1f} | "
                   + (f"{a / 1e6:.1f} | {hbm / a:.3f} |" if a else "| |"))
    return out


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE",
                 "SQ_INSTS_LDS", "TCC_HIT_sum", "TCC_MISS_sum")
PEAK_BF16_TFLOPS = 2500.0


def summarize_mfma(mfma_dir, trace_dir, command):
    """MFMA, LDS and L2 counters of every library kernel (one rocprofv3 --pmc
    pass of this script) against the kernel-trace durations."""
    acc = {}
    for r in _csv_rows(mfma_dir, "counter_collection.csv"):
        if "bole::" in r["Kernel_Name"] and r["Counter_Name"] in MFMA_COUNTERS:
            acc.setdefault(_short(r["Kernel_Name"]), {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
    dur = {_short(r["Name"]): float(r["AverageNs"]) for r in _csv_rows(trace_dir, "kernel_stats.csv")}
    lines = ["# MFMA, LDS and L2 counters, target workload (rocprofv3 --pmc)", "", "Command:", "", "```",
             command, "```", "", "Summarized from its output (durations from the kernel trace) by:",
             "", "```", summarizer_command(), "```", "",
             "Per dispatch, averaged over the run. bf16 MFMA rate = 512 x "
             "SQ_INSTS_VALU_MFMA_MOPS_BF16 / the kernel's average duration in the kernel trace, "
             f"against the {PEAK_BF16_TFLOPS:.0f} TFLOP/s dense bf16 peak. LDS bank-conflict share = "
             "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE. L2 hit rate = TCC_HIT_sum / (TCC_HIT_sum + "
             "TCC_MISS_sum); the two-call verify (`verify_kernel<1, false, ...>`) reads G and C right "
             "after the producer wrote them.", "",
             "| kernel | bf16 MFMA TFLOP/s | of peak | LDS instructions | "
             "LDS bank-conflict share | L2 hit rate |", "|---|---|---|---|---|---|"]
    for k in sorted(acc):
        c = {n: sum(v) / len(v) for n, v in acc[k].items()}
        if len(c) < len(MFMA_COUNTERS) or k not in dur:
            continue
        tflops = 512.0 * c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] / (dur[k] * 1e-9) / 1e12
        conf = c["SQ_LDS_BANK_CONFLICT"] / max(c["SQ_LDS_IDX_ACTIVE"], 1.0)
        hit = c["TCC_HIT_sum"] / max(c["TCC_HIT_sum"] + c["TCC_MISS_sum"], 1.0)
        lines.append(f"| `{k}` | {tflops:.1f} | {tflops / PEAK_BF16_TFLOPS:.3f} | "
                     f"{c['SQ_INSTS_LDS']:.0f} | {conf:.3f} | {hit:.3f} |")
    with open(os.path.join(PROFILES, "bole_kernels_target_mfma_lds.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def marked_windows(trace_dir, kernel):
    """The stretches of a kernel trace between two consecutive marker
    dispatches (torch's sleep kernel, named spin_kernel) that hold `kernel`'s
    dispatches and nothing else, in order: each a list of (start, end)
    timestamps in ns.  The bench marks its timed K steps first, then the two
    regions of the dominant kernel's marginal time (graphs of 128 and of 64
    launches, 8 replays each)."""
    rows = sorted(_csv_rows(trace_dir, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"]))
    marks = [i for i, r in enumerate(rows) if "spin_kernel" in r["Kernel_Name"]]
    out = []
    for a, b in zip(marks, marks[1:]):
        win = rows[a + 1:b]
        if win and all(kernel in r["Kernel_Name"] for r in win):
            out.append([(int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in win])
    return out


def timed_window(trace_dir, kernel):
    """Durations (ns) of `kernel`'s dispatches in the first marked window (the
    timed K steps), or None."""
    w = marked_windows(trace_dir, kernel)
    return [e - s for s, e in w[0]] if w else None


def trace_marginal_us(windows, r=64, replays=8):
    """The marginal time per launch from a trace's own timestamps: the span of
    the window of 2r x replays dispatches minus that of r x replays, over
    r x replays (each span holds `replays` replay starts, which cancel).
    None without both windows."""
    spans = {}
    for w in windows:
        spans.setdefault(len(w), (w[-1][1] - w[0][0]) / 1e3)
    if 2 * r * replays not in spans or r * replays not in spans:
        return None
    return (spans[2 * r * replays] - spans[r * replays]) / (r * replays)


def summarizer_command():
    """This script's command line as invoked, without the (long) recorded
    profiling commands."""
    out, skip = ["python3", "bench.py"], False
    for a in sys.argv[1:]:
        if skip:
            skip = False
        elif a == "--profile-commands":
            skip = True
        elif not a.startswith("--profile-commands="):
            out.append(a)
    return " ".join(out)


def summarize_profiles(trace_dir, fetch_dir, write_dir, calib_mib, commands, n_sets,
                       bench_line=None):
    """Turn three rocprofv3 runs of this script (a kernel trace, a FETCH_SIZE
    pass and a WRITE_SIZE pass, the counter passes preceded by a plain copy of
    calib_mib MiB, all three over the same n_sets rotated input sets) into the
    text summaries under profiles/ and the counter record the bench line reads
    its `traffic` from."""
    os.makedirs(PROFILES, exist_ok=True)
    stats = _csv_rows(trace_dir, "kernel_stats.csv")
    cfg = W.CONFIGS["target"]
    forests = [W.make_forest(cfg, seed) for seed in range(n_sets)]
    # the default step's launches each commit their own batch's previous round
    algo = float(np.mean([commit_tree_verify_algorithmic_bytes(f.sizes(), f, cfg.H, cfg.d_k,
                                                               cfg.d_v, 2) for f in forests]))
    lines = ["# Kernel durations, target workload (rocprofv3 --kernel-trace --stats)", "",
             "Command:", "", "```", commands["trace"], "```", "",
             "Summarized from its output by:", "", "```", summarizer_command(), "```", ""]
    wins = marked_windows(trace_dir, DOMINANT_KERNEL)
    if wins:
        w = np.array([e - s for s, e in wins[0]], np.float64) / 1e3
        span = (wins[0][-1][1] - wins[0][0][0]) / 1e3 / len(w)
        lines += ["## The timed region", "",
                  "Dispatches of `bole_commit_tree_verify` between the two marker kernels "
                  "the bench launches around its timed replays (the K steps its JSON line "
                  "reports):", "",
                  "| dispatches | mean us | median us | min us | max us | span / K us | "
                  "algorithmic MB | GB/s at the mean | of 8 TB/s |",
                  "|---|---|---|---|---|---|---|---|---|",
                  f"| {len(w)} | {w.mean():.2f} | {np.median(w):.2f} | {w.min():.2f} | "
                  f"{w.max():.2f} | {span:.2f} | {algo / 1e6:.1f} | {algo / (w.mean() * 1e3):.0f} | "
                  f"{algo / (w.mean() * 1e3) / PEAK_HBM_GBS:.3f} |", ""]
        m = trace_marginal_us(wins)
        if m is not None:
            lines += ["## The roofline's duration", "",
                      "`roofline.ms_per_launch` is a marginal time: graphs of 128 and of 64 "
                      "back-to-back launches, 8 replays each, each region between marker "
                      "kernels. From this trace's own timestamps, (span of the 1 024 dispatches "
                      "- span of the 512) / 512:", "",
                      "| marginal us per launch | algorithmic MB | GB/s | of 8 TB/s |",
                      "|---|---|---|---|",
                      f"| {m:.2f} | {algo / 1e6:.1f} | {algo / (m * 1e3):.0f} | "
                      f"{algo / (m * 1e3) / PEAK_HBM_GBS:.3f} |", "",
                      ]
            if bench_line:
                d = json.load(open(bench_line))
                ro = d["roofline"]
                lines += ["The JSON line the traced run printed, timed with HIP events over the "
                          "same dispatches:", "",
                          "| ms_per_step | roofline.ms_per_launch | roofline.frac | "
                          "frac from the trace's marginal | ratio |", "|---|---|---|---|---|",
                          f"| {d['ms_per_step'] * 1e3:.2f} us | {ro['ms_per_launch'] * 1e3:.2f} us | "
                          f"{ro['frac']:.4f} | {algo / (m * 1e3) / PEAK_HBM_GBS:.4f} | "
                          f"{ro['frac'] / (algo / (m * 1e3) / PEAK_HBM_GBS):.3f} |", ""]
    lines += ["## Every dispatch of the run (warm-up, captures and other paths included)", "",
              "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        if "bole::" in r["Name"] or "copyBuffer" in r["Name"]:
            lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | "
                         f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                         f"{float(r['MaxNs']) / 1e3:.2f} |")
    with open(os.path.join(PROFILES, "bole_kernels_target_trace.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")

    def per_dispatch(d, counter):
        rows = sorted((r for r in _csv_rows(d, "counter_collection.csv")
                       if r["Counter_Name"] == counter), key=lambda r: int(r["Dispatch_Id"]))
        dom = [float(r["Counter_Value"]) for r in rows if DOMINANT_KERNEL in r["Kernel_Name"]]
        # the calibration copies run before any library kernel (later copies,
        # such as the bench's own bandwidth figure, have other sizes)
        first = next((i for i, r in enumerate(rows) if "bole::" in r["Kernel_Name"]), len(rows))
        copies = [float(r["Counter_Value"]) for r in rows[:first] if "copyBuffer" in r["Kernel_Name"]]
        if not dom or not copies:
            raise SystemExit(f"{counter}: dominant kernel or calibration copy missing in {d}")
        return sum(dom) / len(dom), len(dom), float(np.median(copies))

    fetch, n_f, copy_fetch = per_dispatch(fetch_dir, "FETCH_SIZE")
    write, n_w, copy_write = per_dispatch(write_dir, "WRITE_SIZE")
    calib_kib = calib_mib * 1024.0
    f_fetch, f_write = calib_kib / copy_fetch, calib_kib / copy_write
    traffic = (fetch * f_fetch + write * f_write) * 1024.0
    rec = {"kernel": DOMINANT_KERNEL, "kernel_source_hash": kernel_source_hash(),
           "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
           "dispatches": [n_f, n_w], "copy_mib": calib_mib,
           "copy_fetch_kib": copy_fetch, "copy_write_kib": copy_write,
           "fetch_scale": f_fetch, "write_scale": f_write,
           "hbm_bytes_per_launch": traffic, "algorithmic_bytes_per_launch": float(algo)}
    with open(PROFILE_COUNTERS, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    md = ["# HBM traffic of `bole_commit_tree_verify`, target workload (rocprofv3 --pmc)", "",
          "Commands (one counter per pass; each pass first copies "
          f"{calib_mib} MiB device-to-device for the calibration):", "", "```",
          commands["fetch"], commands["write"], "```", "",
          "Summarized from their output by:", "", "```", summarizer_command(), "```", "",
          "| quantity | value |", "|---|---|",
          f"| FETCH_SIZE per dispatch (KiB) | {fetch:.0f} over {n_f} dispatches |",
          f"| WRITE_SIZE per dispatch (KiB) | {write:.0f} over {n_w} dispatches |",
          f"| copy of {calib_mib} MiB: FETCH_SIZE / WRITE_SIZE (KiB) | {copy_fetch:.0f} / "
          f"{copy_write:.0f} |",
          f"| scale factors (true / counted) | fetch {f_fetch:.3f}, write {f_write:.3f} |",
          f"| HBM bytes per launch (scaled) | {traffic / 1e6:.1f} MB |",
          f"| algorithmic bytes per launch | {algo / 1e6:.1f} MB |",
          f"| ratio | {traffic / algo:.3f} |", "",
          f"Kernel source hash: `{rec['kernel_source_hash']}` ({', '.join(KERNEL_SOURCE_NAMES)}); "
          "bench.py reports `traffic` only while it matches.", ""]
    md += all_kernel_traffic(fetch_dir, write_dir, f_fetch, f_write, n_sets)
    with open(os.path.join(PROFILES, "bole_commit_tree_verify_target_counters.md"), "w") as fh:
        fh.write("\n".join(md) + "\n")
    print(json.dumps(rec))


def build_states_on_gpu(cfg, B, layer, seed, torch, TreeRound, dev):
    """Committed states from the prefix recipe (sequential recurrence over
    cfg.prefix seeded tokens from a zero state), produced by the library itself:
    the prefix is fed as chain trees of up to 64 nodes, each verified and
    committed in turn."""
    pb = W.make_prefix_bulk(cfg, B, layer, seed)
    pool = torch.zeros(B, cfg.H, cfg.d_v, cfg.d_k, dtype=torch.float32, device=dev)
    slot = torch.arange(B, dtype=torch.int32, device=dev)
    P = cfg.prefix
    done = 0
    while done < P:
        T = min(64, P - done)
        f = W.chain_forest(B, T)
        rnd = TreeRound(f.parent, f.tree_off, cfg.H, device=dev)
        sl = slice(done, done + T)

        def tokens(a, storage=True):  # [T, B, H, ...] -> [B*T, H, ...], tree-major
            a = np.ascontiguousarray(np.swapaxes(a[sl], 0, 1)).reshape(B * T, *a.shape[2:])
            if storage and cfg.dtype == "bf16":
                return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(a).to(dev)

        q, k, v = tokens(pb.q), tokens(pb.k), tokens(pb.v)
        g, beta = tokens(pb.g, False), tokens(pb.beta, False)
        logP = rnd.prep(g[None])[0]
        _, U = rnd.layer(q, k, v, logP, beta, pool, slot)
        rnd.commit(pool[None], slot, k[None], U[None], logP[None], f.accept)
        done += T
    torch.cuda.synchronize()
    return pool


class InputSet:
    """One request batch's round inputs on the device: its forest, token
    operands and slot states.  The deferred step (each launch commits the same
    requests' previous round) reads the previous round's U, logP and topology
    while writing its own, so those outputs rotate through GROUPS buffer groups
    (group 0 is also what the other paths use)."""

    GROUPS = 3

    def __init__(self, cfg, seed, torch, TreeRound, dev):
        f = W.make_forest(cfg, seed)
        x = W.make_layer(cfg, f.N, 0, seed)
        self.forest = f
        self.sizes = f.sizes()

        def tok(a):
            a = np.ascontiguousarray(a)
            if cfg.dtype == "bf16":
                return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(a).to(dev)

        self.q, self.k, self.v = tok(x.q), tok(x.k), tok(x.v)
        self.g = torch.from_numpy(x.g).to(dev)[None]
        self.beta = torch.from_numpy(x.beta).to(dev)
        self.pool = build_states_on_gpu(cfg, f.B, 0, seed, torch, TreeRound, dev)
        self.slot = torch.arange(f.B, dtype=torch.int32, device=dev)
        self.accept = torch.from_numpy(f.accept).to(dev)
        self.rnd = TreeRound(f.parent, f.tree_off, cfg.H, device=dev)
        N, H = f.N, cfg.H
        self.logP = torch.empty_like(self.g)
        self.O = torch.empty(N, H, cfg.d_v, dtype=self.v.dtype, device=dev)
        self.U = torch.empty(N, H, cfg.d_v, dtype=torch.float32, device=dev)
        t = self.rnd.topo
        self.groups = [dict(U=self.U, logP=self.logP[0], depth=t.depth, anc=t.anc,
                            order=t.order, tree_depth=t.tree_depth)]
        for _ in range(self.GROUPS - 1):
            self.groups.append(dict(
                U=torch.empty_like(self.U), logP=torch.empty_like(self.logP[0]),
                depth=torch.empty_like(t.depth), anc=torch.empty_like(t.anc),
                order=torch.empty_like(t.order), tree_depth=torch.empty_like(t.tree_depth)))

    def fill_groups(self, bole):
        """Every group holds a verified round of this batch (bole_tree_verify
        from the current slot states, which it leaves unchanged)."""
        t = self.rnd.topo
        for gr in self.groups:
            bole.bole_tree_verify(self.q, self.k, self.v, t.parent, self.g[0], self.beta,
                                  self.pool, self.slot, t.tree_off, self.O, gr["U"], gr["depth"],
                                  gr["anc"], gr["order"], gr["tree_depth"], gr["logP"],
                                  self.rnd.err)


def cycle_colour(m, n):
    """Output group of a batch's m-th round when its n >= 2 rounds repeat as a
    cycle (graph replays): a proper colouring of the cycle, so a round never
    writes the group its predecessor (round m - 1, or n - 1 for m = 0) wrote."""
    if n % 2 == 0 or m < n - 1:
        return m % 2
    return 2


def deferred_schedule(R, S):
    """(set, written group, read group) of each of R deferred steps over S sets
    in rotation: step i runs set i % S, whose rounds in the R steps form a cycle
    (each needs at least two)."""
    if R < 2 * S:
        raise SystemExit(f"the deferred step needs at least {2 * S} steps per graph "
                         f"(two rounds per input set); got {R}")
    out = []
    for i in range(R):
        j, m = i % S, i // S
        n = (R - j + S - 1) // S
        out.append((j, cycle_colour(m, n), cycle_colour((m - 1) % n, n)))
    return out


def launch(s, bole, which, cur=0, prev=1):
    t = s.rnd.topo
    lp = s.logP[0]
    if which == "tree_prep":
        bole.bole_tree_prep(t.parent, t.tree_off, s.g, t.depth, t.anc, t.order, t.tree_depth,
                            s.logP, s.rnd.err)
    elif which == "factor_gc":
        bole.bole_factor_gc(s.q, s.k, lp, s.beta, t.anc, t.order, t.tree_off, s.rnd.G, s.rnd.C,
                            s.rnd.err)
    elif which == "verify":
        bole.bole_verify(s.q, s.k, s.v, lp, s.beta, s.pool, s.slot, s.rnd.G, s.rnd.C, t.order,
                         t.depth, t.tree_off, t.tree_depth, s.O, s.U, s.rnd.err)
    elif which == "verify_neumann":
        bole.bole_verify_neumann(s.q, s.k, s.v, lp, s.beta, s.pool, s.slot, s.rnd.G, s.rnd.C,
                                 t.order, t.depth, t.tree_off, t.tree_depth, s.O, s.U, s.rnd.err)
    elif which == "factor_inverse":
        bole.bole_factor_inverse(s.q, s.k, lp, s.beta, t.anc, t.order, t.tree_off, s.rnd.G,
                                 s.rnd.C, s.rnd.err)
    elif which == "verify_inverse":
        bole.bole_verify_inverse(s.q, s.k, s.v, lp, s.beta, s.pool, s.slot, s.rnd.G, s.rnd.C,
                                 t.order, t.depth, t.tree_off, t.tree_depth, s.O, s.U, s.rnd.err)
    elif which == "tree_verify":
        bole.bole_tree_verify(s.q, s.k, s.v, t.parent, s.g[0], s.beta, s.pool, s.slot, t.tree_off,
                              s.O, s.U, t.depth, t.anc, t.order, t.tree_depth, lp, s.rnd.err)
    elif which == "factor_verify":
        bole.bole_factor_verify(s.q, s.k, s.v, lp, s.beta, s.pool, s.slot, t.anc, t.order,
                                t.depth, t.tree_off, t.tree_depth, s.O, s.U, s.rnd.err)
    elif which == "commit":
        bole.bole_commit_path(s.pool, s.slot, s.k, s.U, lp, t.anc, t.tree_off, s.accept,
                              s.rnd.err)
    elif which == "commit_tree_verify":
        # the same requests' previous round (group `prev`) is committed into
        # their slots, and this round is verified and written to group `cur`
        gc, gp = s.groups[cur], s.groups[prev]
        bole.bole_commit_tree_verify(s.q, s.k, s.v, t.parent, s.g[0], s.beta, s.pool, s.slot,
                                     t.tree_off, s.O, gc["U"], gc["depth"], gc["anc"],
                                     gc["order"], gc["tree_depth"], gc["logP"], s.k, gp["U"],
                                     gp["logP"], gp["anc"], t.tree_off, s.accept, s.rnd.err)
    else:
        raise ValueError(which)


STEPS = {
    # the previous round's commit, preparation, G/C and verify in one launch
    # (the default): one round's commit and one round's verify per step
    "deferred": ("commit_tree_verify",),
    # preparation, G/C and verify in one launch, then the commit
    "tree": ("tree_verify", "commit"),
    # preparation on its own, G/C produced and consumed in one launch
    "fused": ("tree_prep", "factor_verify", "commit"),
    # the four-call path: G/C written by the producer, read back by verify
    "split": ("tree_prep", "factor_gc", "verify", "commit"),
    # the four-call path with the other exact solves of (I + G) U = R: the
    # d-step Neumann propagation, and the explicit inverse W = (I+G)^-1, M = C W
    "split_neumann": ("tree_prep", "factor_gc", "verify_neumann", "commit"),
    "split_inverse": ("tree_prep", "factor_inverse", "verify_inverse", "commit"),
}


def run_step(s, bole, path="tree", cur=0, prev=1):
    """One pass of the whole path on the current stream (cur / prev: the
    deferred step's written and read output groups)."""
    for which in STEPS[path]:
        launch(s, bole, which, cur, prev)


def capture(torch, fn):
    """A HIP graph of the launches fn() makes on the current stream (captured on
    a side stream, as torch requires)."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # one uncaptured pass on the capture stream first
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graphs(graphs, reps, torch):
    """Average ms per replay of graphs[i % len(graphs)], i < reps, bracketed by
    events on the replaying (current) stream.  An untimed replay of each graph
    goes first, not waited for, so the GPU is busy when the timed region
    opens."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    for g in graphs:
        g.replay()
    e0.record()
    for i in range(reps):
        graphs[i % len(graphs)].replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def graph_steps(k, cap=2048):
    """Steps per captured graph for a run of exactly k steps: k itself, or the
    largest divisor of k not above cap."""
    if k <= cap:
        return k
    return next(r for r in range(cap, 0, -1) if k % r == 0)


def input_sets(sets, steps, path):
    """Rotated input sets a run of `steps` steps uses: `sets`, or fewer for the
    deferred step, whose captured graph must give each set at least two rounds
    (each set's rounds form a cycle)."""
    if path != "deferred":
        return sets
    r = graph_steps(steps)
    if r < 4:
        raise SystemExit(f"the deferred step needs a graph of at least 4 steps; "
                         f"--steps {steps} gives {r}")
    return min(sets, r // 2)


# A short kernel (torch.cuda._sleep cycles) before and after a timed region:
# markers that delimit its dispatches in a kernel trace.
MARKER_CYCLES = 1000


# Untimed steps replayed right before a timed region (tens of milliseconds of
# GPU work): a region timed straight after host-side setup, with the GPU idle
# meanwhile, ran about 5% slower over its first few hundred steps.
PREROLL_STEPS = 2000


def graph_ms(torch, g, r, replays, marker=False):
    """ms per step of `replays` back-to-back replays of the captured graph g
    of r steps.  Untimed pre-roll replays (at least PREROLL_STEPS steps) are
    enqueued right before the timed ones with no wait between: the GPU is
    still busy with them while the host enqueues the timed replays, so the
    timed region holds no host launch time, only the GPU's own start of each
    replay, and it opens on a GPU that has been at full load for a while.
    marker: short kernels right before and after the timed replays delimit
    them in a kernel trace."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    for _ in range(max(1, -(-PREROLL_STEPS // r))):
        g.replay()
    if marker:
        torch.cuda._sleep(MARKER_CYCLES)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    if marker:
        torch.cuda._sleep(MARKER_CYCLES)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (replays * r)


def marginal_ms(torch, calls, r=64, replays=8, marker=False):
    """Marginal ms per launch of back-to-back launches: the difference between
    captured graphs of 2r and r launches (calls(n) gives n zero-argument
    launch calls), each replayed `replays` times after the pre-roll.  The
    GPU's start of each replay cancels, so this is the kernel's own duration
    in a stream of launches, the figure a kernel trace reports per dispatch.
    marker: each of the two timed regions is delimited by marker kernels, so
    a kernel trace can give the same figure from its own timestamps (the
    2r-launch region first)."""
    def one(n):
        cs = calls(n)
        return graph_ms(torch, capture(torch, lambda: [c() for c in cs]), n, replays, marker) * n
    return (one(2 * r) - one(r)) / r


def time_steps_eager(sets, bole, path, K, torch):
    """The same steps launched one call at a time from Python (bound by the
    host's launch rate rather than the GPU)."""
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(K):
        run_step(sets[i % len(sets)], bole, path)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / K


def check_graph_replay(s, graph, bole, path, torch):
    """A captured step must reproduce the eager step exactly: from the same
    state pool, eager and replayed O, U and committed pool agree bit for bit,
    on several replays with eager work between them."""
    pool0 = s.pool.clone()
    for _ in range(3):
        s.pool.copy_(pool0)
        run_step(s, bole, path)
        ref = (s.O.clone(), s.U.clone(), s.pool.clone())
        s.pool.copy_(pool0)
        s.O.zero_()
        s.U.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, (s.O, s.U, s.pool)):
            if not torch.equal(a, b):
                raise SystemExit("graph replay differs from the eager step")
    s.pool.copy_(pool0)
    torch.cuda.synchronize()


def cpu_model():
    """The host CPU's model name as /proc/cpuinfo gives it, with its family and
    model numbers (a virtualised host may give only a generic name)."""
    info = {}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if not line.strip():
                    break  # the first processor's block
                key, _, val = line.partition(":")
                info.setdefault(key.strip(), val.strip())
    except OSError:
        pass
    name = info.get("model name")
    if not name:
        import platform
        return platform.processor() or "unknown"
    if "cpu family" in info and "model" in info:
        name += f" (family {info['cpu family']}, model {info['model']})"
    return name


def cpu_baseline(cfg, seed, budget_s=12.0):
    """The fp64 oracle (tree walk + commit) on the host cores, on the same
    workload; repeats the whole layer until about budget_s of CPU work."""
    import oracle
    f = W.make_forest(cfg, seed)
    x = W.make_layer(cfg, f.N, 0, seed)
    rng = np.random.default_rng(seed)
    # states only need the right shape here: the walk's cost does not depend on them
    S = (rng.standard_normal((f.B, cfg.H, cfg.d_v, cfg.d_k)) * 0.1).astype(np.float32)
    slot = np.arange(f.B, dtype=np.int32)
    threads = oracle.default_threads()

    def timed(nthreads, budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.tree_prep(f.parent, f.tree_off, x.g[None])
            oracle.verify(f.parent, f.tree_off, x.q64, x.k64, x.v64, x.g64, x.beta64, S, slot,
                          f.accept, nthreads=nthreads)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget or reps >= 1000:
                return reps, el

    reps, el = timed(threads, budget_s)
    reps1, el1 = timed(1, budget_s / 4)
    rate = reps * f.N * cfg.H / el
    return {"value": rate, "unit": "node-heads/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "sample": f"{reps} full repetitions of the workload's layer (prep + walk + commit, "
                      f"{f.N} nodes x {cfg.H} heads, float64) in {el:.1f} s",
            "single_thread_value": reps1 * f.N * cfg.H / el1}


def conv_algorithmic_bytes(N, B, C, Wd, e):
    """bole_tree_conv: inputs read and outputs written once, each request's
    committed conv state and the weights read once."""
    return N * C * e * 2 + B * (Wd - 1) * C * e + C * (Wd + 1) * 4


# bytes a timed rotation of inputs touches at least: several times the 256 MB
# last-level cache.  The count of rotated inputs is capped: a small workload
# would otherwise need hundreds of thousands of them (and a captured graph of
# as many launches); its rotation then stays cache-sized, as its record says.
ROTATION_BYTES = 1 << 30
MAX_ROTATED_INPUTS = 64    # per-launch inputs (the convolution, the streaming kernel)
MAX_ROTATED_SETS = 16      # whole input sets (verify workloads)


def rotation_count(nbytes, lo, cap):
    """Inputs to rotate so that they touch ROTATION_BYTES, between lo and cap."""
    return int(min(cap, max(lo, -(-ROTATION_BYTES // max(int(nbytes), 1)))))


def time_tree_conv(cfg, sets, torch, bole, dev, reps):
    """The first-stage tree convolution at the workload's shape: C = H (2 d_k +
    d_v) channels (the mixed q, k, v projection), width W.CONV_WIDTH.  Returns
    (ms per launch, algorithmic bytes per launch, ms per conv-state commit)."""
    C, Wd = W.conv_channels(cfg), W.CONV_WIDTH
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    e = 2 if cfg.dtype == "bf16" else 4
    nbytes = np.mean([conv_algorithmic_bytes(s_.forest.N, s_.forest.B, C, Wd, e) for s_ in sets])
    # inputs and outputs of their own, rotated over at least ROTATION_BYTES so
    # that the last-level cache serves none of them
    n_in = rotation_count(nbytes, 4 * len(sets), MAX_ROTATED_INPUTS)
    runs = []
    for k in range(n_in):
        s_ = sets[k % len(sets)]
        t = s_.rnd.topo
        N, B = s_.forest.N, s_.forest.B
        x = torch.randn(N, C, generator=gen, device=dev).to(tdt)
        st = torch.randn(B, Wd - 1, C, generator=gen, device=dev).to(tdt)
        wgt = torch.randn(C, Wd, generator=gen, device=dev) / Wd ** 0.5
        bias = 0.1 * torch.randn(C, generator=gen, device=dev)
        runs.append((x, wgt, bias, st, s_.slot, t.parent, t.tree_off, torch.empty_like(x),
                     s_.rnd.err))
    g = capture(torch, lambda: [bole.bole_tree_conv(*runs[i]) for i in range(n_in)])
    ms = time_graphs([g], max(reps // n_in, 5), torch) / n_in
    # the conv-state commit of the accepted paths (moves W - 1 rows per request)
    commits = [(r[3], r[4], r[0], r[5], r[6], sets[k % len(sets)].accept, r[8])
               for k, r in enumerate(runs)]
    gc = capture(torch, lambda: [bole.bole_conv_commit(*commits[i % len(commits)])
                                 for i in range(n_in)])
    ms_commit = time_graphs([gc], max(reps // n_in, 5), torch) / n_in
    return ms, nbytes, ms_commit, n_in


def copy_bandwidth(torch, dev, footprint_bytes, reps):
    """GB/s of a plain device copy (read + write) whose source and destination
    together span footprint_bytes, timed as graph replays."""
    n = footprint_bytes // 8
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    g = capture(torch, lambda: dst.copy_(src))
    ms = time_graphs([g], reps, torch)
    return 2 * n * 4 / (ms * 1e-3) / 1e9


def time_depth16(cfg, torch, TreeRound, bole, dev, reps):
    """Sensitivity: bole_tree_verify on the workload's shape with trees drawn
    under a depth cap of 16 instead of cfg.D (ms per launch, algorithmic bytes)."""
    from dataclasses import replace
    c16 = replace(cfg, D=16)
    e = 2 if cfg.dtype == "bf16" else 4
    probe = InputSet(c16, 0, torch, TreeRound, dev)
    nb0 = tree_verify_algorithmic_bytes(probe.sizes, cfg.H, cfg.d_k, cfg.d_v, e)
    # enough sets that a rotation touches ROTATION_BYTES
    n_sets = rotation_count(nb0, 2, MAX_ROTATED_SETS)
    sets = [probe] + [InputSet(c16, seed, torch, TreeRound, dev) for seed in range(1, n_sets)]
    for s_ in sets:
        run_step(s_, bole, "tree")
    n_in = 2 * n_sets
    g = capture(torch, lambda: [launch(sets[i % n_sets], bole, "tree_verify") for i in range(n_in)])
    ms = time_graphs([g], max(reps // n_in, 5), torch) / n_in
    depth = max(int(s_.rnd.topo.tree_depth.max().item()) for s_ in sets)
    nb = np.mean([tree_verify_algorithmic_bytes(s_.sizes, cfg.H, cfg.d_k, cfg.d_v, e)
                  for s_ in sets])
    return ms, nb, depth, n_sets


def time_forest_build(cfg, torch, ForestBuilder, dev, reps, capacity):
    """Budget selection and packing for the workload's requests: drafted
    candidate trees (depth 8, top-k 4) of cfg.B requests, the given forest
    capacity, at most 64 nodes per request.  Returns ms per call (two launches)."""
    c = W.make_candidates(cfg.B, seed=77)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    cp, pd, co = d(c.cand_parent), d(c.p_draft), d(c.cand_off)
    fb = ForestBuilder(c.B, len(c.cand_parent), capacity, device=dev)
    n_in = 16
    g = capture(torch, lambda: [fb.build(cp, pd, co) for _ in range(n_in)])
    ms = time_graphs([g], max(reps // n_in, 5), torch) / n_in
    assert int(fb.err.item()) == 0, "device error bits set"
    return ms, int(c.cand_off[-1]), int(fb.tree_off[-1].item())


def commit_algorithmic_bytes(forest, L, H, d_k, d_v, e):
    """Compulsory HBM bytes of one commit over L layers: every committed slot
    read and written once (float32), plus the accepted path's key and U rows."""
    depth = np.zeros(forest.N, np.int64)
    for b in range(forest.B):
        o = forest.tree_off[b]
        for i in range(forest.tree_off[b + 1] - o):  # parents precede children or not: walk up
            j, d = i, 0
            while forest.parent[o + j] >= 0:
                j, d = forest.parent[o + j], d + 1
            depth[o + i] = d
    path_len = [int(depth[forest.tree_off[b] + a]) + 1
                for b, a in enumerate(forest.accept) if a >= 0]
    per_head = sum(8 * d_k * d_v + la * (e * d_k + 4 * d_v) for la in path_len)
    return L * H * per_head


def build_states_device(cfg, B, layer, seed, torch, TreeRound, dev):
    """As build_states_on_gpu, with the prefix tokens drawn on the device."""
    pre = W.device_prefix(cfg, B, layer, seed, torch, dev)
    pool = torch.zeros(B, cfg.H, cfg.d_v, cfg.d_k, dtype=torch.float32, device=dev)
    slot = torch.arange(B, dtype=torch.int32, device=dev)
    P, done = cfg.prefix, 0
    while done < P:
        T = min(64, P - done)
        f = W.chain_forest(B, T)
        rnd = TreeRound(f.parent, f.tree_off, cfg.H, device=dev)

        def tok(a):  # [P, B, H, ...] -> [B*T, H, ...], tree-major
            return a[done:done + T].transpose(0, 1).reshape(B * T, *a.shape[2:]).contiguous()

        q, k, v, g, beta = tok(pre.q), tok(pre.k), tok(pre.v), tok(pre.g), tok(pre.beta)
        logP = rnd.prep(g[None])[0]
        _, U = rnd.layer(q, k, v, logP, beta, pool, slot)
        rnd.commit(pool[None], slot, k[None], U[None], logP[None], f.accept)
        done += T
    return pool


def time_bucketed_rounds(cfg, x, pool, slot, torch, dev, K):
    """Whole rounds from drafted candidates: budget selection and packing, the
    L per-layer tree_verify launches and one commit, captured once per capacity
    bucket (BucketedRound) and timed as graph replays.  Token operands are the
    round's device-drawn layers; each tree accepts its last packed node."""
    from linear_attention_tree_amd import BucketedRound
    B, L, N = cfg.B, cfg.L, x.q.shape[1]
    cands = W.make_candidates(B, seed=5)
    buckets = [N // 2, N]
    br = BucketedRound(B, L, cfg.H, cfg.d_k, cfg.d_v, x.v.dtype, int(cands.cand_off[-1]), buckets,
                       device=dev)
    for name in ("q", "k", "v", "g", "beta"):
        getattr(br, name).copy_(getattr(x, name))
    br.cand_parent.copy_(torch.from_numpy(cands.cand_parent))
    br.p_draft.copy_(torch.from_numpy(cands.p_draft))
    br.cand_off.copy_(torch.from_numpy(cands.cand_off))
    pool_b = pool.clone()
    sizes = {}
    for c in buckets:  # each bucket's forest, for its accepted nodes
        br.forest[c].build(br.cand_parent, br.p_draft, br.cand_off)
        sizes[c] = np.diff(br.forest[c].tree_off.cpu().numpy())
    br.accept.zero_()  # the roots: valid in every bucket's forest for the capture passes
    br.capture(pool_b, slot)
    out = {}
    for c in buckets:
        br.accept.copy_(torch.from_numpy((sizes[c] - 1).astype(np.int32)))
        ms = time_graphs([br.graphs[(c, 0)]], max(K // 4, 5), torch)
        out[str(c)] = {"ms_per_round": ms, "nodes": int(sizes[c].sum()),
                       "node_heads_per_s": float(sizes[c].sum()) * cfg.H * L / (ms * 1e-3)}
    assert int(br.err.item()) == 0, "device error bits set"
    del br
    # the same rounds with each layer's launch carrying its commit of the
    # previous round (graphs of the two parities replayed in turn; each round
    # commits the previous round's accepted nodes of the same bucket)
    bd = BucketedRound(B, L, cfg.H, cfg.d_k, cfg.d_v, x.v.dtype, int(cands.cand_off[-1]), buckets,
                       device=dev, deferred=True)
    for par in (0, 1):
        for name in ("q", "k", "v", "g", "beta"):
            bd.tokens(par)[name].copy_(getattr(x, name))
    bd.cand_parent.copy_(torch.from_numpy(cands.cand_parent))
    bd.p_draft.copy_(torch.from_numpy(cands.p_draft))
    bd.cand_off.copy_(torch.from_numpy(cands.cand_off))
    bd.accept.fill_(-1)
    pool_d = pool.clone()
    bd.capture(pool_d, slot)
    out_d = {}
    for c in buckets:
        bd.accept.fill_(-1)  # the first round of this bucket commits nothing
        bd.graphs[(c, 0)].replay()
        bd.accept.copy_(torch.from_numpy((sizes[c] - 1).astype(np.int32)))
        bd.graphs[(c, 1)].replay()  # from here each round commits the previous one
        ms = time_graphs([bd.graphs[(c, 0)], bd.graphs[(c, 1)]], 2 * max(K // 8, 3), torch)
        out_d[str(c)] = {"ms_per_round": ms, "nodes": int(sizes[c].sum()),
                         "node_heads_per_s": float(sizes[c].sum()) * cfg.H * L / (ms * 1e-3)}
    assert int(bd.err.item()) == 0, "device error bits set"
    return {"note": "per capacity bucket: bole_forest_build over drafted candidates "
                    f"({int(cands.cand_off[-1])} for {B} requests), {L} x bole_tree_verify, one "
                    "bole_commit_path; one captured graph per bucket",
            "by_capacity": out,
            "deferred_note": f"the same with {L} x bole_commit_tree_verify (each layer carries "
                             "its commit of the previous round) and no commit launch",
            "deferred_by_capacity": out_d}


def workload_record(cname, torch, TreeRound, bole, dev):
    """One layer of another of the pages' workload shapes: the marginal time per
    launch of bole_commit_tree_verify (the default step's kernel) and of
    bole_tree_verify, over enough rotated input sets that a rotation touches
    ROTATION_BYTES."""
    cfg = W.CONFIGS[cname]
    e = 2 if cfg.dtype == "bf16" else 4
    probe = InputSet(cfg, 0, torch, TreeRound, dev)
    b0 = commit_tree_verify_algorithmic_bytes(probe.sizes, probe.forest, cfg.H, cfg.d_k, cfg.d_v, e)
    n = rotation_count(b0, 2, MAX_ROTATED_SETS)
    sets = [probe] + [InputSet(cfg, seed, torch, TreeRound, dev) for seed in range(1, n)]
    for s_ in sets:
        s_.fill_groups(bole)

    def deferred(r):
        return [lambda j=j, c=c, pv=pv: launch(sets[j], bole, "commit_tree_verify", c, pv)
                for j, c, pv in deferred_schedule(r, n)]

    def tree(r):
        return [lambda i=i: launch(sets[i % n], bole, "tree_verify") for i in range(r)]

    r = max(64, 2 * n)
    ms_c = marginal_ms(torch, deferred, r)
    ms_t = marginal_ms(torch, tree, r)
    for s_ in sets:
        assert s_.rnd.error_bits() == 0, "device error bits set"
    nodes = float(np.mean([s_.forest.N for s_ in sets]))
    bc = float(np.mean([commit_tree_verify_algorithmic_bytes(s_.sizes, s_.forest, cfg.H, cfg.d_k,
                                                              cfg.d_v, e) for s_ in sets]))
    bt = float(np.mean([tree_verify_algorithmic_bytes(s_.sizes, cfg.H, cfg.d_k, cfg.d_v, e)
                        for s_ in sets]))

    def rec(ms, nb):
        return {"us_per_launch": ms * 1e3, "algorithmic_MB": nb / 1e6,
                "frac_of_hbm_peak": nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                "node_heads_per_s": nodes * cfg.H / (ms * 1e-3)}

    out = {"workload": f"{cfg.name}: B={cfg.B} trees ({cfg.tree}, up to {cfg.T} nodes, depth<="
                       f"{cfg.D}), H={cfg.H}, d_k=d_v={cfg.d_k}, {cfg.dtype} q/k/v, one layer",
           "nodes": nodes, "input_sets": n, "rotation_MB": round(bc * n / 1e6, 1),
           "timing": "marginal time per launch between captured graphs of 2r and r back-to-back "
                     f"launches (r = {r}), 8 replays each",
           "bole_commit_tree_verify": rec(ms_c, bc), "bole_tree_verify": rec(ms_t, bt)}
    del sets, probe
    torch.cuda.empty_cache()
    return out


def multilayer_record(torch, TreeRound, bole, dev, reps):
    """The multi-layer round at its full shape (36 layers, 32 trees x 64 nodes,
    32 heads, d = 128, bf16; token operands and states drawn on the device)
    beside the per-node full-state-snapshot baseline run in the same harness:
    round times, the per-layer kernels against their roofline, the commit over
    all layers, bytes written per layer and the snapshots' resident memory."""
    from linear_attention_tree_amd.baselines import SnapshotVerifier
    cfg = W.CONFIGS["multilayer"]
    L, H, d_k, d_v = cfg.L, cfg.H, cfg.d_k, cfg.d_v
    f = W.make_forest(cfg, 0)
    B, N = f.B, f.N
    e = 2 if cfg.dtype == "bf16" else 4
    x = W.device_layer(cfg, N, 0, 0, torch, dev, lead=(L,))
    pool0 = W.device_states(cfg, B, 0, torch, dev, lead=(L,))
    slot = torch.arange(B, dtype=torch.int32, device=dev)
    accept = torch.from_numpy(f.accept).to(dev)
    rnd = TreeRound(f.parent, f.tree_off, H, device=dev)
    t = rnd.topo
    O = torch.empty(L, N, H, d_v, dtype=x.v.dtype, device=dev)
    # two output sets: a deferred round reads the previous round's U, logP and
    # ancestor sets while it writes its own
    bufs = [(torch.empty(L, N, H, d_v, dtype=torch.float32, device=dev),
             torch.empty(L, N, H, dtype=torch.float32, device=dev),
             tuple(torch.empty_like(a) for a in (t.depth, t.anc, t.order, t.tree_depth)))
            for _ in range(2)]
    pool = pool0.clone()

    def tree_layer(l, U, lp, topo):
        bole.bole_tree_verify(x.q[l], x.k[l], x.v[l], t.parent, x.g[l], x.beta[l], pool[l], slot,
                              t.tree_off, O[l], U[l], *topo, lp[l], rnd.err)

    def deferred_layer(l, cur):
        (U, lp, topo), (Up, lpp, topop) = bufs[cur], bufs[1 - cur]
        bole.bole_commit_tree_verify(x.q[l], x.k[l], x.v[l], t.parent, x.g[l], x.beta[l],
                                     pool[l], slot, t.tree_off, O[l], U[l], *topo, lp[l],
                                     x.k[l], Up[l], lpp[l], topop[1], t.tree_off, accept, rnd.err)

    def tree_round(cur=0):  # L x bole_tree_verify, then one commit over all layers
        U, lp, topo = bufs[cur]
        for l in range(L):
            tree_layer(l, U, lp, topo)
        bole.bole_commit_path(pool, slot, x.k, U, lp, topo[1], t.tree_off, accept, rnd.err)

    def deferred_rounds():  # two rounds of L x bole_commit_tree_verify
        for cur in (0, 1):
            for l in range(L):
                deferred_layer(l, cur)

    def commit_only():
        U, lp, topo = bufs[0]
        bole.bole_commit_path(pool, slot, x.k, U, lp, topo[1], t.tree_off, accept, rnd.err)

    def timed(fn, n_rep):
        """ms per replay of fn's captured graph: two pre-roll replays (whole
        rounds, milliseconds of GPU work) enqueued right before the timed ones
        keep the GPU busy while the host enqueues those."""
        g = capture(torch, fn)
        torch.cuda.synchronize()
        for _ in range(2):
            g.replay()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n_rep):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n_rep

    tree_round(0)  # real rounds in both buffer sets
    tree_round(1)
    torch.cuda.synchronize()
    ms_deferred = timed(deferred_rounds, max(reps // 8, 3)) / 2
    ms_tree = timed(tree_round, max(reps // 8, 3))
    ms_commit = timed(commit_only, max(reps // 4, 5))
    # per launch: marginal time between one and two deferred rounds' launches,
    # and between L and 2L tree_verify launches
    t1 = timed(lambda: [deferred_layer(l, 0) for l in range(L)], 3)
    t2 = timed(deferred_rounds, 3)
    ms_ctv = (t2 - t1) / L
    U0, lp0, topo0 = bufs[0]
    t1 = timed(lambda: [tree_layer(l, U0, lp0, topo0) for l in range(L)], 3)
    t2 = timed(lambda: [tree_layer(l % L, U0, lp0, topo0) for l in range(2 * L)], 3)
    ms_tv = (t2 - t1) / L
    assert rnd.error_bits() == 0, "device error bits set"
    ctv_bytes = commit_tree_verify_algorithmic_bytes(f.sizes(), f, H, d_k, d_v, e)
    tv_bytes = tree_verify_algorithmic_bytes(f.sizes(), H, d_k, d_v, e)
    c_bytes = commit_algorithmic_bytes(f, L, H, d_k, d_v, e)

    # the per-node snapshot baseline on the same inputs: every layer's node
    # states kept until the round's commit, as a serial tree verifier keeps them
    snap_layer = N * H * d_v * d_k * 4
    free, _ = torch.cuda.mem_get_info()
    all_layers = free > L * snap_layer + (8 << 30)
    snap = torch.empty((L if all_layers else 1), N, H, d_v, d_k, dtype=torch.float32, device=dev)
    sv = SnapshotVerifier(f.parent, f.tree_off, H, device=dev)
    pool_s = pool0.clone()
    O_s = torch.empty_like(O)
    U_s = torch.empty_like(bufs[0][0])

    def snapshot_layer(l):
        sl = snap[l if all_layers else 0]
        sv.layer(x.q[l], x.k[l], x.v[l], x.g[l], x.beta[l], pool_s[l], slot, sl, O_s[l], U_s[l])
        if not all_layers:  # commit before the next layer overwrites the snapshots
            sv.commit(sl, pool_s[l], slot, accept)

    def snapshot_round():
        for l in range(L):
            snapshot_layer(l)
        if all_layers:
            for l in range(L):
                sv.commit(snap[l], pool_s[l], slot, accept)

    snapshot_round()
    torch.cuda.synchronize()
    ms_snap = timed(snapshot_round, 3)
    ms_snap_layer = timed(lambda: snapshot_layer(0), 5)
    del snap
    torch.cuda.empty_cache()
    o_u_bytes = N * H * d_v * (e + 4)
    prep_bytes = N * (4 * H + 20)
    snap_written = snap_layer + o_u_bytes
    snap_moved = 2 * snap_layer + N * H * (2 * e * d_k + e * d_v + 8) + o_u_bytes
    return {
        "workload": f"L={L} layers, B={B} trees x T={cfg.T} nodes (random recursive, "
                    f"depth<={cfg.D}), H={H}, d_k=d_v={d_k}, {cfg.dtype} q/k/v, f32 gates and "
                    "state; tokens and states drawn on the device",
        "round_ms": {"deferred: L x commit_tree_verify": ms_deferred,
                     "tree: L x tree_verify + one commit over all layers": ms_tree},
        "node_heads_per_s_per_layer": N * H * L / (ms_deferred * 1e-3),
        "commit_tree_verify_per_layer": {
            "ms": ms_ctv, "algorithmic_bytes": ctv_bytes,
            "frac_of_hbm_peak": ctv_bytes / (ms_ctv * 1e-3) / 1e9 / PEAK_HBM_GBS},
        "tree_verify_per_layer": {
            "ms": ms_tv, "algorithmic_bytes": tv_bytes,
            "frac_of_hbm_peak": tv_bytes / (ms_tv * 1e-3) / 1e9 / PEAK_HBM_GBS},
        "commit_over_all_layers": {
            "ms": ms_commit, "algorithmic_bytes": c_bytes,
            "frac_of_hbm_peak": c_bytes / (ms_commit * 1e-3) / 1e9 / PEAK_HBM_GBS},
        "gc_bytes_per_round": {"tree and deferred paths (on chip)": 0,
                               "split path: one workspace reused by every layer":
                               int(bole.bole_gc_workspace_bytes(B, H))},
        "bytes_written_per_layer": {
            "bole_tree_verify (O, U, logP, topology)": o_u_bytes + prep_bytes,
            "bole_commit_tree_verify (also the committed slots)":
                o_u_bytes + prep_bytes + B * H * d_v * d_k * 4,
            "snapshot baseline (node states, O, U)": snap_written},
        "snapshot_baseline": {
            "note": "per-node full-state snapshots, level-synchronous (one launch per depth; "
                    "every node's float32 state written, then read by its children); commit = "
                    "copy of the accepted node's state",
            "ms_per_round": ms_snap, "ms_per_layer": ms_snap_layer,
            "bytes_moved_per_layer": snap_moved,
            "GBs_per_layer": snap_moved / (ms_snap_layer * 1e-3) / 1e9,
            "resident_snapshot_GiB": (L if all_layers else 1) * snap_layer / 2 ** 30,
            "snapshots_kept": "every layer until the commit" if all_layers
                              else "one layer at a time (not enough free memory for all)",
        },
        "round_speedup_vs_snapshot": ms_snap / ms_deferred,
        "transient_bytes_per_round": {"U + logP": L * N * H * (4 * d_v + 4),
                                      "per-node snapshots": L * snap_layer},
    }


def round_main(cfg, args, torch, TreeRound, bole, dev):
    """One step = one verification round over cfg.L layers: the per-layer
    verify launches, then one commit over all layers (in place, so each round
    verifies against the states the previous round committed).  With --path
    deferred each layer's launch carries that layer's commit of the previous
    round instead (bole_commit_tree_verify) and there is no separate commit;
    the per-round outputs (U, logP, topology) alternate between two buffer
    sets, so a round reads the previous one's while writing its own."""
    if args.path.startswith("split"):
        raise SystemExit("the multi-layer round runs --path deferred, tree or fused")
    L, H = cfg.L, cfg.H
    f = W.make_forest(cfg, 0)
    B, N = f.B, f.N
    x = W.device_layer(cfg, N, 0, 0, torch, dev, lead=(L,))
    pool = torch.stack([build_states_device(cfg, B, l, 0, torch, TreeRound, dev)
                        for l in range(L)])
    slot = torch.arange(B, dtype=torch.int32, device=dev)
    accept = torch.from_numpy(f.accept).to(dev)
    rnd = TreeRound(f.parent, f.tree_off, H, device=dev)
    t = rnd.topo
    logP = torch.empty(L, N, H, dtype=torch.float32, device=dev)
    O = torch.empty(L, N, H, cfg.d_v, dtype=x.v.dtype, device=dev)
    U = torch.empty(L, N, H, cfg.d_v, dtype=torch.float32, device=dev)

    def verify_layers(path):
        if path == "tree":
            for l in range(L):
                bole.bole_tree_verify(x.q[l], x.k[l], x.v[l], t.parent, x.g[l], x.beta[l],
                                      pool[l], slot, t.tree_off, O[l], U[l], t.depth, t.anc,
                                      t.order, t.tree_depth, logP[l], rnd.err)
        else:
            bole.bole_tree_prep(t.parent, t.tree_off, x.g, t.depth, t.anc, t.order,
                                t.tree_depth, logP, rnd.err)
            for l in range(L):
                bole.bole_factor_verify(x.q[l], x.k[l], x.v[l], logP[l], x.beta[l], pool[l],
                                        slot, t.anc, t.order, t.depth, t.tree_off, t.tree_depth,
                                        O[l], U[l], rnd.err)

    def commit():
        bole.bole_commit_path(pool, slot, x.k, U, logP, t.anc, t.tree_off, accept, rnd.err)

    # the second buffer set of the deferred rounds (the first is U, logP, t)
    U2 = torch.empty_like(U)
    logP2 = torch.empty_like(logP)
    topo2 = [torch.empty_like(a) for a in (t.depth, t.anc, t.order, t.tree_depth)]
    sets_d = [(U, logP, (t.depth, t.anc, t.order, t.tree_depth)), (U2, logP2, tuple(topo2))]

    def deferred_round(cur):
        (Uc, lpc, (dc, ac, oc, tdc)), (Up, lpp, (_, ap, _, _)) = sets_d[cur], sets_d[1 - cur]
        for l in range(L):
            bole.bole_commit_tree_verify(x.q[l], x.k[l], x.v[l], t.parent, x.g[l], x.beta[l],
                                         pool[l], slot, t.tree_off, O[l], Uc[l], dc, ac, oc, tdc,
                                         lpc[l], x.k[l], Up[l], lpp[l], ap, t.tree_off, accept,
                                         rnd.err)

    def one_round(path):
        if path == "deferred":  # two rounds, one on each buffer set
            deferred_round(0)
            deferred_round(1)
            return
        verify_layers(path)
        commit()

    one_round("tree")  # a real round in buffer set 0, copied to set 1
    U2.copy_(U)
    logP2.copy_(logP)
    for a, b in zip(topo2, (t.depth, t.anc, t.order, t.tree_depth)):
        a.copy_(b)
    for _ in range(max(args.warmup, 1)):
        for p in ("tree", "fused", "deferred"):
            one_round(p)
    torch.cuda.synchronize()
    assert rnd.error_bits() == 0, "device error bits set"
    K = args.steps
    graphs = {p: capture(torch, lambda p_=p: one_round(p_)) for p in ("deferred", "tree", "fused")}
    for g in graphs.values():  # untimed pre-roll
        g.replay()
    ms_round = {p: time_graphs([g], K, torch) / (2 if p == "deferred" else 1)
                for p, g in graphs.items()}
    g_ver = capture(torch, lambda: verify_layers("tree" if args.path == "deferred" else args.path))
    ms_verify = time_graphs([g_ver], max(K // 4, 5), torch)
    g_com = capture(torch, commit)
    ms_commit = time_graphs([g_com], max(K // 4, 5), torch)
    assert rnd.error_bits() == 0, "device error bits set"

    e = 2 if cfg.dtype == "bf16" else 4
    if args.path == "deferred":
        dominant = "commit_tree_verify"
        vbytes = commit_tree_verify_algorithmic_bytes(f.sizes(), f, H, cfg.d_k, cfg.d_v, e)
        # per-layer launches of the deferred rounds, timed alone (graphs of two rounds)
        g_dv = capture(torch, lambda: (deferred_round(0), deferred_round(1)))
        ms_layer_deferred = time_graphs([g_dv], max(K // 4, 5), torch) / (2 * L)
    else:
        dominant, bytes_fn = DOMINANT[args.path]
        vbytes = bytes_fn(f.sizes(), H, cfg.d_k, cfg.d_v, e)
    cbytes = commit_algorithmic_bytes(f, L, H, cfg.d_k, cfg.d_v, e)
    ms_layer = ms_verify / L
    step = ms_round[args.path]
    ms_dom = ms_layer_deferred if args.path == "deferred" else ms_layer
    buckets = time_bucketed_rounds(cfg, x, pool, slot, torch, dev, K)
    achieved = vbytes / (ms_dom * 1e-3) / 1e9
    c_achieved = cbytes / (ms_commit * 1e-3) / 1e9
    out = {
        "metric": "tree nodes x heads verified/sec per GDN layer",
        "value": N * H * L / (step * 1e-3),
        "unit": "node-heads/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: one round over L={L} layers, B={B} trees x T={cfg.T} nodes "
                        f"(random recursive, depth<={cfg.D}), H={H}, d_k=d_v={cfg.d_k}, "
                        f"{cfg.dtype} q/k/v, f32 gates and state; step = {L} x "
                        + (f"{dominant} (each layer's verify with its commit of the previous "
                           "round inside)" if args.path == "deferred"
                           else f"{dominant} + one commit over all layers"),
            "L": L, "B": B, "T": cfg.T, "H": H, "d_k": cfg.d_k, "d_v": cfg.d_v, "nodes": N,
            "path": args.path,
            "timing": "HIP graph replays of whole rounds; verify and commit also alone",
            "ms_per_round": ms_round,
            "verify_ms_per_layer": ms_layer,
            "commit_tree_verify_ms_per_layer": ms_dom if args.path == "deferred" else None,
            "commit_ms_per_round": ms_commit,
            "gc_bytes_per_round": {"tree/fused (on chip)": 0,
                                   "split: one workspace reused by every layer":
                                   int(bole.bole_gc_workspace_bytes(B, H))},
            "transient_bytes_per_round": {"U + logP": L * N * H * (4 * cfg.d_v + 4)},
            "bucketed_rounds": buckets,
        },
        "roofline": {
            "kernel": "bole_" + dominant,
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": None,
            "algorithmic_bytes_per_launch": vbytes,
        },
        "commit_roofline": {
            "kernel": "bole_commit_path",
            "bound": "hbm",
            "achieved": c_achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": c_achieved / PEAK_HBM_GBS,
            "algorithmic_bytes_per_launch": cbytes,
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, 0, args.cpu_budget)
    print(json.dumps(out), flush=True)


def main():
    global PREROLL_STEPS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="target", choices=sorted(W.CONFIGS))
    ap.add_argument("--sets", type=int, default=8,
                    help="rotated independent input sets (fewer when the deferred step's "
                         "graph of --steps steps cannot give each set two rounds)")
    ap.add_argument("--path", default="deferred", choices=sorted(STEPS),
                    help="deferred: commit_tree_verify (the previous round's commit inside this "
                         "round's verify); tree: tree_verify + commit; "
                         "fused: prep + factor_verify + commit; "
                         "split: the four calls; split_neumann, split_inverse: the four calls "
                         "with the other exact solves")
    ap.add_argument("--preroll-steps", type=int, default=PREROLL_STEPS,
                    help="untimed steps replayed ahead of every timed region (a counter pass, "
                         "which times nothing, can take fewer and dispatch less)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="leave out the one-layer records of the batched and ragged workloads")
    ap.add_argument("--no-multilayer", action="store_true",
                    help="leave out the 36-layer round and its per-node snapshot baseline")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("MFMA_DIR", "TRACE_DIR"),
                    help="write the MFMA/LDS counter summary under profiles/ and exit")
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write the profiles/ summaries from three rocprofv3 runs of this script "
                         "(no GPU needed)")
    ap.add_argument("--trace-bench-line", default=None,
                    help="with --summarize-profiles: the JSON line the traced run printed")
    ap.add_argument("--profile-commands", default="",
                    help="JSON {trace, fetch, write} of the commands that made the runs")
    args = ap.parse_args()
    PREROLL_STEPS = max(1, args.preroll_steps)
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma, args.profile_commands or "?")
        return
    if args.summarize_profiles:
        # the runs' --steps / --sets / --path give the sets they rotated
        summarize_profiles(*args.summarize_profiles, args.calibrate_copy_mib or 256,
                           json.loads(args.profile_commands or "{}") or
                           {"trace": "?", "fetch": "?", "write": "?"},
                           input_sets(args.sets, args.steps, args.path), args.trace_bench_line)
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(every (request, head, layer) unit is independent, so a multi-GPU run would "
              "shard requests or heads with no exchange on the data path)", file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_attention_tree_amd import TreeRound, bole
    dev = torch.device("cuda:0")
    cfg = W.CONFIGS[args.config]
    if cfg.L != 1:
        round_main(cfg, args, torch, TreeRound, bole, dev)
        return
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.sets < 2:
        raise SystemExit("--sets must be at least 2 (a step commits the previous set's round)")
    n_sets = input_sets(args.sets, args.steps, args.path)
    sets = [InputSet(cfg, seed, torch, TreeRound, dev) for seed in range(n_sets)]
    S = len(sets)
    e = 2 if cfg.dtype == "bf16" else 4
    for s_ in sets:
        s_.fill_groups(bole)

    for i in range(args.warmup):
        for p in STEPS:
            run_step(sets[i % S], bole, p)
    torch.cuda.synchronize()
    for s in sets:
        assert s.rnd.error_bits() == 0, "device error bits set"

    # Steps are timed as replays of one captured graph of R steps (R = K, or a
    # divisor of K for long runs): launching a kernel per step from Python
    # costs more host time than the GPU spends on it.  Batches rotate over the
    # input sets; with the deferred step each set's rounds form a cycle in
    # which every launch commits the same requests' previous round.
    K = args.steps
    check_graph_replay(sets[0], capture(torch, lambda: run_step(sets[0], bole, args.path)),
                       bole, args.path, torch)

    def launches(which, r):
        """r launches of one kernel (or one step when `which` is a path) over
        the rotated sets, as a list of zero-argument calls."""
        if which in ("deferred", "commit_tree_verify"):
            name = "commit_tree_verify"
            return [lambda j=j, c=c, pv=pv: launch(sets[j], bole, name, c, pv)
                    for j, c, pv in deferred_schedule(r, S)]
        if which in STEPS:
            return [lambda i=i: run_step(sets[i % S], bole, which) for i in range(r)]
        return [lambda i=i: launch(sets[i % S], bole, which) for i in range(r)]

    def time_graph(g, r, replays, marker=False):
        return graph_ms(torch, g, r, replays, marker)

    def capture_steps(which, r):
        calls = launches(which, r)
        return capture(torch, lambda: [c() for c in calls])

    def time_k(which, k, marker=False):
        """ms per step over exactly k back-to-back steps (k / r replays of one
        graph of r steps)."""
        r = graph_steps(k)
        return time_graph(capture_steps(which, r), r, k // r, marker)

    def time_per_launch(which, r=64, replays=8, marker=False):
        return marginal_ms(torch, lambda n: launches(which, n), r, replays, marker)

    torch.cuda._sleep(1)  # load the marker kernel before the timed regions
    ms_step = time_k(args.path, K, marker=True)
    # the dominant kernel's own duration per launch (the step's one launch
    # for the deferred path), and the verify kernel alone (the step's verify
    # without the commit), each as the marginal time per back-to-back launch
    ms_launch = time_per_launch(args.path if args.path == "deferred" else DOMINANT[args.path][0],
                                marker=True)
    ms_tree_verify = time_per_launch("tree_verify")
    ms_other = {p: time_k(p, max(K // 2, 2 * S)) for p in STEPS if p != args.path}
    ms_eager = time_steps_eager(sets, bole, args.path, max(K // 2, 10), torch)
    # per-kernel averages: each kernel alone, 4 x len(sets) launches per graph
    # over the rotated sets (same inputs, same stream)
    kernels = ("tree_prep", "factor_gc", "verify", "factor_verify", "tree_verify", "commit",
               "commit_tree_verify", "verify_neumann", "factor_inverse", "verify_inverse")
    avg = {}
    for which in kernels:
        n_in = 4 * S
        calls = launches(which, n_in)
        g = capture(torch, lambda c_=calls: [c() for c in c_])
        avg[which] = time_graphs([g], max(K // n_in, 5), torch) / n_in
    conv_ms, conv_bytes, conv_commit_ms, conv_inputs = time_tree_conv(cfg, sets, torch, bole, dev, K)
    # the streaming kernel with the convolution's bytes: y is the written part
    conv_written = float(np.mean([s_.forest.N for s_ in sets])) * W.conv_channels(cfg) * e
    conv_ceil = stream_ceiling(torch, dev, conv_bytes - conv_written, conv_written,
                               rotation_count(conv_bytes, 2, MAX_ROTATED_INPUTS))
    d16_ms, d16_bytes, d16_depth, d16_sets = time_depth16(cfg, torch, TreeRound, bole, dev, K)
    from linear_attention_tree_amd import ForestBuilder
    forest_runs = {}
    for cap in (cfg.B * cfg.T, 768):
        f_ms, m_total, packed = time_forest_build(cfg, torch, ForestBuilder, dev, K, cap)
        forest_runs[str(cap)] = {"ms": f_ms, "nodes_packed": packed}
    for s_ in sets:
        assert s_.rnd.error_bits() == 0, "device error bits set"
    dominant, bytes_fn = DOMINANT[args.path]

    # per step of the timed sequence: set i % S (the mix when K % S != 0)
    mix = [i % S for i in range(graph_steps(K))]
    nodes = float(np.mean([sets[j].forest.N for j in mix]))
    value = nodes * cfg.H / (ms_step * 1e-3)
    tv_bytes = float(np.mean([tree_verify_algorithmic_bytes(sets[j].sizes, cfg.H, cfg.d_k, cfg.d_v,
                                                            e) for j in mix]))
    if args.path == "deferred":
        # each launch commits its own batch's previous round
        vbytes = float(np.mean([commit_tree_verify_algorithmic_bytes(
            sets[j].sizes, sets[j].forest, cfg.H, cfg.d_k, cfg.d_v, e) for j in mix]))
    else:
        vbytes = float(np.mean([bytes_fn(sets[j].sizes, cfg.H, cfg.d_k, cfg.d_v, e) for j in mix]))
    # the kernel's duration per launch in a stream of back-to-back launches
    # (for the deferred path, the timed step's single launch)
    ms_dom = ms_launch
    dom_timing = ("marginal time per launch between captured graphs of 128 and 64 back-to-back "
                  "launches, each replayed 8 times (HIP events; the GPU's start of each replay "
                  "cancels)")
    achieved = vbytes / (ms_dom * 1e-3) / 1e9
    tv_achieved = tv_bytes / (ms_tree_verify * 1e-3) / 1e9
    # a plain copy over the same footprint as the rotated input sets
    copy_gbs = copy_bandwidth(torch, dev, int(vbytes * S), 20)
    # the streaming kernel at each verify kernel's footprint and read:write mix
    tv_written = float(np.mean([tree_verify_written_bytes(sets[j].sizes, cfg.H, cfg.d_k, cfg.d_v,
                                                          e) for j in mix]))
    if args.path == "deferred":
        dom_written = float(np.mean([commit_tree_verify_written_bytes(
            sets[j].sizes, sets[j].forest, cfg.H, cfg.d_k, cfg.d_v, e) for j in mix]))
        ceil_dom = stream_ceiling(torch, dev, vbytes - dom_written, dom_written, S)
    else:
        ceil_dom = None
    ceil_tv = stream_ceiling(torch, dev, tv_bytes - tv_written, tv_written, S)
    # the committed counter record is the default path's dominant kernel
    traffic = traffic_from_profile(kernel_source_hash()) if args.path == "deferred" else None

    out = {
        "metric": "tree nodes x heads verified/sec per GDN layer",
        "value": value,
        "unit": "node-heads/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: B={cfg.B} trees x T={cfg.T} nodes (random recursive, "
                        f"depth<={cfg.D}), H={cfg.H}, d_k=d_v={cfg.d_k}, {cfg.dtype} q/k/v, "
                        f"f32 gates and state; step = {' + '.join(STEPS[args.path])}"
                        + (" (this round's verify with the same requests' previous round's "
                           "accepted-path commit inside: one commit and one verify per step)"
                           if args.path == "deferred" else ""),
            "B": cfg.B, "T": cfg.T, "H": cfg.H, "d_k": cfg.d_k, "d_v": cfg.d_v,
            "nodes": nodes, "input_sets": S,
            "rotation_MB": round(vbytes * S / 1e6, 1),
            # measured: 480 MB rotated made the default kernel 20% faster than
            # 957 MB; 673 MB and more measured the same as 1.3 GB
            "rotation_note": (None if vbytes * S >= 600e6 else
                              "the rotated inputs touch less than about 600 MB: the figures may "
                              "be partly served from the 256 MB last-level cache (more --sets, "
                              "with --steps at least twice --sets, avoid it)"),
            "path": args.path,
            "timing": f"{K} back-to-back steps as {K // graph_steps(K)} replay(s) of a captured "
                      f"graph of {graph_steps(K)} steps, after untimed pre-roll replays; input "
                      f"sets rotated; per-kernel figures from graphs of {4 * S} launches",
            "ms_per_step_other_path": ms_other,
            "ms_per_step_eager_launches": ms_eager,
            "kernel_ms_back_to_back": avg,
            "tree_verify_depth_cap_16": {
                "note": "sensitivity: the same shape with trees drawn under a depth cap of 16",
                "ms": d16_ms, "deepest_tree": d16_depth,
                "rotation_MB": round(d16_bytes * d16_sets / 1e6, 1),
                "achieved_GBs": d16_bytes / (d16_ms * 1e-3) / 1e9,
                "frac_of_hbm_peak": d16_bytes / (d16_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            },
            "stage1_tree_conv": {
                "note": "first pipeline stage: the short causal convolution over each node's "
                        "ancestors, with bias and SiLU; not part of the step",
                "channels": W.conv_channels(cfg), "width": W.CONV_WIDTH, "ms": conv_ms,
                "rotation_MB": round(conv_bytes * conv_inputs / 1e6, 1),
                "achieved_GBs": conv_bytes / (conv_ms * 1e-3) / 1e9,
                "frac_of_hbm_peak": conv_bytes / (conv_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                "algorithmic_bytes_per_launch": conv_bytes,
                "stream_ceiling": {"written_bytes_per_launch": conv_written, "GBs": conv_ceil,
                                   "frac_of_peak": conv_ceil / PEAK_HBM_GBS,
                                   "kernel_frac_of_ceiling":
                                       conv_bytes / (conv_ms * 1e-3) / 1e9 / conv_ceil},
                "conv_commit_ms": conv_commit_ms,
            },
            "forest_build": {
                "note": "budget selection by cumulative draft probability and forest packing "
                        "(two launches), not part of the step; latency-bound",
                "requests": cfg.B, "candidates": m_total, "max_tree": 64,
                "by_capacity": forest_runs,
            },
        },
        "roofline": {
            "kernel": "bole_" + dominant,
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": vbytes,
            "ms_per_launch": ms_dom,
            "timing": dom_timing,
            # the same bytes over the K timed steps' own time (for the deferred
            # path a step is this one launch; the step time also holds the
            # graph replay's start)
            "frac_at_step_time": (vbytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS
                                  if args.path == "deferred" else None),
            "copy_GBs": copy_gbs,
            "frac_of_copy": achieved / copy_gbs,
            "stream_ceiling": None if ceil_dom is None else {
                "note": "a plain streaming kernel (baselines/stream.hip) moving the same read and "
                        "written bytes per launch over the same rotated footprint",
                "written_bytes_per_launch": dom_written, "GBs": ceil_dom,
                "frac_of_peak": ceil_dom / PEAK_HBM_GBS, "kernel_frac_of_ceiling": achieved / ceil_dom},
        },
        "roofline_tree_verify": {
            "note": "the verify alone (bole_tree_verify: preparation, factors, solve and "
                    "readout of one layer, no commit)",
            "kernel": "bole_tree_verify",
            "bound": "hbm",
            "ms": ms_tree_verify,
            "achieved": tv_achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": tv_achieved / PEAK_HBM_GBS,
            "algorithmic_bytes_per_launch": tv_bytes,
            "timing": "as the roofline's dominant kernel",
            "stream_ceiling": {
                "written_bytes_per_launch": tv_written, "GBs": ceil_tv,
                "frac_of_peak": ceil_tv / PEAK_HBM_GBS, "kernel_frac_of_ceiling": tv_achieved / ceil_tv},
        },
    }
    if not args.no_workloads:
        out["config"]["other_workloads"] = {c: workload_record(c, torch, TreeRound, bole, dev)
                                            for c in ("batched", "ragged")}
    if not args.no_multilayer:
        out["config"]["multilayer"] = multilayer_record(torch, TreeRound, bole, dev, K)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, 0, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Throughput of closed-form tree verification for one GDN layer on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
tree preparation (topology + log-space gate products), the G/C factors,
value-tiled verify and the accepted-path commit.  The default path runs all
of it in one launch (bole_commit_tree_verify: this round's preparation,
factors and verify with the previous round's commit inside); --path tree
times bole_tree_verify + bole_commit_path, and --path fused and --path split
the three- and four-launch forms.  Default workload: 16 requests,
64-node random trees (depth <= 12), 32 state heads, d_k = d_v = 128, bf16
q/k/v with float32 gates and states.  Several independent input sets are
rotated so the bytes touched per rotation exceed the 256 MB last-level cache.

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
DOMINANT_KERNEL = "verify_kernel<1, true, true, true, 0, true>"
# the same without the commit (bole_tree_verify)
TREE_VERIFY_KERNEL = "verify_kernel<1, true, true, true, 0, false>"


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


def all_kernel_traffic(fetch_dir, write_dir, f_fetch, f_write):
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
    forests = [W.make_forest(cfg, seed) for seed in range(4)]
    algo = {
        "bole::" + DOMINANT_KERNEL: np.mean(
            [commit_tree_verify_algorithmic_bytes(f.sizes(), forests[i - 1], cfg.H, cfg.d_k,
                                                  cfg.d_v, 2) for i, f in enumerate(forests)]),
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
             command, "```", "",
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


def summarize_profiles(trace_dir, fetch_dir, write_dir, calib_mib, commands):
    """Turn three rocprofv3 runs of this script (a kernel trace, a FETCH_SIZE
    pass and a WRITE_SIZE pass, the counter passes preceded by a plain copy of
    calib_mib MiB) into the text summaries under profiles/ and the counter
    record the bench line reads its `traffic` from."""
    os.makedirs(PROFILES, exist_ok=True)
    stats = _csv_rows(trace_dir, "kernel_stats.csv")
    lines = ["# Kernel durations, target workload (rocprofv3 --kernel-trace --stats)", "",
             "Command:", "", "```", commands["trace"], "```", "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        if "bole::" in r["Name"] or "copyBuffer" in r["Name"]:
            lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | "
                         f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                         f"{float(r['MaxNs']) / 1e3:.2f} |")
    with open(os.path.join(PROFILES, "bole_kernels_target_trace.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")

    def per_dispatch(d, counter):
        rows = [r for r in _csv_rows(d, "counter_collection.csv") if r["Counter_Name"] == counter]
        dom = [float(r["Counter_Value"]) for r in rows if DOMINANT_KERNEL in r["Kernel_Name"]]
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        if not dom or not copies:
            raise SystemExit(f"{counter}: dominant kernel or calibration copy missing in {d}")
        return sum(dom) / len(dom), len(dom), max(copies)

    fetch, n_f, copy_fetch = per_dispatch(fetch_dir, "FETCH_SIZE")
    write, n_w, copy_write = per_dispatch(write_dir, "WRITE_SIZE")
    calib_kib = calib_mib * 1024.0
    f_fetch, f_write = calib_kib / copy_fetch, calib_kib / copy_write
    traffic = (fetch * f_fetch + write * f_write) * 1024.0
    cfg = W.CONFIGS["target"]
    forests = [W.make_forest(cfg, seed) for seed in range(4)]
    algo = np.mean([commit_tree_verify_algorithmic_bytes(f.sizes(), forests[i - 1], cfg.H, cfg.d_k,
                                                         cfg.d_v, 2) for i, f in enumerate(forests)])
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
    md += all_kernel_traffic(fetch_dir, write_dir, f_fetch, f_write)
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


def launch(s, bole, which):
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
        # the previous input set's round is committed into this set's slots:
        # the same work as a serving loop's previous round of the same requests
        p, pt = s.prev, s.prev.rnd.topo
        bole.bole_commit_tree_verify(s.q, s.k, s.v, t.parent, s.g[0], s.beta, s.pool, s.slot,
                                     t.tree_off, s.O, s.U, t.depth, t.anc, t.order, t.tree_depth,
                                     lp, p.k, p.U, p.logP[0], pt.anc, pt.tree_off, p.accept,
                                     s.rnd.err)
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


def run_step(s, bole, path="tree"):
    """One pass of the whole path on the current stream."""
    for which in STEPS[path]:
        launch(s, bole, which)


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
    events on the replaying (current) stream."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(reps):
        graphs[i % len(graphs)].replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


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
            "sample": f"{reps} full repetitions of the workload's layer (prep + walk + commit, "
                      f"{f.N} nodes x {cfg.H} heads, float64) in {el:.1f} s",
            "single_thread_value": reps1 * f.N * cfg.H / el1}


def conv_algorithmic_bytes(N, B, C, Wd, e):
    """bole_tree_conv: inputs read and outputs written once, each request's
    committed conv state and the weights read once."""
    return N * C * e * 2 + B * (Wd - 1) * C * e + C * (Wd + 1) * 4


def time_tree_conv(cfg, sets, torch, bole, dev, reps):
    """The first-stage tree convolution at the workload's shape: C = H (2 d_k +
    d_v) channels (the mixed q, k, v projection), width W.CONV_WIDTH.  Returns
    (ms per launch, algorithmic bytes per launch, ms per conv-state commit)."""
    C, Wd = W.conv_channels(cfg), W.CONV_WIDTH
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    runs = []
    for s_ in sets:
        t = s_.rnd.topo
        N, B = s_.forest.N, s_.forest.B
        x = torch.randn(N, C, generator=gen, device=dev).to(tdt)
        st = torch.randn(B, Wd - 1, C, generator=gen, device=dev).to(tdt)
        wgt = torch.randn(C, Wd, generator=gen, device=dev) / Wd ** 0.5
        bias = 0.1 * torch.randn(C, generator=gen, device=dev)
        runs.append((x, wgt, bias, st, s_.slot, t.parent, t.tree_off, torch.empty_like(x),
                     s_.rnd.err))
    n_in = 4 * len(sets)
    g = capture(torch, lambda: [bole.bole_tree_conv(*runs[i % len(runs)]) for i in range(n_in)])
    ms = time_graphs([g], max(reps // n_in, 5), torch) / n_in
    e = 2 if cfg.dtype == "bf16" else 4
    nbytes = np.mean([conv_algorithmic_bytes(s_.forest.N, s_.forest.B, C, Wd, e) for s_ in sets])
    # the conv-state commit of the accepted paths (moves W - 1 rows per request)
    commits = [(r[3], r[4], r[0], r[5], r[6], s_.accept, r[8]) for r, s_ in zip(runs, sets)]
    gc = capture(torch, lambda: [bole.bole_conv_commit(*commits[i % len(commits)])
                                 for i in range(n_in)])
    ms_commit = time_graphs([gc], max(reps // n_in, 5), torch) / n_in
    return ms, nbytes, ms_commit


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
    sets = [InputSet(c16, seed, torch, TreeRound, dev) for seed in range(2)]
    for s_ in sets:
        run_step(s_, bole, "tree")
    n_in = 16
    g = capture(torch, lambda: [launch(sets[i % 2], bole, "tree_verify") for i in range(n_in)])
    ms = time_graphs([g], max(reps // n_in, 5), torch) / n_in
    depth = max(int(s_.rnd.topo.tree_depth.max().item()) for s_ in sets)
    nb = np.mean([tree_verify_algorithmic_bytes(s_.sizes, cfg.H, cfg.d_k, cfg.d_v,
                                                2 if cfg.dtype == "bf16" else 4) for s_ in sets])
    return ms, nb, depth


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
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="target", choices=sorted(W.CONFIGS))
    ap.add_argument("--sets", type=int, default=4, help="rotated independent input sets")
    ap.add_argument("--path", default="deferred", choices=sorted(STEPS),
                    help="deferred: commit_tree_verify (the previous round's commit inside this "
                         "round's verify); tree: tree_verify + commit; "
                         "fused: prep + factor_verify + commit; "
                         "split: the four calls; split_neumann, split_inverse: the four calls "
                         "with the other exact solves")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("MFMA_DIR", "TRACE_DIR"),
                    help="write the MFMA/LDS counter summary under profiles/ and exit")
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write the profiles/ summaries from three rocprofv3 runs of this script "
                         "(no GPU needed)")
    ap.add_argument("--profile-commands", default="",
                    help="JSON {trace, fetch, write} of the commands that made the runs")
    args = ap.parse_args()
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma, args.profile_commands or "?")
        return
    if args.summarize_profiles:
        summarize_profiles(*args.summarize_profiles, args.calibrate_copy_mib or 256,
                           json.loads(args.profile_commands or "{}") or
                           {"trace": "?", "fetch": "?", "write": "?"})
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
    sets = [InputSet(cfg, seed, torch, TreeRound, dev) for seed in range(args.sets)]
    for i, s_ in enumerate(sets):
        s_.prev = sets[i - 1]  # the round before this one, in the rotation
    e = 2 if cfg.dtype == "bf16" else 4

    for i in range(args.warmup):
        for p in STEPS:
            run_step(sets[i % len(sets)], bole, p)
    torch.cuda.synchronize()
    for s in sets:
        assert s.rnd.error_bits() == 0, "device error bits set"

    # The step is timed as HIP graph replays (one captured step per input set,
    # replayed in rotation): launching three kernels per step from Python costs
    # more host time than the GPU spends on them.
    K = args.steps
    others = [p for p in STEPS if p != args.path]
    R = 4 * len(sets)  # steps per rotation graph
    singles = [capture(torch, lambda s_=s_: run_step(s_, bole, args.path)) for s_ in sets]
    check_graph_replay(sets[0], singles[0], bole, args.path, torch)

    def rotation(p):
        return capture(torch, lambda: [run_step(sets[i % len(sets)], bole, p) for i in range(R)])

    def time_k_steps(p, k, singles_p):
        """Exactly k steps: k // R rotation replays, then the rest one by one,
        after an untimed pre-roll of the same graph (the GPU otherwise enters
        the timed region idle, right after the host-side captures)."""
        rot = rotation(p)
        for _ in range(max(1, min(k, 200) // R)):
            rot.replay()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(k // R):
            rot.replay()
        for i in range(k % R):
            singles_p[i % len(sets)].replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / k

    ms_step = time_k_steps(args.path, K, singles)
    ms_other = {}
    for other in others:
        singles_other = [capture(torch, lambda s_=s_, o_=other: run_step(s_, bole, o_))
                         for s_ in sets]
        ms_other[other] = time_k_steps(other, max(K // 2, 10), singles_other)
    ms_eager = time_steps_eager(sets, bole, args.path, max(K // 2, 10), torch)
    # per-kernel averages: each kernel alone, 4 x len(sets) launches per graph
    # over the rotated sets (same inputs, same stream)
    kernels = ("tree_prep", "factor_gc", "verify", "factor_verify", "tree_verify", "commit",
               "commit_tree_verify", "verify_neumann", "factor_inverse", "verify_inverse")
    avg = {}
    for which in kernels:
        n_in = 4 * len(sets)
        g = capture(torch, lambda w_=which: [launch(sets[i % len(sets)], bole, w_)
                                              for i in range(n_in)])
        avg[which] = time_graphs([g], max(K // n_in, 5), torch) / n_in
    conv_ms, conv_bytes, conv_commit_ms = time_tree_conv(cfg, sets, torch, bole, dev, K)
    d16_ms, d16_bytes, d16_depth = time_depth16(cfg, torch, TreeRound, bole, dev, K)
    from linear_attention_tree_amd import ForestBuilder
    forest_runs = {}
    for cap in (cfg.B * cfg.T, 768):
        f_ms, m_total, packed = time_forest_build(cfg, torch, ForestBuilder, dev, K, cap)
        forest_runs[str(cap)] = {"ms": f_ms, "nodes_packed": packed}
    for s_ in sets:
        assert s_.rnd.error_bits() == 0, "device error bits set"
    dominant, bytes_fn = DOMINANT[args.path]

    nodes = sum(s.forest.N for s in sets) / len(sets)
    value = nodes * cfg.H / (ms_step * 1e-3)
    if args.path == "deferred":
        vbytes = np.mean([commit_tree_verify_algorithmic_bytes(s.sizes, s.prev.forest, cfg.H,
                                                               cfg.d_k, cfg.d_v, e) for s in sets])
    else:
        vbytes = np.mean([bytes_fn(s.sizes, cfg.H, cfg.d_k, cfg.d_v, e) for s in sets])
    achieved = vbytes / (avg[dominant] * 1e-3) / 1e9
    # a plain copy over the same footprint as the rotated input sets
    copy_gbs = copy_bandwidth(torch, dev, int(vbytes * len(sets)), 20)
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
                        + (" (this round's verify with the previous round's accepted-path "
                           "commit inside: one commit and one verify per step)"
                           if args.path == "deferred" else ""),
            "B": cfg.B, "T": cfg.T, "H": cfg.H, "d_k": cfg.d_k, "d_v": cfg.d_v,
            "nodes": nodes, "input_sets": len(sets), "path": args.path,
            "timing": "HIP graph replays: 16 captured steps per graph; kernels: 16 launches per graph",
            "ms_per_step_other_path": ms_other,
            "ms_per_step_eager_launches": ms_eager,
            "kernel_ms_back_to_back": avg,
            "tree_verify_depth_cap_16": {
                "note": "sensitivity: the same shape with trees drawn under a depth cap of 16",
                "ms": d16_ms, "deepest_tree": d16_depth,
                "achieved_GBs": d16_bytes / (d16_ms * 1e-3) / 1e9,
                "frac_of_hbm_peak": d16_bytes / (d16_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            },
            "stage1_tree_conv": {
                "note": "first pipeline stage: the short causal convolution over each node's "
                        "ancestors, with bias and SiLU; not part of the step",
                "channels": W.conv_channels(cfg), "width": W.CONV_WIDTH, "ms": conv_ms,
                "achieved_GBs": conv_bytes / (conv_ms * 1e-3) / 1e9,
                "frac_of_hbm_peak": conv_bytes / (conv_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                "algorithmic_bytes_per_launch": conv_bytes,
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
            "copy_GBs": copy_gbs,
            "frac_of_copy": achieved / copy_gbs,
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, 0, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

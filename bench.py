"""Throughput of closed-form tree verification for one GDN layer on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
tree preparation (topology + log-space gate products), the G/C factor producer,
value-tiled verify and the accepted-path commit.  Default workload: 16 requests,
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
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "verify_target_counters.json")
KERNEL_SOURCES = [os.path.join(ROOT, "linear_attention_tree_amd", "csrc", f)
                  for f in ("verify.hip", "common.h")]


def verify_algorithmic_bytes(sizes, H, d_k, d_v, e):
    """Compulsory HBM bytes of one verify launch: S_pre read once; q, k, v, logP,
    beta read once; O (token dtype) and U (float32) written once."""
    per_node = 2 * e * d_k + e * d_v + 8 + e * d_v + 4 * d_v
    return int(sum(H * (4 * d_k * d_v + T * per_node) for T in sizes))


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(expected_hash):
    try:
        d = json.load(open(PROFILE_COUNTERS))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_hash") != expected_hash:
        return None
    return d.get("hbm_bytes_per_launch")


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


def run_step(s, bole, events=None):
    """prep -> factor -> verify -> commit on the current stream."""
    t = s.rnd.topo
    if events:
        events[0].record()
    bole.bole_tree_prep(t.parent, t.tree_off, s.g, t.depth, t.anc, t.order, t.tree_depth,
                        s.logP, s.rnd.err)
    if events:
        events[1].record()
    lp = s.logP[0]
    bole.bole_factor_gc(s.q, s.k, lp, s.beta, t.anc, t.tree_off, s.rnd.G, s.rnd.C, s.rnd.err)
    if events:
        events[2].record()
    bole.bole_verify(s.q, s.k, s.v, lp, s.beta, s.pool, s.slot, s.rnd.G, s.rnd.C, t.anc, t.depth,
                     t.tree_off, t.tree_depth, s.O, s.U, s.rnd.err)
    if events:
        events[3].record()
    bole.bole_commit_path(s.pool, s.slot, s.k, s.U, lp, t.anc, t.tree_off, s.accept, s.rnd.err)
    if events:
        events[4].record()


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
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.tree_prep(f.parent, f.tree_off, x.g[None])
        oracle.verify(f.parent, f.tree_off, x.q64, x.k64, x.v64, x.g64, x.beta64, S, slot,
                      f.accept, nthreads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 1000:
            break
    rate = reps * f.N * cfg.H / el
    return {"value": rate, "unit": "node-heads/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} full repetitions of the workload's layer (prep + walk + commit, "
                      f"{f.N} nodes x {cfg.H} heads, float64) in {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="target", choices=sorted(W.CONFIGS))
    ap.add_argument("--sets", type=int, default=4, help="rotated independent input sets")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    args = ap.parse_args()
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
        cfg = W.Config(**{**cfg.__dict__, "L": 1})
    sets = [InputSet(cfg, seed, torch, TreeRound, dev) for seed in range(args.sets)]
    e = 2 if cfg.dtype == "bf16" else 4

    for i in range(args.warmup):
        run_step(sets[i % len(sets)], bole)
    torch.cuda.synchronize()
    for s in sets:
        assert s.rnd.error_bits() == 0, "device error bits set"

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(K):
        run_step(sets[i % len(sets)], bole, ev[i])
    t_stop.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_stop)
    ms_step = total_ms / K
    per = np.array([[ev[i][j].elapsed_time(ev[i][j + 1]) for j in range(4)] for i in range(K)])
    avg = per.mean(axis=0)          # prep, factor, verify, commit (ms)

    nodes = sum(s.forest.N for s in sets) / len(sets)
    value = nodes * cfg.H / (ms_step * 1e-3)
    vbytes = np.mean([verify_algorithmic_bytes(s.sizes, cfg.H, cfg.d_k, cfg.d_v, e) for s in sets])
    achieved = vbytes / (avg[2] * 1e-3) / 1e9
    traffic = traffic_from_profile(kernel_source_hash())

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
                        "f32 gates and state; step = tree_prep + factor_gc + verify + commit",
            "B": cfg.B, "T": cfg.T, "H": cfg.H, "d_k": cfg.d_k, "d_v": cfg.d_v,
            "nodes": nodes, "input_sets": len(sets),
            "kernel_ms": {"tree_prep": avg[0], "factor_gc": avg[1], "verify": avg[2],
                          "commit": avg[3]},
            "layer_ms_factor_plus_verify": avg[1] + avg[2],
        },
        "roofline": {
            "kernel": "bole_verify",
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": vbytes,
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, 0, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of one ZHA layer's decode step on one MI355X.

A step is one pass of the whole hot path for one new token: append (KV row
write plus the summaries it completes) and a decode step (per-level routing
from the top of the tree down, then exact attention over the selected raw
tokens, the sink and the tail).  The default workload is the light router
(4 KV / 32 query heads, d 128, bf16, 262,144 cached tokens, R 1, chunk 8,
4 levels, p 0.75) with 256 appended+decoded tokens; inputs are seeded
synthetic caches resident in HBM before the timed region.

Prints one JSON line.  `--sweep` adds the latency-vs-context curve
(16K .. 10M tokens, light shape) against dense decode, one JSON line per point.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

METRIC = "ZHA single-layer decode µs/step (batch 1) vs context length; HBM GB/s % peak"
HBM_PEAK_GBS = 8000.0


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="light")
    ap.add_argument("--sweep", action="store_true", help="also run the 16K..10M context sweep")
    ap.add_argument("--sweep-points", default="16384,32768,65536,131072,262144,524288,1048576,2097152,4194304,10485760")
    ap.add_argument("--sweep-steps", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle CPU baseline")
    ap.add_argument("--out", default=None, help="also append the JSON line(s) to this file")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration) and exit")
    return ap.parse_args()


ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "zha_attn_kernel_light_traffic.txt")
ATTN_SOURCES = [os.path.join(ROOT, "hierarchical_tree_indexed_zha_amd", "csrc", f)
                for f in ("zha_attn.hip", "zha_common.h", "zha_internal.h")]


def attn_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per launch of the gather kernel from the committed FETCH_SIZE /
    WRITE_SIZE counter passes (copy-calibrated), or None when they are missing,
    were taken on another workload, or the kernel source changed since."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith((" ", "#", "$")):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("workload") != workload or kv.get("source_digest") != attn_source_digest():
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def copy_calibration(nbytes: int, reps: int):
    """A plain device-to-device copy of nbytes, reps times: the reference kernel
    whose FETCH_SIZE / WRITE_SIZE counters calibrate the gather kernel's."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


def head_tokens(route1, g, hl, n_tokens, c):
    """Distinct tokens head hl of group g attends: its kept chunks, the sink if not among them, the tail."""
    nk = int(route1["n_kept"][g])
    kept = route1["kept"][g, :nk]
    mine = ((route1["mask"][g, :nk] >> hl) & 1) == 1
    n_mine = int(mine.sum())
    kept0 = n_mine > 0 and bool(mine[0]) and int(kept[0]) == 0
    n1 = n_tokens // c
    return n_mine * c + (0 if (kept0 or n1 == 0) else 1) + (n_tokens - c * n1)


def union_tokens(route1, g, n_tokens, c):
    """Distinct tokens the gather reads for group g: kept chunks, the sink if not among them, the tail."""
    nk = int(route1["n_kept"][g])
    kept0 = nk > 0 and int(route1["kept"][g, 0]) == 0
    n1 = n_tokens // c
    return nk * c + (0 if (kept0 or n1 == 0) else 1) + (n_tokens - c * n1)


def run_steps(layer, x, w, n0, steps, append, decode=True, offset=0):
    for t in range(steps):
        i = (offset + t) % x["q"].shape[0]
        if append:
            layer.append(x["k_app"][i], x["v_app"][i])
        if decode:
            layer.decode(x["q"][i])


def timed(fn, torch):
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def bench_workload(args, torch, W, B, ZhaLayer):
    base = W.get(args.workload)
    total = args.warmup + args.steps
    w = dataclasses.replace(base, steps=max(base.steps, total))
    c, d = w.chunk, w.head_dim
    e_kv = 2 if w.kv_dtype == "bf16" else 4
    _log(f"[bench] generating {w.name}: N={w.n_tokens} H_kv={w.n_kv_heads} H_q={w.n_q_heads} c={c} L={w.levels} "
         f"R={w.n_ref} p={w.top_p} append={w.append}")
    x = W.generate(w, device="cuda")
    cfg = B.config_of(w)
    layer = ZhaLayer(cfg, x["k"], x["v"], x["ref_q"])
    N = w.n_tokens

    t_build = timed(lambda: layer.build(N), torch)
    _log(f"[bench] build {t_build * 1e3:.2f} ms")

    # warm-up steps, then rewind: appends overwrite the same rows and nodes again
    run_steps(layer, x, w, N, args.warmup, w.append)
    torch.cuda.synchronize()
    layer.n_tokens = N

    # timed: append + decode per step
    t_step = timed(lambda: run_steps(layer, x, w, N, args.steps, w.append), torch)
    us_step = t_step / args.steps * 1e6
    _log(f"[bench] step (append+decode) {us_step:.1f} us")

    # decode only and append only, same cache
    layer.n_tokens = N
    t_dec = timed(lambda: run_steps(layer, x, w, N, args.steps, False), torch)
    us_dec = t_dec / args.steps * 1e6
    us_app = None
    if w.append:
        layer.n_tokens = N
        us_app = timed(lambda: run_steps(layer, x, w, N, args.steps, True, decode=False), torch) / args.steps * 1e6
    layer.n_tokens = N

    # dense baseline at the same context
    for _ in range(4):
        layer.dense(x["q"][0])
    t_dense = timed(lambda: [layer.dense(x["q"][t % x["q"].shape[0]]) for t in range(args.steps)], torch)
    us_dense = t_dense / args.steps * 1e6
    _log(f"[bench] decode-only {us_dec:.1f} us, append-only {us_app} us, dense {us_dense:.1f} us")

    # Phase timing: the timed append+decode steps replayed from N with HIP events
    # on the decode stream: before routing, at the start and end of the gather
    # kernel (recorded by its dispatch) and after the combine; no host
    # synchronisation inside the replay.
    layer.n_tokens = N
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    stream = torch.cuda.current_stream()
    for row in evs:
        for e in row:
            e.record(stream)          # creates the underlying HIP events
    torch.cuda.synchronize()
    for t in range(args.steps):
        i = t % x["q"].shape[0]
        if w.append:
            layer.append(x["k_app"][i], x["v_app"][i])
        B.zha_decode_step_timed(cfg, layer.bufs, layer.n_tokens, x["q"][i], layer.out,
                                [e.cuda_event for e in evs[t]])
    torch.cuda.synchronize()
    route_ms = sum(r[0].elapsed_time(r[1]) for r in evs)
    gather_ms = sum(r[1].elapsed_time(r[2]) for r in evs)
    comb_ms = sum(r[2].elapsed_time(r[3]) for r in evs)
    step_us = sorted(r[0].elapsed_time(r[3]) * 1e3 for r in evs)      # each decode between its first and last event
    dec_med_us = step_us[len(step_us) // 2]

    # Algorithmic bytes of the same steps: replayed once more, reading each step's
    # kept lists on the host (the selection is deterministic).
    layer.n_tokens = N
    gather_bytes = router_bytes = 0
    keys_read = []
    keys_head = []
    R = w.n_ref
    for t in range(args.steps):
        i = t % x["q"].shape[0]
        if w.append:
            layer.append(x["k_app"][i], x["v_app"][i])
        layer.decode(x["q"][i])
        torch.cuda.synchronize()
        n = layer.n_tokens
        r1 = layer.route_level(1)
        ut = [union_tokens(r1, g, n, c) for g in range(w.n_kv_heads)]
        gather_bytes += sum(ut) * 2 * d * e_kv
        keys_read.append(sum(ut) / (w.n_kv_heads * n))
        G = w.n_q_heads // w.n_kv_heads
        keys_head.append(sum(head_tokens(r1, g, hl, n, c) for g in range(w.n_kv_heads) for hl in range(G))
                         / (w.n_q_heads * n))
        for lv in range(1, w.levels + 1):
            if n // c ** lv:
                router_bytes += int(layer.route_level(lv)["n_cand"].sum()) * R * (d + 1) * 4
    layer.n_tokens = N
    K = args.steps
    gather_us = gather_ms / K * 1e3
    route_us = route_ms / K * 1e3
    gather_gbs = gather_bytes / K / (gather_us * 1e-6) / 1e9
    router_gbs = router_bytes / K / (route_us * 1e-6) / 1e9
    dense_bytes = w.n_kv_heads * N * 2 * d * e_kv
    _log(f"[bench] phases: route {route_us:.1f} us ({router_gbs:.0f} GB/s alg), gather {gather_us:.1f} us "
         f"({gather_gbs:.0f} GB/s alg), combine {comb_ms / K * 1e3:.1f} us; keys read {sum(keys_read) / K:.4f}")
    traffic = read_traffic(w.name)

    result = {
        "metric": METRIC,
        "value": round(us_step, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_step / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.kv_dtype,
        "data": "synthetic (seeded cluster-needle cache, resident in HBM)",
        "config": {"workload": w.name, "n_tokens": N, "n_kv_heads": w.n_kv_heads, "n_q_heads": w.n_q_heads,
                   "head_dim": d, "chunk": c, "levels": w.levels, "n_ref": R, "top_p": w.top_p,
                   "append_per_step": w.append, "batch": 1},
        "tokens_per_s": round(1e6 / us_step, 1),
        "decode_us": round(us_dec, 3),
        "append_us": None if us_app is None else round(us_app, 3),
        "dense_us": round(us_dense, 3),
        "speedup_vs_dense": round(us_dense / us_dec, 3),
        "keys_read_frac": round(sum(keys_read) / K, 5),
        "keys_read_frac_head_mean": round(sum(keys_head) / K, 5),
        "decode_us_events_median": round(dec_med_us, 3),
        "phase_us": {"route": round(route_us, 3), "gather": round(gather_us, 3),
                     "combine": round(comb_ms / K * 1e3, 3)},
        "router_gbs_alg": round(router_gbs, 1),
        "dense_gbs_alg": round(dense_bytes / (us_dense * 1e-6) / 1e9, 1),
        "build_ms": round(t_build * 1e3, 3),
        "roofline": {"bound": "hbm", "kernel": "zha_attn_kernel<bf16, sparse> (gather)",
                     "achieved": round(gather_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gather_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else int(traffic),
                     "bytes_per_launch": int(gather_bytes / K), "avg_launch_us": round(gather_us, 3),
                     "traffic_over_alg": None if traffic is None else round(traffic / (gather_bytes / K), 4)},
    }
    return result, layer, x, w


def cpu_baseline(args, layer, x, w, torch):
    """The fp64 oracle on a bounded sample of the same workload: append + decode steps
    over a tree precomputed outside the timed region (as the GPU's build is)."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    N = w.n_tokens
    kh = x["k"].cpu().view(torch.int16).numpy().view(np.uint16).copy() if w.kv_dtype == "bf16" else x["k"].cpu().numpy().copy()
    vh = x["v"].cpu().view(torch.int16).numpy().view(np.uint16).copy() if w.kv_dtype == "bf16" else x["v"].cpu().numpy().copy()
    conv = (lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16)) if w.kv_dtype == "bf16" else (lambda t: t.cpu().numpy())
    tree = O.SummaryTree(kh, x["ref_q"].cpu().numpy(), N, w.chunk, w.levels)
    t0 = time.perf_counter()
    for lv in range(1, w.levels + 1):
        for g in range(w.n_kv_heads):
            tree.get(lv, g, np.arange(tree.n_nodes(lv)))
    t_pre = time.perf_counter() - t0
    _log(f"[cpu] oracle tree precompute {t_pre:.1f} s")
    n = N
    done, elapsed = 0, 0.0
    while done < 64 and (elapsed < args.cpu_seconds or done < 1):
        i = done % x["q"].shape[0]
        qh = conv(x["q"][i])
        t0 = time.perf_counter()
        if w.append:
            n, _ = O.append_token(kh, vh, tree, n, conv(x["k_app"][i]), conv(x["v_app"][i]))
        O.decode_step(qh, kh, vh, tree, w.top_p)
        elapsed += time.perf_counter() - t0
        done += 1
    us = elapsed / done * 1e6
    _log(f"[cpu] oracle {done} steps, {us / 1e3:.1f} ms/step, threads {threads}")
    # the same steps again on one core (BLAS limited to one thread), a third of the budget
    us1, done1 = None, 0
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            elapsed1 = 0.0
            while done1 < done and (elapsed1 < args.cpu_seconds / 3 or done1 < 1):
                i = done1 % x["q"].shape[0]
                t0 = time.perf_counter()
                O.decode_step(conv(x["q"][i]), kh, vh, tree, w.top_p)
                elapsed1 += time.perf_counter() - t0
                done1 += 1
        us1 = elapsed1 / done1 * 1e6
        _log(f"[cpu] oracle on one core: {done1} decode steps, {us1 / 1e3:.1f} ms/step")
    except Exception as e:
        _log(f"[cpu] one-core timing skipped: {e}")
    return {"value": round(us, 1), "unit": "us/step", "cores": threads, "kind": "oracle",
            "value_one_core": None if us1 is None else round(us1, 1),
            "sample": f"{done} append+decode steps of {w.name} (N={N}) after an untimed fp64 tree "
                      f"precompute of {t_pre:.1f} s; host cores available {os.cpu_count()}; "
                      f"value_one_core: {done1} decode steps with BLAS on one thread"}


def sweep(args, torch, W, B, ZhaLayer):
    base = W.get("light")
    lines = []
    for n in [int(v) for v in args.sweep_points.split(",")]:
        L = W.levels_for(n, base.chunk)
        w = dataclasses.replace(base, name=f"light@{n}", n_tokens=n, levels=L, steps=args.sweep_steps, append=False)
        _log(f"[sweep] N={n} L={L}")
        x = W.generate(w, device="cuda")
        layer = ZhaLayer(B.config_of(w), x["k"], x["v"], x["ref_q"])
        layer.build(n)
        for t in range(4):
            layer.decode(x["q"][t % w.steps])
            layer.dense(x["q"][t % w.steps])
        K = args.sweep_steps
        us_z = timed(lambda: [layer.decode(x["q"][t % w.steps]) for t in range(K)], torch) / K * 1e6
        us_d = timed(lambda: [layer.dense(x["q"][t % w.steps]) for t in range(K)], torch) / K * 1e6
        r1 = layer.route_level(1)
        kr = sum(union_tokens(r1, g, n, w.chunk) for g in range(w.n_kv_heads)) / (w.n_kv_heads * n)
        line = {"sweep": "light", "n_tokens": n, "levels": L, "zha_decode_us": round(us_z, 2),
                "dense_decode_us": round(us_d, 2), "speedup_vs_dense": round(us_d / us_z, 3),
                "keys_read_frac": round(kr, 5),
                "dense_gbs_alg": round(w.n_kv_heads * n * 2 * w.head_dim * 2 / (us_d * 1e-6) / 1e9, 1)}
        _log(json.dumps(line))
        lines.append(line)
        del layer, x
        torch.cuda.empty_cache()
    return lines


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the library has no multi-GPU path (one GPU holds the whole cache at these sizes).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 4)
        return
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from hierarchical_tree_indexed_zha_amd import binding as B
    from hierarchical_tree_indexed_zha_amd import workloads as W
    from hierarchical_tree_indexed_zha_amd.runtime import ZhaLayer
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    B.lib()
    result, layer, x, w = bench_workload(args, torch, W, B, ZhaLayer)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, layer, x, w, torch)
    del layer
    torch.cuda.empty_cache()
    lines = [result]
    if args.sweep:
        result["sweep"] = sweep(args, torch, W, B, ZhaLayer)
    line = json.dumps(result)
    print(line, flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()

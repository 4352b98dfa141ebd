#!/usr/bin/env python3
"""Benchmark of one ZHA layer's decode step on one MI355X.

A step is one pass of the whole hot path for one new token: append (KV row
write plus the summaries it completes) and a decode step (per-level routing
from the top of the tree down, then exact attention over the selected raw
tokens, the sink and the tail).  The default workload is the light router
(4 KV / 32 query heads, d 128, bf16, 262,144 cached tokens, R 1, chunk 8,
4 levels, p 0.75) with 256 appended+decoded tokens; inputs are seeded
synthetic caches resident in HBM before the timed region.

Prints one JSON line: the light workload's step, a per-kernel event trace of the
router, a cold-cache variant of the gather (1 GiB written between steps), the
oracle timed on the host cores on a bounded sample, the latency-vs-context curve
(16K .. 10M tokens, light shape) against dense decode and the ultra-long point
(10,485,760 tokens with appends).  `--geometry` instead sweeps (chunk, levels, R,
p) at 262,144 tokens.
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
    ap.add_argument("--no-sweep", action="store_true", help="skip the 16K..10M context sweep and the ultra point")
    ap.add_argument("--sweep-points", default="16384,65536,262144,1048576,4194304,10485760")
    ap.add_argument("--sweep-steps", type=int, default=16)
    ap.add_argument("--ultra-steps", type=int, default=64)
    ap.add_argument("--trace-steps", type=int, default=32, help="steps of the per-kernel event trace")
    ap.add_argument("--cold-steps", type=int, default=32, help="steps of the cold-cache gather variant")
    ap.add_argument("--flush-bytes", type=int, default=1 << 30, help="bytes written between cold steps")
    ap.add_argument("--geometry", action="store_true", help="only run the (c, L, R, p) geometry sweep")
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
    bd = build_device(layer, N, w, torch)
    _log(f"[bench] build {t_build * 1e3:.2f} ms (device {bd['us']:.1f} us, {bd['gbs']:.0f} GB/s alg)")

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
    app_dev = None
    if w.append:
        layer.n_tokens = N
        us_app = timed(lambda: run_steps(layer, x, w, N, args.steps, True, decode=False), torch) / args.steps * 1e6
    layer.n_tokens = N

    # dense baseline at the same context
    for _ in range(4):
        layer.dense(x["q"][0])
    t_dense = timed(lambda: [layer.dense(x["q"][t % x["q"].shape[0]]) for t in range(args.steps)], torch)
    us_dense = t_dense / args.steps * 1e6
    if w.append:
        layer.n_tokens = N
        app_dev = append_device(layer, x, args.steps, torch, us_dense)
        layer.n_tokens = N
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

    # Algorithmic bytes of the same steps: replayed once more with the step's device
    # stats (the selection is deterministic) and the level-1 kept lists on the host.
    layer.n_tokens = N
    gather_bytes = router_bytes = 0
    keys_read = []
    keys_head = []
    stats = layer.new_stats()
    G = w.n_q_heads // w.n_kv_heads
    R = w.n_ref
    for t in range(args.steps):
        i = t % x["q"].shape[0]
        if w.append:
            layer.append(x["k_app"][i], x["v_app"][i])
        layer.decode(x["q"][i], stats=stats)
        st = layer.read_stats(stats)
        n = layer.n_tokens
        gather_bytes += st["gather_bytes"]
        router_bytes += sum(st["bytes_streamed"])
        keys_read.append(st["gather_tokens"] / (w.n_kv_heads * n))
        r1 = layer.route_level(1)
        keys_head.append(sum(head_tokens(r1, g, hl, n, c) for g in range(w.n_kv_heads) for hl in range(G))
                         / (w.n_q_heads * n))
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
        "build_device": bd,
        "append_device": app_dev,
        "roofline": {"bound": "hbm", "kernel": "zha_attn_kernel<bf16, sparse> (gather)",
                     "achieved": round(gather_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gather_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else int(traffic),
                     "bytes_per_launch": int(gather_bytes / K), "avg_launch_us": round(gather_us, 3),
                     "traffic_over_alg": None if traffic is None else round(traffic / (gather_bytes / K), 4)},
    }
    return result, layer, x, w


def build_device(layer, N, w, torch, reps=3):
    """The tree build's device time (HIP events around zha_build_tree, best of reps) and its
    algorithmic bytes: the keys read once, every level's planes (s, b, lse) written, and
    the child planes each merge launch reads (none at level 2 where the leaf kernel
    writes the level-2 nodes itself: 4 <= R <= 16 with c in {2, 4})."""
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        layer.build(N)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    us = min(ts)
    H, d, R, c = w.n_kv_heads, w.head_dim, w.n_ref, w.chunk
    e_kv = 2 if w.kv_dtype == "bf16" else 4
    node = R * (d + 2) * 4
    byts = H * N * d * e_kv
    fused = 4 <= R <= 16 and c in (2, 4)
    for lv in range(1, w.levels + 1):
        n = N // c ** lv
        byts += H * n * node                      # written
        if lv > 2 or (lv == 2 and not fused):
            byts += H * n * c * node              # children read by the merge
    return {"us": round(us, 2), "alg_bytes": int(byts), "gbs": round(byts / (us * 1e-6) / 1e9, 1)}


def append_device(layer, x, steps, torch, dense_us):
    """Device time of each append (HIP events around zha_append_token: the KV row write and,
    when a chunk completes, its leaf summary and the merges above it), mean and max.
    Dense decodes queued first keep the device busy while the host issues the appends
    (about 60 us of host time each with their events), so that each event pair brackets
    the append's own kernels rather than the device waiting for the host."""
    rows = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    nq = x["q"].shape[0]
    N = layer.n_tokens
    for _ in range(max(1, math.ceil(steps * 60.0 / max(dense_us, 1.0)))):
        layer.dense(x["q"][0])
    for t in range(steps):
        rows[t][0].record()
        layer.append(x["k_app"][t % nq], x["v_app"][t % nq])
        rows[t][1].record()
    torch.cuda.synchronize()
    layer.n_tokens = N
    us = [a.elapsed_time(b) * 1e3 for a, b in rows]
    return {"mean_us": round(sum(us) / len(us), 3), "max_us": round(max(us), 3), "steps": steps}


EXEMPT_MARGIN = 1e-4    # cumulative-mass margin below which a cut has several correct answers


def cpu_model():
    """The host CPU's model name (first processor of /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


_PROC = {}    # the forked workers' view of the oracle state (inherited, never sent)


def _group_decode(job):
    """Oracle decode of one KV group's query heads in a worker process: (group, output rows)."""
    import numpy as np
    import oracle as O
    g, qh = job
    st = _PROC
    q = O.widen(qh)
    G = q.shape[0] // st["n_kv"]
    rows = []
    for h in range(g * G, (g + 1) * G):
        r = O.route_head(q[h], st["tree"], g, st["p"])
        rows.append(O.attend(q[h], st["kh"][g], st["vh"][g], r.tokens, st["tree"].tau))
    return g, np.stack(rows)


def cpu_procs(args, x, w, conv, kh, vh, tree):
    """The oracle's decode on every host core: one forked worker process per KV group (the
    oracle state inherited copy-on-write), each with its share of the BLAS threads; a
    bounded sample of decode steps at the sample's final context.  None if it fails."""
    import multiprocessing as mp
    ncpu = os.cpu_count() or 1
    nproc = max(1, min(w.n_kv_heads, ncpu))
    _PROC.update(tree=tree, kh=kh, vh=vh, p=w.top_p, n_kv=w.n_kv_heads)
    pool = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=max(1, ncpu // nproc)):
            pool = mp.get_context("fork").Pool(nproc)
        done, elapsed = 0, 0.0
        while done < 16 and (elapsed < args.cpu_seconds / 3 or done < 1):
            qh = conv(x["q"][done % x["q"].shape[0]])
            t0 = time.perf_counter()
            pool.map_async(_group_decode, [(g, qh) for g in range(w.n_kv_heads)]).get(timeout=120)
            elapsed += time.perf_counter() - t0
            done += 1
        return {"value": round(elapsed / done * 1e6, 1), "processes": nproc,
                "threads_per_process": max(1, ncpu // nproc), "steps": done}
    except Exception as e:
        _log(f"[cpu] per-group processes skipped: {e!r}")
        return None
    finally:
        if pool is not None:
            pool.terminate()
            pool.join()
        _PROC.clear()


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
    exempt, pairs = 0, 0
    while done < 64 and (elapsed < args.cpu_seconds or done < 1):
        i = done % x["q"].shape[0]
        qh = conv(x["q"][i])
        t0 = time.perf_counter()
        if w.append:
            n, _ = O.append_token(kh, vh, tree, n, conv(x["k_app"][i]), conv(x["v_app"][i]))
        _, routes = O.decode_step(qh, kh, vh, tree, w.top_p)
        elapsed += time.perf_counter() - t0
        done += 1
        # (head, step) pairs with a cut margin below the tie bar: either side of that
        # cut is a correct answer, so their leaf sets are exempt from identity
        exempt += sum(1 for r in routes if r.min_margin < EXEMPT_MARGIN)
        pairs += len(routes)
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
    procs = cpu_procs(args, x, w, conv, kh, vh, tree)
    if procs:
        _log(f"[cpu] oracle decode, one process per KV group: {procs['value'] / 1e3:.1f} ms/step")
    return {"value": round(us, 1), "unit": "us/step", "cores": threads, "kind": "oracle",
            "value_one_core": None if us1 is None else round(us1, 1), "cpu_model": cpu_model(),
            "decode_processes": procs,
            "exempt_heads": {"count": exempt, "of": pairs, "margin": EXEMPT_MARGIN},
            "sample": f"{done} append+decode steps of {w.name} (N={N}) after an untimed fp64 tree "
                      f"precompute of {t_pre:.1f} s; host cores available {os.cpu_count()}; "
                      f"value_one_core: {done1} decode steps with BLAS on one thread"}


def _events(torch, n):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    st = torch.cuda.current_stream()
    for e in evs:
        e.record(st)          # creates the underlying HIP events
    torch.cuda.synchronize()
    return evs


def trace_kernels(args, layer, x, w, torch, B):
    """Per-kernel device time of decode steps (an event after every kernel, on the
    step's stream) and each kernel's algorithmic bytes from the step's own stats
    (the same query decoded again with stats: the routing is deterministic)."""
    N, c, G = layer.n_tokens, w.chunk, w.n_q_heads // w.n_kv_heads
    evs = _events(torch, 40)
    handles = [e.cuda_event for e in evs]
    stats = layer.new_stats()
    acc = {}
    K = args.trace_steps
    for t in range(K):
        q = x["q"][t % x["q"].shape[0]]
        kinds = B.zha_decode_step_traced(layer.cfg, layer.bufs, N, q, layer.out, handles)
        torch.cuda.synchronize()
        layer.decode(q, stats=stats)
        st = layer.read_stats(stats)
        kinds_l = [k for k in kinds]
        crossed = {lv for k, lv in kinds_l if k == "cross"}
        chain_lv = []
        if any(k == "chain" for k, _ in kinds_l):
            top = kinds_l[0][1]
            scored = [lv for k, lv in kinds_l if k == "score"]
            low = (max(scored) + 1) if scored else 1
            chain_lv = list(range(low, top + 1))
        # the first level below the chain, when the chain launch scored its every node
        # (its streamed bytes then exceed its candidates' bytes)
        spec_lv = None
        if chain_lv and min(chain_lv) > 1:
            lb = min(chain_lv) - 1
            if st["bytes_streamed"][lb - 1] != st["bytes_read"][lb - 1]:
                spec_lv = lb
        for i in range(1, len(kinds_l)):
            name, lv = kinds_l[i]
            us = evs[i - 1].elapsed_time(evs[i]) * 1e3
            if name == "score_all":
                byts = sum(st["bytes_streamed"][l - 1] + (N // c ** l) * w.n_q_heads * 4 for l in chain_lv)
            elif name == "chain":
                byts = sum((N // c ** l) * w.n_q_heads * 4 for l in chain_lv)
                if spec_lv:
                    byts += st["bytes_streamed"][spec_lv - 1] + (N // c ** spec_lv) * w.n_q_heads * 4
            elif name == "score" and lv == spec_lv:
                byts = 2 * st["group_cand"][lv - 1] * G * 4     # node-indexed scores copied to the candidates
            elif name == "score":
                byts = st["bytes_read"][lv - 1] + st["group_cand"][lv - 1] * G * 4
            elif name == "select":
                byts = st["group_cand"][lv - 1] * G * 4
            elif name == "cross":
                byts = st["group_cand"][lv - 1] * G * 4
            elif name == "resolve":
                byts = 0
            elif name == "apply":
                # the heads' kept bitmaps (G bits per candidate), or with the cross launch
                # their scores; the kept list written
                per = G * 4 if lv in crossed else G / 8
                byts = st["group_cand"][lv - 1] * per + st["group_kept"][lv - 1] * 8
            elif name == "gather":
                byts = st["gather_bytes"]
            else:
                byts = None
            key = f"{name} L{lv}" if name in ("score", "select", "cross", "resolve", "apply") else name
            a = acc.setdefault(key, {"us": 0.0, "bytes": 0, "n": 0, "counted": byts is not None})
            a["us"] += us
            a["n"] += 1
            if byts is not None:
                a["bytes"] += byts
    out = []
    for key, a in acc.items():
        us = a["us"] / a["n"]
        row = {"kernel": key, "us": round(us, 3)}
        if a["counted"]:
            byts = a["bytes"] / a["n"]
            row["alg_bytes"] = int(byts)
            row["gbs"] = round(byts / (us * 1e-6) / 1e9, 1)
            row["frac"] = round(byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        out.append(row)
    return out


def cold_gather(args, layer, x, w, torch, B):
    """Decode steps with args.flush_bytes written to a scratch buffer before each (outside
    the step's events): the 256 MB Infinity Cache and the L2s hold none of the cache's
    rows when the gather starts.  Returns the gather kernel's and the step's device time."""
    N = layer.n_tokens
    flush = torch.empty(args.flush_bytes, dtype=torch.uint8, device="cuda")
    K = args.cold_steps
    if K < 1:
        return None
    rows = [_events(torch, 4) for _ in range(K)]
    stats = layer.new_stats()
    gb = 0
    for t in range(K):
        q = x["q"][t % x["q"].shape[0]]
        flush.fill_(t & 255)
        B.zha_decode_step_timed(layer.cfg, layer.bufs, N, q, layer.out, [e.cuda_event for e in rows[t]])
    torch.cuda.synchronize()
    for t in range(K):
        layer.decode(x["q"][t % x["q"].shape[0]], stats=stats)
        gb += layer.read_stats(stats)["gather_bytes"]
    g_us = sum(r[1].elapsed_time(r[2]) for r in rows) / K * 1e3
    d_us = sum(r[0].elapsed_time(r[3]) for r in rows) / K * 1e3
    del flush
    torch.cuda.empty_cache()
    return {"gather_us": round(g_us, 3), "decode_us": round(d_us, 3),
            "gather_gbs": round(gb / K / (g_us * 1e-6) / 1e9, 1), "flush_bytes": args.flush_bytes}


def fidelity_of(layer, x, steps):
    """Mean over `steps` decode steps and all query heads of the router's per-level
    exact-mass recall and of the attended set's captured mass (zha_route_fidelity)."""
    import numpy as np
    nq = x["q"].shape[0]
    recs = []
    for t in range(steps):
        q = x["q"][t % nq]
        layer.decode(q)
        recs.append(layer.fidelity(q).cpu().numpy())
    r = np.stack(recs).mean(axis=(0, 1))
    L = layer.cfg.levels
    return {"recall_by_level": {f"L{l}": round(float(r[l - 1]), 5) for l in range(1, L + 1)},
            "captured_mass": round(float(r[L]), 5), "steps": steps}


def point(torch, W, B, ZhaLayer, w, steps, dense_steps, append, plane_format=0, fid_steps=0):
    """Decode latency of workload w at its own size against dense, with the route/gather
    split (HIP events), keys read and summary bytes; appends before each step if asked;
    with fid_steps, the router's fidelity over that many steps."""
    x = W.generate(w, device="cuda")
    layer = ZhaLayer(B.config_of(w, plane_format=plane_format), x["k"], x["v"], x["ref_q"])
    n = w.n_tokens
    t0 = time.perf_counter()
    layer.build(n)
    torch.cuda.synchronize()
    build_ms = (time.perf_counter() - t0) * 1e3
    nq = x["q"].shape[0]
    for t in range(4):
        layer.decode(x["q"][t % nq])
        layer.dense(x["q"][t % nq])
    if append:
        run_steps(layer, x, w, n, min(8, steps), True)
        layer.n_tokens = n
    us_z = timed(lambda: run_steps(layer, x, w, n, steps, append), torch) / steps * 1e6
    layer.n_tokens = n
    us_d = timed(lambda: [layer.dense(x["q"][t % nq]) for t in range(dense_steps)], torch) / dense_steps * 1e6
    rows = [_events(torch, 4) for _ in range(min(steps, 16))]
    for t, r in enumerate(rows):
        if append:
            layer.append(x["k_app"][t % nq], x["v_app"][t % nq])
        B.zha_decode_step_timed(layer.cfg, layer.bufs, layer.n_tokens, x["q"][t % nq], layer.out,
                                [e.cuda_event for e in r])
    torch.cuda.synchronize()
    route = sum(r[0].elapsed_time(r[1]) for r in rows) / len(rows) * 1e3
    gather = sum(r[1].elapsed_time(r[2]) for r in rows) / len(rows) * 1e3
    stats = layer.new_stats()
    layer.decode(x["q"][0], stats=stats)
    st = layer.read_stats(stats)
    H = w.n_kv_heads
    line = {"n_tokens": n, "levels": w.levels, "chunk": w.chunk, "n_ref": w.n_ref, "top_p": w.top_p,
            "zha_decode_us": round(us_z, 2), "dense_decode_us": round(us_d, 2),
            "speedup_vs_dense": round(us_d / us_z, 3), "route_us": round(route, 2), "gather_us": round(gather, 2),
            "keys_read_frac": round(st["gather_tokens"] / (H * layer.n_tokens), 5),
            "router_bytes": int(sum(st["bytes_streamed"])),
            "dense_gbs_alg": round(H * layer.n_tokens * 2 * w.head_dim * (2 if w.kv_dtype == "bf16" else 4)
                                   / (us_d * 1e-6) / 1e9, 1),
            "build_ms": round(build_ms, 2)}
    line["build_device"] = build_device(layer, n, w, torch, reps=2)
    if append:
        layer.n_tokens = n
    if plane_format:
        line["plane_format"] = {v: k for k, v in B.PLANE_FORMATS.items()}[plane_format]
    if fid_steps:
        line["fidelity"] = fidelity_of(layer, x, fid_steps)
    del layer, x
    torch.cuda.empty_cache()
    return line


def sweep(args, torch, W, B, ZhaLayer):
    """Light-shape decode latency against dense from 16K to 10M tokens (levels chosen so
    the top level has at most 64 nodes), no appends."""
    base = W.get("light")
    lines = []
    for n in [int(v) for v in args.sweep_points.split(",")]:
        L = W.levels_for(n, base.chunk)
        w = dataclasses.replace(base, name=f"light@{n}", n_tokens=n, levels=L, steps=max(args.sweep_steps, 8),
                                append=False)
        _log(f"[sweep] N={n} L={L}")
        line = point(torch, W, B, ZhaLayer, w, args.sweep_steps, args.sweep_steps, False)
        _log(json.dumps(line))
        lines.append(line)
    return lines


def ultra_point(args, torch, W, B, ZhaLayer):
    """The ultra-long light workload (10,485,760 tokens, 7 levels): append + decode steps."""
    w = dataclasses.replace(W.get("ultra"), steps=max(W.get("ultra").steps, args.ultra_steps))
    _log(f"[ultra] N={w.n_tokens} L={w.levels} steps={args.ultra_steps}")
    line = point(torch, W, B, ZhaLayer, w, args.ultra_steps, 8, True, fid_steps=2)
    line["workload"] = "ultra"
    line["append_per_step"] = True
    _log(json.dumps(line))
    return line


def others(args, torch, W, B, ZhaLayer):
    """deep at full size (route time, keys read, fidelity), and light and wide with
    float32, bfloat16 and 8-bit router planes (router time and bytes, fidelity)."""
    out = {}
    w = dataclasses.replace(W.get("deep"), steps=16, append=False)
    _log("[deep] full size")
    out["deep"] = point(torch, W, B, ZhaLayer, w, 16, 16, False, fid_steps=2)
    planes = {}
    for name in ("light", "wide"):
        w = dataclasses.replace(W.get(name), steps=16, append=False)
        planes[name] = {}
        for fname, fmt in B.PLANE_FORMATS.items():
            _log(f"[planes] {name} plane_format={fname}")
            line = point(torch, W, B, ZhaLayer, w, 16, 16, False, plane_format=fmt, fid_steps=2)
            planes[name][fname] = {k: line[k] for k in (
                "zha_decode_us", "route_us", "gather_us", "router_bytes", "keys_read_frac", "fidelity")}
    out["planes"] = planes
    out["batch"] = batch_points(torch, W, B, ZhaLayer)
    return out


def batch_points(torch, W, B, ZhaLayer, sizes=(1, 2, 4, 8, 16)):
    """light at full size: batches of Q queries routed together (zha_decode_batch),
    device time per batch and per query, against Q single steps."""
    w = dataclasses.replace(W.get("light"), steps=max(sizes), append=False)
    x = W.generate(w, device="cuda")
    layer = ZhaLayer(B.config_of(w), x["k"], x["v"], x["ref_q"])
    layer.build(w.n_tokens)
    out = []
    for nq in sizes:
        q = x["q"][:nq].contiguous()
        for _ in range(3):
            layer.decode_batch(q)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        for _ in range(10):
            layer.decode_batch(q)
        e[1].record()
        for _ in range(10):
            for i in range(nq):
                layer.decode(q[i])
        e[2].record()
        torch.cuda.synchronize()
        tb = e[0].elapsed_time(e[1]) / 10 * 1e3
        ts = e[1].elapsed_time(e[2]) / 10 * 1e3
        out.append({"queries": nq, "batch_us": round(tb, 2), "us_per_query": round(tb / nq, 2),
                    "single_steps_us": round(ts, 2), "speedup_vs_single": round(ts / tb, 3)})
        _log(f"[batch] {out[-1]}")
    del layer, x
    torch.cuda.empty_cache()
    return out


GEOMETRY = [  # (chunk, levels, n_ref, top_p) at 262,144 tokens, light heads and generator
    (4, 8, 1, 0.75), (8, 4, 1, 0.75), (16, 3, 1, 0.75), (32, 2, 1, 0.75), (64, 2, 1, 0.75), (256, 1, 1, 0.75),
    (8, 4, 4, 0.75), (8, 4, 16, 0.75), (4, 6, 16, 0.95), (256, 1, 16, 0.95),
    (8, 4, 1, 0.5), (8, 4, 1, 0.9), (8, 4, 1, 0.95), (8, 4, 1, 0.99),
]


def geometry(args, torch, W, B, ZhaLayer):
    base = W.get("light")
    lines = []
    for c, L, R, p in GEOMETRY:
        w = dataclasses.replace(base, name=f"light-c{c}-L{L}-R{R}-p{p}", chunk=c, levels=L, n_ref=R, top_p=p,
                                steps=16, append=False)
        _log(f"[geometry] c={c} L={L} R={R} p={p}")
        line = point(torch, W, B, ZhaLayer, w, 16, 16, False)
        _log(json.dumps(line))
        lines.append(line)
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
    if args.geometry:
        line = json.dumps({"geometry": geometry(args, torch, W, B, ZhaLayer), "tokens": 262144})
        print(line, flush=True)
        if args.out:
            with open(args.out, "a") as f:
                f.write(line + "\n")
        return
    result, layer, x, w = bench_workload(args, torch, W, B, ZhaLayer)
    kern = trace_kernels(args, layer, x, w, torch, B)
    result["router_kernels"] = [r for r in kern if r["kernel"] not in ("gather", "combine")]
    rt_us = sum(r["us"] for r in result["router_kernels"])
    rt_b = sum(r.get("alg_bytes", 0) for r in result["router_kernels"])
    result["router_roofline"] = {"bound": "latency", "us": round(rt_us, 3), "alg_bytes": rt_b,
                                 "achieved": round(rt_b / (rt_us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                                 "unit": "GB/s", "frac": round(rt_b / (rt_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                 "note": "traced steps, an event after every kernel (its dispatch gap included)"}
    cold = cold_gather(args, layer, x, w, torch, B)
    rf = result["roofline"]
    rf["warm_source"] = "hbm_or_mall"
    if cold is not None:
        rf["achieved_cold"] = cold["gather_gbs"]
        rf["frac_cold"] = round(cold["gather_gbs"] / HBM_PEAK_GBS, 4)
        result["cold"] = cold
        _log(f"[bench] cold gather {cold['gather_us']:.1f} us ({cold['gather_gbs']:.0f} GB/s), "
             f"cold decode {cold['decode_us']:.1f} us")
    _log(f"[bench] router kernels {rt_us:.1f} us")
    result["fidelity"] = {w.name: fidelity_of(layer, x, 4)}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, layer, x, w, torch)
    del layer, x
    torch.cuda.empty_cache()
    if not args.no_sweep:
        oth = others(args, torch, W, B, ZhaLayer)
        result["deep"] = oth["deep"]
        result["fidelity"]["deep"] = oth["deep"]["fidelity"]
        result["planes"] = oth["planes"]
        result["batch"] = oth["batch"]
        result["sweep"] = sweep(args, torch, W, B, ZhaLayer)
        result["ultra"] = ultra_point(args, torch, W, B, ZhaLayer)
        result["fidelity"]["ultra"] = result["ultra"]["fidelity"]
    line = json.dumps(result)
    print(line, flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()

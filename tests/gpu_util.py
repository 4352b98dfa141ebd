"""Shared helpers of the GPU tests: device inputs, host copies for the oracle, comparisons."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle as O
from hierarchical_tree_indexed_zha_amd import binding as B
from hierarchical_tree_indexed_zha_amd import workloads as W
from hierarchical_tree_indexed_zha_amd.runtime import ZhaLayer

# Tolerances.  Selection: leaf sets identical unless a level's cut margin is
# below MARGIN (then either side of the cut is correct).  Attention: max-abs
# ATOL against the oracle on the same selected set (bf16 inputs, fp32
# accumulation).
MARGIN = 1e-4
ATOL = 2e-2
# With bfloat16 router planes a rare element rounds one way on the GPU (from its
# float32 planes) and the other way in the oracle (from float64): a score moves by
# up to tau |q_d| 2**-7 |s_d| for such an element (about 1e-3 for one flip at these
# sizes), so cuts closer than this to changing are either side's.
NARROW_MARGIN = 1e-2
# With 8-bit planes a flipped element moves a score by up to tau |q_d| 2**-3 |s_d|
# (one E4M3 spacing), about ten times the bfloat16 figure.
FP8_MARGIN = 3e-2
# Routing checks on the GPU's own candidate sets: scores (relative to 1 + |sigma|),
# cumulative mass, and the ordering of kept vs dropped probabilities.  fp32 scores
# and sums carry ~1e-6 relative error.
SCORE_RTOL = 1e-4
MASS_TOL = 1e-5
ORDER_RTOL = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_host(t: torch.Tensor) -> np.ndarray:
    """Exact host copy for the oracle: bf16 as raw uint16 bits, fp32 as float32."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def make_layer(w: W.Workload, device="cuda", seed=None, top_p=None, capacity=None, plane_format=0):
    x = W.generate(w, device=device, seed=seed)
    cfg = B.config_of(w, capacity=capacity if capacity is not None else w.capacity, plane_format=plane_format)
    if top_p is not None:
        cfg.top_p = top_p
    layer = ZhaLayer(cfg, x["k"], x["v"], x["ref_q"])
    return layer, x


def oracle_tree(layer: ZhaLayer, n_tokens: int, keys_host=None):
    kh = to_host(layer.k) if keys_host is None else keys_host
    fmt = {v: k for k, v in B.PLANE_FORMATS.items()}[layer.cfg.plane_format]
    return kh, O.SummaryTree(kh, to_host(layer.ref_q), n_tokens, layer.cfg.chunk, layer.cfg.levels, plane_format=fmt)


PLANE_REL = 2e-5   # the GPU's float32 planes against the oracle's, relative to the plane's largest element


def narrow_tolerance(q, s, tree) -> np.ndarray:
    """s: the candidates' exact (unrounded) planes.  Per candidate, how far the GPU's score may sit from the oracle's when the router
    reads narrow planes.  The GPU rounds its float32 planes, the oracle its float64
    ones; they differ by at most PLANE_REL times the plane's largest element (the
    tree summaries' bar), and rounding is monotone, so the GPU's narrow element lies
    between the roundings of the two ends of that interval, as does the oracle's: the
    width of that bracket is the element's possible difference (zero unless the
    element sits next to a rounding boundary).  For 8-bit planes whose scale could
    differ between the two ends, every element may move by a spacing at the coarser
    scale (at most 2**-3 |s_d|, or 2**-9 times the scale below the smallest normal).
    The score moves by tau sum_d |q_d| times those differences, maximised over
    planes.  Zero for float32 planes."""
    fmt = getattr(tree, "plane_format", "f32")
    if fmt == "f32" or s is None or len(s) == 0:
        return np.zeros(0 if s is None else len(s))
    qa = np.abs(O.widen(q))
    m = np.abs(s).max(axis=-1, keepdims=True) * PLANE_REL
    lo, hi = s - m, s + m
    if fmt == "bf16":
        step = np.abs(O.round_bf16(hi) - O.round_bf16(lo))
    else:
        m0 = np.abs(s).max(axis=-1)
        k0 = O.fp8_plane_scale_exp(m0[..., None] * (1 - PLANE_REL))
        k1 = O.fp8_plane_scale_exp(m0[..., None] * (1 + PLANE_REL))
        step = np.abs(O.round_fp8(hi, k0) - O.round_fp8(lo, k0))
        loose = np.maximum(np.abs(s) * 2.0 ** -3, np.ldexp(1.0, k1[..., None] - 8))
        step = np.where((k0 != k1)[..., None], loose, step)
    return tree.tau * (qa[None, None, :] * step).sum(-1).max(-1)


def _kept_by_head(route, g, G):
    nk = int(route["n_kept"][g])
    nodes = route["kept"][g, :nk].numpy().astype(np.int64)
    masks = route["mask"][g, :nk].numpy().astype(np.int64)
    return [nodes[(masks >> hl) & 1 == 1] for hl in range(G)]


def check_routing(layer: ZhaLayer, qh, n_tokens: int, tree: O.SummaryTree, p: float, label: str = "",
                  groups=None):
    """Level by level, check the GPU's routing against the oracle's arithmetic on the GPU's own
    candidate sets: candidate sets follow the expansion rule, scores match, stats are exact,
    and each head's kept set is a valid minimal top-p cut of the oracle's probabilities
    (mass reaches p, dropping its lightest node falls below p, no dropped node outweighs a
    kept one), all within rounding tolerances.  `groups` restricts the check to those KV groups; the
    oracle tree then holds exactly those groups, in that order.  Returns (worst score error,
    per-level kept sets)."""
    cfg = layer.cfg
    c, L, H = cfg.chunk, cfg.levels, cfg.n_kv_heads
    G = cfg.n_q_heads // H
    top = max([lv for lv in range(1, L + 1) if n_tokens // c ** lv > 0], default=0)
    routes = {lv: layer.route_level(lv) for lv in range(1, top + 1)}
    # the chain's last level: the group kept list the device derived from the heads'
    # bitmaps (in the next level's score kernel, or a merge at level 1) is theirs
    chained = [lv for lv in routes if routes[lv]["chained"]]
    if chained:
        lo = min(chained)
        r = routes[lo]
        for g in (range(H) if groups is None else groups):
            nk = int(r["n_kept"][g])
            assert int(r["dev_n_kept"][g]) == nk, f"{label} level {lo} group {g}: device kept count"
            assert torch.equal(r["dev_kept"][g, :nk], r["kept"][g, :nk]), f"{label} level {lo} group {g}: kept list"
            assert torch.equal(r["dev_mask"][g, :nk], r["mask"][g, :nk]), f"{label} level {lo} group {g}: masks"
    worst = 0.0
    kept_all = {lv: [None] * cfg.n_q_heads for lv in routes}
    for g in (range(H) if groups is None else groups):
        tg = g if groups is None else list(groups).index(g)
        prev_kept = None
        for lv in range(top, 0, -1):
            r = routes[lv]
            n_here = n_tokens // c ** lv
            if lv == top:
                nodes = np.arange(n_here, dtype=np.int64)
            else:
                rp = routes[lv + 1]
                nk = int(rp["n_kept"][g])
                parents = rp["kept"][g, :nk].numpy().astype(np.int64)
                nodes = np.concatenate([(parents[:, None] * c + np.arange(c)[None, :]).ravel(),
                                        np.arange(c * (n_tokens // c ** (lv + 1)), n_here, dtype=np.int64)])
            assert int(r["n_cand"][g]) == len(nodes), f"{label} level {lv} group {g}: candidate count"
            sig = r["sigma"][g, :, :len(nodes)].numpy().astype(np.float64)
            kept_h = _kept_by_head(r, g, G)
            s_all, b_all = tree.router_planes(lv, tg, nodes) if len(nodes) else (None, None)
            # the exact planes, around which the narrow copies' rounding is bracketed
            s_ex = tree.get(lv, tg, nodes)[0] if len(nodes) and tree.plane_format != "f32" else s_all
            for hl in range(G):
                h = g * G + hl
                is_c = sig[hl] > -np.inf
                cand = nodes[is_c]
                if lv == top:
                    expect = nodes
                else:
                    up = n_tokens // c ** (lv + 1)
                    expect = np.sort(np.concatenate([(prev_kept[hl][:, None] * c + np.arange(c)[None, :]).ravel(),
                                                     np.arange(c * up, n_here, dtype=np.int64)]))
                assert cand.tolist() == expect.tolist(), f"{label} level {lv} head {h}: candidate set"
                kept = kept_h[hl]
                assert int(r["stats"][h, 0]) == len(cand) and int(r["stats"][h, 1]) == len(kept), \
                    f"{label} level {lv} head {h}: stats"
                if len(cand) == 0:
                    assert len(kept) == 0
                    continue
                so = O.plane_scores(qh[h], s_all[is_c], b_all[is_c], tree.tau)
                tol = narrow_tolerance(qh[h], s_ex[is_c], tree)      # 0 for float32 planes
                err = float((np.maximum(np.abs(sig[hl][is_c] - so) - tol, 0.0) / (1.0 + np.abs(so))).max())
                worst = max(worst, err)
                assert err <= SCORE_RTOL, f"{label} level {lv} head {h}: score error {err:.3g}"
                slack = 2.0 * float(tol.max()) if len(tol) else 0.0  # probability ratios move by e^{2 tol}
                e = np.exp(so - so.max())
                pi = e / e.sum()
                inkept = np.isin(cand, kept)
                assert set(kept.tolist()) <= set(cand.tolist())
                if p >= 1.0:
                    assert inkept.all(), f"{label} level {lv} head {h}: p=1 must keep all"
                    continue
                assert len(kept) >= 1
                # The GPU's own order, exactly: keys formed from its fp32 scores as the
                # kernels form them (delta to the head's maximum in 2^-27 steps).  Every
                # candidate below the largest kept key is kept, and among the candidates
                # equal to it the kept ones are the lowest positions.
                s32 = r["sigma"][g, hl, :len(nodes)].numpy()[is_c]
                dl = (np.float32(s32.max()) - s32).astype(np.float32)
                kq = (np.minimum(dl, np.float32(31.999998092651367)) * np.float32(134217728.0)).astype(np.uint32)
                keys = np.where(dl < np.float32(32.0), kq, np.uint32(0xFFFFFFFE))
                kcut = keys[inkept].max()
                assert inkept[keys < kcut].all(), f"{label} level {lv} head {h}: a key below the cut dropped"
                at = inkept[keys == kcut]
                assert at[:int(at.sum())].all(), f"{label} level {lv} head {h}: ties not taken in position order"
                mass = pi[inkept].sum()
                lightest = pi[inkept].min()
                assert mass >= p - MASS_TOL - slack, f"{label} level {lv} head {h}: kept mass {mass:.6f} < p"
                assert mass - lightest < p + MASS_TOL + slack, f"{label} level {lv} head {h}: cut not minimal"
                if (~inkept).any():
                    heaviest_dropped = pi[~inkept].max()
                    assert heaviest_dropped <= lightest * (1 + ORDER_RTOL) * math.exp(slack) + 1e-15, \
                        f"{label} level {lv} head {h}: dropped {heaviest_dropped:.3g} > kept {lightest:.3g}"
            prev_kept = kept_h
            for hl in range(G):
                kept_all[lv][g * G + hl] = kept_h[hl].tolist()
    return worst, kept_all


def compare_decode(layer: ZhaLayer, x_q: torch.Tensor, n_tokens: int, tree: O.SummaryTree, kh, vh,
                   p: float, label: str = "", check_outputs_vs_oracle: bool = True, heads=None, groups=None):
    """Decode on the GPU and compare with the oracle.

    Every head: routing checked level by level (check_routing) and attention checked on
    the GPU's own selection.  Heads whose oracle cut margins are all >= MARGIN: per-level
    node sets identical to the oracle's own routing and output within ATOL of it.
    With `groups`, only those KV groups are checked and tree, kh and vh hold exactly
    those groups, in that order.  Returns (n_exempt, max attention error, worst score error)."""
    out = layer.decode(x_q).clone()
    torch.cuda.synchronize()
    out_h = out.cpu().numpy().astype(np.float64)
    qh = to_host(x_q)
    worst_sig, gk = check_routing(layer, qh, n_tokens, tree, p, label, groups=groups)
    G = layer.cfg.n_q_heads // layer.cfg.n_kv_heads
    c = layer.cfg.chunk
    n_exempt, max_err = 0, 0.0
    n_exact = n_ambiguous = 0
    if heads is None:
        heads = range(layer.cfg.n_q_heads) if groups is None else [g * G + j for g in groups for j in range(G)]
    margin_bar = {"bf16": NARROW_MARGIN, "fp8": FP8_MARGIN}.get(getattr(tree, "plane_format", "f32"), MARGIN)
    for h in heads:
        tg = h // G if groups is None else list(groups).index(h // G)
        r = O.route_head(qh[h], tree, tg, p)
        exempt = r.min_margin < margin_bar
        n_exempt += exempt
        # Levels from the top down to the first ambiguous cut must keep exactly the
        # oracle's nodes; below it either side of that cut is correct and the candidate
        # sets may differ (the routing is then checked for validity only).
        for lv in r.levels:
            got_h = gk[lv.level][h] if lv.level in gk else []
            if lv.margin < margin_bar:
                n_ambiguous += 1
                break
            n_exact += 1
            assert got_h == lv.kept.tolist(), (
                f"{label} head {h} level {lv.level}: GPU kept {got_h[:20]}... ({len(got_h)}) vs oracle "
                f"{lv.kept.tolist()[:20]}... ({len(lv.kept)}), margin {lv.margin:.3g}")
        leaves = gk[1][h] if 1 in gk else []
        toks = O.final_token_set(np.array(leaves, dtype=np.int64), n_tokens, c)
        ref = O.attend(qh[h], kh[tg], vh[tg], toks, tree.tau)
        err = float(np.abs(out_h[h] - ref).max())
        max_err = max(max_err, err)
        assert err <= ATOL, f"{label} head {h}: attention error {err:.3g} on the GPU's selected set"
        if check_outputs_vs_oracle and not exempt:
            o_ref = O.attend(qh[h], kh[tg], vh[tg], r.tokens, tree.tau)
            err2 = float(np.abs(out_h[h] - o_ref).max())
            assert err2 <= ATOL, f"{label} head {h}: output error {err2:.3g} vs oracle decode"
    say(f"  {label}: (head, level) cuts identical to the oracle {n_exact}, ambiguous (margin < {margin_bar}) "
        f"{n_ambiguous}")
    return n_exempt, max_err, worst_sig


def compare_tree(layer: ZhaLayer, tree: O.SummaryTree, n_tokens: int, sample: int | None = None, seed: int = 0,
                 rtol: float = 2e-5):
    """Summary planes of the GPU tree against the oracle's (all nodes, or a sample per level)."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for lv in range(1, layer.cfg.levels + 1):
        n = n_tokens // layer.cfg.chunk ** lv
        if n == 0:
            continue
        s_g, b_g, l_g = (t.cpu().numpy() for t in layer.tree_level(lv))
        for g in range(layer.cfg.n_kv_heads):
            nodes = np.arange(n) if sample is None or n <= sample else np.sort(rng.choice(n, sample, replace=False))
            s_o, b_o, l_o = tree.get(lv, g, nodes)
            for name, a, b in (("lse", l_g[g, nodes], l_o), ("b", b_g[g, nodes], b_o), ("s", s_g[g, nodes], s_o)):
                err = np.abs(a - b) / (1.0 + np.abs(b))
                e = float(err.max())
                worst = max(worst, e)
                assert e <= rtol, f"level {lv} head {g} {name}: max rel err {e:.3g}"
    return worst


def check_sel_stats(layer: ZhaLayer, sel: torch.Tensor, stats: torch.Tensor, n_tokens: int, tree: O.SummaryTree,
                    qh, p: float, label: str = "", chained_levels=()):
    """The decode step's optional outputs against the oracle.

    sel: per head, the kept level-1 chunks; for a head whose oracle cuts all have margin
    >= MARGIN they must be the oracle's kept leaves, and the attended token set built
    from them must be the oracle's token set; for every head they must be what the
    routing in scratch says.  stats: per level, candidate and kept sums over heads, the
    union candidates per group and the router bytes sum_g |U_g| * R * (d e + 4)
    (e = 4 for float32 planes, 2 for their bfloat16 copy), with U_g the union of the group's per-head candidate
    sets (the oracle's where all of the group's heads are unambiguous); the gathered
    tokens and bytes."""
    cfg = layer.cfg
    c, L, H, R, d = cfg.chunk, cfg.levels, cfg.n_kv_heads, cfg.n_ref, cfg.head_dim
    G = cfg.n_q_heads // H
    st = layer.read_stats(stats)
    got_sel = layer.read_sel(sel)
    top = max([lv for lv in range(1, L + 1) if n_tokens // c ** lv > 0], default=0)
    assert st["n_tokens"] == n_tokens and st["top_level"] == top and st["levels"] == L, label
    if top >= 1:
        kept1 = layer.kept_sets(1)
        assert got_sel == kept1, f"{label}: sel differs from the level-1 routing in scratch"
    else:
        assert all(len(s) == 0 for s in got_sel), label
    routes = [O.route_head(qh[h], tree, h // G, p) for h in range(cfg.n_q_heads)]
    for h, r in enumerate(routes):
        if r.min_margin >= MARGIN:
            assert got_sel[h] == r.kept_leaves().tolist(), f"{label} head {h}: sel vs oracle leaves"
            toks = O.final_token_set(np.array(got_sel[h], dtype=np.int64), n_tokens, c)
            assert toks.tolist() == r.tokens.tolist(), f"{label} head {h}: token set vs oracle"
    if cfg.plane_format == B.PLANE_FORMATS["fp8"]:
        plane = R * (d + 8)                     # codes, the plane's scale and b
    else:
        plane = R * (d * (2 if cfg.plane_format == B.PLANE_FORMATS["bf16"] else 4) + 4)
    e_kv = 2 if cfg.kv_dtype == B.ZHA_BF16 else 4
    for lv in range(1, B.STATS_MAX_LEVELS + 1):
        i = lv - 1
        if lv > top:
            for k in ("cand", "kept", "group_cand", "group_kept", "bytes_read", "bytes_streamed"):
                assert st[k][i] == 0, f"{label} level {lv}: {k} should be 0"
            continue
        r = layer.route_level(lv)
        assert st["cand"][i] == int(r["stats"][:, 0].sum()), f"{label} level {lv}: cand"
        assert st["kept"][i] == int(r["stats"][:, 1].sum()), f"{label} level {lv}: kept"
        assert st["group_kept"][i] == int(r["n_kept"].sum()), f"{label} level {lv}: group_kept"
        union = 0
        for g in range(H):
            hs = range(g * G, (g + 1) * G)
            if all(routes[h].min_margin >= MARGIN for h in hs):
                u = set()
                for h in hs:
                    for lr in routes[h].levels:
                        if lr.level == lv:
                            u |= set(lr.candidates.tolist())
                n_u = len(u)
            else:
                n_u = int(r["n_cand"][g])
            assert int(r["n_cand"][g]) == n_u, f"{label} level {lv} group {g}: union candidates"
            union += n_u
        assert st["group_cand"][i] == union, f"{label} level {lv}: group_cand"
        assert st["bytes_read"][i] == union * plane, f"{label} level {lv}: bytes_read formula"
        if lv in chained_levels:
            assert st["bytes_streamed"][i] == (n_tokens // c ** lv) * H * plane, f"{label} level {lv}: streamed"
        else:
            assert st["bytes_streamed"][i] >= st["bytes_read"][i]
    toks = 0
    for g in range(H):
        u = set()
        for h in range(g * G, (g + 1) * G):
            u |= set(O.final_token_set(np.array(got_sel[h], dtype=np.int64), n_tokens, c).tolist())
        toks += len(u)
    assert st["gather_tokens"] == toks, f"{label}: gather tokens {st['gather_tokens']} vs {toks}"
    assert st["gather_bytes"] == toks * 2 * d * e_kv
    return st

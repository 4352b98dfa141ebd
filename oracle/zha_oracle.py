"""Plain fp64 CPU oracle for one ZHA decode step and the tree that feeds it.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run
this module: only the tests, the smoke check and the benchmark's CPU-baseline
leg use it.  It shares no code, table or constant with the HIP library.

Sources (web pages on Zyphra Hierarchical Attention, ZHA), cited by title and
section throughout:

  [kg]   "Zyphra 分层注意力（ZHA）：通向真次二次注意力的新路径，挑战长上下文瓶颈"
         (kg.zhiyong.dev), sections 机制拆解 (mechanism), 局限与权衡 (limits).
  [fe]   "ZHA 用树形稀疏注意力改造现有大模型" (feinterview.poetries.top),
         sections 稀疏注意力为什么还会被索引拖慢 (index), 256K 的质量结果
         (quality), 几百倍加速 (speed).
  [rit]  rit.work/blog/zha-tree-indexer-long-context, section
         "Дерево сокращает сам поиск нужных ключей" (tree).
  [gt]   "階層型疎Attention「ZHA」──長文LLMの探索コストを削る新設計"
         (geek-terminal.com), section 技術的ディープダイブ (deep dive).
  [cap]  "Zyphra Luncurkan ZHA: Attention Sparse Tree-based yang Beneran
         Subquadratic?" (news.captivela.com), opening section.

What the pages fix, restated:
  * Contiguous keys are cut into chunks; each chunk gets a summary; summaries
    are grouped the same way level after level, so the fanout equals the chunk
    size ([kg] mechanism; [fe] index: chunk 4 and 6 levels make a 4,096-token
    top node; [cap] opening).
  * Summaries come from a few reference queries; each gives a tangent-plane
    estimate of the log attention mass of the block, and the estimate used is
    the maximum over the planes ([fe] index; [kg] mechanism).
  * Decoding scores the top level, keeps the smallest node set whose
    cumulative estimated probability reaches p, expands only the children of
    kept nodes and repeats down to the raw KV ([kg] mechanism; [fe] index;
    [rit] tree; [gt] deep dive).
  * The final attention is exact, over the raw keys of the selected leaves
    ([rit] tree; [gt] deep dive); the first token is always kept as the
    attention sink ([fe] index; [cap] opening); the full KV cache is kept
    ([kg] limits; [fe] index; [rit] tree).

Readings taken where the pages are silent (the same list is kept in the design
notes of the repository):
  R1  logits use the attention's temperature tau = 1/sqrt(d) everywhere:
      b_r = LSE_r - tau q_r.s_r and sigma(q) = max_r (tau q.s_r + b_r).
  R2  a node's summary is defined over the raw keys it covers (the recursive
      construction gives the same planes when reference queries are shared).
  R3  one set of R reference queries per KV head, shared by all levels.
  R4  fanout c at every level; level 1 holds chunks of c raw tokens; a level-l
      node covers c**l tokens.
  R5  the softmax that turns scores into probabilities runs over the current
      level's candidates only.
  R6  the cut is inclusive (cumulative >= p), keeps at least one node, breaks
      ties by ascending node index; p >= 1 keeps every candidate.
  R7  every query head routes on its own.
  R8  a node that is not complete has no summary; its complete children join
      the candidates of their own level (orphans); the raw tail of fewer than
      c tokens is always attended.
  R9  token 0 is always attended; sets are unions, so it is never counted twice.
  R10 a decode step attends over the cache as it stands (append first).

All arithmetic is float64.  Inputs may be float32/float64 arrays or bfloat16
given as raw uint16 bit patterns; they are widened exactly.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "widen",
    "round_bf16",
    "fp8_plane_scale_exp",
    "round_fp8",
    "n_complete",
    "summarize_nodes",
    "SummaryTree",
    "plane_scores",
    "top_p_cut",
    "route_head",
    "final_token_set",
    "attend",
    "decode_step",
    "dense_decode",
    "append_token",
    "level_mass_recall",
    "HeadRoute",
    "LevelRoute",
]

# Largest number of raw key rows widened to float64 at once while summarising.
_BATCH_TOKENS = 1 << 16


def widen(a) -> np.ndarray:
    """Exact widening to float64.  uint16 arrays are bfloat16 bit patterns."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64, copy=False)


def round_bf16(x) -> np.ndarray:
    """Round float64 values to bfloat16 (8 significant bits, float32's exponent
    range), to nearest with ties to even, and return them as float64.

    The narrow-format router of [fe] speed (几百倍加速, a router reading its
    summaries in a narrow format): the planes are computed in full precision and
    rounded once.  Written from the definition: x = m 2**e with 1/2 <= |m| < 1,
    the representable neighbours are multiples of 2**(e - 8), and np.round rounds
    half to even.  Values here are normal and finite (no subnormal or overflow case).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)


FP8_MAX = 448.0   # largest finite FP8 E4M3 value (1.75 * 2**8)


def fp8_plane_scale_exp(s) -> np.ndarray:
    """Per plane (the last axis holds its d elements), the exponent k of the smallest
    power of two with max_d |s_d| <= 448 * 2**k, clamped to k >= -126; 0 for an
    all-zero plane.

    The scale of the 8-bit router planes: a plane is stored as 2**k times FP8 E4M3
    values (4 exponent bits, bias 7, 3 mantissa bits, subnormals, largest 448), so
    its largest element lands in (224, 448] and none overflows.  With
    max = f 2**e, 1/2 <= f < 1: k = e - 9 when f <= 7/8, else e - 8.
    """
    m = np.abs(np.asarray(s, dtype=np.float64)).max(axis=-1)
    f, e = np.frexp(m)
    k = np.where(f <= 0.875, e - 9, e - 8)
    return np.where(m == 0, 0, np.maximum(k, -126)).astype(np.int64)


def round_fp8(s, k=None) -> np.ndarray:
    """Each plane of s (last axis) rounded to its 8-bit router form and returned as
    float64: 2**k * RNE_e4m3(s / 2**k) with k = fp8_plane_scale_exp(s) (or the
    per-plane exponents given, whose scaled values must stay within 448).

    The narrow router of [fe] speed (几百倍加速) at 8 bits.  Written from the
    format's definition: a scaled value x with 2**(e-1) <= |x| < 2**e (frexp) has
    spacing 2**(e - 4) when e >= -5 (three mantissa bits), and below the smallest
    normal 2**-6 the spacing stays 2**-9 (subnormals); np.round rounds half to
    even.  Scaled values never pass 448, so no overflow case arises.
    """
    s = np.asarray(s, dtype=np.float64)
    k = (fp8_plane_scale_exp(s) if k is None else np.asarray(k, dtype=np.int64))[..., None]
    x = np.ldexp(s, -k)
    _, ex = np.frexp(x)
    qe = np.maximum(ex, -5) - 4
    return np.ldexp(np.round(np.ldexp(x, -qe)), qe + k)


def n_complete(n_tokens: int, chunk: int, level: int) -> int:
    """Number of complete level-`level` nodes over tokens [0, n_tokens).

    A level-l node covers c**l consecutive tokens (reading R4 of [fe] index:
    chunk 4 with 6 levels gives a 4,096-token top node).
    """
    return n_tokens // (chunk ** level)


def summarize_nodes(keys_g, qref_g, chunk: int, level: int, nodes, tau: float):
    """Tangent-plane summaries of level-`level` nodes, from the raw keys.

    For node n covering tokens T_n and reference query q_r ([fe] index: the
    planes estimate each block's log attention mass; [kg] mechanism):
        z_t   = tau * q_r . k_t                    for t in T_n
        LSE_r = log sum_t exp(z_t)                 (max-subtracted)
        s_r   = sum_t exp(z_t - LSE_r) * k_t       (softmax-weighted key mean)
        b_r   = LSE_r - tau * q_r . s_r
    so that the plane tau*q.s_r + b_r touches LSE_n(q) at q = q_r.

    Returns (s [n, R, d], b [n, R], lse [n, R]) in float64.
    """
    nodes = np.asarray(nodes, dtype=np.int64)
    qref = widen(qref_g)
    n_ref, d = qref.shape
    span = chunk ** level
    s_out = np.empty((len(nodes), n_ref, d))
    b_out = np.empty((len(nodes), n_ref))
    lse_out = np.empty((len(nodes), n_ref))
    per_batch = max(1, _BATCH_TOKENS // span)
    offs = np.arange(span, dtype=np.int64)
    for lo in range(0, len(nodes), per_batch):
        sel = nodes[lo:lo + per_batch]
        toks = sel[:, None] * span + offs[None, :]              # [n, span]
        keys = widen(keys_g[toks.ravel()]).reshape(len(sel), span, d)
        z = tau * np.matmul(keys, qref.T).transpose(0, 2, 1)      # [n, R, span]
        zmax = z.max(axis=2, keepdims=True)
        lse = zmax[..., 0] + np.log(np.exp(z - zmax).sum(axis=2))
        w = np.exp(z - lse[..., None])                           # [n, R, span]
        s = np.matmul(w, keys)                                   # [n, R, d]
        b = lse - tau * np.einsum("rd,nrd->nr", qref, s)
        s_out[lo:lo + len(sel)] = s
        b_out[lo:lo + len(sel)] = b
        lse_out[lo:lo + len(sel)] = lse
    return s_out, b_out, lse_out


class SummaryTree:
    """The summary tree beside a full KV cache, computed node by node on demand.

    Every node's planes are computed from the raw keys it covers (reading R2),
    never from its children, so that the GPU's recursive merge is checked
    against the definition.  Only complete nodes have summaries (reading R8).
    Reference queries are one set per KV head shared by all levels (R3).
    """

    def __init__(self, keys, qref, n_tokens: int, chunk: int, levels: int, tau: float | None = None,
                 plane_format: str = "f32"):
        if plane_format not in ("f32", "bf16", "fp8"):
            raise ValueError(f"plane_format must be 'f32', 'bf16' or 'fp8' (got {plane_format!r})")
        self.plane_format = plane_format     # what the router reads: exact planes, or s rounded to bf16 / fp8
        self.keys = keys                     # [H_kv][>= n_tokens][d] (any float or bf16 bits)
        self.qref = widen(qref)              # [H_kv][R][d]
        self.n_tokens = int(n_tokens)
        self.chunk = int(chunk)
        self.levels = int(levels)
        d = self.qref.shape[-1]
        self.tau = (1.0 / math.sqrt(d)) if tau is None else float(tau)
        self._cache: dict[tuple[int, int], dict[int, tuple]] = {}

    def n_nodes(self, level: int) -> int:
        return n_complete(self.n_tokens, self.chunk, level)

    def get(self, level: int, g: int, nodes):
        """Planes (s [n,R,d], b [n,R], lse [n,R]) of complete nodes `nodes` of KV head g."""
        nodes = np.asarray(nodes, dtype=np.int64)
        if len(nodes) and (nodes.min() < 0 or nodes.max() >= self.n_nodes(level)):
            raise IndexError("only complete nodes have summaries")
        cache = self._cache.setdefault((level, g), {})
        missing = np.array([n for n in nodes.tolist() if n not in cache], dtype=np.int64)
        if len(missing):
            s, b, lse = summarize_nodes(self.keys[g], self.qref[g], self.chunk, level, missing, self.tau)
            for i, n in enumerate(missing.tolist()):
                cache[n] = (s[i], b[i], lse[i])
        n_ref, d = self.qref.shape[1:]
        s = np.empty((len(nodes), n_ref, d))
        b = np.empty((len(nodes), n_ref))
        lse = np.empty((len(nodes), n_ref))
        for i, n in enumerate(nodes.tolist()):
            s[i], b[i], lse[i] = cache[n]
        return s, b, lse

    def router_planes(self, level: int, g: int, nodes):
        """The planes the router scores with: (s, b), s rounded to bfloat16 or to its
        scaled 8-bit form when the tree's plane_format is 'bf16' or 'fp8' (b is kept
        in full precision)."""
        s, b, _ = self.get(level, g, nodes)
        if self.plane_format == "bf16":
            s = round_bf16(s)
        elif self.plane_format == "fp8":
            s = round_fp8(s)
        return s, b

    def full_level(self, level: int, g: int):
        """Planes of every complete node of one level (for whole-tree comparisons)."""
        n = self.n_nodes(level)
        s, b, lse = summarize_nodes(self.keys[g], self.qref[g], self.chunk, level,
                                    np.arange(n, dtype=np.int64), self.tau)
        return s, b, lse

    def invalidate(self):
        self._cache.clear()


def plane_scores(q, s, b, tau: float):
    """Estimated log attention mass of each node for query q.

    sigma_n(q) = max_r (tau * q . s_{n,r} + b_{n,r}): the largest of the
    node's tangent planes ([fe] index: the maximum over several estimating
    planes).  s [n,R,d], b [n,R]; returns [n].
    """
    q = widen(q)
    return (tau * np.einsum("d,nrd->nr", q, s) + b).max(axis=1)


def top_p_cut(sigma, node_ids, p: float):
    """Minimal top-p node set of one level.

    pi = softmax(sigma) over the candidates; order by pi descending, ties by
    ascending node index; keep the shortest prefix whose cumulative
    probability reaches p ([kg] mechanism; [fe] index; [gt] deep dive: not a
    fixed top-k).  p >= 1 keeps every candidate.

    Returns (kept node ids in rank order, pi in candidate order, margin) where
    margin is the distance of this cut from changing under a small
    perturbation of the scores:
        min(S_K - p,  p - S_{K-1}  (p when K = 1),  1 - pi_(K+1) / pi_(K)  (inf when K = |C|)).
    The first two terms are cumulative probability; the last is the relative
    gap between the last kept and the first dropped candidate (about their
    score difference), which is what decides their order under score error.
    """
    sigma = np.asarray(sigma, dtype=np.float64)
    node_ids = np.asarray(node_ids, dtype=np.int64)
    n = len(sigma)
    if n == 0:
        return node_ids[:0], sigma[:0], math.inf
    e = np.exp(sigma - sigma.max())
    pi = e / e.sum()
    order = np.lexsort((node_ids, -pi))
    if p >= 1.0:
        return node_ids[order], pi, math.inf
    cum = np.cumsum(pi[order])
    reach = np.nonzero(cum >= p)[0]
    k = int(reach[0]) + 1 if len(reach) else n
    margin = cum[k - 1] - p
    margin = min(margin, p - (cum[k - 2] if k >= 2 else 0.0))
    if k < n:
        margin = min(margin, 1.0 - pi[order[k]] / pi[order[k - 1]])
    return node_ids[order[:k]], pi, float(margin)


@dataclass
class LevelRoute:
    level: int
    candidates: np.ndarray      # ascending node ids
    sigma: np.ndarray           # per candidate
    pi: np.ndarray              # per candidate
    kept: np.ndarray            # ascending node ids
    margin: float


@dataclass
class HeadRoute:
    levels: list = field(default_factory=list)   # LevelRoute, top level first
    tokens: np.ndarray | None = None              # final attended token set T_h (ascending)

    @property
    def min_margin(self) -> float:
        return min([lv.margin for lv in self.levels], default=math.inf)

    def kept_leaves(self) -> np.ndarray:
        for lv in self.levels:
            if lv.level == 1:
                return lv.kept
        return np.zeros(0, dtype=np.int64)


def route_head(q_h, tree: SummaryTree, g: int, p: float) -> HeadRoute:
    """Top-down routing of one query head through the tree of KV head g.

    Level L: every complete node is a candidate.  Level l < L: the children of
    the nodes kept at level l+1, plus the complete level-l nodes whose parent
    is not complete (orphans, reading R8).  Each level keeps its minimal
    top-p set (top_p_cut); dropped branches are never revisited ([kg]
    mechanism; [fe] index; [rit] tree).
    """
    c, L, N = tree.chunk, tree.levels, tree.n_tokens
    route = HeadRoute()
    kept_above = np.zeros(0, dtype=np.int64)
    for level in range(L, 0, -1):
        n_here = n_complete(N, c, level)
        if level == L:
            cand = np.arange(n_here, dtype=np.int64)
        else:
            n_up = n_complete(N, c, level + 1)
            children = (kept_above[:, None] * c + np.arange(c, dtype=np.int64)[None, :]).ravel()
            orphans = np.arange(c * n_up, n_here, dtype=np.int64)
            cand = np.sort(np.concatenate([children, orphans]))
        if len(cand) == 0:
            lv = LevelRoute(level, cand, np.zeros(0), np.zeros(0), cand, math.inf)
        else:
            s, b = tree.router_planes(level, g, cand)
            sigma = plane_scores(q_h, s, b, tree.tau)
            kept, pi, margin = top_p_cut(sigma, cand, p)
            lv = LevelRoute(level, cand, sigma, pi, np.sort(kept), margin)
        route.levels.append(lv)
        kept_above = lv.kept
    route.tokens = final_token_set(route.kept_leaves(), N, c)
    return route


def final_token_set(kept_leaves, n_tokens: int, chunk: int) -> np.ndarray:
    """T_h = {0} | tokens of kept leaf chunks | raw tail [c*n_1, N), as a set.

    Token 0 is the attention sink ([fe] index; [cap] opening); the tail holds
    fewer than c tokens and has no summary (reading R8).
    """
    kept_leaves = np.asarray(kept_leaves, dtype=np.int64)
    n1 = n_complete(n_tokens, chunk, 1)
    parts = [np.zeros(1, dtype=np.int64) if n_tokens > 0 else np.zeros(0, dtype=np.int64),
             (kept_leaves[:, None] * chunk + np.arange(chunk, dtype=np.int64)[None, :]).ravel(),
             np.arange(chunk * n1, n_tokens, dtype=np.int64)]
    return np.unique(np.concatenate(parts))


def attend(q_h, keys_g, values_g, tokens, tau: float):
    """Exact softmax attention of one query over the given raw tokens.

    o = sum_t softmax_t(tau * q . k_t) v_t ([rit] tree: the final attention
    uses the raw keys of the selected leaves, not their summaries).
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    q = widen(q_h)
    k = widen(keys_g[tokens])
    v = widen(values_g[tokens])
    z = tau * (k @ q)
    w = np.exp(z - z.max())
    return (w / w.sum()) @ v


def decode_step(q, keys, values, tree: SummaryTree, p: float):
    """One ZHA decode step for all query heads.

    q [H_q][d]; query head h reads KV head g = h // (H_q / H_kv) (grouped-query
    attention).  Returns (out [H_q][d] float64, routes list[HeadRoute]).
    """
    q = widen(q)
    n_q = q.shape[0]
    n_kv = tree.qref.shape[0]
    group = n_q // n_kv
    out = np.empty((n_q, q.shape[1]))
    routes = []
    for h in range(n_q):
        g = h // group
        r = route_head(q[h], tree, g, p)
        out[h] = attend(q[h], keys[g], values[g], r.tokens, tree.tau)
        routes.append(r)
    return out, routes


def level_mass_recall(q_h, keys_g, kept_by_level: dict, tokens, n_tokens: int, chunk: int, levels: int,
                      tau: float):
    """How much of the exact attention the routing of one query head kept.

    p_t = softmax_t(tau q.k_t) over all n_tokens tokens (the dense attention the
    method approximates; [fe] quality 256K 的质量结果 judges the router by it).
    For level l (1..levels): recall_l = sum of p_t over the tokens whose level-l
    node is in kept_by_level[l] (node ids), tokens under no complete level-l node
    counting as kept (they are never dropped at that level; R8).  A level absent
    from kept_by_level keeps every node.  captured = sum of p_t over `tokens`,
    the attended set.  Returns (recall [levels], captured).
    """
    keys = widen(keys_g[:n_tokens])
    z = tau * (keys @ widen(q_h))
    z = z - z.max()
    p = np.exp(z)
    p = p / p.sum()
    t = np.arange(n_tokens, dtype=np.int64)
    recall = np.ones(levels)
    for level in range(1, levels + 1):
        if level not in kept_by_level:
            continue
        span = chunk ** level
        node = t // span
        keep = (node >= n_complete(n_tokens, chunk, level)) | np.isin(node, np.asarray(kept_by_level[level]))
        recall[level - 1] = p[keep].sum()
    captured = p[np.asarray(tokens, dtype=np.int64)].sum()
    return recall, float(captured)


def dense_decode(q, keys, values, n_tokens: int, tau: float | None = None):
    """Exact attention of every query head over all n_tokens cached tokens (baseline)."""
    q = widen(q)
    n_q, d = q.shape
    n_kv = keys.shape[0]
    group = n_q // n_kv
    tau = (1.0 / math.sqrt(d)) if tau is None else tau
    toks = np.arange(n_tokens, dtype=np.int64)
    return np.stack([attend(q[h], keys[h // group], values[h // group], toks, tau) for h in range(n_q)])


def append_token(keys, values, tree: SummaryTree, n_before: int, k_new, v_new):
    """Append one token: write row n_before of K and V, then summarise each node it completes.

    The completed levels are exactly those l with (n_before + 1) % c**l == 0;
    each gets node (l, (n_before + 1) / c**l - 1), computed from raw keys
    ([rit] tree: levels are added as the context grows).  Returns the new
    token count and the list of (level, node) summarised.
    """
    keys[:, n_before] = k_new
    values[:, n_before] = v_new
    n = n_before + 1
    tree.n_tokens = n
    done = []
    level = 1
    while level <= tree.levels and n % (tree.chunk ** level) == 0:
        node = n // (tree.chunk ** level) - 1
        for g in range(keys.shape[0]):
            tree.get(level, g, [node])
        done.append((level, node))
        level += 1
    return n, done

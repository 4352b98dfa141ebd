"""Pins of the fp64 oracle to facts fixed outside itself (CPU only).

Each test checks the oracle against a closed form, an invariant, a textbook or
library routine, a brute-force enumeration or a hand-derived example, so that
a plausible slip in it (a dropped term, a wrong sign or index, a transposed
operand, a missed orphan) fails at least one of them.  test_oracle_mutations.py
plants such slips and checks that these pins catch them.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng


def _rand_cache(n_kv, n, d, seed, scale=1.0):
    r = RNG(seed)
    return r.normal(size=(n_kv, n, d)) * scale, r.normal(size=(n_kv, n, d))


# ---------------------------------------------------------------- summaries (P1-P6)

@pytest.mark.parametrize("span_level,chunk", [(1, 4), (2, 4), (3, 2), (1, 8)])
def test_p1_plane_at_ref_query_is_exact_lse(span_level, chunk):
    """P1: plane r evaluated at q_r equals the node's exact log-sum-exp at q_r."""
    d, R = 16, 5
    keys, _ = _rand_cache(1, chunk ** span_level * 3, d, 1)
    qref = RNG(2).normal(size=(R, d)) * 2
    tau = 1 / math.sqrt(d)
    s, b, lse = O.summarize_nodes(keys[0], qref, chunk, span_level, [0, 1, 2], tau)
    span = chunk ** span_level
    for n in range(3):
        k = keys[0, n * span:(n + 1) * span]
        for r in range(R):
            exact = scipy.special.logsumexp(tau * k @ qref[r])
            assert abs(tau * qref[r] @ s[n, r] + b[n, r] - exact) < 1e-12
            assert abs(lse[n, r] - exact) < 1e-12


def test_p2_max_of_planes_never_exceeds_lse():
    """P2: log-sum-exp is convex, so every tangent plane lies below it."""
    d, R, c = 32, 8, 4
    keys, _ = _rand_cache(1, 64, d, 3)
    qref = RNG(4).normal(size=(R, d)) * 3
    tau = 1 / math.sqrt(d)
    s, b, _ = O.summarize_nodes(keys[0], qref, c, 2, [0, 1, 2, 3], tau)
    qs = RNG(5).normal(size=(500, d)) * 3
    for n in range(4):
        k = keys[0, 16 * n:16 * (n + 1)]
        exact = scipy.special.logsumexp(tau * qs @ k.T, axis=1)
        est = np.stack([O.plane_scores(q, s[n:n + 1], b[n:n + 1], tau)[0] for q in qs])
        assert np.all(est <= exact + 1e-12)
        # the bound is not vacuous: it is tight somewhere near the reference queries
        near = O.plane_scores(qref[0] + 1e-3, s[n:n + 1], b[n:n + 1], tau)[0]
        assert abs(near - scipy.special.logsumexp(tau * k @ (qref[0] + 1e-3))) < 1e-4


def test_p3_score_at_ref_query_equals_lse():
    """P3: sigma_n(q_r) = LSE_n(q_r) exactly (the r-th plane touches; the others lie below)."""
    d, R = 16, 6
    keys, _ = _rand_cache(1, 32, d, 6)
    qref = RNG(7).normal(size=(R, d)) * 2
    tau = 1 / math.sqrt(d)
    s, b, _ = O.summarize_nodes(keys[0], qref, 4, 1, np.arange(8), tau)
    for n in range(8):
        for r in range(R):
            exact = scipy.special.logsumexp(tau * keys[0, 4 * n:4 * n + 4] @ qref[r])
            assert abs(O.plane_scores(qref[r], s[n:n + 1], b[n:n + 1], tau)[0] - exact) < 1e-12


@pytest.mark.parametrize("level,chunk", [(1, 4), (2, 4), (3, 2), (1, 256)])
def test_p4_identical_keys_closed_form(level, chunk):
    """P4: a node of identical keys kappa has sigma(q) = level*log(c) + tau*q.kappa for every q."""
    d, R = 8, 4
    kappa = RNG(8).normal(size=d)
    span = chunk ** level
    keys = np.tile(kappa, (span, 1))[None]
    qref = RNG(9).normal(size=(R, d))
    tau = 1 / math.sqrt(d)
    s, b, _ = O.summarize_nodes(keys[0], qref, chunk, level, [0], tau)
    assert np.allclose(s[0], kappa[None, :], atol=1e-12)
    assert np.allclose(b[0], level * math.log(chunk), atol=1e-12)
    for q in RNG(10).normal(size=(20, d)) * 4:
        assert abs(O.plane_scores(q, s, b, tau)[0] - (level * math.log(chunk) + tau * q @ kappa)) < 1e-10


def test_p5_merge_of_children_equals_summary_from_raw():
    """P5: the recursive construction (merging c child planes) gives the from-raw planes.

    Merge written from the pages' recursive description: LSE_P = logsumexp_j LSE_j,
    s_P = sum_j exp(LSE_j - LSE_P) s_j, b_P = LSE_P - tau q_r.s_P.
    """
    d, R, c = 16, 4, 4
    keys, _ = _rand_cache(1, 4 * 16, d, 11)
    qref = RNG(12).normal(size=(R, d)) * 2
    tau = 1 / math.sqrt(d)
    s1, b1, l1 = O.summarize_nodes(keys[0], qref, c, 1, np.arange(16), tau)
    s2, b2, l2 = O.summarize_nodes(keys[0], qref, c, 2, np.arange(4), tau)
    for p in range(4):
        ch = slice(c * p, c * p + c)
        lse_p = scipy.special.logsumexp(l1[ch], axis=0)                     # [R]
        a = np.exp(l1[ch] - lse_p[None, :])                                 # [c, R]
        s_p = np.einsum("jr,jrd->rd", a, s1[ch])
        b_p = lse_p - tau * np.einsum("rd,rd->r", qref, s_p)
        assert np.allclose(lse_p, l2[p], atol=1e-12)
        assert np.allclose(s_p, s2[p], atol=1e-12)
        assert np.allclose(b_p, b2[p], atol=1e-12)


def test_p6_summary_invariant_to_key_order():
    """P6: a node's planes do not depend on the order of its keys."""
    d, R, c = 16, 3, 8
    keys, _ = _rand_cache(1, 8, d, 13)
    qref = RNG(14).normal(size=(R, d))
    tau = 1 / math.sqrt(d)
    s, b, _ = O.summarize_nodes(keys[0], qref, c, 1, [0], tau)
    perm = RNG(15).permutation(8)
    s2, b2, _ = O.summarize_nodes(keys[0][perm], qref, c, 1, [0], tau)
    assert np.allclose(s, s2, atol=1e-12) and np.allclose(b, b2, atol=1e-12)


# ---------------------------------------------------------------- routing and attention (P7-P12)

def _tree(n_kv, n, d, R, c, L, seed, scale=1.0):
    keys, values = _rand_cache(n_kv, n, d, seed, scale)
    qref = RNG(seed + 100).normal(size=(n_kv, R, d))
    return keys, values, O.SummaryTree(keys, qref, n, c, L)


def _sdpa(q, k, v):
    """Textbook attention through torch's CPU routine (a different code path)."""
    qt = torch.tensor(q)[None, None, None]          # [1,1,1,d]
    kt = torch.tensor(k)[None, None]
    vt = torch.tensor(v)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, 0, 0].numpy()


@pytest.mark.parametrize("n", [64, 100, 257])
def test_p7_p_one_reproduces_dense(n):
    """P7: p = 1 keeps every leaf, so the decode equals dense softmax attention."""
    d = 16
    keys, values, tree = _tree(2, n, d, 4, 4, 3, 20)
    q = RNG(21).normal(size=(4, d)) * 3
    out, routes = O.decode_step(q, keys, values, tree, 1.0)
    for h in range(4):
        assert len(routes[h].tokens) == n
        assert np.allclose(out[h], _sdpa(q[h], keys[h // 2, :n], values[h // 2, :n]), atol=1e-12)


def test_p8_tiny_p_is_argmax_descent():
    """P8: a vanishing p keeps exactly the best-scoring candidate at every level."""
    d = 16
    keys, values, tree = _tree(1, 256, d, 4, 4, 3, 30)
    for q in RNG(31).normal(size=(10, d)) * 3:
        r = O.route_head(q, tree, 0, 1e-9)
        for lv in r.levels:
            assert len(lv.kept) == 1
            assert lv.kept[0] == lv.candidates[np.argmax(lv.sigma)]


def _ancestor_candidates(n_tokens, c, L, kept_by_level, level):
    """Candidate set at `level` from the ancestor formulation (independent of the oracle's
    parent-plus-orphan rule): a complete node is a candidate iff each of its complete
    ancestors was kept."""
    out = []
    for j in range(O.n_complete(n_tokens, c, level)):
        ok = True
        for up in range(level + 1, L + 1):
            a = j // c ** (up - level)
            if a < O.n_complete(n_tokens, c, up) and a not in kept_by_level[up]:
                ok = False
                break
        if ok:
            out.append(j)
    return out


@pytest.mark.parametrize("n,c,L,p,seed", [(64, 4, 2, 0.8, 40), (60, 4, 2, 0.6, 41), (63, 2, 3, 0.7, 42),
                                          (50, 2, 4, 0.9, 43), (64, 8, 1, 0.75, 44), (30, 4, 2, 0.95, 45)])
def test_p9_brute_force_small(n, c, L, p, seed):
    """P9: at N <= 64 every level's kept set is the unique minimum-size, maximum-mass set
    reaching p among all subsets of the candidates; candidates match the ancestor rule;
    attention matches direct summation over the final set."""
    d = 8
    keys, values, tree = _tree(1, n, d, 3, c, L, seed, scale=2.0)
    tau = tree.tau
    for q in RNG(seed + 1).normal(size=(4, d)) * 3:
        r = O.route_head(q, tree, 0, p)
        kept_by_level = {}
        for lv in r.levels:
            kept_by_level[lv.level] = set(lv.kept.tolist())
        for lv in r.levels:
            assert lv.candidates.tolist() == _ancestor_candidates(n, c, L, kept_by_level, lv.level)
            m = len(lv.candidates)
            if m == 0:
                continue
            assert m <= 16
            e = np.exp(lv.sigma - lv.sigma.max())
            pi = e / e.sum()
            best = None
            for size in range(1, m + 1):
                for sub in itertools.combinations(range(m), size):
                    mass = pi[list(sub)].sum()
                    if mass >= p and (best is None or mass > best[0]):
                        best = (mass, sub)
                if best is not None:
                    break
            assert sorted(lv.candidates[list(best[1])].tolist()) == lv.kept.tolist()
        # final set and attention by direct summation
        leaves = kept_by_level[1]
        T = sorted({0} | {c * j + i for j in leaves for i in range(c)} | set(range(c * (n // c), n)))
        assert r.tokens.tolist() == T
        w = np.array([math.exp(tau * q @ keys[0, t]) for t in T])
        ref = sum(w[i] * values[0, t] for i, t in enumerate(T)) / w.sum()
        assert np.allclose(O.attend(q, keys[0], values[0], r.tokens, tau), ref, atol=1e-12)


def test_p10_build_equals_build_then_appends():
    """P10: the tree over N + m tokens equals the tree over N tokens grown by m appends."""
    d, c, L, R = 8, 4, 3, 2
    n0, m = 37, 29
    keys, values = _rand_cache(2, n0 + m, d, 50)
    qref = RNG(51).normal(size=(2, R, d))
    full = O.SummaryTree(keys.copy(), qref, n0 + m, c, L)
    k_grow = keys.copy()
    k_grow[:, n0:] = 0.0
    v_grow = values.copy()
    v_grow[:, n0:] = 0.0
    grown = O.SummaryTree(k_grow, qref, n0, c, L)
    done = []
    n = n0
    for t in range(m):
        n, completed = O.append_token(k_grow, v_grow, grown, n, keys[:, n0 + t], values[:, n0 + t])
        done += completed
    assert n == n0 + m
    # completed nodes are exactly the ones whose last token was appended
    expect = [(lv, (t + 1) // c ** lv - 1) for t in range(n0, n0 + m) for lv in range(1, L + 1)
              if (t + 1) % c ** lv == 0]
    assert done == expect
    for lv in range(1, L + 1):
        for g in range(2):
            a = full.full_level(lv, g)
            b = grown.full_level(lv, g)
            for x, y in zip(a, b):
                assert np.array_equal(x, y)
            assert np.array_equal(grown.get(lv, g, np.arange(grown.n_nodes(lv)))[0], a[0])


def test_p11_dense_is_textbook_attention():
    """P11: dense decode equals softmax(q K^T / sqrt(d)) V from torch's CPU routine."""
    d = 32
    keys, values = _rand_cache(2, 300, d, 60)
    q = RNG(61).normal(size=(8, d)) * 2
    out = O.dense_decode(q, keys, values, 300)
    for h in range(8):
        assert np.allclose(out[h], _sdpa(q[h], keys[h // 4], values[h // 4]), atol=1e-12)


@pytest.mark.parametrize("n,p", [(200, 0.7), (203, 0.9)])
def test_p12_single_level_is_flat_chunk_top_p(n, p):
    """P12a: with one level, routing is a flat top-p over all complete chunks."""
    d, c = 16, 8
    keys, values, tree = _tree(1, n, d, 4, c, 1, 70, scale=2.0)
    for q in RNG(71).normal(size=(5, d)) * 3:
        r = O.route_head(q, tree, 0, p)
        assert len(r.levels) == 1
        n1 = n // c
        # flat scores of every chunk, from raw keys, by the definition
        sig = []
        for j in range(n1):
            k = keys[0, c * j:c * j + c]
            planes = [tree.tau * q @ (scipy.special.softmax(tree.tau * k @ qr) @ k)
                      + scipy.special.logsumexp(tree.tau * k @ qr)
                      - tree.tau * qr @ (scipy.special.softmax(tree.tau * k @ qr) @ k)
                      for qr in tree.qref[0]]
            sig.append(max(planes))
        sig = np.array(sig)
        pi = np.exp(sig - sig.max())
        pi /= pi.sum()
        order = sorted(range(n1), key=lambda j: (-pi[j], j))
        cum, kept = 0.0, []
        for j in order:
            kept.append(j)
            cum += pi[j]
            if cum >= p:
                break
        assert r.levels[0].kept.tolist() == sorted(kept)


@pytest.mark.parametrize("n", [1, 2, 3])
def test_p12_short_context_is_dense(n):
    """P12b: with N < c there is no complete chunk, so every token is attended (dense)."""
    d = 8
    keys, values, tree = _tree(1, n, d, 2, 4, 2, 80)
    q = RNG(81).normal(size=(2, d))
    out, routes = O.decode_step(q, keys, values, tree, 0.5)
    assert routes[0].tokens.tolist() == list(range(n))
    assert np.allclose(out, O.dense_decode(q, keys, values, n), atol=1e-14)


# ---------------------------------------------------------------- hand-derived golden examples

def _golden():
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        return json.load(f)


def _golden_cases():
    g = _golden()
    return [(ex, case) for ex in g["examples"] for case in ex["cases"]]


@pytest.mark.parametrize("ex,case", _golden_cases(), ids=lambda x: x.get("name", x.get("p")) if isinstance(x, dict) else str(x))
def test_golden_worked_examples(ex, case):
    g = _golden()
    d, c, L = g["head_dim"], g["chunk"], g["levels"]
    n = ex["n_tokens"]
    a = np.log(np.array(ex["exp_a"], dtype=np.float64))
    keys = np.zeros((1, n, d))
    keys[0, :, 0] = a                                  # tau * (2 e1) . (a e1) = a
    values = np.zeros((1, n, d))
    values[0, :, 1] = np.arange(n)
    values[0, :, 2] = 1.0
    q = np.zeros((1, d))
    q[0, 0] = 2.0
    tree = O.SummaryTree(keys, q[None].copy(), n, c, L)
    assert tree.tau == 0.5
    out, routes = O.decode_step(q, keys, values, tree, case["p"])
    for lv in routes[0].levels:
        assert lv.kept.tolist() == case["kept"][str(lv.level)]
        assert lv.margin > 1e-3
    assert routes[0].tokens.tolist() == case["tokens"]
    assert abs(out[0, 1] - float(Fraction(case["out_e2"]))) < 1e-12
    assert abs(out[0, 2] - 1.0) < 1e-12 and abs(out[0, 0]) < 1e-12


# ---------------------------------------------------------------- cut rule details

def test_cut_ties_break_by_ascending_index_and_margin_flags_them():
    sigma = np.array([1.0, 2.0, 2.0, 0.5])
    ids = np.array([10, 11, 12, 13])
    kept, pi, margin = O.top_p_cut(sigma, ids, 0.35)
    # 11 and 12 tie (pi = 0.386 each); 11 ranks first and alone reaches 0.35
    assert kept.tolist() == [11]
    assert margin == 0.0          # a tie straddles the cut: either side is correct


def test_cut_margin_terms():
    """The margin is the smallest of the two cumulative distances from p and the
    relative gap between the last kept and the first dropped probability."""
    pis = np.array([0.5, 0.25, 0.25 - 5e-5, 5e-5])
    sigma = np.log(pis)                      # softmax(log pi) = pi (they sum to 1)
    kept, pi, margin = O.top_p_cut(sigma, np.arange(4), 0.6)
    assert kept.tolist() == [0, 1]
    # S_K - p = 0.15, p - S_{K-1} = 0.1, relative tie gap 5e-5 / 0.25 = 2e-4
    assert abs(margin - 2e-4) < 1e-12
    kept, pi, margin = O.top_p_cut(sigma, np.arange(4), 0.75 - 5e-5)
    assert kept.tolist() == [0, 1] and abs(margin - 5e-5) < 1e-12      # S_K - p
    kept, pi, margin = O.top_p_cut(sigma, np.arange(4), 0.5 + 1e-6)
    assert kept.tolist() == [0, 1] and abs(margin - 1e-6) < 1e-12      # p - S_{K-1}


def test_cut_keeps_at_least_one_and_all_at_p_one():
    sigma = np.array([5.0, -5.0, -6.0])
    assert O.top_p_cut(sigma, np.arange(3), 1e-12)[0].tolist() == [0]
    assert sorted(O.top_p_cut(sigma, np.arange(3), 1.0)[0].tolist()) == [0, 1, 2]
    assert O.top_p_cut(sigma, np.arange(3), 1.0)[2] == math.inf


def test_bf16_bits_widen_exactly():
    x = torch.randn(1000).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.widen(bits), x.double().numpy())


# ---------------------------------------------------------------- narrow router planes (P14)

def test_p14_round_bf16_matches_library_rounding_of_float32_values():
    """On float32-representable inputs one rounding to bfloat16 is the library's own
    float32 -> bfloat16 conversion (round to nearest, ties to even)."""
    x32 = (torch.randn(20000, dtype=torch.float64) * torch.exp(torch.randn(20000, dtype=torch.float64) * 4)).float()
    ref = x32.to(torch.bfloat16).double().numpy()
    assert np.array_equal(O.round_bf16(x32.double().numpy()), ref)


def test_p14_round_bf16_hand_values():
    """bfloat16 spacing is 2**-7 on [1, 2): exact ties go to the even neighbour, values
    past a tie go up, signs are symmetric, and a float64 value just past a tie is not
    first rounded to float32 (that double rounding would land on the tie and go down)."""
    u = 2.0 ** -7
    cases = [
        (1.0 + u / 2, 1.0),                     # tie: 1 (even) vs 1 + u (odd)
        (1.0 + 3 * u / 2, 1.0 + 2 * u),         # tie: 1 + u (odd) vs 1 + 2u (even)
        (1.0 + u / 2 + 2.0 ** -30, 1.0 + u),    # just past the tie
        (1.0 + u / 2 + 2.0 ** -40, 1.0 + u),    # past the tie by less than float32 resolves
        (-(1.0 + 3 * u / 2), -(1.0 + 2 * u)),
        (3.0 * 2.0 ** 20 + 2.0 ** 13, 3.0 * 2.0 ** 20),   # spacing 2**14 on [2**21, 2**22): tie to even
        (0.0, 0.0),
        (2.0 ** -100 * (1 + u / 4), 2.0 ** -100),
    ]
    got = O.round_bf16(np.array([c[0] for c in cases]))
    assert got.tolist() == [c[1] for c in cases]


def test_p14_bf16_router_scores_use_rounded_planes_only():
    """A 'bf16' tree scores with s rounded to bfloat16 and b unchanged: the score equals
    the plane formula on round_bf16(s), and differs from the exact score by at most
    tau * sum_d |q_d| |s_d| 2**-8 (half a bfloat16 spacing per element)."""
    keys, _ = _rand_cache(1, 256, 32, seed=11)
    qref = RNG(12).normal(size=(1, 2, 32))
    t32 = O.SummaryTree(keys, qref, 256, 4, 2)
    t16 = O.SummaryTree(keys, qref, 256, 4, 2, plane_format="bf16")
    q = RNG(13).normal(size=32)
    nodes = np.arange(16)
    s, b, _ = t32.get(2, 0, nodes)
    s16, b16 = t16.router_planes(2, 0, nodes)
    assert np.array_equal(b16, b) and np.array_equal(s16, O.round_bf16(s))
    exact = O.plane_scores(q, s, b, t32.tau)
    narrow = O.plane_scores(q, s16, b16, t16.tau)
    bound = t32.tau * (np.abs(q)[None, None, :] * np.abs(s) * 2.0 ** -8).sum(-1).max(-1)
    assert np.all(np.abs(narrow - exact) <= bound + 1e-12)
    assert not np.array_equal(narrow, exact)
    with pytest.raises(ValueError):
        O.SummaryTree(keys, qref, 256, 4, 2, plane_format="fp4")


def test_p14_round_fp8_matches_library_rounding_of_scaled_float32_values():
    """Each plane divided by its power-of-two scale and rounded is the library's own
    float32 -> float8_e4m3fn conversion (round to nearest, ties to even), over planes
    whose magnitudes span many binades and reach the subnormals."""
    g = torch.Generator().manual_seed(5)
    s32 = (torch.randn(400, 2, 128, dtype=torch.float64, generator=g)
           * torch.exp(torch.randn(400, 2, 1, dtype=torch.float64, generator=g) * 5)
           * torch.exp(torch.randn(400, 2, 128, dtype=torch.float64, generator=g) * 2)).float()
    s = s32.double().numpy()
    k = O.fp8_plane_scale_exp(s)
    x = torch.from_numpy(np.ldexp(s, -k[..., None]))        # exact: power-of-two scaling
    assert torch.equal(x.float().double(), x)                # still float32-representable
    ref = np.ldexp(x.float().to(torch.float8_e4m3fn).double().numpy(), k[..., None])
    assert np.array_equal(O.round_fp8(s), ref)
    assert np.abs(np.ldexp(s, -k[..., None])).max() <= 448.0


def test_p14_fp8_scale_and_hand_values():
    """The scale puts a plane's largest magnitude in (224, 448]; E4M3 spacing is 2**-3
    on [1, 2), 32 on [256, 512) and 2**-9 below 2**-6 (subnormals); ties go to the
    even neighbour."""
    planes = np.array([[448.0, 1.0], [449.0, 1.0], [1.0, -0.5], [0.875, 0.1], [0.8750001, 0.1],
                       [0.0, 0.0], [-3.0, 2.0 ** -130]])
    assert O.fp8_plane_scale_exp(planes).tolist() == [0, 1, -8, -9, -8, 0, -7]
    u = 2.0 ** -9
    cases = [(1.0625, 1.0), (1.1875, 1.25), (1.97, 2.0), (-3.3, -3.25), (300.0, 288.0), (304.0, 320.0),
             (2.0 ** -10, 0.0), (1.5 * u, 2 * u), (2.5 * u, 2 * u), (0.51 * u, u), (2.0 ** -6 + u / 2, 2.0 ** -6),
             (0.0, 0.0)]
    x = np.array([[448.0] + [c[0] for c in cases]])          # scale 1 (k = 0) for every case
    got = O.round_fp8(x)[0, 1:]
    assert got.tolist() == [c[1] for c in cases]
    assert O.round_fp8(np.zeros((1, 4))).tolist() == [[0.0] * 4]


def test_p14_fp8_router_scores_use_rounded_planes_only():
    """An 'fp8' tree scores with s rounded to its scaled 8-bit form and b unchanged,
    within half a spacing per element of the exact score."""
    keys, _ = _rand_cache(1, 256, 32, seed=11)
    qref = RNG(12).normal(size=(1, 2, 32))
    t32 = O.SummaryTree(keys, qref, 256, 4, 2)
    t8 = O.SummaryTree(keys, qref, 256, 4, 2, plane_format="fp8")
    q = RNG(13).normal(size=32)
    nodes = np.arange(16)
    s, b, _ = t32.get(2, 0, nodes)
    s8, b8 = t8.router_planes(2, 0, nodes)
    assert np.array_equal(b8, b) and np.array_equal(s8, O.round_fp8(s))
    k = O.fp8_plane_scale_exp(s)[..., None]
    exact = O.plane_scores(q, s, b, t32.tau)
    narrow = O.plane_scores(q, s8, b8, t8.tau)
    half = np.maximum(2.0 ** -4 * np.abs(s), np.ldexp(1.0, k - 10))
    bound = t32.tau * (np.abs(q)[None, None, :] * half).sum(-1).max(-1)
    assert np.all(np.abs(narrow - exact) <= bound + 1e-12)
    assert not np.array_equal(narrow, exact)


# ---------------------------------------------------------------- router fidelity (P15)

def _route_kept(r):
    return {lv.level: lv.kept for lv in r.levels}


def test_p15_recall_is_one_everywhere_at_p_one():
    keys, _ = _rand_cache(1, 300, 16, seed=21)
    tree = O.SummaryTree(keys, RNG(22).normal(size=(1, 2, 16)), 300, 4, 3)
    q = RNG(23).normal(size=16) * 2
    r = O.route_head(q, tree, 0, 1.0)
    rec, cap = O.level_mass_recall(q, keys[0], _route_kept(r), r.tokens, 300, 4, 3, tree.tau)
    assert np.allclose(rec, 1.0, atol=1e-12) and abs(cap - 1.0) < 1e-12


def test_p15_recall_equals_node_logsumexp_form_and_is_monotone():
    """recall_l = sum over kept nodes n of e^{LSE_n - LSE} (node log-sum-exp over its raw
    keys, a separate formula) plus the mass of the tokens under no complete level-l
    node; it never grows going down the levels; captured = recall_1 plus the sink's
    mass when its chunk was dropped."""
    n, c, L, d = 203, 3, 3, 8
    keys, _ = _rand_cache(1, n, d, seed=31, scale=1.5)
    tree = O.SummaryTree(keys, RNG(32).normal(size=(1, 1, d)), n, c, L)
    for seed in range(6):
        q = RNG(40 + seed).normal(size=d) * 3
        r = O.route_head(q, tree, 0, 0.6)
        kept = _route_kept(r)
        rec, cap = O.level_mass_recall(q, keys[0], kept, r.tokens, n, c, L, tree.tau)
        z = tree.tau * (keys[0] @ q)
        lse_all = scipy.special.logsumexp(z)
        for level in range(1, L + 1):
            span = c ** level
            nl = n // span
            s = sum(math.exp(scipy.special.logsumexp(z[k * span:(k + 1) * span]) - lse_all) for k in kept[level])
            if nl * span < n:
                s += math.exp(scipy.special.logsumexp(z[nl * span:]) - lse_all)
            assert abs(rec[level - 1] - s) < 1e-12
        assert np.all(np.diff(rec) >= -1e-12)               # recall_1 <= recall_2 <= ... <= recall_L
        p0 = math.exp(z[0] - lse_all)
        sink_dropped = 0 not in set(kept[1].tolist())
        assert abs(cap - (rec[0] + (p0 if sink_dropped else 0.0))) < 1e-12

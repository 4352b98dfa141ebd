"""Plant plausible slips in the oracle (on the CPU) and check that a pin catches each.

Each mutation replaces one oracle function by a subtly wrong variant; at least
one pin from test_oracle_pins must then fail.  This guards the pins
themselves: a pin that cannot see a dropped term is not a pin.
"""
import math

import numpy as np
import pytest

import oracle as O
import oracle.zha_oracle as Z
import tests.test_oracle_pins as P

_orig_summarize = Z.summarize_nodes
_orig_cut = Z.top_p_cut
_orig_final = Z.final_token_set
_orig_attend = Z.attend
_orig_round = Z.round_bf16
_orig_recall = Z.level_mass_recall


def _recall_tail_dropped(q_h, keys_g, kept_by_level, tokens, n_tokens, chunk, levels, tau):
    # tokens under no complete node counted as dropped
    keys = O.widen(keys_g[:n_tokens])
    z = tau * (keys @ O.widen(q_h))
    p = np.exp(z - z.max())
    p /= p.sum()
    t = np.arange(n_tokens)
    rec = np.ones(levels)
    for level, kept in kept_by_level.items():
        rec[level - 1] = p[np.isin(t // chunk ** level, np.asarray(kept))].sum()
    return rec, float(p[np.asarray(tokens)].sum())


def _recall_unnormalised_by_level(q_h, keys_g, kept_by_level, tokens, n_tokens, chunk, levels, tau):
    rec, cap = _orig_recall(q_h, keys_g, kept_by_level, tokens, n_tokens, chunk, levels, tau)
    return rec[::-1].copy(), cap


def _round_truncate(x):
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.trunc(np.ldexp(m, 8)), e - 8)


def _round_via_float32(x):
    return _orig_round(np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64))


def _round_half_away(x):
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    y = np.ldexp(m, 8)
    return np.ldexp(np.sign(y) * np.floor(np.abs(y) + 0.5), e - 8)


def _summ_no_tau_in_b(keys_g, qref_g, chunk, level, nodes, tau):
    s, b, lse = _orig_summarize(keys_g, qref_g, chunk, level, nodes, tau)
    qref = O.widen(qref_g)
    return s, lse - np.einsum("rd,nrd->nr", qref, s), lse


def _summ_plain_mean(keys_g, qref_g, chunk, level, nodes, tau):
    s, b, lse = _orig_summarize(keys_g, qref_g, chunk, level, nodes, tau)
    span = chunk ** level
    qref = O.widen(qref_g)
    for i, n in enumerate(np.asarray(nodes)):
        mean = O.widen(keys_g[n * span:(n + 1) * span]).mean(0)
        s[i] = mean[None, :]
    return s, lse - tau * np.einsum("rd,nrd->nr", qref, s), lse


def _summ_sign_flip(keys_g, qref_g, chunk, level, nodes, tau):
    s, b, lse = _orig_summarize(keys_g, qref_g, chunk, level, nodes, tau)
    return s, -b, lse


def _cut_ties_desc(sigma, node_ids, p):
    return _orig_cut(sigma, -np.asarray(node_ids), p)[0] * -1, *_orig_cut(sigma, node_ids, p)[1:]


def _cut_global_softmax_floor(sigma, node_ids, p):
    # keeps one node fewer than needed whenever it can (exclusive cut)
    kept, pi, m = _orig_cut(sigma, node_ids, p)
    return (kept[:-1] if len(kept) > 1 else kept), pi, m


def _final_no_sink(kept_leaves, n_tokens, chunk):
    t = _orig_final(kept_leaves, n_tokens, chunk)
    kept = set((np.asarray(kept_leaves) * chunk).tolist())
    return t if 0 in kept else t[t != 0]


def _final_no_tail(kept_leaves, n_tokens, chunk):
    t = _orig_final(kept_leaves, n_tokens, chunk)
    return t[(t < chunk * (n_tokens // chunk)) | (t == 0)]


def _attend_no_max_shift_wrong_scale(q_h, keys_g, values_g, tokens, tau):
    return _orig_attend(q_h, keys_g, values_g, tokens, tau * 2)


def _route_no_orphans(q_h, tree, g, p):
    c, L, N = tree.chunk, tree.levels, tree.n_tokens
    route = Z.HeadRoute()
    kept_above = np.zeros(0, dtype=np.int64)
    for level in range(L, 0, -1):
        n_here = Z.n_complete(N, c, level)
        if level == L:
            cand = np.arange(n_here, dtype=np.int64)
        else:
            cand = np.sort((kept_above[:, None] * c + np.arange(c)[None, :]).ravel())
        if len(cand) == 0:
            lv = Z.LevelRoute(level, cand, np.zeros(0), np.zeros(0), cand, math.inf)
        else:
            s, b, _ = tree.get(level, g, cand)
            sigma = Z.plane_scores(q_h, s, b, tree.tau)
            kept, pi, margin = Z.top_p_cut(sigma, cand, p)
            lv = Z.LevelRoute(level, cand, sigma, pi, np.sort(kept), margin)
        route.levels.append(lv)
        kept_above = lv.kept
    route.tokens = Z.final_token_set(route.kept_leaves(), N, c)
    return route


_orig_fp8_scale = Z.fp8_plane_scale_exp


def _fp8_truncate(s, k=None):
    s = np.asarray(s, dtype=np.float64)
    k = _orig_fp8_scale(s)[..., None]
    x = np.ldexp(s, -k)
    _, ex = np.frexp(x)
    qe = np.maximum(ex, -5) - 4
    return np.ldexp(np.trunc(np.ldexp(x, -qe)), qe + k)


def _fp8_node_scale(s, k=None):
    s = np.asarray(s, dtype=np.float64)
    k = _orig_fp8_scale(s.reshape(s.shape[:-2] + (-1,)) if s.ndim >= 2 else s)
    k = k[..., None, None] if s.ndim >= 2 else k[..., None]
    x = np.ldexp(s, -k)
    _, ex = np.frexp(x)
    qe = np.maximum(ex, -5) - 4
    return np.ldexp(np.round(np.ldexp(x, -qe)), qe + k)


def _fp8_no_subnormals(s, k=None):
    s = np.asarray(s, dtype=np.float64)
    k = _orig_fp8_scale(s)[..., None]
    x = np.ldexp(s, -k)
    _, ex = np.frexp(x)
    qe = ex - 4
    y = np.ldexp(np.round(np.ldexp(x, -qe)), qe)
    return np.ldexp(np.where(np.abs(x) < 2.0 ** -6, 0.0, y), k)


def _fp8_scale_low(s):
    m = np.abs(np.asarray(s, dtype=np.float64)).max(axis=-1)
    _, e = np.frexp(m)
    return np.where(m == 0, 0, np.maximum(e - 9, -126)).astype(np.int64)


def _pins():
    """The pins run against every mutation (name, callable)."""
    out = []
    for sl, c in [(1, 4), (2, 4)]:
        out.append((f"p1[{sl},{c}]", lambda sl=sl, c=c: P.test_p1_plane_at_ref_query_is_exact_lse(sl, c)))
    out.append(("p2", P.test_p2_max_of_planes_never_exceeds_lse))
    out.append(("p3", P.test_p3_score_at_ref_query_equals_lse))
    out.append(("p4", lambda: P.test_p4_identical_keys_closed_form(2, 4)))
    out.append(("p7", lambda: P.test_p7_p_one_reproduces_dense(100)))
    out.append(("p8", P.test_p8_tiny_p_is_argmax_descent))
    for args in [(60, 4, 2, 0.6, 41), (63, 2, 3, 0.7, 42)]:
        out.append((f"p9{args}", lambda a=args: P.test_p9_brute_force_small(*a)))
    out.append(("p11", P.test_p11_dense_is_textbook_attention))
    for ex, case in P._golden_cases():
        out.append((f"golden[{ex['name']},{case['p']}]", lambda ex=ex, case=case: P.test_golden_worked_examples(ex, case)))
    out.append(("ties", P.test_cut_ties_break_by_ascending_index_and_margin_flags_them))
    out.append(("p14-library", P.test_p14_round_bf16_matches_library_rounding_of_float32_values))
    out.append(("p14-hand", P.test_p14_round_bf16_hand_values))
    out.append(("p14-scores", P.test_p14_bf16_router_scores_use_rounded_planes_only))
    out.append(("p14-fp8-library", P.test_p14_round_fp8_matches_library_rounding_of_scaled_float32_values))
    out.append(("p14-fp8-hand", P.test_p14_fp8_scale_and_hand_values))
    out.append(("p14-fp8-scores", P.test_p14_fp8_router_scores_use_rounded_planes_only))
    out.append(("p15-one", P.test_p15_recall_is_one_everywhere_at_p_one))
    out.append(("p15-lse", P.test_p15_recall_equals_node_logsumexp_form_and_is_monotone))
    return out


MUTATIONS = {
    "b_without_tau": ("summarize_nodes", _summ_no_tau_in_b),
    "s_plain_mean": ("summarize_nodes", _summ_plain_mean),
    "b_sign_flip": ("summarize_nodes", _summ_sign_flip),
    "ties_by_descending_index": ("top_p_cut", _cut_ties_desc),
    "cut_one_short": ("top_p_cut", _cut_global_softmax_floor),
    "no_sink": ("final_token_set", _final_no_sink),
    "no_tail": ("final_token_set", _final_no_tail),
    "wrong_attention_scale": ("attend", _attend_no_max_shift_wrong_scale),
    "no_orphans": ("route_head", _route_no_orphans),
    "bf16_truncates": ("round_bf16", _round_truncate),
    "bf16_double_rounding_via_float32": ("round_bf16", _round_via_float32),
    "bf16_ties_away_from_zero": ("round_bf16", _round_half_away),
    "fp8_truncates": ("round_fp8", _fp8_truncate),
    "fp8_one_scale_per_node": ("round_fp8", _fp8_node_scale),
    "fp8_flushes_subnormals": ("round_fp8", _fp8_no_subnormals),
    "fp8_scale_one_binade_low": ("fp8_plane_scale_exp", _fp8_scale_low),
    "recall_drops_the_tail": ("level_mass_recall", _recall_tail_dropped),
    "recall_levels_reversed": ("level_mass_recall", _recall_unnormalised_by_level),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_each_planted_slip_is_caught(name, monkeypatch):
    fn_name, bad = MUTATIONS[name]
    monkeypatch.setattr(Z, fn_name, bad)
    monkeypatch.setattr(O, fn_name, bad, raising=False)
    caught = []
    for pin_name, pin in _pins():
        try:
            pin()
        except AssertionError:
            caught.append(pin_name)
    assert caught, f"no pin caught the planted slip {name}"


def test_pins_pass_on_the_unmutated_oracle():
    for pin_name, pin in _pins():
        pin()

"""Batched multi-query decode (zha_decode_batch): a batch of queries over one cache and
tree, routed by one launch sequence, against the fp64 oracle query by query, and
against zha_decode_step on each query alone (identical selections; outputs equal up
to the attention's summation order)."""
import numpy as np
import pytest
import torch

import oracle as O
from hierarchical_tree_indexed_zha_amd import workloads as W
from tests.gpu_util import ATOL, MARGIN, make_layer, oracle_tree, say, to_host

pytestmark = pytest.mark.gpu


def _w(name, n, levels=None, steps=8, **kw):
    return W.scaled(W.get(name), n, steps=steps, levels=levels, **kw)


CASES = [
    ("tiny", W.get("tiny"), 3),
    ("light@32768", _w("light", 32768), 4),
    ("deep@16384", _w("deep", 16384, levels=6), 3),
    ("ultra@65536", _w("ultra", 65536, levels=5), 2),
    ("light@600000", _w("light", 600000, levels=4), 2),
]


@pytest.mark.parametrize("name,w,nq", CASES, ids=[c[0] for c in CASES])
def test_batch_matches_single_and_oracle(name, w, nq):
    say(f"[batch] {name}: {nq} queries")
    layer, x = make_layer(w)
    n = w.n_tokens
    layer.build(n)
    q = x["q"][:nq].contiguous()
    sel_b = torch.zeros((nq,) + layer.sel_shape(), dtype=torch.int32, device=q.device)
    out_b = layer.decode_batch(q, sel=sel_b).clone()
    torch.cuda.synchronize()
    kh, tree = oracle_tree(layer, n)
    vh = to_host(layer.v)
    G = w.n_q_heads // w.n_kv_heads
    checked = exempt = 0
    for i in range(nq):
        sel1 = layer.new_sel()
        out1 = layer.decode(q[i], sel=sel1).clone()
        torch.cuda.synchronize()
        assert torch.equal(sel_b[i], sel1), f"{name} query {i}: batch selection differs from the single step's"
        d1 = float((out_b[i] - out1).abs().max())
        assert d1 <= 1e-4, f"{name} query {i}: batch vs single output {d1:.3g}"
        qh = to_host(q[i])
        leaves = layer.read_sel(sel_b[i])
        ob = out_b[i].cpu().numpy().astype(np.float64)
        for h in range(w.n_q_heads):
            g = h // G
            toks = O.final_token_set(np.asarray(leaves[h], dtype=np.int64), n, w.chunk)
            ref = O.attend(qh[h], kh[g], vh[g], toks, tree.tau)
            assert float(np.abs(ob[h] - ref).max()) <= ATOL, f"{name} query {i} head {h}: attention"
            if h % 4 == 0:
                r = O.route_head(qh[h], tree, g, w.top_p)
                checked += 1
                if r.min_margin < MARGIN:
                    exempt += 1
                    continue
                assert leaves[h] == r.kept_leaves().tolist(), f"{name} query {i} head {h}: kept leaves"
    say(f"[batch] {name}: {nq} queries, {checked} routed heads against the oracle ({exempt} ambiguous)")


def test_batch_after_appends_and_timing():
    """light's shape with appends, a batch of 8 against 8 single steps: identical
    selections, and the batch's device time reported."""
    w = _w("light", 131072, levels=4, steps=16)
    layer, x = make_layer(w)
    layer.build(w.n_tokens)
    for t in range(9):
        layer.append(x["k_app"][t], x["v_app"][t])
    q = x["q"][:8].contiguous()
    sel_b = torch.zeros((8,) + layer.sel_shape(), dtype=torch.int32, device=q.device)
    layer.decode_batch(q, sel=sel_b)
    for i in range(8):
        sel1 = layer.new_sel()
        layer.decode(q[i], sel=sel1)
        assert torch.equal(sel_b[i], sel1), f"query {i}"
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for _ in range(3):
        layer.decode_batch(q)
    e[0].record()
    for _ in range(10):
        layer.decode_batch(q)
    e[1].record()
    for _ in range(10):
        for i in range(8):
            layer.decode(q[i])
    e[2].record()
    torch.cuda.synchronize()
    tb = e[0].elapsed_time(e[1]) / 10 * 1e3
    ts = e[1].elapsed_time(e[2]) / 10 * 1e3
    say(f"[batch] light@131072+9, 8 queries: batch {tb:.1f} us, 8 single steps {ts:.1f} us")

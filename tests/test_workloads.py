"""Seeded input generators: determinism (P13) and the shapes/distributions they promise (CPU)."""
import math

import torch

from hierarchical_tree_indexed_zha_amd import workloads as W


def test_p13_same_seed_same_bytes():
    for name in ["tiny", "light", "deep", "ultra"]:
        w = W.scaled(W.get(name), 4096, steps=3)
        a, b = W.generate(w), W.generate(w)
        assert a.keys() == b.keys()
        for k in a:
            assert torch.equal(a[k].view(torch.uint8) if a[k].dtype == torch.bfloat16 else a[k],
                               b[k].view(torch.uint8) if b[k].dtype == torch.bfloat16 else b[k])
        c = W.generate(w, seed=12345)
        assert not torch.equal(a["k"].float(), c["k"].float())


def test_shapes_and_dtypes_follow_workload():
    w = W.scaled(W.get("light"), 8192, steps=5)
    x = W.generate(w)
    assert x["k"].shape == (4, 8192 + 5, 128) and x["k"].dtype == torch.bfloat16
    assert x["ref_q"].shape == (4, 1, 128) and x["ref_q"].dtype == torch.float32
    assert x["q"].shape == (5, 32, 128) and x["k_app"].shape == (5, 4, 128)
    assert torch.count_nonzero(x["k"][:, 8192:].float()) == 0


def test_full_size_configs_match_the_named_shapes():
    assert W.get("light").levels == W.levels_for(262144, 8) == 4
    assert 262144 // 4 ** 6 == 64 and W.get("deep").levels == 6
    assert 10485760 // 8 ** 7 == 5 and W.get("ultra").levels == 7
    assert 16384 // 4 ** 6 == 4 and W.get("tiny").levels == 6
    assert W.get("wide").chunk == 256 and W.get("wide").levels == 1


def test_tiny_needles_and_query_correlation():
    w = W.get("tiny")
    x = W.generate(w)
    k = x["k"][0]
    norms = k.norm(dim=1)
    # 4 planted needles have norm ~6, the N(0,1) background ~sqrt(128)
    assert int((norms < 8).sum()) == 4
    qhat = k[norms < 8].mean(0)
    qhat = qhat / qhat.norm()
    cos = (x["q"].reshape(-1, 128) @ qhat) / x["q"].reshape(-1, 128).norm(dim=1)
    assert 0.45 < float(cos.min()) and float(cos.max()) < 0.95
    assert abs(float(x["q"].reshape(-1, 128).norm(dim=1).mean()) - math.sqrt(128)) < 0.5


def test_topic_needles_match_their_queries():
    w = W.scaled(W.get("deep"), 16384, steps=4)
    x = W.generate(w)
    q = x["q"].float()
    for g in range(4):
        qbar = q[:, 8 * g:8 * g + 8].mean(1)           # [steps, d]
        sims = (x["k"][g].float() @ qbar.T)             # tokens x steps
        # each step's needle: 16 tokens whose key is ~qbar
        for t in range(4):
            close = ((x["k"][g].float() - qbar[t]).norm(dim=1) < 3.0).sum()
            assert int(close) >= 16
        assert sims.shape[1] == 4

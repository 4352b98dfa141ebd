"""The no-allocation decode entry point (library-held scratch) against zha_decode_step
(caller scratch): the same kernels, so the outputs must be identical, on two calls in a
row on one GPU, the second with a smaller input than the first."""
import pytest
import torch

from hierarchical_tree_indexed_zha_amd import binding as B
from hierarchical_tree_indexed_zha_amd import workloads as W
from tests.gpu_util import make_layer, say

pytestmark = pytest.mark.gpu


def _noalloc(layer, q, n):
    out = torch.full_like(layer.out, float("nan"))
    B.zha_decode_step_noalloc(layer.cfg, layer.k, layer.v, layer.tree, n, q, out)
    return out


def test_noalloc_matches_decode_step_twice_shrinking():
    cases = [("light (262,144 tokens)", W.get("light"), None),
             ("deep@16384", W.scaled(W.get("deep"), 16384, steps=2, levels=6), None)]
    for name, w, n in cases:
        n = w.n_tokens if n is None else n
        cfg = B.config_of(w)
        assert B.zha_scratch_bytes(cfg) <= B.NOALLOC_SCRATCH_BYTES
        say(f"[noalloc] {name}: n={n}, scratch {B.zha_scratch_bytes(cfg)} bytes")
        layer, x = make_layer(w)
        layer.build(n)
        for t in range(2):
            q = x["q"][t]
            ref = layer.decode(q).clone()
            got = _noalloc(layer, q, n)
            torch.cuda.synchronize()
            assert torch.equal(ref, got), f"{name} step {t}: max diff {(ref - got).abs().max().item()}"
        del layer, x
        torch.cuda.empty_cache()


def test_noalloc_rejects_oversized_configs_before_launching():
    w = W.get("ultra")
    cfg = B.config_of(w)
    assert B.zha_scratch_bytes(cfg) > B.NOALLOC_SCRATCH_BYTES
    fake = 4096
    with pytest.raises(B.ZhaError) as e:
        B.zha_decode_step_noalloc(cfg, fake, fake, fake, w.n_tokens, fake, fake, stream=0)
    assert e.value.code == B.ZHA_ERR_UNSUPPORTED and "no-allocation" in B.last_error()

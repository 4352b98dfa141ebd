"""The C ABI library loads, exports every symbol include/zha.h declares, and validates
arguments on the host (no GPU and no compute calls needed)."""
import ctypes
import os
import re

import pytest

from hierarchical_tree_indexed_zha_amd import binding as B
from hierarchical_tree_indexed_zha_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "zha.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert "zha_decode_step" in names and "dense_decode" in names and len(names) >= 12
    lib = B.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(B.EXPORTS) == names


def _cfg(**kw):
    base = dict(n_kv_heads=4, n_q_heads=32, head_dim=128, chunk=8, levels=4, n_ref=1, top_p=0.75,
                kv_dtype="bf16", capacity=262144)
    base.update(kw)
    return B.make_config(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(n_kv_heads=0), B.ZHA_ERR_ARG),
    (dict(n_q_heads=30), B.ZHA_ERR_ARG),
    (dict(n_q_heads=4 * 17), B.ZHA_ERR_UNSUPPORTED),
    (dict(head_dim=64), B.ZHA_ERR_UNSUPPORTED),
    (dict(head_dim=0), B.ZHA_ERR_ARG),
    (dict(chunk=1), B.ZHA_ERR_ARG),
    (dict(chunk=2048), B.ZHA_ERR_UNSUPPORTED),
    (dict(levels=0), B.ZHA_ERR_ARG),
    (dict(n_ref=0), B.ZHA_ERR_ARG),
    (dict(n_ref=3), B.ZHA_ERR_UNSUPPORTED),
    (dict(n_ref=64), B.ZHA_ERR_UNSUPPORTED),
    (dict(top_p=0.0), B.ZHA_ERR_ARG),
    (dict(top_p=1.5), B.ZHA_ERR_ARG),
    (dict(top_p=float("nan")), B.ZHA_ERR_ARG),
    (dict(kv_dtype=7), B.ZHA_ERR_ARG),
    (dict(capacity=0), B.ZHA_ERR_ARG),
    (dict(capacity=1 << 31), B.ZHA_ERR_UNSUPPORTED),
])
def test_config_validation(kw, code):
    with pytest.raises(B.ZhaError) as e:
        B.zha_check_config(_cfg(**kw))
    assert e.value.code == code
    assert B.last_error()


def test_valid_configs_pass_and_sizes_match_layout():
    for name in W.WORKLOADS:
        w = W.get(name)
        cfg = B.config_of(w)
        B.zha_check_config(cfg)
        # tree: per level, H_kv * n_cap * R * (d + 2) floats (planes, b, lse), 256-byte aligned pieces
        expect = 0
        for lv in range(1, w.levels + 1):
            n = w.capacity // w.chunk ** lv
            for nbytes in (4 * w.n_kv_heads * n * w.n_ref * w.head_dim, 4 * w.n_kv_heads * n * w.n_ref,
                           4 * w.n_kv_heads * n * w.n_ref):
                expect += (nbytes + 255) // 256 * 256
        assert B.zha_tree_bytes(cfg) == expect
        assert B.zha_scratch_bytes(cfg) > 0 and B.zha_dense_scratch_bytes(cfg) > 0
        o = B.zha_tree_level_offsets(cfg, w.levels)
        assert o["n_cap"] == w.capacity // w.chunk ** w.levels
        r = B.zha_route_level_offsets(cfg, 1)
        assert r["n_cap"] == w.capacity // w.chunk
        assert max(r["n_cand"], r["sigma"], r["kept"], r["mask"], r["stats"]) < B.zha_scratch_bytes(cfg)


def test_entry_points_reject_bad_arguments_before_touching_the_device():
    cfg = _cfg(capacity=1000)
    fake = 4096   # never dereferenced: validation fails first
    bufs = B.Buffers(fake, fake, fake, fake, fake)
    cases = [
        (lambda: B.zha_build_tree(cfg, bufs, 1001, 0), B.ZHA_ERR_CAPACITY),
        (lambda: B.zha_build_tree(cfg, bufs, -1, 0), B.ZHA_ERR_ARG),
        (lambda: B.zha_build_tree(cfg, B.Buffers(None, fake, fake, fake, fake), 10, 0), B.ZHA_ERR_ARG),
        (lambda: B.zha_append_token(cfg, bufs, 1000, fake, fake, 0), B.ZHA_ERR_CAPACITY),
        (lambda: B.zha_append_token(cfg, bufs, 10, None, fake, 0), B.ZHA_ERR_ARG),
        (lambda: B.zha_decode_step(cfg, bufs, 0, fake, fake, 0), B.ZHA_ERR_ARG),
        (lambda: B.zha_decode_step(cfg, bufs, 1001, fake, fake, 0), B.ZHA_ERR_CAPACITY),
        (lambda: B.zha_decode_step(cfg, B.Buffers(fake, fake, fake, fake, None), 10, fake, fake, 0), B.ZHA_ERR_ARG),
        (lambda: B.dense_decode(cfg, fake, fake, 1001, fake, fake, fake, 0), B.ZHA_ERR_CAPACITY),
        (lambda: B.dense_decode(cfg, fake, fake, 10, fake, fake, None, 0), B.ZHA_ERR_ARG),
        (lambda: B.zha_tree_level_offsets(cfg, 0), B.ZHA_ERR_ARG),
        (lambda: B.zha_route_level_offsets(cfg, 5), B.ZHA_ERR_ARG),
    ]
    for fn, code in cases:
        with pytest.raises(B.ZhaError) as e:
            fn()
        assert e.value.code == code, B.last_error()


def test_null_config_is_rejected():
    lib = B.lib()
    assert lib.zha_check_config(None) == B.ZHA_ERR_ARG
    assert lib.zha_tree_bytes(None) == 0
    assert b"NULL" in lib.zha_last_error()

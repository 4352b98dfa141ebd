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


def _base():
    return dict(n_kv_heads=4, n_q_heads=32, head_dim=128, chunk=8, levels=4, n_ref=1, top_p=0.75,
                kv_dtype="bf16", capacity=262144)


def _cfg(**kw):
    base = _base()
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
    (dict(sink=0), B.ZHA_ERR_UNSUPPORTED),
    (dict(sink=2), B.ZHA_ERR_ARG),
    (dict(sink=-1), B.ZHA_ERR_ARG),
    (dict(plane_format=3), B.ZHA_ERR_ARG),
    (dict(plane_format=-1), B.ZHA_ERR_ARG),
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
        assert B.zha_sel_bytes(cfg) == 4 * w.n_q_heads * (w.capacity // w.chunk + 1)
        o = B.zha_tree_level_offsets(cfg, w.levels)
        assert o["n_cap"] == w.capacity // w.chunk ** w.levels
        assert o["s16"] == o["s8"] == o["sc"] == -1
        r = B.zha_route_level_offsets(cfg, w.n_tokens, 1)
        assert r["n_cap"] == w.capacity // w.chunk
        assert max(r["n_cand"], r["sigma"], r["kept"], r["mask"], r["stats"]) < B.zha_scratch_bytes(cfg)


def test_narrow_plane_layouts():
    """bf16 planes add a [H][n][R][d] 2-byte copy per level; 8-bit planes a 1-byte copy
    and a float32 scale per plane, each 256-byte aligned after the float32 pieces."""
    w = W.get("light")
    base = B.zha_tree_bytes(B.config_of(w))
    al = lambda x: (x + 255) // 256 * 256
    extra16 = extra8 = 0
    for lv in range(1, w.levels + 1):
        n = w.capacity // w.chunk ** lv
        extra16 += al(2 * w.n_kv_heads * n * w.n_ref * w.head_dim)
        extra8 += al(w.n_kv_heads * n * w.n_ref * w.head_dim) + al(4 * w.n_kv_heads * n * w.n_ref)
    c16, c8 = B.config_of(w, plane_format="bf16"), B.config_of(w, plane_format="fp8")
    assert B.zha_tree_bytes(c16) == base + extra16
    assert B.zha_tree_bytes(c8) == base + extra8
    o16, o8 = B.zha_tree_level_offsets(c16, 1), B.zha_tree_level_offsets(c8, 1)
    assert o16["s16"] > o16["lse"] and o16["s8"] == o16["sc"] == -1
    assert o8["s16"] == -1 and o8["lse"] < o8["s8"] < o8["sc"] and o8["s8"] % 256 == 0 and o8["sc"] % 256 == 0


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
        (lambda: B.zha_decode_step(cfg, bufs, 0, fake, fake, stream=0), B.ZHA_ERR_ARG),
        (lambda: B.zha_decode_step(cfg, bufs, 1001, fake, fake, fake, fake, stream=0), B.ZHA_ERR_CAPACITY),
        (lambda: B.zha_decode_step(cfg, B.Buffers(fake, fake, fake, fake, None), 10, fake, fake, stream=0),
         B.ZHA_ERR_ARG),
        (lambda: B.zha_decode_step(B.make_config(**{**_base(), "capacity": 1000, "sink": 0}), bufs, 10, fake, fake,
                                   stream=0), B.ZHA_ERR_UNSUPPORTED),
        (lambda: B.zha_decode_step_traced(cfg, bufs, 10, fake, fake, [], stream=0), B.ZHA_ERR_ARG),
        (lambda: B.zha_decode_batch(cfg, bufs, 10, 0, fake, fake, stream=0), B.ZHA_ERR_ARG),
        (lambda: B.zha_decode_batch(cfg, bufs, 1001, 2, fake, fake, stream=0), B.ZHA_ERR_CAPACITY),
        (lambda: B.zha_batch_scratch_bytes(cfg, 0), B.ZHA_ERR_ARG),
        (lambda: B.zha_decode_step_traced(cfg, bufs, 10, fake, fake, [fake, None], stream=0), B.ZHA_ERR_ARG),
        (lambda: B.dense_decode(cfg, fake, fake, 1001, fake, fake, fake, 0), B.ZHA_ERR_CAPACITY),
        (lambda: B.dense_decode(cfg, fake, fake, 10, fake, fake, None, 0), B.ZHA_ERR_ARG),
        (lambda: B.zha_tree_level_offsets(cfg, 0), B.ZHA_ERR_ARG),
        (lambda: B.zha_route_level_offsets(cfg, 10, 5), B.ZHA_ERR_ARG),
        (lambda: B.zha_route_level_offsets(cfg, 0, 1), B.ZHA_ERR_ARG),
        (lambda: B.zha_route_level_offsets(cfg, 1001, 1), B.ZHA_ERR_ARG),
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


def test_stats_struct_layout_matches_header():
    """The ctypes mirror of zha_stats has the header's field order and size: two leading
    scalars (8 + 4 + 4 bytes), six per-level int64 arrays, two trailing int64 totals."""
    import ctypes
    n = B.STATS_MAX_LEVELS
    assert ctypes.sizeof(B.Stats) == 16 + 6 * 8 * n + 16
    src = open(os.path.join(ROOT, "include", "zha.h")).read()
    body = src[src.index("typedef struct zha_stats"):src.index("} zha_stats;")]
    names = re.findall(r"^\s*(?:int64_t|int32_t)\s+(\w+)", body, flags=re.M)
    assert names == [f for f, _ in B.Stats._fields_]
    assert f"#define ZHA_STATS_MAX_LEVELS {n}" in src


def test_config_struct_layout_matches_header():
    src = open(os.path.join(ROOT, "include", "zha.h")).read()
    body = src[src.index("typedef struct zha_config"):src.index("} zha_config;")]
    names = re.findall(r"^\s*(?:int64_t|int32_t|float)\s+(\w+)", body, flags=re.M)
    assert names == [f for f, _ in B.Config._fields_]


def test_chained_levels_follow_the_slot_and_plane_bounds():
    """The first routed levels form the chain while each has at most 8,192 node slots and
    together at most 32,768 planes per group; the rest are routed over group candidates."""
    def chained(name, n=None):
        w = W.get(name)
        n = w.n_tokens if n is None else n
        cfg = B.config_of(w, capacity=max(w.capacity, n))
        return [lv for lv in range(1, w.levels + 1) if B.zha_route_level_offsets(cfg, n, lv)["chained"]]
    assert chained("light") == [2, 3, 4]          # 4096 + 512 + 64 planes; level 1 has 32,768 slots
    assert chained("light", 262144 + 272) == [2, 3, 4]   # after the bench's appends: 4,100 level-2 nodes
    assert chained("tiny") == [2, 3, 4, 5, 6]     # R = 16: 21,824 planes; level 1 would add 65,536
    assert chained("deep") == [4, 5, 6]           # 1,344 nodes * 16 planes; level 3's 4,096 nodes would add 65,536 planes
    assert chained("wide") == [1]                 # 1,024 nodes * 16 planes
    assert chained("ultra") == [4, 5, 6, 7]       # 2,560 + 320 + 40 + 5 nodes
    assert chained("light", 100) == [1, 2]        # 12 level-1 nodes, one level-2 node
    assert chained("light", 60) == [1]            # only level 1 complete: 7 nodes


def test_batch_scratch_covers_every_query():
    """The batch's scratch grows with the number of queries and one query needs exactly
    the single step's scratch."""
    cfg = _cfg(capacity=50000)
    one = B.zha_scratch_bytes(cfg)
    assert B.zha_batch_scratch_bytes(cfg, 1) == one
    sizes = [B.zha_batch_scratch_bytes(cfg, q) for q in (1, 2, 4, 8)]
    assert all(b > a for a, b in zip(sizes, sizes[1:]))
    assert sizes[-1] >= 8 * (one // 2)

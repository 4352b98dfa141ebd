"""ctypes binding of libzha.so (C ABI in include/zha.h).

Argument marshalling only: every computation runs in the library's HIP
kernels.  Torch tensors are accepted wherever the ABI takes a device pointer;
the current torch HIP stream is passed as the stream.  A missing library is an
error (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libzha.so")

ZHA_OK = 0
ZHA_ERR_ARG = -1
ZHA_ERR_CAPACITY = -2
ZHA_ERR_UNSUPPORTED = -3
ZHA_ERR_HIP = -4
ZHA_BF16 = 0
ZHA_F32 = 1

EXPORTS = [
    "zha_check_config", "zha_tree_bytes", "zha_scratch_bytes", "zha_dense_scratch_bytes", "zha_sel_bytes",
    "zha_tree_level_offsets", "zha_route_level_offsets", "zha_build_tree", "zha_append_token",
    "zha_decode_step", "zha_decode_step_timed", "zha_decode_step_traced", "dense_decode", "zha_last_error",
    "zha_decode_step_noalloc", "zha_fidelity_work_bytes", "zha_route_fidelity", "zha_batch_scratch_bytes",
    "zha_decode_batch",
]
# kinds of a traced step's kernels (kinds[i] = 100 * kind + level)
TRACE_KINDS = {0: "start", 1: "score_all", 2: "chain", 3: "merge_ids", 4: "score", 5: "select", 6: "apply",
               7: "gather", 8: "combine", 9: "cross", 10: "resolve"}
NOALLOC_SCRATCH_BYTES = 32 << 20
STATS_MAX_LEVELS = 32


class ZhaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [
        ("n_kv_heads", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("chunk", ctypes.c_int32),
        ("levels", ctypes.c_int32),
        ("n_ref", ctypes.c_int32),
        ("top_p", ctypes.c_float),
        ("kv_dtype", ctypes.c_int32),
        ("capacity", ctypes.c_int64),
        ("sink", ctypes.c_int32),
        ("plane_format", ctypes.c_int32),
    ]


class Buffers(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("ref_q", ctypes.c_void_p),
        ("tree", ctypes.c_void_p),
        ("scratch", ctypes.c_void_p),
    ]


class Stats(ctypes.Structure):
    """zha_stats (include/zha.h): per-level counts and bytes of one decode step."""
    _fields_ = [
        ("n_tokens", ctypes.c_int64),
        ("top_level", ctypes.c_int32),
        ("levels", ctypes.c_int32),
        ("cand", ctypes.c_int64 * STATS_MAX_LEVELS),
        ("kept", ctypes.c_int64 * STATS_MAX_LEVELS),
        ("group_cand", ctypes.c_int64 * STATS_MAX_LEVELS),
        ("group_kept", ctypes.c_int64 * STATS_MAX_LEVELS),
        ("bytes_read", ctypes.c_int64 * STATS_MAX_LEVELS),
        ("bytes_streamed", ctypes.c_int64 * STATS_MAX_LEVELS),
        ("gather_tokens", ctypes.c_int64),
        ("gather_bytes", ctypes.c_int64),
    ]


def stats_from_bytes(raw: bytes) -> dict:
    """A zha_stats read back from device memory, as a dict of ints and lists (index l-1 = level l)."""
    st = Stats.from_buffer_copy(raw)
    out = {}
    for name, typ in Stats._fields_:
        v = getattr(st, name)
        out[name] = list(v) if hasattr(typ, "_length_") else int(v)
    return out


class RouteOffsets(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("n_cand", "sigma", "n_kept", "kept", "mask", "stats", "kbm", "n_cap",
                                              "wcap", "chained", "sig_stride")]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run `python -m hierarchical_tree_indexed_zha_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        cfgp = P(Config)
        sig = {
            "zha_check_config": (ctypes.c_int, [cfgp]),
            "zha_tree_bytes": (ctypes.c_size_t, [cfgp]),
            "zha_scratch_bytes": (ctypes.c_size_t, [cfgp]),
            "zha_dense_scratch_bytes": (ctypes.c_size_t, [cfgp]),
            "zha_sel_bytes": (ctypes.c_size_t, [cfgp]),
            "zha_tree_level_offsets": (ctypes.c_int, [cfgp, ctypes.c_int32, P(ctypes.c_int64), P(ctypes.c_int64),
                                                      P(ctypes.c_int64), P(ctypes.c_int64), P(ctypes.c_int64),
                                                      P(ctypes.c_int64), P(ctypes.c_int64)]),
            "zha_route_level_offsets": (ctypes.c_int, [cfgp, ctypes.c_int64, ctypes.c_int32, P(RouteOffsets)]),
            "zha_build_tree": (ctypes.c_int, [cfgp, P(Buffers), ctypes.c_int64, ctypes.c_void_p]),
            "zha_append_token": (ctypes.c_int, [cfgp, P(Buffers), ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_void_p]),
            "zha_decode_step": (ctypes.c_int, [cfgp, P(Buffers), ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
            "zha_decode_step_timed": (ctypes.c_int, [cfgp, P(Buffers), ctypes.c_int64, ctypes.c_void_p,
                                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                     P(ctypes.c_void_p), ctypes.c_void_p]),
            "zha_decode_step_traced": (ctypes.c_int, [cfgp, P(Buffers), ctypes.c_int64, ctypes.c_void_p,
                                                      ctypes.c_void_p, P(ctypes.c_void_p), ctypes.c_int32,
                                                      P(ctypes.c_int32), P(ctypes.c_int32), ctypes.c_void_p]),
            "zha_fidelity_work_bytes": (ctypes.c_size_t, [cfgp, ctypes.c_int64]),
            "zha_batch_scratch_bytes": (ctypes.c_size_t, [cfgp, ctypes.c_int32]),
            "zha_decode_batch": (ctypes.c_int, [cfgp, P(Buffers), ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
            "zha_route_fidelity": (ctypes.c_int, [cfgp, P(Buffers), ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                                  ctypes.c_void_p, ctypes.c_void_p]),
            "dense_decode": (ctypes.c_int, [cfgp, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
            "zha_last_error": (ctypes.c_char_p, []),
            "zha_decode_step_noalloc": (ctypes.c_int, [cfgp, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                       ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                                       ctypes.c_void_p]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().zha_last_error().decode()


def _check(rc: int):
    if rc != ZHA_OK:
        raise ZhaError(rc, last_error())


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


PLANE_FORMATS = {"f32": 0, "bf16": 1, "fp8": 2}   # ZHA_PLANES_F32, ZHA_PLANES_BF16, ZHA_PLANES_FP8


def make_config(n_kv_heads, n_q_heads, head_dim, chunk, levels, n_ref, top_p, kv_dtype, capacity, sink=1,
                plane_format=0) -> Config:
    if isinstance(kv_dtype, str):
        kv_dtype = ZHA_BF16 if kv_dtype == "bf16" else ZHA_F32
    if isinstance(plane_format, str):
        plane_format = PLANE_FORMATS[plane_format]
    return Config(n_kv_heads, n_q_heads, head_dim, chunk, levels, n_ref, top_p, kv_dtype, capacity, sink,
                  plane_format)


def config_of(w, capacity: int | None = None, plane_format=0) -> Config:
    """Config of a workloads.Workload (router planes float32 unless plane_format says otherwise)."""
    return make_config(w.n_kv_heads, w.n_q_heads, w.head_dim, w.chunk, w.levels, w.n_ref, w.top_p, w.kv_dtype,
                       w.capacity if capacity is None else capacity, plane_format=plane_format)


def zha_check_config(cfg: Config) -> None:
    _check(lib().zha_check_config(ctypes.byref(cfg)))


def zha_tree_bytes(cfg: Config) -> int:
    n = lib().zha_tree_bytes(ctypes.byref(cfg))
    if n == 0:
        raise ZhaError(ZHA_ERR_ARG, last_error())
    return n


def zha_scratch_bytes(cfg: Config) -> int:
    n = lib().zha_scratch_bytes(ctypes.byref(cfg))
    if n == 0:
        raise ZhaError(ZHA_ERR_ARG, last_error())
    return n


def zha_dense_scratch_bytes(cfg: Config) -> int:
    n = lib().zha_dense_scratch_bytes(ctypes.byref(cfg))
    if n == 0:
        raise ZhaError(ZHA_ERR_ARG, last_error())
    return n


def zha_sel_bytes(cfg: Config) -> int:
    n = lib().zha_sel_bytes(ctypes.byref(cfg))
    if n == 0:
        raise ZhaError(ZHA_ERR_ARG, last_error())
    return n


def zha_tree_level_offsets(cfg: Config, level: int) -> dict:
    s, b, l, n, s16, s8, sc = (ctypes.c_int64() for _ in range(7))
    _check(lib().zha_tree_level_offsets(ctypes.byref(cfg), level, ctypes.byref(s), ctypes.byref(b), ctypes.byref(l),
                                        ctypes.byref(n), ctypes.byref(s16), ctypes.byref(s8), ctypes.byref(sc)))
    return {"s": s.value, "b": b.value, "lse": l.value, "n_cap": n.value, "s16": s16.value, "s8": s8.value,
            "sc": sc.value}


def zha_route_level_offsets(cfg: Config, n_tokens: int, level: int) -> dict:
    o = RouteOffsets()
    _check(lib().zha_route_level_offsets(ctypes.byref(cfg), n_tokens, level, ctypes.byref(o)))
    return {n: getattr(o, n) for n, _ in RouteOffsets._fields_}


def buffers(k, v, ref_q, tree, scratch) -> Buffers:
    return Buffers(_ptr(k), _ptr(v), _ptr(ref_q), _ptr(tree), _ptr(scratch))


def zha_build_tree(cfg: Config, bufs: Buffers, n_tokens: int, stream=None) -> None:
    _check(lib().zha_build_tree(ctypes.byref(cfg), ctypes.byref(bufs), n_tokens, _stream(stream)))


def zha_append_token(cfg: Config, bufs: Buffers, n_before: int, k_new, v_new, stream=None) -> None:
    _check(lib().zha_append_token(ctypes.byref(cfg), ctypes.byref(bufs), n_before, _ptr(k_new), _ptr(v_new),
                                  _stream(stream)))


def zha_decode_step(cfg: Config, bufs: Buffers, n_tokens: int, q, out, sel=None, stats=None,
                    stream=None) -> None:
    """sel: None or device int32 [H_q][1 + capacity // chunk]; stats: None or a device buffer of
    ctypes.sizeof(Stats) bytes."""
    _check(lib().zha_decode_step(ctypes.byref(cfg), ctypes.byref(bufs), n_tokens, _ptr(q), _ptr(out), _ptr(sel),
                                 _ptr(stats), _stream(stream)))


def zha_decode_step_timed(cfg: Config, bufs: Buffers, n_tokens: int, q, out, events, sel=None, stats=None,
                          stream=None) -> None:
    """events: four raw hipEvent_t handles (ints, or None) recorded around the step's phases."""
    arr = (ctypes.c_void_p * 4)(*[e if e else None for e in events])
    _check(lib().zha_decode_step_timed(ctypes.byref(cfg), ctypes.byref(bufs), n_tokens, _ptr(q), _ptr(out),
                                       _ptr(sel), _ptr(stats), arr, _stream(stream)))


def zha_decode_step_traced(cfg: Config, bufs: Buffers, n_tokens: int, q, out, events, stream=None):
    """events: raw hipEvent_t handles (ints), one recorded before the step and one after each
    kernel.  Returns [(kind name, level)] for events[0 .. n) as recorded."""
    n_ev = len(events)
    arr = (ctypes.c_void_p * n_ev)(*events)
    kinds = (ctypes.c_int32 * n_ev)()
    got = ctypes.c_int32(0)
    _check(lib().zha_decode_step_traced(ctypes.byref(cfg), ctypes.byref(bufs), n_tokens, _ptr(q), _ptr(out), arr,
                                        n_ev, kinds, ctypes.byref(got), _stream(stream)))
    return [(TRACE_KINDS.get(kinds[i] // 100, "?"), kinds[i] % 100) for i in range(got.value)]


def zha_batch_scratch_bytes(cfg: Config, n_queries: int) -> int:
    n = lib().zha_batch_scratch_bytes(ctypes.byref(cfg), n_queries)
    if n == 0:
        raise ZhaError(ZHA_ERR_ARG, last_error())
    return n


def zha_decode_batch(cfg: Config, bufs: Buffers, n_tokens: int, n_queries: int, q, out, sel=None,
                     stream=None) -> None:
    _check(lib().zha_decode_batch(ctypes.byref(cfg), ctypes.byref(bufs), n_tokens, n_queries, _ptr(q), _ptr(out),
                                  _ptr(sel), _stream(stream)))


def zha_fidelity_work_bytes(cfg: Config, n_tokens: int) -> int:
    n = lib().zha_fidelity_work_bytes(ctypes.byref(cfg), n_tokens)
    if n == 0:
        raise ZhaError(ZHA_ERR_ARG, last_error())
    return n


def zha_route_fidelity(cfg: Config, bufs: Buffers, n_tokens: int, q, recall, work, stream=None) -> None:
    _check(lib().zha_route_fidelity(ctypes.byref(cfg), ctypes.byref(bufs), n_tokens, _ptr(q), _ptr(recall),
                                    _ptr(work), _stream(stream)))


def dense_decode(cfg: Config, k, v, n_tokens: int, q, out, scratch, stream=None) -> None:
    _check(lib().dense_decode(ctypes.byref(cfg), _ptr(k), _ptr(v), n_tokens, _ptr(q), _ptr(out), _ptr(scratch),
                              _stream(stream)))


def zha_decode_step_noalloc(cfg: Config, k, v, tree, n_tokens: int, q, out, stream=None) -> None:
    """zha_decode_step on the library's own per-GPU scratch (no caller scratch, nothing allocated)."""
    _check(lib().zha_decode_step_noalloc(ctypes.byref(cfg), _ptr(k), _ptr(v), _ptr(tree), n_tokens, _ptr(q),
                                         _ptr(out), _stream(stream)))

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
    "zha_check_config", "zha_tree_bytes", "zha_scratch_bytes", "zha_dense_scratch_bytes",
    "zha_tree_level_offsets", "zha_route_level_offsets", "zha_build_tree", "zha_append_token",
    "zha_decode_step", "zha_decode_step_timed", "dense_decode", "zha_last_error",
]


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
    ]


class Buffers(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("ref_q", ctypes.c_void_p),
        ("tree", ctypes.c_void_p),
        ("scratch", ctypes.c_void_p),
    ]


class RouteOffsets(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("n_cand", "sigma", "n_kept", "kept", "mask", "stats", "n_cap")]


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
            "zha_tree_level_offsets": (ctypes.c_int, [cfgp, ctypes.c_int32, P(ctypes.c_int64), P(ctypes.c_int64),
                                                      P(ctypes.c_int64), P(ctypes.c_int64)]),
            "zha_route_level_offsets": (ctypes.c_int, [cfgp, ctypes.c_int32, P(RouteOffsets)]),
            "zha_build_tree": (ctypes.c_int, [cfgp, P(Buffers), ctypes.c_int64, ctypes.c_void_p]),
            "zha_append_token": (ctypes.c_int, [cfgp, P(Buffers), ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_void_p]),
            "zha_decode_step": (ctypes.c_int, [cfgp, P(Buffers), ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_void_p]),
            "zha_decode_step_timed": (ctypes.c_int, [cfgp, P(Buffers), ctypes.c_int64, ctypes.c_void_p,
                                                     ctypes.c_void_p, P(ctypes.c_void_p), ctypes.c_void_p]),
            "dense_decode": (ctypes.c_int, [cfgp, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
            "zha_last_error": (ctypes.c_char_p, []),
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


def make_config(n_kv_heads, n_q_heads, head_dim, chunk, levels, n_ref, top_p, kv_dtype, capacity) -> Config:
    if isinstance(kv_dtype, str):
        kv_dtype = ZHA_BF16 if kv_dtype == "bf16" else ZHA_F32
    return Config(n_kv_heads, n_q_heads, head_dim, chunk, levels, n_ref, top_p, kv_dtype, capacity)


def config_of(w, capacity: int | None = None) -> Config:
    """Config of a workloads.Workload."""
    return make_config(w.n_kv_heads, w.n_q_heads, w.head_dim, w.chunk, w.levels, w.n_ref, w.top_p, w.kv_dtype,
                       w.capacity if capacity is None else capacity)


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


def zha_tree_level_offsets(cfg: Config, level: int) -> dict:
    s, b, l, n = (ctypes.c_int64() for _ in range(4))
    _check(lib().zha_tree_level_offsets(ctypes.byref(cfg), level, ctypes.byref(s), ctypes.byref(b), ctypes.byref(l),
                                        ctypes.byref(n)))
    return {"s": s.value, "b": b.value, "lse": l.value, "n_cap": n.value}


def zha_route_level_offsets(cfg: Config, level: int) -> dict:
    o = RouteOffsets()
    _check(lib().zha_route_level_offsets(ctypes.byref(cfg), level, ctypes.byref(o)))
    return {n: getattr(o, n) for n, _ in RouteOffsets._fields_}


def buffers(k, v, ref_q, tree, scratch) -> Buffers:
    return Buffers(_ptr(k), _ptr(v), _ptr(ref_q), _ptr(tree), _ptr(scratch))


def zha_build_tree(cfg: Config, bufs: Buffers, n_tokens: int, stream=None) -> None:
    _check(lib().zha_build_tree(ctypes.byref(cfg), ctypes.byref(bufs), n_tokens, _stream(stream)))


def zha_append_token(cfg: Config, bufs: Buffers, n_before: int, k_new, v_new, stream=None) -> None:
    _check(lib().zha_append_token(ctypes.byref(cfg), ctypes.byref(bufs), n_before, _ptr(k_new), _ptr(v_new),
                                  _stream(stream)))


def zha_decode_step(cfg: Config, bufs: Buffers, n_tokens: int, q, out, stream=None) -> None:
    _check(lib().zha_decode_step(ctypes.byref(cfg), ctypes.byref(bufs), n_tokens, _ptr(q), _ptr(out),
                                 _stream(stream)))


def zha_decode_step_timed(cfg: Config, bufs: Buffers, n_tokens: int, q, out, events, stream=None) -> None:
    """events: four raw hipEvent_t handles (ints, or None) recorded around the step's phases."""
    arr = (ctypes.c_void_p * 4)(*[e if e else None for e in events])
    _check(lib().zha_decode_step_timed(ctypes.byref(cfg), ctypes.byref(bufs), n_tokens, _ptr(q), _ptr(out), arr,
                                       _stream(stream)))


def dense_decode(cfg: Config, k, v, n_tokens: int, q, out, scratch, stream=None) -> None:
    _check(lib().dense_decode(ctypes.byref(cfg), _ptr(k), _ptr(v), n_tokens, _ptr(q), _ptr(out), _ptr(scratch),
                              _stream(stream)))

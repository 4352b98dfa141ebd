"""Device buffers for one ZHA layer, held as torch tensors, and views into them.

Torch provides device memory and the stream; every step of the method runs in
libzha.so through `binding`.
"""
from __future__ import annotations

import torch

from . import binding as B


class ZhaLayer:
    """K/V cache, reference queries, summary tree and scratch of one attention layer."""

    def __init__(self, cfg: B.Config, k: torch.Tensor, v: torch.Tensor, ref_q: torch.Tensor):
        B.zha_check_config(cfg)
        dev = k.device
        if dev.type != "cuda":
            raise ValueError("ZhaLayer needs device tensors")
        H, cap, d = cfg.n_kv_heads, cfg.capacity, cfg.head_dim
        want = torch.bfloat16 if cfg.kv_dtype == B.ZHA_BF16 else torch.float32
        for name, t in (("k", k), ("v", v)):
            if tuple(t.shape) != (H, cap, d) or t.dtype != want or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous {want} tensor of shape {(H, cap, d)}")
        if tuple(ref_q.shape) != (H, cfg.n_ref, d) or ref_q.dtype != torch.float32 or not ref_q.is_contiguous():
            raise ValueError(f"ref_q must be a contiguous float32 tensor of shape {(H, cfg.n_ref, d)}")
        self.cfg = cfg
        self.k, self.v, self.ref_q = k, v, ref_q
        self.tree = torch.empty(B.zha_tree_bytes(cfg), dtype=torch.uint8, device=dev)
        self.scratch = torch.empty(B.zha_scratch_bytes(cfg), dtype=torch.uint8, device=dev)
        self.dense_scratch = torch.empty(B.zha_dense_scratch_bytes(cfg), dtype=torch.uint8, device=dev)
        self.bufs = B.buffers(k, v, ref_q, self.tree, self.scratch)
        self.out = torch.empty((cfg.n_q_heads, d), dtype=torch.float32, device=dev)
        self.n_tokens = 0

    # -- the C ABI entry points
    def build(self, n_tokens: int):
        B.zha_build_tree(self.cfg, self.bufs, n_tokens)
        self.n_tokens = n_tokens

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor):
        B.zha_append_token(self.cfg, self.bufs, self.n_tokens, k_new, v_new)
        self.n_tokens += 1

    def decode(self, q: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
        out = self.out if out is None else out
        B.zha_decode_step(self.cfg, self.bufs, self.n_tokens, q, out)
        return out

    def dense(self, q: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
        out = self.out if out is None else out
        B.dense_decode(self.cfg, self.k, self.v, self.n_tokens, q, out, self.dense_scratch)
        return out

    # -- views for tests and diagnostics
    def _view(self, buf, off, dtype, shape):
        n = 1
        for s in shape:
            n *= s
        nbytes = n * torch.tensor([], dtype=dtype).element_size()
        return buf[off:off + nbytes].view(dtype).view(*shape)

    def tree_level(self, level: int):
        """(s [H][n_cap][R][d], b [H][n_cap][R], lse [H][n_cap][R]) float32 views of the tree."""
        o = B.zha_tree_level_offsets(self.cfg, level)
        H, R, d, n = self.cfg.n_kv_heads, self.cfg.n_ref, self.cfg.head_dim, o["n_cap"]
        return (self._view(self.tree, o["s"], torch.float32, (H, n, R, d)),
                self._view(self.tree, o["b"], torch.float32, (H, n, R)),
                self._view(self.tree, o["lse"], torch.float32, (H, n, R)))

    def route_level(self, level: int) -> dict:
        """Routing the last decode step left for `level` (copied to host)."""
        o = B.zha_route_level_offsets(self.cfg, level)
        H, G, n = self.cfg.n_kv_heads, self.cfg.n_q_heads // self.cfg.n_kv_heads, o["n_cap"]
        v = lambda off, dt, shape: self._view(self.scratch, off, dt, shape).cpu()
        return {
            "n_cand": v(o["n_cand"], torch.int32, (H,)),
            "sigma": v(o["sigma"], torch.float32, (H, G, n)),
            "n_kept": v(o["n_kept"], torch.int32, (H,)),
            "kept": v(o["kept"], torch.int32, (H, n)),
            "mask": v(o["mask"], torch.int32, (H, n)),
            "stats": v(o["stats"], torch.int32, (H * G, 2)),
        }

    def kept_sets(self, level: int) -> list[list[int]]:
        """Per query head, the ascending node ids it kept at `level` in the last decode step."""
        r = self.route_level(level)
        H, G = self.cfg.n_kv_heads, self.cfg.n_q_heads // self.cfg.n_kv_heads
        out = []
        for g in range(H):
            nk = int(r["n_kept"][g])
            nodes = r["kept"][g, :nk].tolist()
            masks = r["mask"][g, :nk].tolist()
            for hl in range(G):
                out.append([n for n, m in zip(nodes, masks) if (m >> hl) & 1])
        return out

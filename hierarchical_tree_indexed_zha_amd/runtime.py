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

    # -- argument checks: the ABI takes raw pointers, so shape, dtype, device and
    # layout are checked here before any pointer crosses it
    def _need(self, name, t, shape, dtype):
        if not isinstance(t, torch.Tensor) or t.device != self.k.device or t.dtype != dtype \
                or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
            got = (tuple(t.shape), t.dtype, str(t.device), t.is_contiguous()) if isinstance(t, torch.Tensor) else type(t)
            raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on "
                             f"{self.k.device}; got {got}")

    @property
    def kv_torch_dtype(self):
        return torch.bfloat16 if self.cfg.kv_dtype == B.ZHA_BF16 else torch.float32

    def _check_q_out(self, q, out):
        d = self.cfg.head_dim
        self._need("q", q, (self.cfg.n_q_heads, d), self.kv_torch_dtype)
        self._need("out", out, (self.cfg.n_q_heads, d), torch.float32)

    # -- the C ABI entry points
    def build(self, n_tokens: int):
        B.zha_build_tree(self.cfg, self.bufs, n_tokens)
        self.n_tokens = n_tokens

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor):
        shape = (self.cfg.n_kv_heads, self.cfg.head_dim)
        self._need("k_new", k_new, shape, self.kv_torch_dtype)
        self._need("v_new", v_new, shape, self.kv_torch_dtype)
        B.zha_append_token(self.cfg, self.bufs, self.n_tokens, k_new, v_new)
        self.n_tokens += 1

    def decode(self, q: torch.Tensor, out: torch.Tensor | None = None, sel: torch.Tensor | None = None,
               stats: torch.Tensor | None = None) -> torch.Tensor:
        """One decode step.  sel: optional int32 [H_q][1 + capacity // chunk] (per-head kept
        chunk lists); stats: optional uint8 tensor of stats_nbytes() bytes (a zha_stats)."""
        out = self.out if out is None else out
        self._check_q_out(q, out)
        if sel is not None:
            self._need("sel", sel, self.sel_shape(), torch.int32)
        if stats is not None:
            self._need("stats", stats, (self.stats_nbytes(),), torch.uint8)
        B.zha_decode_step(self.cfg, self.bufs, self.n_tokens, q, out, sel, stats)
        return out

    def dense(self, q: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
        out = self.out if out is None else out
        self._check_q_out(q, out)
        B.dense_decode(self.cfg, self.k, self.v, self.n_tokens, q, out, self.dense_scratch)
        return out

    # -- optional decode outputs
    def sel_shape(self):
        return (self.cfg.n_q_heads, self.cfg.capacity // self.cfg.chunk + 1)

    def new_sel(self) -> torch.Tensor:
        return torch.zeros(self.sel_shape(), dtype=torch.int32, device=self.k.device)

    @staticmethod
    def stats_nbytes() -> int:
        import ctypes
        return ctypes.sizeof(B.Stats)

    def new_stats(self) -> torch.Tensor:
        return torch.zeros(self.stats_nbytes(), dtype=torch.uint8, device=self.k.device)

    @staticmethod
    def read_stats(stats: torch.Tensor) -> dict:
        return B.stats_from_bytes(bytes(stats.cpu().numpy().tobytes()))

    @staticmethod
    def read_sel(sel: torch.Tensor) -> list[list[int]]:
        """Per query head, the ascending kept chunk indices a `sel` output holds."""
        s = sel.cpu()
        return [s[h, 1:1 + int(s[h, 0])].tolist() for h in range(s.shape[0])]

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

    def decode_batch(self, q: torch.Tensor, out: torch.Tensor | None = None,
                     sel: torch.Tensor | None = None) -> torch.Tensor:
        """A batch of decode queries q [Q][H_q][d] routed together over the current cache
        (zha_decode_batch); returns out [Q][H_q][d] float32.  sel: optional int32
        [Q][H_q][1 + capacity // chunk]."""
        cfg = self.cfg
        if q.dim() != 3 or tuple(q.shape[1:]) != (cfg.n_q_heads, cfg.head_dim):
            raise ValueError(f"q must be [Q][{cfg.n_q_heads}][{cfg.head_dim}] (got {tuple(q.shape)})")
        nq = q.shape[0]
        self._need("q", q, tuple(q.shape), self.kv_torch_dtype)
        if out is None:
            out = torch.empty((nq, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32, device=self.k.device)
        self._need("out", out, (nq, cfg.n_q_heads, cfg.head_dim), torch.float32)
        if sel is not None:
            self._need("sel", sel, (nq,) + self.sel_shape(), torch.int32)
        need = B.zha_batch_scratch_bytes(cfg, nq)
        if getattr(self, "_bscratch", None) is None or self._bscratch.numel() < need:
            self._bscratch = torch.empty(need, dtype=torch.uint8, device=self.k.device)
        bufs = B.Buffers(self.bufs.k, self.bufs.v, self.bufs.ref_q, self.bufs.tree, self._bscratch.data_ptr())
        B.zha_decode_batch(cfg, bufs, self.n_tokens, nq, q, out, sel)
        return out

    def tree_level16(self, level: int) -> torch.Tensor:
        """The router's bfloat16 copy of level `level`'s planes s [H][n_cap][R][d] (plane_format bf16)."""
        o = B.zha_tree_level_offsets(self.cfg, level)
        if o["s16"] < 0:
            raise ValueError("the tree keeps no bfloat16 planes (plane_format is not bf16)")
        H, R, d, n = self.cfg.n_kv_heads, self.cfg.n_ref, self.cfg.head_dim, o["n_cap"]
        return self._view(self.tree, o["s16"], torch.bfloat16, (H, n, R, d))

    def tree_level8(self, level: int):
        """The router's 8-bit copy of level `level`'s planes s (plane_format fp8): the FP8
        E4M3 codes uint8 [H][n_cap][R][d] and the per-plane scales float32 [H][n_cap][R]."""
        o = B.zha_tree_level_offsets(self.cfg, level)
        if o["s8"] < 0:
            raise ValueError("the tree keeps no 8-bit planes (plane_format is not fp8)")
        H, R, d, n = self.cfg.n_kv_heads, self.cfg.n_ref, self.cfg.head_dim, o["n_cap"]
        return (self._view(self.tree, o["s8"], torch.uint8, (H, n, R, d)),
                self._view(self.tree, o["sc"], torch.float32, (H, n, R)))

    def fidelity(self, q: torch.Tensor) -> torch.Tensor:
        """Router fidelity of the step the last decode(q) ran (same q, same n_tokens): float32
        [H_q][L + 1], per level the exact attention mass of the tokens the head kept, and
        last the mass of the attended token set."""
        self._check_q_out(q, self.out)
        recall = torch.empty((self.cfg.n_q_heads, self.cfg.levels + 1), dtype=torch.float32, device=self.k.device)
        work = torch.empty(B.zha_fidelity_work_bytes(self.cfg, self.n_tokens), dtype=torch.uint8,
                           device=self.k.device)
        B.zha_route_fidelity(self.cfg, self.bufs, self.n_tokens, q, recall, work)
        return recall

    def route_level(self, level: int) -> dict:
        """Routing the last decode step left for `level` (copied to host), in the layout of
        a level scored over its group candidates: n_cand [H], sigma [H][G][n_cap] by
        group candidate position, n_kept [H], kept [H][n_cap], mask [H][n_cap] and per-head
        stats [H_q][2].  A chained level (every node scored, per-head kept bitmaps over node
        ids) is laid out that way on the host from the device's node scores, bitmaps and
        stats; its group kept list as the device wrote it (at the chain's last level only)
        is returned as `dev_n_kept`, `dev_kept`, `dev_mask`."""
        o = B.zha_route_level_offsets(self.cfg, self.n_tokens, level)
        cfg = self.cfg
        H, G, n = cfg.n_kv_heads, cfg.n_q_heads // cfg.n_kv_heads, o["n_cap"]
        v = lambda off, dt, shape: self._view(self.scratch, off, dt, shape).cpu()
        out = {
            "n_cand": v(o["n_cand"], torch.int32, (H,)),
            "sigma": v(o["sigma"], torch.float32, (H, G, o["sig_stride"]))[:, :, :n],
            "n_kept": v(o["n_kept"], torch.int32, (H,)),
            "kept": v(o["kept"], torch.int32, (H, n)),
            "mask": v(o["mask"], torch.int32, (H, n)),
            "stats": v(o["stats"], torch.int32, (H * G, 2)),
            "chained": bool(o["chained"]),
        }
        if not o["chained"]:
            return out
        import numpy as np
        c, N = cfg.chunk, self.n_tokens
        words = v(o["kbm"], torch.int64, (H, G, o["wcap"])).numpy().view(np.uint64)
        nn = N // c ** level
        bits = ((words[..., :, None] >> np.arange(64, dtype=np.uint64)) & np.uint64(1)).reshape(H, G, -1)[..., :nn]
        kept_h = [[np.nonzero(bits[g, hl])[0] for hl in range(G)] for g in range(H)]
        top = max(lv for lv in range(1, cfg.levels + 1) if N // c ** lv > 0)
        if level < top:
            up = self.route_level(level + 1)
            assert up["chained"], "the chain is a contiguous run of levels from the top"
            prev = up["kept_by_head"]
            orph = np.arange(c * (N // c ** (level + 1)), nn, dtype=np.int64)
        sig_nodes = out["sigma"].numpy()
        sigma = np.full((H, G, n), -np.inf, dtype=np.float32)
        n_cand = np.zeros(H, dtype=np.int32)
        n_kept = np.zeros(H, dtype=np.int32)
        kept = np.zeros((H, n), dtype=np.int32)
        mask = np.zeros((H, n), dtype=np.int32)
        for g in range(H):
            if level == top:
                cands = [np.arange(nn, dtype=np.int64)] * G
            else:
                cands = [np.concatenate([(prev[g][hl][:, None] * c + np.arange(c)[None, :]).ravel(), orph])
                         for hl in range(G)]
            union = np.unique(np.concatenate(cands))
            n_cand[g] = len(union)
            for hl in range(G):
                pos = np.searchsorted(union, cands[hl])
                sigma[g, hl, pos] = sig_nodes[g, hl, cands[hl]]
            uk = np.unique(np.concatenate(kept_h[g]))
            n_kept[g] = len(uk)
            kept[g, :len(uk)] = uk
            for hl in range(G):
                mask[g, np.searchsorted(uk, kept_h[g][hl])] |= 1 << hl
        out.update({"dev_n_kept": out["n_kept"], "dev_kept": out["kept"], "dev_mask": out["mask"],
                    "n_cand": torch.from_numpy(n_cand), "sigma": torch.from_numpy(sigma),
                    "n_kept": torch.from_numpy(n_kept), "kept": torch.from_numpy(kept),
                    "mask": torch.from_numpy(mask), "kept_by_head": kept_h})
        return out

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

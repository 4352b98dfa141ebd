"""Named workloads and their seeded synthetic inputs.

This module only draws numbers: it holds none of the method's arithmetic, so
that the HIP path and the fp64 oracle can both consume the very same arrays.

The five workloads follow the shapes the ZHA pages evaluate:
  * tiny  — 1 KV head, 8 query heads, fp32, 16,384 tokens, chunk 4, 6 levels,
            R = 16, p = 0.95, i.i.d. Gaussian cache with 4 planted needles.
  * light — the "light" router of the pages' speed model (R = 1, chunk 8,
            p = 0.75; page "ZHA 用树形稀疏注意力改造现有大模型", section 几百倍加速),
            4 KV / 32 query heads, bf16, 262,144 tokens, 4 levels.
  * deep  — the deep tree (chunk 4, 6 levels, R = 16, p = 0.95; same page,
            section 256K 的质量结果), 262,144 tokens.
  * wide  — the wide tree (chunk 256, 1 level, R = 16, p = 0.95), 262,144 tokens.
  * ultra — the light router at 10,485,760 tokens, chunk 8, 7 levels.

The pages measure quality on benchmark suites with a trained model; those are
not reproduced.  The generators stand in for them: planted needles for
retrieval probes, contiguous topic segments for the locality of natural text,
and an i.i.d. background for the worst case in which nothing is compressible.
"""
from __future__ import annotations

import math
import zlib
from dataclasses import dataclass, replace

import torch

__all__ = ["Workload", "WORKLOADS", "get", "scaled", "generate", "stream_seed", "levels_for"]


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    n_kv_heads: int
    n_q_heads: int
    head_dim: int
    kv_dtype: str          # "f32" | "bf16"
    n_tokens: int
    chunk: int
    levels: int
    n_ref: int
    top_p: float
    steps: int
    append: bool           # steps append one token each before decoding
    generator: str         # "needles" | "clusters" | "topics"

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def torch_dtype(self):
        return torch.float32 if self.kv_dtype == "f32" else torch.bfloat16

    @property
    def capacity(self) -> int:
        return self.n_tokens + (self.steps if self.append else 0)


def levels_for(n_tokens: int, chunk: int, max_top: int = 64) -> int:
    """Smallest depth whose top level holds at most `max_top` complete nodes."""
    levels = 1
    while n_tokens // chunk ** levels > max_top:
        levels += 1
    return levels


WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 8, 128, "f32", 16384, 4, 6, 16, 0.95, 64, False, "needles"),
    "light": Workload("light", 1, 4, 32, 128, "bf16", 262144, 8, 4, 1, 0.75, 256, True, "clusters"),
    "deep": Workload("deep", 2, 4, 32, 128, "bf16", 262144, 4, 6, 16, 0.95, 256, False, "topics"),
    "wide": Workload("wide", 3, 4, 32, 128, "bf16", 262144, 256, 1, 16, 0.95, 256, False, "topics"),
    "ultra": Workload("ultra", 4, 4, 32, 128, "bf16", 10485760, 8, 7, 1, 0.75, 64, True, "topics"),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def scaled(w: Workload, n_tokens: int, steps: int | None = None, levels: int | None = None, **kw) -> Workload:
    """A smaller copy of a workload (same generator and router settings)."""
    if levels is None:
        levels = min(w.levels, max(1, levels_for(n_tokens, w.chunk)))
    return replace(w, name=f"{w.name}@{n_tokens}", n_tokens=n_tokens,
                   steps=w.steps if steps is None else steps, levels=levels, **kw)


def stream_seed(base: int, *names) -> int:
    """Deterministic 63-bit seed for a named sub-stream of a base seed."""
    h = base & 0xFFFFFFFF
    for n in names:
        h = (h * 1000003) ^ zlib.crc32(str(n).encode())
        h &= (1 << 63) - 1
    return h


def _gen(base: int, device, *names) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(stream_seed(base, *names))
    return g


def _randn(shape, base, device, *names):
    return torch.randn(shape, generator=_gen(base, device, *names), device=device, dtype=torch.float32)


def _rand(shape, base, device, *names):
    return torch.rand(shape, generator=_gen(base, device, *names), device=device, dtype=torch.float32)


def _unit(x):
    return x / x.norm(dim=-1, keepdim=True)


def _orth_unit(x, u):
    """Unit vectors from x with the component along unit u removed."""
    x = x - (x * u).sum(-1, keepdim=True) * u
    return _unit(x)


_BLOCK = 1 << 20  # tokens generated per (head, block) stream


def generate(w: Workload, device="cpu", seed: int | None = None) -> dict:
    """Seeded inputs of workload w on `device`.

    Returns a dict of tensors:
      k, v        [H_kv][capacity][d]   cache, rows >= n_tokens zero
      ref_q       [H_kv][R][d]          fp32 reference queries
      q           [steps][H_q][d]       decode queries (cache dtype)
      k_app,v_app [steps][H_kv][d]      appended tokens (cache dtype), if w.append
    Values are drawn in fp32 and rounded once to the cache dtype (RNE); every
    consumer sees those rounded values.  The same (workload, seed, device kind)
    gives byte-identical tensors.
    """
    base = 1000 + w.index if seed is None else seed
    dev = torch.device(device)
    H, Hq, d, N, G = w.n_kv_heads, w.n_q_heads, w.head_dim, w.n_tokens, w.group
    dt = w.torch_dtype
    cap = w.capacity
    k = torch.zeros((H, cap, d), dtype=dt, device=dev)
    v = torch.zeros((H, cap, d), dtype=dt, device=dev)
    ref_q = _randn((H, w.n_ref, d), base, dev, "refs")
    q = torch.empty((w.steps, Hq, d), dtype=torch.float32, device=dev)
    rd = math.sqrt(d)

    # Background cache, per (head, block) stream so large caches stream in blocks.
    for g in range(H):
        for b0 in range(0, N, _BLOCK):
            b1 = min(N, b0 + _BLOCK)
            blk = b0 // _BLOCK
            v[g, b0:b1] = _randn((b1 - b0, d), base, dev, "values", g, blk).to(dt)
            if w.generator in ("needles", "clusters"):
                k[g, b0:b1] = _randn((b1 - b0, d), base, dev, "keys", g, blk).to(dt)

    if w.generator == "needles":
        # One seeded direction; 4 needle keys 6*qhat + 0.1*eps at distinct positions in [1, N).
        qhat = _unit(_randn((d,), base, dev, "qhat"))
        for g in range(H):
            pos = torch.randperm(N - 1, generator=_gen(base, "cpu", "needles", g))[:4] + 1
            eps = _randn((4, d), base, dev, "needle_eps", g)
            k[g, pos.to(dev)] = (6.0 * qhat + 0.1 * eps).to(dt)
        rho = 0.5 + 0.4 * _rand((w.steps, Hq, 1), base, dev, "rho")
        wv = _orth_unit(_randn((w.steps, Hq, d), base, dev, "qnoise"), qhat)
        q[:] = rd * (rho * qhat + torch.sqrt(1 - rho * rho) * wv)

    elif w.generator == "clusters":
        # 64 unit cluster directions per head; each cluster is 8 contiguous tokens at a
        # non-overlapping start in [1, N-8) whose keys have cosine 0.5..0.9 with it.
        span = 8
        n_cl = max(1, min(64, (N - 1) // (2 * span)))   # fewer clusters only when N is tiny
        for g in range(H):
            u = _unit(_randn((n_cl, d), base, dev, "cl_dir", g))
            # slot i spans [1 + 2*span*i, 1 + 2*span*(i+1)); an offset < span keeps clusters disjoint
            slots = torch.randperm((N - 1) // (2 * span), generator=_gen(base, "cpu", "cl_pos", g))[:n_cl]
            starts = 1 + slots * 2 * span + torch.randint(0, span, (n_cl,), generator=_gen(base, "cpu", "cl_off", g))
            rho = 0.5 + 0.4 * _rand((n_cl, span, 1), base, dev, "cl_rho", g)
            wv = _orth_unit(_randn((n_cl, span, d), base, dev, "cl_w", g), u[:, None, :])
            keys = rd * (rho * u[:, None, :] + torch.sqrt(1 - rho * rho) * wv)
            idx = (starts[:, None] + torch.arange(span)[None, :]).reshape(-1).to(dev)
            k[g, idx] = keys.reshape(-1, d).to(dt)
            target = torch.randint(0, n_cl, (w.steps,), generator=_gen(base, "cpu", "cl_target", g)).to(dev)
            noise = _randn((w.steps, G, d), base, dev, "cl_qnoise", g)
            q[:, g * G:(g + 1) * G] = rd * u[target][:, None, :] + 0.25 * noise

    elif w.generator == "topics":
        # 1024 Gaussian topic means per head; 256-token segments with a uniform topic;
        # keys mu + 0.5*eps.  Each (step, group) targets the topic of a random segment,
        # heads q = mu + 0.5*eps, and a 16-token needle q_bar + 0.1*eps is planted
        # at a distinct 16-aligned slot (+1) before any tree is built.
        n_top, seg = 1024, 256
        n_seg = (N + seg - 1) // seg
        for g in range(H):
            mu = _randn((n_top, d), base, dev, "topic_mu", g)
            topic = torch.randint(0, n_top, (n_seg,), generator=_gen(base, "cpu", "topic_of_seg", g)).to(dev)
            for b0 in range(0, N, _BLOCK):
                b1 = min(N, b0 + _BLOCK)
                blk = b0 // _BLOCK
                t = torch.arange(b0, b1, device=dev) // seg
                k[g, b0:b1] = (mu[topic[t]] + 0.5 * _randn((b1 - b0, d), base, dev, "keys", g, blk)).to(dt)
            tseg = torch.randint(0, n_seg, (w.steps,), generator=_gen(base, "cpu", "q_seg", g)).to(dev)
            qn = _randn((w.steps, G, d), base, dev, "topic_qnoise", g)
            qg = mu[topic[tseg]][:, None, :] + 0.5 * qn
            q[:, g * G:(g + 1) * G] = qg
            n_slots = max(0, (N - 1 - 16) // 16)
            n_nd = min(w.steps, n_slots)                              # one needle per step while they fit
            slots = torch.randperm(n_slots, generator=_gen(base, "cpu", "needle_slot", g))[:n_nd]
            qbar = qg.mean(dim=1)                                     # [steps, d]
            eps = _randn((w.steps, 16, d), base, dev, "needle_eps", g)
            needles = (qbar[:, None, :] + 0.1 * eps)[:n_nd]
            idx = (1 + slots[:, None] * 16 + torch.arange(16)[None, :]).reshape(-1).to(dev)
            k[g, idx] = needles.reshape(-1, d).to(dt)
    else:
        raise ValueError(w.generator)

    out = {"k": k, "v": v, "ref_q": ref_q.contiguous(), "q": q.to(dt).contiguous()}
    if w.append:
        if w.generator == "topics":
            # Appended tokens continue the topic stream (new 256-token segments).
            ka = torch.empty((w.steps, H, d), dtype=torch.float32, device=dev)
            for g in range(H):
                mu = _randn((n_top, d), base, dev, "topic_mu", g)
                n_new = (w.steps + seg - 1) // seg + 1
                tp = torch.randint(0, n_top, (n_new,), generator=_gen(base, "cpu", "append_topic", g)).to(dev)
                pos = torch.arange(N, N + w.steps, device=dev)
                seg_idx = pos // seg - N // seg
                ka[:, g] = mu[tp[seg_idx]] + 0.5 * _randn((w.steps, d), base, dev, "append_k", g)
        else:
            ka = _randn((w.steps, H, d), base, dev, "append_k")
        out["k_app"] = ka.to(dt).contiguous()
        out["v_app"] = _randn((w.steps, H, d), base, dev, "append_v").to(dt).contiguous()
    return out

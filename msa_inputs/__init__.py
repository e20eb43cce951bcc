"""Seeded synthetic inputs for the MSA training hot path.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It only draws and rounds random tensors and packs documents; it
holds none of the arithmetic of the attention method itself (no scoring, no
selection, no softmax).

Workloads
---------
The pages describe MiniMax Sparse Attention training at 128k-1M tokens with
GQA and 128-token KV blocks chosen by a proxy head (ai-minor "Dramatically
Speeding Up Million-Token Training!", News Overview; keelcrux "Flash-MSA: Ein
Training mit einer Million Tokens", Under the hood).  They name no dataset and
print no tensors, so every workload here is synthetic:

* ``tiny-2k-fp32``: every tensor i.i.d. N(0, 1), kept in fp32.
* the bf16 workloads: a base of 0.5*N(0, 1), plus a block-constant rank-8
  component.  One latent c ~ N(0, I_8) is drawn per (document, 128-token KV
  block); per KV group g two projections P_g (8 x d) and R_g (8 x dp) are drawn
  with N(0, 1) entries.  0.5*c@P_g/sqrt(8) is added to q (every head of g) and
  to k[g]; 0.5*c@R_g/sqrt(8) is added to qp[g] and kp[g].  v and dO are base
  only.  The latent gives proxy block scores a non-uniform block structure
  that the main attention shares.
* ``varlen-1m-packed``: document lengths floor(exp(U(ln 4096, ln 262144))),
  drawn until they cover 2**20 tokens; the last one is truncated so the total
  is exactly 2**20.

Random streams
--------------
On the host, numpy PCG64 with ``SeedSequence(seed)`` spawned into named child
streams in a fixed order (lengths, latents, proj_main, proj_proxy, q, k, v, qp,
kp, dO).  Lengths are always drawn on the host.  For large workloads the same
recipe can be drawn on a torch device (``device="cuda"``) with torch's own
generator: same distribution, different values.  Floating inputs are rounded
once to bf16 (round to nearest even) for the bf16 workloads, and every consumer
reads the same rounded tensors.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import numpy as np

STREAMS = ("lengths", "latents", "proj_main", "proj_proxy", "q", "k", "v", "qp", "kp", "dO")


@dataclass(frozen=True)
class Workload:
    name: str
    seqlens: tuple            # document lengths (empty -> drawn, see doc_mode)
    heads_q: int
    heads_kv: int
    head_dim: int
    proxy_dim: int
    q_block: int
    topk: int
    local_window: int = 0
    kv_block: int = 128
    dtype: str = "bf16"       # "bf16" or "f32"
    recipe: str = "lowrank"   # "iid" or "lowrank"
    doc_mode: str = "fixed"   # "fixed" or "loguniform"
    total_tokens: int = 0     # for doc_mode == "loguniform"
    proxy_loss_weight: float = 1.0
    dilation: int = 1         # stride of the forced window blocks
    proxy_heads: int = 0      # 0: one proxy head per KV group; 1: one shared proxy head

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv


WORKLOADS: Dict[str, Workload] = {
    "tiny-2k-fp32": Workload("tiny-2k-fp32", (2048,), 8, 2, 64, 32, 64, 4, 0,
                             dtype="f32", recipe="iid"),
    "layer-32k": Workload("layer-32k", (32768,), 32, 8, 128, 64, 64, 16, 0),
    "layer-128k-gqa8": Workload("layer-128k-gqa8", (131072,), 64, 8, 128, 64, 128, 32, 0),
    "layer-512k-window2": Workload("layer-512k-window2", (524288,), 32, 8, 128, 64, 128, 32, 2),
    "varlen-1m-packed": Workload("varlen-1m-packed", (), 32, 8, 128, 64, 128, 64, 0,
                                 doc_mode="loguniform", total_tokens=1 << 20),
}


def _streams(seed: int) -> Dict[str, np.random.Generator]:
    children = np.random.SeedSequence(seed).spawn(len(STREAMS))
    return {name: np.random.Generator(np.random.PCG64(ss)) for name, ss in zip(STREAMS, children)}


def draw_loguniform_lengths(total: int, seed: int, lo: int = 4096, hi: int = 262144) -> List[int]:
    rng = _streams(seed)["lengths"]
    out: List[int] = []
    acc = 0
    while acc < total:
        L = int(math.floor(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
        L = min(L, total - acc)
        out.append(L)
        acc += L
    return out


def seqlens_of(w: Workload, seed: int = 0) -> List[int]:
    if w.doc_mode == "loguniform":
        return draw_loguniform_lengths(w.total_tokens, seed)
    return list(w.seqlens)


def cu_seqlens_of(seqlens) -> np.ndarray:
    cu = np.zeros(len(seqlens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(seqlens, dtype=np.int64))
    return cu


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return them as fp32."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


@dataclass
class Case:
    """One seeded input set.  Arrays are fp32 numpy holding exactly the values the
    kernels consume (bf16-representable for bf16 workloads)."""
    workload: Workload
    seed: int
    seqlens: List[int]
    cu_seqlens: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    qp: np.ndarray
    kp: np.ndarray
    dO: np.ndarray
    extra: dict = field(default_factory=dict)


def _kv_block_latents(rng, seqlens, kv_block, rank=8):
    """One latent vector per (document, KV block), broadcast to tokens."""
    T = int(sum(seqlens))
    lat = np.zeros((T, rank), dtype=np.float32)
    s = 0
    for L in seqlens:
        nk = -(-L // kv_block)
        c = rng.standard_normal((nk, rank), dtype=np.float32)
        tok = np.arange(L) // kv_block
        lat[s:s + L] = c[tok]
        s += L
    return lat


def make_case(w: Workload, seed: int = 0, seqlens: Optional[List[int]] = None,
              exact_proxy: bool = False) -> Case:
    """Draw a workload on the host with numpy (canonical values for a seed).

    ``exact_proxy``: qp and kp are drawn from {-1, -1/2, 0, 1/2, 1}, so every
    partial sum of a proxy dot product is a multiple of 1/4 and is exact in fp32
    under any summation order (test-only mode).
    """
    if seqlens is None:
        seqlens = seqlens_of(w, seed)
    T = int(sum(seqlens))
    st = _streams(seed)
    Hq, Hkv, d, dp = w.heads_q, w.heads_kv, w.head_dim, w.proxy_dim
    G = w.group

    def normal(name, shape):
        return st[name].standard_normal(shape, dtype=np.float32)

    if w.recipe == "iid":
        q, k, v = normal("q", (T, Hq, d)), normal("k", (T, Hkv, d)), normal("v", (T, Hkv, d))
        qp, kp = normal("qp", (T, Hkv, dp)), normal("kp", (T, Hkv, dp))
        dO = normal("dO", (T, Hq, d))
    else:
        lat = _kv_block_latents(st["latents"], seqlens, w.kv_block)
        Pm = st["proj_main"].standard_normal((Hkv, 8, d), dtype=np.float32)
        Rp = st["proj_proxy"].standard_normal((Hkv, 8, dp), dtype=np.float32)
        add_main = 0.5 * np.einsum("tr,grd->tgd", lat, Pm) / math.sqrt(8.0)
        add_prox = 0.5 * np.einsum("tr,grd->tgd", lat, Rp) / math.sqrt(8.0)
        q = 0.5 * normal("q", (T, Hq, d))
        q += np.repeat(add_main, G, axis=1)
        k = 0.5 * normal("k", (T, Hkv, d)) + add_main
        v = 0.5 * normal("v", (T, Hkv, d))
        qp = 0.5 * normal("qp", (T, Hkv, dp)) + add_prox
        kp = 0.5 * normal("kp", (T, Hkv, dp)) + add_prox
        dO = 0.5 * normal("dO", (T, Hq, d))
    if exact_proxy:
        vals = np.array([-1.0, -0.5, 0.0, 0.5, 1.0], dtype=np.float32)
        qp = vals[st["qp"].integers(0, 5, size=(T, Hkv, dp))]
        kp = vals[st["kp"].integers(0, 5, size=(T, Hkv, dp))]
    arrs = [q, k, v, qp, kp, dO]
    if w.dtype == "bf16":
        arrs = [round_bf16(a) for a in arrs]
    else:
        arrs = [np.ascontiguousarray(a, dtype=np.float32) for a in arrs]
    q, k, v, qp, kp, dO = arrs
    if w.proxy_heads == 1:            # one shared proxy head: the first group's projection
        qp, kp = np.ascontiguousarray(qp[:, :1]), np.ascontiguousarray(kp[:, :1])
    return Case(w, seed, list(seqlens), cu_seqlens_of(seqlens), q, k, v, qp, kp, dO)


def make_case_torch(w: Workload, seed: int = 0, device="cuda", seqlens: Optional[List[int]] = None):
    """Draw the same recipe directly on a torch device (fast path for 128k-1M
    token workloads).  Returns a dict of torch tensors in the workload dtype plus
    ``cu_seqlens`` (int32, on the device) and ``seqlens`` (host list)."""
    import torch
    if seqlens is None:
        seqlens = seqlens_of(w, seed)
    T = int(sum(seqlens))
    Hq, Hkv, d, dp, G = w.heads_q, w.heads_kv, w.head_dim, w.proxy_dim, w.group
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1000003 + 17)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def normal(shape, scale):
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        return x

    out = {}
    if w.recipe == "iid":
        for name, shape in (("q", (T, Hq, d)), ("k", (T, Hkv, d)), ("v", (T, Hkv, d)),
                            ("qp", (T, Hkv, dp)), ("kp", (T, Hkv, dp)), ("dO", (T, Hq, d))):
            out[name] = normal(shape, 1.0).to(dt)
    else:
        # block-constant latents: one per (document, KV block)
        nks = [-(-L // w.kv_block) for L in seqlens]
        c = normal((sum(nks), 8), 1.0)
        tok_blk = torch.cat([torch.arange(L, device=device) // w.kv_block + off
                             for L, off in zip(seqlens, np.cumsum([0] + nks[:-1]).tolist())])
        Pm = normal((Hkv, 8, d), 1.0)
        Rp = normal((Hkv, 8, dp), 1.0)
        s = 0.5 / math.sqrt(8.0)
        add_main_blk = torch.einsum("br,grd->bgd", c, Pm) * s     # per block
        add_prox_blk = torch.einsum("br,grd->bgd", c, Rp) * s
        q = normal((T, Hq, d), 0.5)
        q.view(T, Hkv, G, d).add_(add_main_blk[tok_blk].unsqueeze(2))
        out["q"] = q.to(dt); del q
        k = normal((T, Hkv, d), 0.5); k.add_(add_main_blk[tok_blk]); out["k"] = k.to(dt); del k
        out["v"] = normal((T, Hkv, d), 0.5).to(dt)
        qp = normal((T, Hkv, dp), 0.5); qp.add_(add_prox_blk[tok_blk]); out["qp"] = qp.to(dt); del qp
        kp = normal((T, Hkv, dp), 0.5); kp.add_(add_prox_blk[tok_blk]); out["kp"] = kp.to(dt); del kp
        out["dO"] = normal((T, Hq, d), 0.5).to(dt)
    if w.proxy_heads == 1:            # one shared proxy head: the first group's projection
        out["qp"] = out["qp"][:, :1].contiguous()
        out["kp"] = out["kp"][:, :1].contiguous()
    out["cu_seqlens"] = torch.from_numpy(cu_seqlens_of(seqlens)).to(device)
    out["seqlens"] = list(seqlens)
    return out


def small_variant(w: Workload, total_tokens: int, **kw) -> Workload:
    """The same head/block geometry on fewer tokens (for oracle-sized parity cases)."""
    return replace(w, name=f"{w.name}@{total_tokens}", seqlens=(total_tokens,),
                   doc_mode="fixed", total_tokens=0, **kw)

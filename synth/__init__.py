"""Seeded synthetic workloads for tree-summarised (ZHA) decode attention.

This module only draws random inputs: a KV cache, reference queries and decode
queries with the shapes and structure of the workloads the ZHA summary page
discusses (long clustered contexts, GQA heads, RoPE models).  It holds none of the
method's arithmetic (no attention, no summaries, no routing); both the CPU oracle
and the HIP path consume what it produces, so neither depends on the other.

Key structure (stand-in for the long-novel / RULER-style contexts of the ZHA page,
section "how it works" / "premises and limits", which are not available here):
  * ``runs``: tokens come in contiguous runs whose length is Geometric with mean C;
    each run draws a cluster from a uniform or Zipf(s) law; a key is its cluster
    centroid (N(0, I)) plus N(0, sigma^2) noise.  Locality makes chunks coherent the
    way document text is.
  * ``iid``: every token draws its cluster independently (uniform mass, adversarial).
  * ``hier``: a 4-level Gaussian mixture with branching 8 laid out in contiguous
    equal segments, so routing mass concentrates at upper tree levels.
Token 0 is an attention-sink key scaled x4.  Values are N(0, I).  Reference
queries are N(0, 1)/sqrt(d).  A decode query is a cluster centroid plus
N(0, 0.5^2) noise.  For RoPE workloads the cache holds keys already rotated at
their positions and the decode query is rotated at position T-1, the way a RoPE
model produces them (rotate-half pairing, fp64 angles); this is workload
synthesis, the ZHA path itself receives post-RoPE K and q.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

__all__ = ["Workload", "WORKLOADS", "make_cache", "make_qref", "make_query",
           "make_queries", "rope_rotate"]

SEED_BASE = 20261203


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H_kv: int
    G: int                 # query heads per KV head
    d: int
    C: int                 # chunk size (children per node)
    L: int                 # tree levels
    R: int                 # reference queries per tree
    p: float               # top-p mass fraction per level
    kv_dtype: str          # "f32" or "bf16"
    N: int                 # summarised prefix length
    open_len: int          # open-chunk length at the first decode step
    steps: int             # decode steps the workload runs
    n_clusters: int = 32
    freq: str = "uniform"  # cluster law: "uniform" or "zipf"
    zipf_s: float = 1.1
    placement: str = "runs"  # "runs", "iid" or "hier"
    sigma: float = 0.3
    q_sigma: float = 0.5
    sink_scale: float = 4.0
    rope: bool = False
    rope_base: float = 1.0e6
    index: int = 0

    @property
    def Hq(self) -> int:
        return self.H_kv * self.G

    @property
    def T0(self) -> int:
        return self.N + self.open_len

    @property
    def T_final(self) -> int:
        return self.T0 + self.steps

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # 1 KV head x 1 query head, d=64, NoPE, fp32, 4096 keys from 32 clusters.
    "tiny": Workload("tiny", B=1, H_kv=1, G=1, d=64, C=16, L=2, R=4, p=0.9,
                     kv_dtype="f32", N=4096, open_len=0, steps=8, n_clusters=32,
                     index=0),
    # GQA 8x4, d=128, bf16, 131072 keys, 1024 clusters, open chunk C/2.
    "gqa128k": Workload("gqa128k", B=1, H_kv=8, G=4, d=128, C=64, L=3, R=16, p=0.9,
                        kv_dtype="bf16", N=131072, open_len=32, steps=64,
                        n_clusters=1024, index=1),
    # Long context: 1M keys, 8192 Zipf(1.1) clusters.
    "long1m": Workload("long1m", B=1, H_kv=8, G=4, d=128, C=64, L=3, R=16, p=0.9,
                       kv_dtype="bf16", N=1 << 20, open_len=32, steps=32,
                       n_clusters=8192, freq="zipf", index=2),
    # Deep tree: C=4, L=6 over a hierarchical mixture.
    "deep": Workload("deep", B=1, H_kv=4, G=8, d=128, C=4, L=6, R=16, p=0.9,
                     kv_dtype="bf16", N=262144, open_len=2, steps=64,
                     n_clusters=512, placement="hier", index=3),
    # RoPE + batch: 16 sequences x 262144 keys, base 1e6.
    "rope_batch": Workload("rope_batch", B=16, H_kv=4, G=8, d=128, C=32, L=3, R=16,
                           p=0.9, kv_dtype="bf16", N=262144, open_len=16, steps=32,
                           n_clusters=1024, rope=True, index=4),
}


def _gen(device, *key: int) -> torch.Generator:
    """A torch generator on ``device`` seeded from (SEED_BASE, *key)."""
    h = SEED_BASE
    for k in key:
        h = (h * 1000003 + int(k) + 0x9E3779B9) % (1 << 62)
    g = torch.Generator(device=device)
    g.manual_seed(h)
    return g


def _cluster_law(wl: Workload, device) -> torch.Tensor:
    c = torch.arange(1, wl.n_clusters + 1, dtype=torch.float64, device=device)
    if wl.freq == "zipf":
        w = c.pow(-wl.zipf_s)
    else:
        w = torch.ones_like(c)
    return (w / w.sum()).to(torch.float32)


def rope_rotate(x: torch.Tensor, pos: torch.Tensor, base: float) -> torch.Tensor:
    """Rotate-half RoPE of the last dim of ``x`` at integer positions ``pos``.

    Pairs (i, i + d/2) are rotated by pos * base^(-2i/d); angles in fp64.
    ``pos`` broadcasts against ``x.shape[:-1]``.
    """
    d = x.shape[-1]
    h = d // 2
    i = torch.arange(h, dtype=torch.float64, device=x.device)
    theta = torch.pow(torch.tensor(base, dtype=torch.float64, device=x.device), -2.0 * i / d)
    ang = pos.to(torch.float64).unsqueeze(-1) * theta
    c = torch.cos(ang)
    s = torch.sin(ang)
    xd = x.to(torch.float64)
    x1, x2 = xd[..., :h], xd[..., h:]
    out = torch.cat([x1 * c - x2 * s, x1 * s + x2 * c], dim=-1)
    return out.to(x.dtype)


def _centroids(wl: Workload, b: int, h: int, device) -> torch.Tensor:
    g = _gen(device, wl.index, b, h, 1)
    if wl.placement == "hier":
        d = wl.d
        mu_a = torch.randn(8, d, generator=g, device=device)
        mu_ab = mu_a.repeat_interleave(8, 0) + 0.5 * torch.randn(64, d, generator=g, device=device)
        mu_abc = mu_ab.repeat_interleave(8, 0) + 0.25 * torch.randn(512, d, generator=g, device=device)
        return mu_abc
    return torch.randn(wl.n_clusters, wl.d, generator=g, device=device)


def _assignment(wl: Workload, b: int, h: int, T: int, device) -> torch.Tensor:
    """Cluster id per token position [T] (int64)."""
    g = _gen(device, wl.index, b, h, 2)
    if wl.placement == "hier":
        seg = wl.N // 512 if wl.N >= 512 else 1
        idx = torch.arange(T, device=device) // seg
        return idx.clamp_max(511)
    law = _cluster_law(wl, device)
    if wl.placement == "iid":
        return torch.multinomial(law, T, replacement=True, generator=g)
    # Contiguous runs, Geometric lengths with mean C, cluster per run from the law.
    n_runs = max(16, int(2 * T / wl.C) + 64)
    lens = torch.empty(n_runs, dtype=torch.float32, device=device).geometric_(1.0 / wl.C, generator=g)
    lens = lens.to(torch.int64)
    while int(lens.sum()) < T:
        more = torch.empty(n_runs, dtype=torch.float32, device=device).geometric_(1.0 / wl.C, generator=g)
        lens = torch.cat([lens, more.to(torch.int64)])
    cl = torch.multinomial(law, lens.numel(), replacement=True, generator=g)
    return torch.repeat_interleave(cl, lens)[:T]


def make_cache(wl: Workload, device="cpu", T_cap: Optional[int] = None):
    """KV cache [B][H_kv][T_cap][d] in the workload's dtype, filled for [0, T_final).

    Also returns the cluster id of every token ([B][H_kv][T_final], int64) so that
    decode queries can be drawn from the same law.
    """
    T = wl.T_final
    if T_cap is None:
        T_cap = T
    assert T_cap >= T
    dt = torch.float32 if wl.kv_dtype == "f32" else torch.bfloat16
    K = torch.zeros(wl.B, wl.H_kv, T_cap, wl.d, dtype=dt, device=device)
    V = torch.zeros(wl.B, wl.H_kv, T_cap, wl.d, dtype=dt, device=device)
    for b in range(wl.B):
        for h in range(wl.H_kv):
            mu = _centroids(wl, b, h, device)
            z = _assignment(wl, b, h, T, device)
            gk = _gen(device, wl.index, b, h, 3)
            gv = _gen(device, wl.index, b, h, 4)
            sig = 0.1 if wl.placement == "hier" else wl.sigma
            k = mu[z] + sig * torch.randn(T, wl.d, generator=gk, device=device)
            k[0] *= wl.sink_scale
            if wl.rope:
                pos = torch.arange(T, device=device)
                k = rope_rotate(k, pos, wl.rope_base)
            K[b, h, :T] = k.to(dt)
            V[b, h, :T] = torch.randn(T, wl.d, generator=gv, device=device).to(dt)
            del k
    return K, V


def make_qref(wl: Workload, device="cpu") -> torch.Tensor:
    """Reference queries [H_kv][R][d] fp32, N(0,1)/sqrt(d)."""
    g = _gen(device, wl.index, 0, 0, 5)
    return torch.randn(wl.H_kv, wl.R, wl.d, generator=g, device=device) / math.sqrt(wl.d)


def make_query(wl: Workload, step: int, T: int, device="cpu") -> torch.Tensor:
    """Decode queries [B][Hq][d] fp32 for one step at cache length T.

    Query head j of sequence b draws a cluster of its KV head's centroids from the
    workload's law (for ``hier`` a leaf cluster uniformly) and adds N(0, q_sigma^2).
    """
    Q = torch.empty(wl.B, wl.Hq, wl.d, dtype=torch.float32, device=device)
    for b in range(wl.B):
        for h in range(wl.H_kv):
            mu = _centroids(wl, b, h, device)
            g = _gen(device, wl.index, b, h, 6, step)
            if wl.placement == "hier":
                c = torch.randint(0, mu.shape[0], (wl.G,), generator=g, device=device)
            else:
                c = torch.multinomial(_cluster_law(wl, device), wl.G, replacement=True, generator=g)
            q = mu[c] + wl.q_sigma * torch.randn(wl.G, wl.d, generator=g, device=device)
            if wl.rope:
                q = rope_rotate(q, torch.full((wl.G,), T - 1, device=device), wl.rope_base)
            Q[b, h * wl.G:(h + 1) * wl.G] = q
    return Q


def make_queries(wl: Workload, n_steps: int, device="cpu") -> torch.Tensor:
    """Queries for steps 0..n_steps-1, step s at T = T0 + s: [n_steps][B][Hq][d]."""
    return torch.stack([make_query(wl, s, wl.T0 + s, device) for s in range(n_steps)])

"""Seeded synthetic inputs for the latent-sparse-attention layer.

This module only draws random numbers. It holds none of the method's arithmetic
(no projection, clustering, scoring or attention), so the HIP path and the CPU
oracle can both be fed from it without sharing any computation.

Workloads follow the shapes of the pages' measurements: a KV cache of clustered
Gaussian keys, a per-KV-head latent projection, and queries that are perturbed
copies of an earlier key (Latent Sparse Attention, bdtechtalks.com, "How latent
sparse attention works" and "LSA in action": single-request decode and
last-chunk prefill at 1M-10M tokens; 128k-token training-shaped layers).

Recipe (one per workload, seeds data = 1000 + i, W = 2000 + i, queries = 3000 + i):
  * every KV head g has its own mixture: centres muK[g], muV[g] ~ N(0, I_d);
    token t of head g draws one component c uniformly and takes
    K = muK[c] + 0.3 eps, V = muV[c] + 0.3 eps' (eps, eps' ~ N(0, I_d));
  * W_lat[g] ~ N(0, 1/d) of shape [d, r];
  * query row i at position pos_i: for each KV head g a target key j is drawn
    uniformly from [0, min(pos_i, n - 1)], and every query head of g's group is
    K[g, j] + 0.1 N(0, I_d);
  * values are drawn in fp32 and rounded once (round-to-nearest-even) to the
    storage dtype.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int            # position in the workload list, used for seeds
    n: int                # keys in the cache
    h_q: int              # query heads
    h_kv: int             # KV heads
    d: int                # head dimension
    dtype: str            # "f32" or "bf16"
    r: int                # latent dimension
    b: int                # branching factor
    L: int                # tree levels below the root
    iters: int            # Lloyd iterations per level
    beam: int             # nodes kept per level
    k: int                # keys retrieved per query group
    centres: int          # Gaussian mixture components per KV head
    m: int                # query rows
    mode: str             # "decode" (pos = n), "chunk" (last m positions), "all" (pos 0..n-1)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def positions(self) -> torch.Tensor:
        if self.mode == "decode":
            return torch.full((self.m,), self.n, dtype=torch.int32)
        if self.mode == "chunk":
            return torch.arange(self.n - self.m, self.n, dtype=torch.int32)
        if self.mode == "all":
            assert self.m == self.n
            return torch.arange(0, self.n, dtype=torch.int32)
        raise ValueError(self.mode)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: a tiny parity case, decode and last-chunk prefill at 1M
# tokens, decode at 10M tokens, and a training-shaped causal layer at 128k.
WORKLOADS = {
    "tiny_4k": Workload("tiny_4k", 0, n=4096, h_q=1, h_kv=1, d=128, dtype="f32", r=32,
                        b=16, L=2, iters=5, beam=4, k=256, centres=256, m=1, mode="decode"),
    "decode_1m": Workload("decode_1m", 1, n=1 << 20, h_q=32, h_kv=4, d=128, dtype="bf16", r=64,
                          b=64, L=3, iters=5, beam=16, k=2048, centres=65536, m=1, mode="decode"),
    "prefill_1m": Workload("prefill_1m", 2, n=1 << 20, h_q=32, h_kv=4, d=128, dtype="bf16", r=64,
                           b=64, L=3, iters=5, beam=16, k=2048, centres=65536, m=4096, mode="chunk"),
    "decode_10m": Workload("decode_10m", 3, n=10 << 20, h_q=32, h_kv=4, d=128, dtype="bf16", r=64,
                           b=64, L=4, iters=5, beam=16, k=4096, centres=1 << 20, m=1, mode="decode"),
    "train_128k": Workload("train_128k", 4, n=1 << 17, h_q=16, h_kv=4, d=128, dtype="bf16", r=64,
                           b=32, L=3, iters=5, beam=16, k=2048, centres=8192, m=1 << 17, mode="all"),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def make_kv(w: Workload, device="cpu", seed: Optional[int] = None):
    """K, V of shape [h_kv, n, d] in the workload dtype, drawn head by head."""
    seed = 1000 + w.index if seed is None else seed
    g = _gen(seed, device)
    K = torch.empty((w.h_kv, w.n, w.d), dtype=w.torch_dtype, device=device)
    V = torch.empty_like(K)
    chunk = 1 << 20
    for h in range(w.h_kv):
        muK = torch.randn((w.centres, w.d), generator=g, device=device)
        muV = torch.randn((w.centres, w.d), generator=g, device=device)
        for s in range(0, w.n, chunk):
            e = min(w.n, s + chunk)
            comp = torch.randint(0, w.centres, (e - s,), generator=g, device=device)
            K[h, s:e] = (muK[comp] + 0.3 * torch.randn((e - s, w.d), generator=g, device=device)).to(w.torch_dtype)
            V[h, s:e] = (muV[comp] + 0.3 * torch.randn((e - s, w.d), generator=g, device=device)).to(w.torch_dtype)
        del muK, muV
    return K, V


def make_w(w: Workload, device="cpu", seed: Optional[int] = None) -> torch.Tensor:
    """W_lat of shape [h_kv, d, r], fp32, N(0, 1/d)."""
    seed = 2000 + w.index if seed is None else seed
    g = _gen(seed, device)
    return torch.randn((w.h_kv, w.d, w.r), generator=g, device=device) * (1.0 / w.d) ** 0.5


def make_queries(w: Workload, K: torch.Tensor, pos: torch.Tensor, seed: Optional[int] = None,
                 sigma: float = 0.1) -> torch.Tensor:
    """Q of shape [m, h_q, d] in K's dtype: perturbed copies of an eligible key."""
    seed = 3000 + w.index if seed is None else seed
    device = K.device
    m = pos.shape[0]
    g = _gen(seed, device)
    G = w.h_q // w.h_kv
    hi = torch.clamp(pos.to(device=device, dtype=torch.int64), max=w.n - 1)
    Q = torch.empty((m, w.h_q, w.d), dtype=K.dtype, device=device)
    chunk = 1 << 16
    for s in range(0, m, chunk):
        e = min(m, s + chunk)
        u = torch.rand((e - s, w.h_kv), generator=g, device=device, dtype=torch.float64)
        tgt = torch.minimum((u * (hi[s:e, None] + 1).double()).floor().long(), hi[s:e, None])
        base = K[torch.arange(w.h_kv, device=device)[None, :], tgt].float()    # [rows, h_kv, d]
        base = base.repeat_interleave(G, dim=1)                                 # [rows, h_q, d]
        noise = torch.randn((e - s, w.h_q, w.d), generator=g, device=device)
        Q[s:e] = (base + sigma * noise).to(K.dtype)
    return Q


def make_lowrank_keys(n: int, h: int, d: int, dtype=torch.bfloat16, seed: int = 4000, decay: float = 0.97,
                      noise: float = 0.05, device="cpu") -> torch.Tensor:
    """Keys with a decaying spectrum, [h, n, d]: per head, K = (Z * s) R^T + mu
    + noise * eps with Z, eps ~ N(0, I), s_i = decay^i (distinct principal
    scales), R a random orthogonal matrix (QR of a Gaussian matrix) and
    mu ~ N(0, I).  Rounded once to `dtype`."""
    g = _gen(seed, device)
    K = torch.empty((h, n, d), dtype=dtype, device=device)
    sc = decay ** torch.arange(d, dtype=torch.float32, device=device)
    chunk = 1 << 20
    for hh in range(h):
        R, _ = torch.linalg.qr(torch.randn((d, d), generator=g, device=device, dtype=torch.float64))
        R = R.float()
        mu = torch.randn((d,), generator=g, device=device)
        for s0 in range(0, n, chunk):
            e = min(n, s0 + chunk)
            Z = torch.randn((e - s0, d), generator=g, device=device) * sc
            eps = torch.randn((e - s0, d), generator=g, device=device)
            K[hh, s0:e] = (Z @ R.T + mu + noise * eps).to(dtype)
    return K


def make_workload(w: Workload, device="cpu", m: Optional[int] = None, pos: Optional[torch.Tensor] = None):
    """Everything one pass of the layer needs: K, V, W_lat, Q and query positions."""
    K, V = make_kv(w, device)
    W = make_w(w, device)
    if pos is None:
        pos = w.positions()
        if m is not None:
            pos = pos[-m:] if w.mode != "decode" else pos[:m]
    pos = pos.to(torch.int32)
    Q = make_queries(w, K, pos)
    return dict(K=K, V=V, W=W, Q=Q, pos=pos.to(device))

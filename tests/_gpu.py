"""Helpers for the GPU parity tests: move the HIP library's outputs to the host
in the oracle's layout, and compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from _ref import node_members


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def np32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy() if t.dtype != torch.float32 else t.detach().cpu().numpy()


def host_index(views, desc) -> "oracle.Index":
    """The GPU-built tree as an oracle.Index (levels concatenated, int64 counts)."""
    L = desc.L
    Cs = [views["C"][l].reshape(-1) for l in range(1, L + 1)]
    cn = [views["cnt"][l].reshape(-1).to(torch.int64) for l in range(1, L + 1)]
    C_all = torch.cat(Cs).cpu().numpy()
    cnt_all = torch.cat(cn).cpu().numpy()
    return oracle.Index(desc.n, desc.h_kv, desc.r, desc.b, L, C_all, cnt_all,
                        views["leaf_off"].to(torch.int64).cpu().numpy(), views["perm"].cpu().numpy())


def assert_same_bits(a: np.ndarray, b: np.ndarray, what: str):
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    if a.dtype == np.float32:
        a, b = a.view(np.int32), b.view(np.int32)
    bad = np.nonzero(a.reshape(-1) != b.reshape(-1))[0]
    assert bad.size == 0, f"{what}: {bad.size} of {a.size} differ, first at flat index {bad[:8]}"


def assert_index_equal(gix: "oracle.Index", oix: "oracle.Index"):
    for l in range(1, oix.L + 1):
        assert_same_bits(gix.cnt(l), oix.cnt(l), f"counts level {l}")
        assert_same_bits(gix.C(l), oix.C(l), f"centroids level {l}")
    assert_same_bits(gix.leaf_off, oix.leaf_off, "leaf offsets")
    assert_same_bits(gix.perm, oix.perm, "leaf members")


def replay_node(K: torch.Tensor, W: torch.Tensor, gix: "oracle.Index", g: int, l: int, u: int, iters: int):
    """Re-run the oracle's k-means of parent u (level l-1) on the members the GPU
    tree gives it and compare the children (counts, centroids, members)."""
    b, L, n = gix.b, gix.L, gix.n
    if l == 1:
        mem = np.arange(n, dtype=np.int64)
    else:
        mem = node_members(gix.leaf_off[g], gix.perm[g], b, L, l - 1, u).astype(np.int64)
    m = len(mem)
    if m == 0:
        assert np.all(gix.cnt(l)[g][u * b:(u + 1) * b] == 0)
        return 0
    Kh = np32(K[g][torch.from_numpy(mem).to(K.device)])
    Z = oracle.project(Kh, np32(W[g]))
    C, asg, cnt = oracle.lloyd_node(Z, np.arange(m, dtype=np.int32), b, iters)
    assert_same_bits(gix.cnt(l)[g][u * b:(u + 1) * b], cnt, f"counts of children of ({g},{l - 1},{u})")
    assert_same_bits(gix.C(l)[g][u * b:(u + 1) * b], C, f"centroids of children of ({g},{l - 1},{u})")
    for c in range(b):
        if cnt[c] == 0:
            continue
        got = node_members(gix.leaf_off[g], gix.perm[g], b, L, l, u * b + c)
        assert np.array_equal(got, mem[asg == c]), f"members of child {c} of ({g},{l - 1},{u})"
    return m


def compact_kv(K: torch.Tensor, V: torch.Tensor, sel: np.ndarray, count: np.ndarray):
    """Gather only the rows a set of selections uses; remap the selections."""
    h = K.shape[0]
    keys = [np.unique(np.concatenate([sel[i, g, :count[i, g]] for i in range(sel.shape[0])] + [np.zeros(1, np.int32)]))
            for g in range(h)]
    width = max(len(x) for x in keys)
    Kc = np.zeros((h, width, K.shape[2]), np.float32)
    Vc = np.zeros_like(Kc)
    sel2 = sel.copy()
    for g in range(h):
        idx = torch.from_numpy(keys[g].astype(np.int64)).to(K.device)
        Kc[g, :len(keys[g])] = np32(K[g][idx])
        Vc[g, :len(keys[g])] = np32(V[g][idx])
        for i in range(sel.shape[0]):
            c = count[i, g]
            sel2[i, g, :c] = np.searchsorted(keys[g], sel[i, g, :c])
    return Kc, Vc, sel2

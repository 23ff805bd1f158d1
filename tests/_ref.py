"""Independent checks used by the tests: brute-force selection, tree walkers and
tolerances.  Written with numpy from the definitions, sharing no code with the
oracle's C source or the HIP library."""
from __future__ import annotations

import numpy as np


def fl32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def group_latent(Q, W, g, G):
    """u for query row Q[h_q, d] and KV head g: fl32(fl32(mean of the group) . W_g)."""
    qbar = fl32(Q[g * G:(g + 1) * G].astype(np.float64).sum(axis=0) / G)
    return fl32(qbar.astype(np.float64) @ W[g].astype(np.float64))


def node_members(leaf_off, perm, b, L, level, v):
    """Members (ascending) of node v at `level`, read off the leaf CSR: the leaves
    below v are the contiguous id range [v*b^(L-level), (v+1)*b^(L-level))."""
    span = b ** (L - level)
    s, e = int(leaf_off[v * span]), int(leaf_off[(v + 1) * span])
    return np.sort(perm[s:e])


def brute_select(Q, pos, Cs, cnts, leaf_off, perm, W, G, beam, k):
    """Score every node of every level (no pruning), then apply the per-level
    top-beam rule and the causal fill.  Q: [h_q, d] of one row; Cs/cnts: lists
    indexed by level-1 of [h_kv, b^l, r] / [h_kv, b^l]; returns per KV head
    (sel in retrieval order, count, cutoff, n_scored)."""
    h_kv = Cs[0].shape[0]
    b = Cs[0].shape[1]
    L = len(Cs)
    out = []
    for g in range(h_kv):
        u = group_latent(Q, W, g, G).astype(np.float64)
        scores = [fl32(Cs[l][g].astype(np.float64) @ u) for l in range(L)]
        cand = [v for v in range(b) if cnts[0][g][v] > 0]
        nsc = 0
        for l in range(L):
            nsc += len(cand)
            order = sorted(cand, key=lambda v: (-float(scores[l][v]), v))
            if l == L - 1:
                leaves = order
                break
            kept = order[:beam]
            cand = [v * b + c for v in kept for c in range(b) if cnts[l + 1][g][v * b + c] > 0]
        taken, cut = [], float("-inf")
        for v in leaves:
            for j in perm[g][leaf_off[g][v]:leaf_off[g][v + 1]]:
                if len(taken) == k:
                    break
                if j <= pos:
                    taken.append(int(j))
                    if len(taken) == k:
                        cut = float(scores[L - 1][v])
        out.append((taken, len(taken), cut, nsc))
    return out


def check_tree(Zs, Cs, cnts, leaf_off, perm, b, L, ulps=1):
    """Structural invariants of a tree plus 'centroid = mean of its members'
    (numpy float64 mean, compared within `ulps` float32 ulps)."""
    h_kv, n = perm.shape
    for g in range(h_kv):
        assert np.array_equal(np.sort(perm[g]), np.arange(n)), "perm is not a permutation"
        lo = leaf_off[g]
        assert lo[0] == 0 and lo[-1] == n and np.all(np.diff(lo) >= 0)
        assert np.array_equal(np.diff(lo), cnts[L - 1][g]), "leaf CSR disagrees with leaf counts"
        for v in range(b ** L):
            seg = perm[g][lo[v]:lo[v + 1]]
            assert np.all(np.diff(seg) > 0), "leaf members not ascending"
        assert cnts[0][g].sum() == n
        for l in range(1, L):
            par = cnts[l - 1][g]
            ch = cnts[l][g].reshape(-1, b).sum(axis=1)
            assert np.array_equal(par, ch), "parent count != sum of children"
        for l in range(1, L + 1):
            for v in np.nonzero(cnts[l - 1][g])[0]:
                mem = node_members(lo, perm[g], b, L, l, int(v))
                mean = fl32(Zs[g][mem].astype(np.float64).mean(axis=0))
                got = Cs[l - 1][g][v]
                assert ulp_diff(got, mean).max() <= ulps, (g, l, v)


def ulp_diff(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    a = np.where(a < 0, np.int64(-2**31) - a, a)
    b = np.where(b < 0, np.int64(-2**31) - b, b)
    return np.abs(a - b)

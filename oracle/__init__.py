"""CPU oracle for the latent-sparse-attention layer (ctypes wrapper over lsa_oracle.c).

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's CPU
baseline may import this package.  It shares no code with the HIP library.

Every function takes and returns numpy arrays on the host.  bf16 inputs are
widened to float32 by the caller (an exact conversion).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lsa_oracle.c")
_LIB = os.path.join(_HERE, "_lib", "liboracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no FP contraction)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.oracle_threads.restype = i32
        L.oracle_project.argtypes = [P, i64, i32, P, i32, P]
        L.oracle_lloyd_node.argtypes = [P, i32, P, i64, i32, i32, P, P, P]
        L.oracle_level_base.argtypes = [i32, i32, i32]
        L.oracle_level_base.restype = i64
        L.oracle_build.argtypes = [P, i64, i32, i32, P, i32, i32, i32, i32, P, P, P, P]
        L.oracle_build.restype = i32
        L.oracle_select.argtypes = [P, i64, i32, i32, P, i64, i32, i32, i32, i32,
                                    P, P, P, P, P, i32, i32, i32, i32, P, P, P, P, P]
        L.oracle_select.restype = i32
        L.oracle_select_flat.argtypes = [P, i64, i32, i32, P, i64, i32, i32, i32, i32,
                                         P, P, P, P, P, i32, i32, i32, P, P, P, P]
        L.oracle_select_flat.restype = i32
        L.oracle_attend.argtypes = [P, P, P, i64, i32, i32, i64, i32, P, P, i32, dbl, P, P]
        L.oracle_attend.restype = i32
        _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def threads() -> int:
    return lib().oracle_threads()


def project(K: np.ndarray, W: np.ndarray) -> np.ndarray:
    """One KV head: K [n, d] float32, W [d, r] float32 -> Z [n, r] float32."""
    K = _c(K, np.float32); W = _c(W, np.float32)
    n, d = K.shape
    r = W.shape[1]
    Z = np.empty((n, r), np.float32)
    lib().oracle_project(_p(K), n, d, _p(W), r, _p(Z))
    return Z


def lloyd_node(Z: np.ndarray, members: np.ndarray, b: int, T: int):
    """k-means of one node: returns (C [b, r], assign [m], cnt [b])."""
    Z = _c(Z, np.float32)
    S = _c(members, np.int32)
    r = Z.shape[1]
    m = S.shape[0]
    C = np.empty((b, r), np.float32)
    asg = np.empty((max(m, 1),), np.int32)
    cnt = np.empty((b,), np.int64)
    lib().oracle_lloyd_node(_p(Z), r, _p(S), m, b, T, _p(C), _p(asg), _p(cnt))
    return C, asg[:m], cnt


class Index:
    """The oracle's tree: per level l = 1..L, centroids C[l] [h, b^l, r] and
    counts cnt[l] [h, b^l]; leaf CSR leaf_off [h, b^L + 1] and perm [h, n]."""

    def __init__(self, n, h_kv, r, b, L, C_all, cnt_all, leaf_off, perm):
        self.n, self.h_kv, self.r, self.b, self.L = n, h_kv, r, b, L
        self.C_all, self.cnt_all, self.leaf_off, self.perm = C_all, cnt_all, leaf_off, perm

    @staticmethod
    def level_base(h_kv, b, l):
        s = 0
        for q in range(1, l):
            s += b ** q
        return s * h_kv

    def C(self, l):
        nodes = self.b ** l
        s = self.level_base(self.h_kv, self.b, l)
        return self.C_all[s * self.r:(s + self.h_kv * nodes) * self.r].reshape(self.h_kv, nodes, self.r)

    def cnt(self, l):
        nodes = self.b ** l
        s = self.level_base(self.h_kv, self.b, l)
        return self.cnt_all[s:s + self.h_kv * nodes].reshape(self.h_kv, nodes)

    @classmethod
    def from_levels(cls, n, h_kv, r, b, L, Cs, cnts, leaf_off, perm):
        """Assemble from per-level arrays (e.g. another implementation's tree)."""
        C_all = np.concatenate([np.ascontiguousarray(c, np.float32).reshape(-1) for c in Cs])
        cnt_all = np.concatenate([np.ascontiguousarray(c, np.int64).reshape(-1) for c in cnts])
        return cls(n, h_kv, r, b, L, C_all, cnt_all,
                   np.ascontiguousarray(leaf_off, np.int64), np.ascontiguousarray(perm, np.int32))


def build_index(K: np.ndarray, W: np.ndarray, b: int, L: int, T: int = 5) -> Index:
    """K [h, n, d] float32, W [h, d, r] float32."""
    K = _c(K, np.float32); W = _c(W, np.float32)
    h, n, d = K.shape
    r = W.shape[2]
    tot = sum(b ** l for l in range(1, L + 1)) * h
    C_all = np.zeros((tot * r,), np.float32)
    cnt_all = np.zeros((tot,), np.int64)
    leaf_off = np.zeros((h, b ** L + 1), np.int64)
    perm = np.zeros((h, n), np.int32)
    lib().oracle_build(_p(K), n, h, d, _p(W), r, b, L, T, _p(C_all), _p(cnt_all), _p(leaf_off), _p(perm))
    return Index(n, h, r, b, L, C_all, cnt_all, leaf_off, perm)


def select(Q: np.ndarray, pos: np.ndarray, index: Index, W: np.ndarray, beam: int, k: int,
           want_kept: bool = False, n_sink: int = 0, window: int = 0):
    """Q [m, h_q, d] float32, pos [m] int32.  Returns dict with sel [m, h_kv,
    k + n_sink + window] (retrieved keys, then sinks, then window, -1 padded),
    count [m, h_kv], cutoff [m, h_kv], nscored [m, h_kv] and optionally kept
    [m, h_kv, L-1, beam]."""
    Q = _c(Q, np.float32); pos = _c(pos, np.int32); W = _c(W, np.float32)
    m, h_q, d = Q.shape
    ix = index
    sel = np.empty((m, ix.h_kv, k + n_sink + window), np.int32)
    cnt = np.empty((m, ix.h_kv), np.int32)
    cut = np.empty((m, ix.h_kv), np.float32)
    nsc = np.empty((m, ix.h_kv), np.int64)
    kept = np.empty((m, ix.h_kv, max(ix.L - 1, 1), beam), np.int32) if want_kept else None
    lib().oracle_select(_p(Q), m, h_q, d, _p(pos), ix.n, ix.h_kv, ix.r, ix.b, ix.L,
                        _p(ix.C_all), _p(ix.cnt_all), _p(ix.leaf_off), _p(ix.perm), _p(W),
                        beam, k, n_sink, window, _p(sel), _p(cnt), _p(cut), _p(kept), _p(nsc))
    out = dict(sel=sel, count=cnt, cutoff=cut, nscored=nsc)
    if want_kept:
        out["kept"] = kept
    return out


def select_flat(Q: np.ndarray, pos: np.ndarray, index: Index, W: np.ndarray, k: int,
                n_sink: int = 0, window: int = 0):
    """Flat search: every non-empty leaf scored.  Same outputs as select()
    (sel [m, h_kv, k + n_sink + window], count, cutoff, nscored)."""
    Q = _c(Q, np.float32); pos = _c(pos, np.int32); W = _c(W, np.float32)
    m, h_q, d = Q.shape
    ix = index
    sel = np.empty((m, ix.h_kv, k + n_sink + window), np.int32)
    cnt = np.empty((m, ix.h_kv), np.int32)
    cut = np.empty((m, ix.h_kv), np.float32)
    nsc = np.empty((m, ix.h_kv), np.int64)
    lib().oracle_select_flat(_p(Q), m, h_q, d, _p(pos), ix.n, ix.h_kv, ix.r, ix.b, ix.L,
                             _p(ix.C_all), _p(ix.cnt_all), _p(ix.leaf_off), _p(ix.perm), _p(W),
                             k, n_sink, window, _p(sel), _p(cnt), _p(cut), _p(nsc))
    return dict(sel=sel, count=cnt, cutoff=cut, nscored=nsc)


def attend(Q: np.ndarray, K: np.ndarray, V: np.ndarray, sel: np.ndarray, count: np.ndarray,
           scale: float | None = None):
    """Q [m, h_q, d], K/V [h_kv, n, d] float32; sel [m, h_kv, k] int32; count
    [m, h_kv].  Returns (out [m, h_q, d] float64, lse [m, h_q] float64)."""
    Q = _c(Q, np.float32); K = _c(K, np.float32); V = _c(V, np.float32)
    sel = _c(sel, np.int32); count = _c(count, np.int32)
    m, h_q, d = Q.shape
    h_kv, n, _ = K.shape
    k = sel.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.empty((m, h_q, d), np.float64)
    lse = np.empty((m, h_q), np.float64)
    lib().oracle_attend(_p(Q), _p(K), _p(V), m, h_q, h_kv, n, d, _p(sel), _p(count), k,
                        float(scale), _p(out), _p(lse))
    return out, lse


def pca_projection(K: np.ndarray, r: int):
    """Training-free latent projection ("Latent sparse attention",
    bdtechtalks.com, "How latent sparse attention works": principal component
    analysis builds the indexing space without trained projections).

    Per KV head g: C = (1/n) sum_j (k_j - mu)(k_j - mu)^T in float64 (mu the
    mean key), its eigenvectors by numpy's symmetric eigensolver, the r with
    the largest eigenvalues as the columns of W_g, largest first.  Each column
    is signed so that its entry of largest magnitude (the first such) is
    positive.  K [h, n, d] float32 -> (W [h, d, r] float32, eigenvalues [h, r]
    float64)."""
    K = np.asarray(K, dtype=np.float32)
    h, n, d = K.shape
    W = np.empty((h, d, r), np.float32)
    ev = np.empty((h, r), np.float64)
    for g in range(h):
        X = K[g].astype(np.float64)
        Xc = X - X.mean(axis=0)
        C = (Xc.T @ Xc) / n
        lam, vec = np.linalg.eigh(C)
        order = np.argsort(-lam, kind="stable")[:r]
        V = vec[:, order]
        for c in range(r):
            j = int(np.argmax(np.abs(V[:, c])))
            if V[j, c] < 0:
                V[:, c] = -V[:, c]
        W[g] = V.astype(np.float32)
        ev[g] = lam[order]
    return W, ev


def index_insert(index: Index, K_new: np.ndarray, W: np.ndarray) -> Index:
    """Incremental insertion of keys appended to the cache ("Latent Sparse
    Attention Breaks Through the Million-Token Context Bottleneck",
    kongchang.com, "How LSA Sidesteps Per-Key Scoring with Hierarchical
    Clustering": the key index is precomputed and updated).

    K_new [h, m, d] float32 are the keys at positions n .. n + m - 1.  Readings:
      - each new key's latent z = fl32(k . W_g) descends from the root to the
        nearest non-empty child at every level (squared Euclidean distance in
        double, dimensions ascending, each difference and square rounded once;
        ties to the smaller child), against the centroids as they were before
        the batch;
      - every node on a path then takes its new keys: with c its old count and
        S the double sum of their latents (keys ascending),
        centroid = fl32((c * centroid + S) / (c + #new)), count = c + #new
        (one new key: the online k-means update);
      - a leaf's members are its old members followed by its new keys
        (ascending positions).
    Returns the tree over n + m keys."""
    ix = index
    K_new = np.ascontiguousarray(K_new, np.float32)
    W = np.ascontiguousarray(W, np.float32)
    h, m, d = K_new.shape
    n, r, b, L = ix.n, ix.r, ix.b, ix.L
    Cs = [ix.C(l).copy() for l in range(1, L + 1)]
    cnts = [ix.cnt(l).copy() for l in range(1, L + 1)]
    nleaf = b ** L
    leaf_off = np.zeros((h, nleaf + 1), np.int64)
    perm = np.zeros((h, n + m), np.int32)
    for g in range(h):
        Z = project(K_new[g], W[g]).astype(np.float64)          # [m, r], exact fp32 values
        paths = np.zeros((m, L), np.int64)
        for j in range(m):
            u = 0
            for l in range(L):
                ch = u * b + np.arange(b)
                cand = ch[ix.cnt(l + 1)[g][ch] > 0]
                Cc = ix.C(l + 1)[g][cand].astype(np.float64)   # centroids before the batch
                dist = np.zeros(len(cand))
                for i in range(r):
                    t = Z[j, i] - Cc[:, i]
                    dist = dist + t * t
                u = int(cand[int(np.argmin(dist))])
                paths[j, l] = u
        for l in range(L):
            for v in np.unique(paths[:, l]):
                js = np.nonzero(paths[:, l] == v)[0]
                S = np.zeros(r)
                for j in js:
                    S = S + Z[j]
                c_old = float(ix.cnt(l + 1)[g][v])
                c0 = ix.C(l + 1)[g][v].astype(np.float64)
                Cs[l][g][v] = ((c_old * c0 + S) / (c_old + len(js))).astype(np.float32)
                cnts[l][g][v] = int(c_old) + len(js)
        lo = ix.leaf_off[g]
        pos = 0
        for v in range(nleaf):
            old = ix.perm[g][lo[v]:lo[v + 1]]
            new = n + np.nonzero(paths[:, L - 1] == v)[0]
            leaf_off[g, v] = pos
            perm[g, pos:pos + len(old)] = old
            perm[g, pos + len(old):pos + len(old) + len(new)] = new
            pos += len(old) + len(new)
        leaf_off[g, nleaf] = pos
    return Index.from_levels(n + m, h, r, b, L, Cs, cnts, leaf_off, perm)

"""Pins of the CPU oracle against things other than itself: a hand-worked
example, a library k-means, a library attention, closed forms and brute force.

All tests here run on the CPU (no GPU marker)."""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from _ref import brute_select, check_tree, fl32, group_latent, node_members, ulp_diff

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _frac32(s):
    return np.float32(float(Fraction(s))) if s not in ("-inf",) else np.float32(-np.inf)


# --------------------------------------------------------------------------- golden
def test_hand_worked_tree_and_selection(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "hand_tree_6keys.json")))
    K = np.array(g["keys"], np.float32)[None]          # [1, 6, 2]
    W = np.array(g["W"], np.float32)[None]             # [1, 2, 2]
    trees = {}
    for name, t in g["trees"].items():
        ix = oracle.build_index(K, W, g["b"], t["L"], g["T"])
        trees[name] = ix
        assert np.array_equal(ix.cnt(1)[0], t["level1_counts"])
        assert np.array_equal(ix.C(1)[0], np.array([[_frac32(x) for x in row] for row in t["level1_centroids"]]))
        if t["L"] == 2:
            assert np.array_equal(ix.cnt(2)[0], t["level2_counts"])
            assert np.array_equal(ix.C(2)[0], np.array([[_frac32(x) for x in row] for row in t["level2_centroids"]]))
        lo = ix.leaf_off[0]
        leaves = [list(ix.perm[0][lo[v]:lo[v + 1]]) for v in range(len(lo) - 1)]
        assert leaves == t["leaf_members"]
    for q in g["queries"]:
        ix = trees[q["tree"]]
        Q = np.array(q["q"], np.float32)[None, None]
        out = oracle.select(Q, np.array([q["pos"]], np.int32), ix, W, q["beam"], q["k"],
                            n_sink=q.get("n_sink", 0), window=q.get("window", 0))
        assert list(out["sel"][0, 0]) == q["sel"]
        assert out["count"][0, 0] == q["count"]
        assert out["cutoff"][0, 0] == _frac32(q["cutoff"])
        assert out["nscored"][0, 0] == q["nscored"]
    for q in g["insertions"]:
        ix = trees[q["tree"]]
        out = oracle.index_insert(ix, np.array(q["keys"], np.float32)[None], W)
        assert out.n == ix.n + len(q["keys"])
        assert np.array_equal(out.cnt(1)[0], q["level1_counts"])
        assert np.array_equal(out.cnt(2)[0], q["level2_counts"])
        assert np.array_equal(out.C(1)[0], np.array([[_frac32(x) for x in row] for row in q["level1_centroids"]]))
        assert np.array_equal(out.C(2)[0], np.array([[_frac32(x) for x in row] for row in q["level2_centroids"]]))
        lo = out.leaf_off[0]
        assert [list(out.perm[0][lo[v]:lo[v + 1]]) for v in range(len(lo) - 1)] == q["leaf_members"]
    for q in g["flat_queries"]:
        ix = trees[q["tree"]]
        Q = np.array(q["q"], np.float32)[None, None]
        out = oracle.select_flat(Q, np.array([q["pos"]], np.int32), ix, W, q["k"],
                                 n_sink=q.get("n_sink", 0), window=q.get("window", 0))
        assert list(out["sel"][0, 0]) == q["sel"]
        assert out["count"][0, 0] == q["count"]
        assert out["cutoff"][0, 0] == _frac32(q["cutoff"])
        assert out["nscored"][0, 0] == q["nscored"]


# --------------------------------------------------------------------------- projection
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_projection_matches_float64_matmul(oracle_lib, dtype):
    g = torch.Generator().manual_seed(7)
    K = torch.randn(777, 128, generator=g).to(dtype).float().numpy()
    W = (torch.randn(128, 48, generator=g) / 128 ** 0.5).numpy()
    Z = oracle.project(K, W)
    ref = fl32(K.astype(np.float64) @ W.astype(np.float64))
    # products are exact in double; only the summation order differs
    assert ulp_diff(Z, ref).max() <= 1
    assert (Z != ref).mean() < 1e-3


# --------------------------------------------------------------------------- k-means
def _seeds(Z, members, b):
    m = len(members)
    a = min(b, m)
    return np.stack([Z[members[(c * m) // a]] for c in range(a)])


@pytest.mark.parametrize("case", [(4096, 16, 5, 0), (1500, 8, 3, 1), (300, 5, 5, 2), (2000, 32, 5, 3)])
def test_lloyd_node_matches_sklearn(oracle_lib, case):
    from sklearn.cluster import KMeans
    n, b, T, seed = case
    w = synth.WORKLOADS["tiny_4k"].replace(n=n, centres=max(b * 4, 16))
    K, _ = synth.make_kv(w, seed=100 + seed)
    W = synth.make_w(w, seed=200 + seed)
    Z = oracle.project(K[0].numpy(), W[0].numpy())
    rng = np.random.default_rng(seed)
    members = np.sort(rng.choice(n, size=n * 3 // 4, replace=False)).astype(np.int32)
    C, asg, cnt = oracle.lloyd_node(Z, members, b, T)
    init = _seeds(Z, members, b).astype(np.float64)
    km = KMeans(n_clusters=len(init), init=init, n_init=1, max_iter=T, tol=0.0, algorithm="lloyd")
    km.fit(Z[members].astype(np.float64))
    assert np.all(cnt > 0)
    # sklearn keeps float64 centres, the oracle rounds each update to float32
    np.testing.assert_allclose(C, km.cluster_centers_, rtol=1e-5, atol=1e-5)
    # the partition is the assignment to the centres before the last update
    assert np.array_equal(np.bincount(asg, minlength=b), cnt)


def test_lloyd_small_node_rules(oracle_lib):
    Z = np.array([[0, 0], [1, 1], [5, 5]], np.float32)
    # fewer members than children: one singleton child per member, the rest empty
    C, asg, cnt = oracle.lloyd_node(Z, np.array([0, 1, 2], np.int32), 4, 5)
    assert list(cnt) == [1, 1, 1, 0] and list(asg) == [0, 1, 2]
    assert np.array_equal(C[:3], Z) and np.all(C[3] == 0)
    # ties go to the smaller child: both seeds equal, so every member picks child 0
    Z2 = np.array([[1, 1], [1, 1], [1, 1], [1, 1]], np.float32)
    C, asg, cnt = oracle.lloyd_node(Z2, np.arange(4, dtype=np.int32), 2, 3)
    assert list(cnt) == [4, 0] and np.all(asg == 0)
    # empty node
    C, asg, cnt = oracle.lloyd_node(Z2, np.zeros((0,), np.int32), 3, 3)
    assert np.all(cnt == 0) and np.all(C == 0)


# --------------------------------------------------------------------------- build
def _tree_lists(ix):
    return ([ix.C(l) for l in range(1, ix.L + 1)], [ix.cnt(l) for l in range(1, ix.L + 1)])


@pytest.mark.parametrize("shape", [(4096, 1, 16, 2), (1000, 2, 4, 3), (333, 1, 8, 1), (50, 2, 3, 3),
                                   (5, 1, 4, 2), (1, 1, 2, 2)])
def test_build_invariants(oracle_lib, shape):
    n, h, b, L = shape
    w = synth.WORKLOADS["tiny_4k"].replace(n=n, h_kv=h, h_q=h, b=b, L=L, centres=64)
    K, _ = synth.make_kv(w)
    W = synth.make_w(w)
    ix = oracle.build_index(K.numpy(), W.numpy(), b, L, 5)
    Zs = [oracle.project(K[g].numpy(), W[g].numpy()) for g in range(h)]
    Cs, cnts = _tree_lists(ix)
    check_tree(Zs, Cs, cnts, ix.leaf_off, ix.perm, b, L, ulps=1)
    # every level-l node's partition is the Lloyd partition of its parent's members
    for g in range(h):
        for l in range(1, L + 1):
            for u in range(b ** (l - 1)):
                mem = (np.arange(n, dtype=np.int32) if l == 1
                       else node_members(ix.leaf_off[g], ix.perm[g], b, L, l - 1, u)).astype(np.int32)
                C, asg, cnt = oracle.lloyd_node(Zs[g], mem, b, 5)
                assert np.array_equal(cnt, cnts[l - 1][g][u * b:(u + 1) * b])
                assert np.array_equal(C, Cs[l - 1][g][u * b:(u + 1) * b])
                if u > 40:
                    break


# --------------------------------------------------------------------------- select
def _small_case(n=600, h_q=4, h_kv=2, b=4, L=3, seed=0, m=6):
    w = synth.WORKLOADS["tiny_4k"].replace(n=n, h_q=h_q, h_kv=h_kv, d=32, r=8, b=b, L=L, centres=32, m=m,
                                            mode="chunk")
    K, V = synth.make_kv(w, seed=seed)
    W = synth.make_w(w, seed=seed + 1)
    pos = torch.tensor(sorted(np.random.default_rng(seed).choice(n + 1, size=m, replace=False)), dtype=torch.int32)
    Q = synth.make_queries(w, K, pos, seed=seed + 2)
    return w, K.numpy(), V.numpy(), W.numpy(), Q.numpy(), pos.numpy()


@pytest.mark.parametrize("params", [(4, 3, 1, 17, 600), (4, 3, 2, 40, 600), (3, 2, 3, 100, 600), (5, 1, 1, 30, 600),
                                    (2, 4, 2, 64, 600), (4, 3, 100, 10000, 600), (4, 2, 2, 3, 3), (8, 2, 1, 5, 7)])
def test_select_matches_brute_force(oracle_lib, params):
    b, L, beam, k, n = params
    w, K, V, W, Q, pos = _small_case(b=b, L=L, seed=b * 10 + L, n=n, m=min(6, n + 1))
    # one all-zero query: every score ties, so only the id order decides
    Q[0] = 0.0
    ix = oracle.build_index(K, W, b, L, 5)
    out = oracle.select(Q, pos, ix, W, beam, k)
    Cs, cnts = _tree_lists(ix)
    G = w.h_q // w.h_kv
    for i in range(len(pos)):
        ref = brute_select(Q[i], int(pos[i]), Cs, cnts, ix.leaf_off, ix.perm, W, G, beam, k)
        for g, (s, c, cut, nsc) in enumerate(ref):
            assert out["count"][i, g] == c
            assert list(out["sel"][i, g, :c]) == s
            assert np.all(out["sel"][i, g, c:] == -1)
            assert ulp_diff(out["cutoff"][i, g], np.float32(cut)).max() <= 1 or (
                np.isinf(cut) and np.isinf(out["cutoff"][i, g]))
            assert out["nscored"][i, g] == nsc
            # scoring budget: b at level 1, at most beam*b below (O(log n) rows per query)
            assert nsc <= b + (L - 1) * beam * b


def test_select_full_beam_takes_every_eligible_key(oracle_lib):
    w, K, V, W, Q, pos = _small_case(b=3, L=3, seed=5)
    ix = oracle.build_index(K, W, 3, 3, 5)
    out = oracle.select(Q, pos, ix, W, beam=3 ** 2, k=w.n)
    for i, p in enumerate(pos):
        want = np.arange(min(int(p), w.n - 1) + 1)
        for g in range(w.h_kv):
            assert out["count"][i, g] == len(want)
            assert np.array_equal(np.sort(out["sel"][i, g, :len(want)]), want)
            assert np.isinf(out["cutoff"][i, g]) or len(want) == w.n


def test_flat_select_is_top_k_by_leaf_score(oracle_lib):
    """L = 1 (one level of clusters, every cluster scored): the selection is the
    first k eligible keys in (leaf score desc, leaf id asc, position asc) order,
    listed in that order."""
    w, K, V, W, Q, pos = _small_case(b=16, L=1, seed=9)
    ix = oracle.build_index(K, W, 16, 1, 5)
    k = 50
    out = oracle.select(Q, pos, ix, W, beam=1, k=k)
    G = w.h_q // w.h_kv
    from _ref import group_latent
    for i, p in enumerate(pos):
        for g in range(w.h_kv):
            u = group_latent(Q[i], W, g, G).astype(np.float64)
            leaf_score = fl32(ix.C(1)[g].astype(np.float64) @ u)
            leaf_of = np.empty(w.n, np.int64)
            for v in range(16):
                leaf_of[ix.perm[g][ix.leaf_off[g][v]:ix.leaf_off[g][v + 1]]] = v
            keys = np.arange(w.n)
            elig = keys[keys <= p]
            order = np.lexsort((elig, leaf_of[elig], -leaf_score[leaf_of[elig]].astype(np.float64)))
            want = elig[order][:k]
            c = out["count"][i, g]
            assert c == min(k, len(elig))
            assert np.array_equal(out["sel"][i, g, :c], want)


def test_selected_keys_precede_query(oracle_lib):
    w, K, V, W, Q, pos = _small_case(b=4, L=3, seed=11, m=12)
    ix = oracle.build_index(K, W, 4, 3, 5)
    out = oracle.select(Q, pos, ix, W, beam=2, k=64)
    for i, p in enumerate(pos):
        for g in range(w.h_kv):
            c = out["count"][i, g]
            s = out["sel"][i, g, :c]
            assert np.all(s <= p) and np.all(s >= 0)
            assert len(np.unique(s)) == c


# --------------------------------------------------------------------------- attend
def _sdpa_masked(Q, K, V, mask, scale):
    """torch SDPA in float64 with a boolean mask [m, h_q, n]."""
    q = torch.from_numpy(Q.astype(np.float64))[:, :, None, :]          # [m, h_q, 1, d]
    h_q, h_kv = Q.shape[1], K.shape[0]
    G = h_q // h_kv
    k = torch.from_numpy(K.astype(np.float64)).repeat_interleave(G, 0)[None]   # [1, h_q, n, d]
    v = torch.from_numpy(V.astype(np.float64)).repeat_interleave(G, 0)[None]
    msk = torch.from_numpy(mask)[:, :, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=msk, scale=scale)
    return o[:, :, 0, :].numpy()


def test_attend_matches_sdpa_with_mask(oracle_lib):
    rng = np.random.default_rng(3)
    m, h_q, h_kv, n, d, k = 5, 8, 2, 300, 64, 40
    Q = rng.standard_normal((m, h_q, d)).astype(np.float32)
    K = rng.standard_normal((h_kv, n, d)).astype(np.float32)
    V = rng.standard_normal((h_kv, n, d)).astype(np.float32)
    sel = np.full((m, h_kv, k), -1, np.int32)
    cnt = rng.integers(1, k + 1, size=(m, h_kv)).astype(np.int32)
    mask = np.zeros((m, h_q, n), bool)
    for i in range(m):
        for g in range(h_kv):
            s = np.sort(rng.choice(n, size=cnt[i, g], replace=False))
            sel[i, g, :cnt[i, g]] = s
            mask[i, g * (h_q // h_kv):(g + 1) * (h_q // h_kv), s] = True
    out, lse = oracle.attend(Q, K, V, sel, cnt)
    ref = _sdpa_masked(Q, K, V, mask, 1.0 / np.sqrt(d))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    # log-sum-exp against a direct evaluation with torch's logsumexp
    for i in range(m):
        for h in range(h_q):
            g = h // (h_q // h_kv)
            s = sel[i, g, :cnt[i, g]]
            sc = torch.from_numpy(K[g, s].astype(np.float64) @ Q[i, h].astype(np.float64) / np.sqrt(d))
            assert abs(lse[i, h] - torch.logsumexp(sc, 0).item()) < 1e-12


def test_attend_empty_selection(oracle_lib):
    Q = np.ones((1, 2, 8), np.float32)
    K = np.ones((1, 4, 8), np.float32)
    sel = np.full((1, 1, 3), -1, np.int32)
    out, lse = oracle.attend(Q, K, K, sel, np.zeros((1, 1), np.int32))
    assert np.all(out == 0) and np.all(np.isneginf(lse))


@pytest.mark.parametrize("shape", [(3, 2), (4, 3), (8, 1)])
def test_dense_equivalence(oracle_lib, shape):
    """beam covering every cluster and k = n reproduces dense causal attention."""
    b, L = shape
    w, K, V, W, Q, pos = _small_case(b=b, L=L, seed=21 + b, m=8)
    ix = oracle.build_index(K, W, b, L, 5)
    out = oracle.select(Q, pos, ix, W, beam=b ** max(L - 1, 0), k=w.n)
    o, _ = oracle.attend(Q, K, V, out["sel"], out["count"])
    keys = np.arange(w.n)
    mask = np.broadcast_to((keys[None, :] <= pos[:, None])[:, None, :], (len(pos), w.h_q, w.n)).copy()
    ref = _sdpa_masked(Q, K, V, mask, 1.0 / np.sqrt(w.d))
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- sinks and window
_LOCAL = [(0, 0), (4, 0), (0, 16), (3, 25), (50, 700), (1, 1)]


@pytest.mark.parametrize("n_sink,window", _LOCAL)
def test_local_keys_filter_the_plain_retrieval_order(oracle_lib, n_sink, window):
    """With sinks and a window, the retrieved part is the plain retrieval order
    (no local keys, k = n: the whole walk over the candidate leaves) restricted
    to [n_sink, hi - window], cut at k; the rest of the row is the sinks, then
    the window, each ascending; the parts are disjoint."""
    w, K, V, W, Q, pos = _small_case(b=4, L=3, seed=31, m=8)
    ix = oracle.build_index(K, W, 4, 3, 5)
    beam, k = 2, 37
    walk = oracle.select(Q, pos, ix, W, beam, w.n)
    out = oracle.select(Q, pos, ix, W, beam, k, n_sink=n_sink, window=window)
    assert out["sel"].shape[2] == k + n_sink + window
    for i, p in enumerate(pos):
        hi = min(int(p), w.n - 1)
        sinks = list(range(0, min(n_sink, hi + 1)))
        win = list(range(max(n_sink, hi - window + 1), hi + 1))
        for g in range(w.h_kv):
            full = walk["sel"][i, g, :walk["count"][i, g]]
            ret = [int(j) for j in full if n_sink <= j <= hi - window][:k]
            c = out["count"][i, g]
            row = list(out["sel"][i, g])
            assert c == len(ret) + len(sinks) + len(win)
            assert row[:c] == ret + sinks + win
            assert all(x == -1 for x in row[c:])
            assert len(set(row[:c])) == c
            # the latest min(window, hi + 1) visible keys are all attended
            assert set(range(max(0, hi - window + 1), hi + 1)) <= set(row[:c])
            if len(ret) == k:
                # the score of the leaf that holds the k-th retrieved key
                u = group_latent(Q[i], W, g, w.h_q // w.h_kv).astype(np.float64)
                lo = ix.leaf_off[g]
                leaf = int(np.searchsorted(lo, np.nonzero(ix.perm[g] == ret[-1])[0][0], side="right") - 1)
                assert out["cutoff"][i, g] == fl32(ix.C(3)[g][leaf].astype(np.float64) @ u)
            else:
                assert np.isneginf(out["cutoff"][i, g])


@pytest.mark.parametrize("n_sink,window", [(3, 10), (0, 64), (200, 1)])
def test_dense_equivalence_with_local_keys(oracle_lib, n_sink, window):
    """beam covering every cluster and k = n: sinks, window and retrieved keys
    together are every visible key once, so attention is dense causal."""
    b, L = 3, 3
    w, K, V, W, Q, pos = _small_case(b=b, L=L, seed=41, m=8)
    ix = oracle.build_index(K, W, b, L, 5)
    out = oracle.select(Q, pos, ix, W, beam=b ** (L - 1), k=w.n, n_sink=n_sink, window=window)
    o, _ = oracle.attend(Q, K, V, out["sel"], out["count"])
    keys = np.arange(w.n)
    mask = np.broadcast_to((keys[None, :] <= pos[:, None])[:, None, :], (len(pos), w.h_q, w.n)).copy()
    ref = _sdpa_masked(Q, K, V, mask, 1.0 / np.sqrt(w.d))
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_window_covering_the_context_is_dense_whatever_the_index(oracle_lib):
    """A window at least as long as the visible context leaves nothing to
    retrieve: any beam and k give dense causal attention."""
    w, K, V, W, Q, pos = _small_case(b=4, L=2, seed=43, m=6)
    ix = oracle.build_index(K, W, 4, 2, 5)
    out = oracle.select(Q, pos, ix, W, beam=1, k=3, n_sink=2, window=w.n)
    o, _ = oracle.attend(Q, K, V, out["sel"], out["count"])
    keys = np.arange(w.n)
    mask = np.broadcast_to((keys[None, :] <= pos[:, None])[:, None, :], (len(pos), w.h_q, w.n)).copy()
    ref = _sdpa_masked(Q, K, V, mask, 1.0 / np.sqrt(w.d))
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    assert np.all(np.isneginf(out["cutoff"]))


# --------------------------------------------------------------------------- flat search
@pytest.mark.parametrize("b,L,k,n_sink,window", [(4, 3, 40, 0, 0), (3, 2, 17, 2, 9), (8, 2, 200, 0, 31),
                                                 (16, 1, 50, 5, 0), (5, 3, 1, 0, 0), (4, 2, 10000, 3, 3)])
def test_flat_select_matches_numpy_ranking(oracle_lib, b, L, k, n_sink, window):
    """Flat search against a numpy ranking of every key by (leaf score desc,
    leaf id asc, position asc), the leaf scores computed from the leaf
    centroids with a float64 matmul; then the sinks and the window."""
    w, K, V, W, Q, pos = _small_case(b=b, L=L, seed=50 + b * 3 + L, m=6)
    Q[0] = 0.0
    ix = oracle.build_index(K, W, b, L, 5)
    out = oracle.select_flat(Q, pos, ix, W, k, n_sink=n_sink, window=window)
    G = w.h_q // w.h_kv
    keys = np.arange(w.n)
    for i, p in enumerate(pos):
        hi = min(int(p), w.n - 1)
        for g in range(w.h_kv):
            u = group_latent(Q[i], W, g, G).astype(np.float64)
            leaf_score = fl32(ix.C(L)[g].astype(np.float64) @ u)
            leaf_of = np.empty(w.n, np.int64)
            lo = ix.leaf_off[g]
            for v in range(b ** L):
                leaf_of[ix.perm[g][lo[v]:lo[v + 1]]] = v
            elig = keys[(keys >= n_sink) & (keys <= hi - window)]
            order = np.lexsort((elig, leaf_of[elig], -leaf_score[leaf_of[elig]].astype(np.float64)))
            ret = list(elig[order][:k])
            local = list(range(0, min(n_sink, hi + 1))) + list(range(max(n_sink, hi - window + 1), hi + 1))
            c = out["count"][i, g]
            assert c == len(ret) + len(local)
            assert list(out["sel"][i, g, :c]) == ret + local
            assert np.all(out["sel"][i, g, c:] == -1)
            if len(ret) == k:
                assert out["cutoff"][i, g] == leaf_score[leaf_of[ret[-1]]]
            else:
                assert np.isneginf(out["cutoff"][i, g])
            assert out["nscored"][i, g] == int(np.count_nonzero(ix.cnt(L)[g]))


@pytest.mark.parametrize("b,L", [(4, 3), (3, 2), (16, 1)])
def test_flat_select_equals_descent_with_every_branch_kept(oracle_lib, b, L):
    """A beam that keeps every node at every level leaves nothing pruned: the
    hierarchical search then visits exactly the flat search's leaves."""
    w, K, V, W, Q, pos = _small_case(b=b, L=L, seed=70 + b, m=8)
    ix = oracle.build_index(K, W, b, L, 5)
    for k, ns, nw in [(25, 0, 0), (300, 2, 7)]:
        f = oracle.select_flat(Q, pos, ix, W, k, n_sink=ns, window=nw)
        h = oracle.select(Q, pos, ix, W, b ** max(L - 1, 0), k, n_sink=ns, window=nw)
        assert np.array_equal(f["sel"], h["sel"]) and np.array_equal(f["count"], h["count"])
        assert np.array_equal(f["cutoff"], h["cutoff"])


# --------------------------------------------------------------------------- PCA projection
def test_pca_closed_form_covariance(oracle_lib):
    """Keys mu +- s_i R_i (i < d) have mean mu and covariance R diag(2 s_i^2 / n) R^T
    exactly: the projection's columns are R's columns (signed), its eigenvalues
    2 s_i^2 / n."""
    rng = np.random.default_rng(5)
    d, r = 24, 10
    R, _ = np.linalg.qr(rng.standard_normal((d, d)))
    s = 2.0 ** (-np.arange(d) / 3.0)
    mu = rng.standard_normal(d)
    rows = []
    for i in range(d):
        rows += [mu + s[i] * R[:, i], mu - s[i] * R[:, i]]
    K = np.array(rows, np.float32)[None]                      # [1, 2d, d]
    W, ev = oracle.pca_projection(K, r)
    n = 2 * d
    np.testing.assert_allclose(ev[0], 2 * s[:r] ** 2 / n, rtol=2e-5)
    for c in range(r):
        v = R[:, c] * np.sign(R[np.argmax(np.abs(R[:, c])), c])
        np.testing.assert_allclose(W[0][:, c], v, atol=3e-5)


def test_pca_matches_sklearn_and_is_orthonormal(oracle_lib):
    from sklearn.decomposition import PCA
    K = synth.make_lowrank_keys(3000, 2, 32, dtype=torch.float32, seed=11).numpy()
    r = 12
    W, ev = oracle.pca_projection(K, r)
    for g in range(2):
        p = PCA(n_components=r, svd_solver="full").fit(K[g].astype(np.float64))
        comp = p.components_                                   # rows, any sign
        for c in range(r):
            assert abs(abs(float(comp[c] @ W[g][:, c].astype(np.float64))) - 1.0) < 1e-6
            j = int(np.argmax(np.abs(W[g][:, c])))
            assert W[g][j, c] > 0
        # sklearn divides by n - 1
        np.testing.assert_allclose(ev[g] * 3000 / 2999, p.explained_variance_, rtol=1e-9)
        np.testing.assert_allclose(W[g].T.astype(np.float64) @ W[g].astype(np.float64), np.eye(r), atol=1e-6)
        assert np.all(np.diff(ev[g]) < 0)
        X = K[g].astype(np.float64)
        Xc = X - X.mean(0)
        C = Xc.T @ Xc / 3000
        resid = C @ W[g].astype(np.float64) - W[g].astype(np.float64) * ev[g][None, :]
        assert np.abs(resid).max() < 1e-6 * ev[g][0]


# --------------------------------------------------------------------------- incremental insertion
@pytest.mark.parametrize("b,L,m", [(4, 3, 1), (4, 3, 37), (8, 2, 200), (3, 2, 5), (16, 1, 50)])
def test_insert_invariants_and_descent(oracle_lib, b, L, m):
    """After inserting m keys: the tree is a valid tree over n + m keys, every
    old key keeps its leaf, every node's count grows by the new keys below it,
    each new key sits in the leaf a greedy nearest-non-empty-child descent
    (numpy distances, pre-batch centroids) reaches, and every centroid stays
    within float32 rounding of its members' mean when the tree's centroids
    were exact means."""
    n = 500
    w, K, V, W, Q, pos = _small_case(b=b, L=L, seed=80 + b + m, n=n + m, m=3)
    ix = oracle.build_index(K[:, :n], W, b, L, 5)
    out = oracle.index_insert(ix, K[:, n:], W)
    Zs = [oracle.project(K[g], W[g]) for g in range(w.h_kv)]
    Cs = [out.C(l) for l in range(1, L + 1)]
    cnts = [out.cnt(l) for l in range(1, L + 1)]
    # structure (the centroid check is loose: a running mean from rounded centroids)
    check_tree(Zs, Cs, cnts, out.leaf_off, out.perm, b, L, ulps=64)
    for g in range(w.h_kv):
        leaf_old = np.empty(n, np.int64)
        for v in range(b ** L):
            leaf_old[ix.perm[g][ix.leaf_off[g][v]:ix.leaf_off[g][v + 1]]] = v
        leaf_new = np.empty(n + m, np.int64)
        for v in range(b ** L):
            leaf_new[out.perm[g][out.leaf_off[g][v]:out.leaf_off[g][v + 1]]] = v
        assert np.array_equal(leaf_new[:n], leaf_old)
        for j in range(m):
            z = Zs[g][n + j].astype(np.float64)
            u = 0
            for l in range(1, L + 1):
                ch = u * b + np.arange(b)
                ch = ch[ix.cnt(l)[g][ch] > 0]
                dist = ((ix.C(l)[g][ch].astype(np.float64) - z) ** 2).sum(axis=1)
                u = int(ch[np.argmin(dist)])
            assert leaf_new[n + j] == u
        for l in range(1, L + 1):
            added = np.zeros(b ** l, np.int64)
            for j in range(m):
                added[leaf_new[n + j] // b ** (L - l)] += 1
            assert np.array_equal(out.cnt(l)[g], ix.cnt(l)[g] + added)


def test_insert_then_dense_select_sees_new_keys(oracle_lib):
    """Every key, old or new, is reachable after insertion: beam over every
    cluster and k = n + m give dense causal attention over the grown cache."""
    b, L, n, m = 3, 3, 400, 60
    w, K, V, W, Q, pos = _small_case(b=b, L=L, seed=91, n=n + m, m=6)
    ix = oracle.build_index(K[:, :n], W, b, L, 5)
    out = oracle.index_insert(ix, K[:, n:], W)
    sel = oracle.select(Q, pos, out, W, beam=b ** (L - 1), k=n + m)
    o, _ = oracle.attend(Q, K, V, sel["sel"], sel["count"])
    keys = np.arange(n + m)
    mask = np.broadcast_to((keys[None, :] <= pos[:, None])[:, None, :], (len(pos), w.h_q, n + m)).copy()
    ref = _sdpa_masked(Q, K, V, mask, 1.0 / np.sqrt(w.d))
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)

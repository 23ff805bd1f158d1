"""GPU parity: the HIP library against the CPU oracle on identical seeded inputs.

Index build and selection must match bit for bit (both sides accumulate in
double in the same order); attention must match within max-abs 1e-4 (fp32
inputs) or 2e-2 (bf16 inputs)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import (assert_index_equal, assert_same_bits, compact_kv, host_index, np32, replay_node, say)

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


@pytest.fixture(scope="module")
def lsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hierarchical_key_indexing_amd as m
    m.lib()
    return m


def _wl(name, **kw):
    return synth.WORKLOADS[name].replace(**kw) if kw else synth.WORKLOADS[name]


# small and ragged shapes: (name, overrides)
SMALL = [
    ("tiny_4k", {}),
    ("ragged_bf16_b5", dict(n=1000, h_q=4, h_kv=2, d=64, dtype="bf16", r=16, b=5, L=3, beam=3, k=100,
                            centres=40, m=7, mode="chunk")),
    ("wide_b64_sparse", dict(n=777, h_q=3, h_kv=3, d=32, dtype="f32", r=8, b=64, L=2, beam=2, k=50,
                             centres=30, m=5, mode="chunk")),
    ("multi_piece_root", dict(n=20000, h_q=16, h_kv=2, d=128, dtype="bf16", r=64, b=64, L=2, beam=8, k=1000,
                              centres=1024, m=3, mode="decode")),
    ("odd_r_deep", dict(n=9000, h_q=8, h_kv=1, d=48, dtype="f32", r=24, b=8, L=3, beam=5, k=333,
                        centres=200, m=9, mode="chunk")),
    ("n_below_b", dict(n=3, h_q=2, h_kv=1, d=16, dtype="f32", r=4, b=4, L=2, beam=2, k=5, centres=2,
                       m=4, mode="chunk")),
    ("single_key", dict(n=1, h_q=1, h_kv=1, d=8, dtype="bf16", r=2, b=2, L=3, beam=1, k=1, centres=1,
                        m=1, mode="decode")),
    ("flat_L1", dict(n=5000, h_q=4, h_kv=1, d=64, dtype="bf16", r=32, b=64, L=1, beam=1, k=700,
                     centres=300, m=6, mode="chunk")),
    # level 1 over 2048 members per node (one workgroup per node for the mean),
    # level 3 with 4 x 256 parents (one wave per parent), odd latent dimension
    ("big_nodes_odd_r", dict(n=40000, h_q=8, h_kv=4, d=48, dtype="f32", r=33, b=16, L=3, beam=4, k=500,
                             centres=500, m=4, mode="chunk")),
    # bf16, d = 128, r = 64 and b <= 4 beam with a level between the first and the
    # leaves: the decode kernel takes level 2 from rows loaded before level 1
    ("pre_level2_b16", dict(n=30000, h_q=16, h_kv=2, d=128, dtype="bf16", r=64, b=16, L=3, beam=4, k=700,
                            centres=500, m=3, mode="decode")),
    # r = 64 with 16 or more rows: flat scoring on the matrix cores, a ragged
    # last wave (37 = 2 x 16 + 5 rows), every leaf in the list (4096 leaves)
    ("flat_mfma_rows", dict(n=20000, h_q=8, h_kv=2, d=128, dtype="bf16", r=64, b=64, L=2, beam=8, k=1000,
                            centres=800, m=37, mode="chunk")),
]

# flat search only (b^L above the top-down search's limits): r = 64 with 21
# rows over 262144 mostly empty leaves, the sampled threshold path
FLAT_ONLY = {"flat_mfma_sampled": dict(n=20000, h_q=8, h_kv=2, d=128, dtype="bf16", r=64, b=64, L=3, beam=4,
                                       k=600, centres=800, m=21, mode="chunk")}


def _inputs(w, dev, m=None):
    data = synth.make_workload(w, device="cpu", m=m)
    out = {k: v.to(dev) for k, v in data.items()}
    out["cpu"] = data
    return out


def _build_both(lsa, w, data):
    say("build", w.name, w.n, w.h_kv, w.b, w.L)
    index, desc = lsa.build_index(data["K"], data["W"], w.b, w.L, w.iters)
    torch.cuda.synchronize()
    views = lsa.index_views(index, desc)
    gix = host_index(views, desc)
    c = data["cpu"]
    oix = oracle.build_index(np32(c["K"]), c["W"].numpy(), w.b, w.L, w.iters)
    return index, desc, gix, oix


@pytest.mark.parametrize("name,over", SMALL, ids=[s[0] for s in SMALL])
def test_small_pipeline_matches_oracle(lsa, name, over):
    dev = torch.device("cuda:0")
    w = _wl("tiny_4k", **over) if name != "tiny_4k" else _wl("tiny_4k")
    w = w.replace(name=name)
    data = _inputs(w, dev)
    index, desc, gix, oix = _build_both(lsa, w, data)
    assert_index_equal(gix, oix)

    c = data["cpu"]
    Qh = np32(c["Q"])
    pos = c["pos"].numpy()
    tol = TOL[w.torch_dtype]
    for beam, k in [(w.beam, w.k), (1, 1), (w.b ** max(w.L - 1, 0), min(w.n + 3, 8192))]:
        ref = oracle.select(Qh, pos, oix, c["W"].numpy(), beam, k)
        o_ref, lse_ref = oracle.attend(Qh, np32(c["K"]), np32(c["V"]), ref["sel"], ref["count"])
        # one workgroup per (row, KV head), then the multi-workgroup kernel (when it applies)
        nws = lsa.select_workspace_bytes(w.m, w.h_q, w.d, desc, beam, k)
        for label, ws in (("single-wg", None), ("multi-wg", lsa.workspace(nws, dev))):
            if label == "multi-wg" and ws is None:
                continue
            say("select", name, label, beam, k)
            sel, cnt, cut = lsa.select(data["Q"], data["pos"], index, desc, data["W"], beam, k, ws=ws)
            torch.cuda.synchronize()
            assert_same_bits(cnt.cpu().numpy(), ref["count"], f"sel_count ({label})")
            assert_same_bits(sel.cpu().numpy(), ref["sel"], f"sel ({label})")
            assert_same_bits(cut.cpu().numpy(), ref["cutoff"], f"cutoff ({label})")
            if ws is not None:
                cus = torch.cuda.get_device_properties(0).multi_processor_count
                if w.m * w.h_kv * beam <= cus:          # the multi-workgroup kernel ran
                    _assert_exchange_zeroed(ws, w.m * w.h_kv, beam, w.h_q // w.h_kv, w.d)
                # whichever path ran, a one-row call on the same workspace follows
                say("select", name, "one row after", label, beam, k)
                s1, c1, u1 = lsa.select(data["Q"][:1], data["pos"][:1], index, desc, data["W"], beam, k, ws=ws)
                torch.cuda.synchronize()
                assert_same_bits(c1.cpu().numpy(), ref["count"][:1], "sel_count (one row after)")
                assert_same_bits(s1.cpu().numpy(), ref["sel"][:1], "sel (one row after)")
                assert_same_bits(u1.cpu().numpy(), ref["cutoff"][:1], "cutoff (one row after)")
        # every selected key precedes (or is) its query
        s = sel.cpu().numpy()
        assert np.all((s == -1) | (s <= pos[:, None, None]))

        say("attend", name, beam, k)
        out, lse = lsa.attend(data["Q"], data["K"], data["V"], sel, cnt)
        torch.cuda.synchronize()
        _check_attention(out, lse, o_ref, lse_ref, tol)

        say("select_attend", name, beam, k)
        # (sized for this batch and for the one-row call that follows)
        fws = lsa.workspace(max(lsa.select_attend_workspace_bytes(w.m, w.h_q, w.d, desc, beam, k),
                                lsa.select_attend_workspace_bytes(1, w.h_q, w.d, desc, beam, k)), dev)
        for rep in range(2):     # the workspace is reusable
            sel2, cnt2, cut2, out2, lse2 = lsa.select_attend(data["Q"], data["K"], data["V"], data["pos"], index,
                                                             desc, data["W"], beam, k, ws=fws)
            torch.cuda.synchronize()
            assert_same_bits(cnt2.cpu().numpy(), ref["count"], "sel_count (fused)")
            assert_same_bits(sel2.cpu().numpy(), ref["sel"], "sel (fused)")
            assert_same_bits(cut2.cpu().numpy(), ref["cutoff"], "cutoff (fused)")
            _check_attention(out2, lse2, o_ref, lse_ref, tol)
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        if lsa.select_workspace_bytes(w.m, w.h_q, w.d, desc, beam, k) > 0 and w.m * w.h_kv * beam <= cus:
            _assert_exchange_zeroed(fws, w.m * w.h_kv, beam, w.h_q // w.h_kv, w.d)
        # a one-row call on the same workspace follows whichever path ran
        say("select_attend", name, "one row after", beam, k)
        sel3, cnt3, cut3, out3, lse3 = lsa.select_attend(data["Q"][:1], data["K"], data["V"], data["pos"][:1], index,
                                                         desc, data["W"], beam, k, ws=fws)
        torch.cuda.synchronize()
        assert_same_bits(cnt3.cpu().numpy(), ref["count"][:1], "sel_count (fused, one row after)")
        assert_same_bits(sel3.cpu().numpy(), ref["sel"][:1], "sel (fused, one row after)")
        assert_same_bits(cut3.cpu().numpy(), ref["cutoff"][:1], "cutoff (fused, one row after)")
        _check_attention(out3, lse3, o_ref[:1], lse_ref[:1], tol)


# r = 64 builds take the projection on the fp64 matrix cores: fp32 keys with
# d = 256 (its largest key tile, over 64 KB of LDS) and bf16 keys with
# d = 136 (34 blocks of four dims), both with a ragged last tile of keys
PROJ_CASES = [("proj_f32_d256", dict(n=1000, h_q=2, h_kv=2, d=256, dtype="f32", r=64, b=8, L=2, beam=2, k=100,
                                     centres=50, m=3, mode="chunk")),
              ("proj_bf16_d136", dict(n=777, h_q=3, h_kv=3, d=136, dtype="bf16", r=64, b=5, L=3, beam=2, k=50,
                                      centres=40, m=2, mode="chunk"))]


@pytest.mark.parametrize("name,over", PROJ_CASES, ids=[c[0] for c in PROJ_CASES])
def test_projection_on_matrix_cores_matches_oracle(lsa, name, over):
    """The index built through the matrix-core projection equals the
    oracle's bit for bit (every centroid is a mean of projected keys)."""
    dev = torch.device("cuda:0")
    w = _wl("tiny_4k", **over).replace(name=name)
    data = _inputs(w, dev)
    say("projection", name)
    index, desc, gix, oix = _build_both(lsa, w, data)
    assert_index_equal(gix, oix)


def _assert_exchange_zeroed(ws, groups, beam, G, d):
    """After a multi-workgroup call everything in its workspace but the trailing
    partial softmax states is zero again (counters and exchange buffers)."""
    a256 = lambda x: (x + 255) // 256 * 256
    part = a256(4 * groups * beam * ((G * d + 2 * G + 3) // 4 * 4))
    head = ws.numel() - part
    assert head > 0 and int(ws[:head].count_nonzero()) == 0, "exchange buffers not left zeroed"


def test_workspace_reused_across_shapes(lsa):
    """One workspace serves calls of different beams (different layouts inside
    it) in any order: every result equals the one from a fresh workspace."""
    dev = torch.device("cuda:0")
    w = _wl("tiny_4k", **dict(SMALL)["ragged_bf16_b5"]).replace(name="ws_reuse")
    data = _inputs(w, dev)
    index, desc = lsa.build_index(data["K"], data["W"], w.b, w.L, w.iters)
    shapes = [(3, 100), (2, 37), (5, 160), (3, 100), (1, 9), (5, 160)]
    size = max(lsa.select_attend_workspace_bytes(w.m, w.h_q, w.d, desc, bm, k) for bm, k in shapes)
    assert size > 0
    shared = lsa.workspace(size, dev)
    for bm, k in shapes:
        say("ws reuse", bm, k)
        fresh = lsa.workspace(lsa.select_attend_workspace_bytes(w.m, w.h_q, w.d, desc, bm, k), dev)
        ref = lsa.select_attend(data["Q"], data["K"], data["V"], data["pos"], index, desc, data["W"], bm, k, ws=fresh)
        got = lsa.select_attend(data["Q"], data["K"], data["V"], data["pos"], index, desc, data["W"], bm, k, ws=shared)
        sel_only = lsa.select(data["Q"], data["pos"], index, desc, data["W"], bm, k, ws=shared)
        torch.cuda.synchronize()
        for a, b_, nm in zip(got, ref, ("sel", "count", "cutoff", "out", "lse")):
            assert torch.equal(a, b_), f"{nm} differs with a reused workspace (beam {bm}, k {k})"
        for a, b_, nm in zip(sel_only, ref[:3], ("sel", "count", "cutoff")):
            assert torch.equal(a, b_), f"select-only {nm} differs with a reused workspace (beam {bm}, k {k})"


# shapes run at their own beam only (their full beam exceeds the selection limits)
BEAM_ONLY = {
    # bf16, d = 128, r = 64, b = 32, L = 3: the decode kernel's waves own
    # level-1 nodes p + beam w; with beam 16 waves 2 and 3 own none
    "owned_b32": dict(n=40000, h_q=16, h_kv=2, d=128, dtype="bf16", r=64, b=32, L=3, beam=16, k=1500,
                      centres=800, m=3, mode="decode"),
}
LOCAL_CASES = [("tiny_4k", {}), ("ragged_bf16_b5", {}), ("multi_piece_root", {}),
               ("multi_piece_root", dict(beam=16)), ("odd_r_deep", {}), ("flat_L1", {}),
               ("owned_b32", {}), ("owned_b32", dict(beam=8))]
LOCAL_SETS = [(4, 16), (0, 300), (7, 0), (50, 100000)]


@pytest.mark.parametrize("name,over", LOCAL_CASES,
                         ids=[c[0] + "".join(f"_{k}{v}" for k, v in c[1].items()) for c in LOCAL_CASES])
def test_sinks_and_window_match_oracle(lsa, name, over):
    """Sinks and a recent window joined to the retrieved keys: every select
    path (one workgroup per row, the multi-workgroup kernel, the fused
    select + attend) gives the oracle's rows bit for bit, and attention over
    them matches the oracle's."""
    dev = torch.device("cuda:0")
    shapes = {**dict(SMALL), **BEAM_ONLY}
    w = _wl("tiny_4k", **shapes[name]) if name != "tiny_4k" else _wl("tiny_4k")
    w = w.replace(name=name, **over)
    data = _inputs(w, dev)
    index, desc, gix, oix = _build_both(lsa, w, data)
    c = data["cpu"]
    Qh = np32(c["Q"])
    pos = c["pos"].numpy()
    tol = TOL[w.torch_dtype]
    for n_sink, window in LOCAL_SETS:
        ref = oracle.select(Qh, pos, gix, c["W"].numpy(), w.beam, w.k, n_sink=n_sink, window=window)
        o_ref, lse_ref = oracle.attend(Qh, np32(c["K"]), np32(c["V"]), ref["sel"], ref["count"])
        nws = lsa.select_workspace_bytes(w.m, w.h_q, w.d, desc, w.beam, w.k, n_sink, window)
        for label, ws in (("single-wg", None), ("multi-wg", lsa.workspace(nws, dev))):
            if label == "multi-wg" and ws is None:
                continue
            say("local select", name, over, label, n_sink, window)
            sel, cnt, cut = lsa.select(data["Q"], data["pos"], index, desc, data["W"], w.beam, w.k, ws=ws,
                                       n_sink=n_sink, window=window)
            torch.cuda.synchronize()
            assert_same_bits(cnt.cpu().numpy(), ref["count"], f"sel_count ({label})")
            assert_same_bits(sel.cpu().numpy(), ref["sel"], f"sel ({label})")
            assert_same_bits(cut.cpu().numpy(), ref["cutoff"], f"cutoff ({label})")
        say("local attend", name, n_sink, window)
        out, lse = lsa.attend(data["Q"], data["K"], data["V"], sel, cnt)
        torch.cuda.synchronize()
        _check_attention(out, lse, o_ref, lse_ref, tol)
        say("local select_attend", name, n_sink, window)
        fws = lsa.workspace(lsa.select_attend_workspace_bytes(w.m, w.h_q, w.d, desc, w.beam, w.k, n_sink, window),
                            dev)
        for rep in range(2):
            sel2, cnt2, cut2, out2, lse2 = lsa.select_attend(data["Q"], data["K"], data["V"], data["pos"], index,
                                                             desc, data["W"], w.beam, w.k, ws=fws,
                                                             n_sink=n_sink, window=window)
            torch.cuda.synchronize()
            assert_same_bits(cnt2.cpu().numpy(), ref["count"], "sel_count (fused)")
            assert_same_bits(sel2.cpu().numpy(), ref["sel"], "sel (fused)")
            assert_same_bits(cut2.cpu().numpy(), ref["cutoff"], "cutoff (fused)")
            _check_attention(out2, lse2, o_ref, lse_ref, tol)
        if lsa.select_workspace_bytes(w.m, w.h_q, w.d, desc, w.beam, w.k) > 0:
            _assert_exchange_zeroed(fws, w.m * w.h_kv, w.beam, w.h_q // w.h_kv, w.d)


FLAT_CASES = ["tiny_4k", "ragged_bf16_b5", "multi_piece_root", "odd_r_deep", "flat_L1", "n_below_b", "single_key",
              "flat_mfma_rows", "flat_mfma_sampled"]


@pytest.mark.parametrize("name", FLAT_CASES)
def test_flat_search_matches_oracle(lsa, name):
    """Flat search (every leaf scored): rows bit for bit equal to the oracle's,
    with and without sinks and a window, in one batch and in batches forced by
    a one-row workspace; attention over them matches the oracle's."""
    dev = torch.device("cuda:0")
    over = FLAT_ONLY[name] if name in FLAT_ONLY else dict(SMALL)[name] if name != "tiny_4k" else {}
    w = _wl("tiny_4k", **over).replace(name=name)
    data = _inputs(w, dev)
    index, desc = lsa.build_index(data["K"], data["W"], w.b, w.L, w.iters)
    torch.cuda.synchronize()
    gix = host_index(lsa.index_views(index, desc), desc)
    c = data["cpu"]
    Qh = np32(c["Q"])
    pos = c["pos"].numpy()
    small_ws = lsa.workspace(lsa.select_flat_workspace_bytes(1, w.h_q, desc), dev)
    for k, n_sink, window in [(w.k, 0, 0), (max(1, w.k // 3), 4, 16), (min(w.n + 5, 8192), 0, 0)]:
        ref = oracle.select_flat(Qh, pos, gix, c["W"].numpy(), k, n_sink=n_sink, window=window)
        for label, ws in (("one batch", None), ("one-row batches", small_ws)):
            say("flat", name, label, k, n_sink, window)
            sel, cnt, cut = lsa.select_flat(data["Q"], data["pos"], index, desc, data["W"], k, ws=ws,
                                            n_sink=n_sink, window=window)
            torch.cuda.synchronize()
            assert_same_bits(cnt.cpu().numpy(), ref["count"], f"sel_count ({label})")
            assert_same_bits(sel.cpu().numpy(), ref["sel"], f"sel ({label})")
            assert_same_bits(cut.cpu().numpy(), ref["cutoff"], f"cutoff ({label})")
        out, lse = lsa.attend(data["Q"], data["K"], data["V"], sel, cnt)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.attend(Qh, np32(c["K"]), np32(c["V"]), ref["sel"], ref["count"])
        _check_attention(out, lse, o_ref, lse_ref, TOL[w.torch_dtype])


def test_flat_search_tied_scores(lsa):
    """All-zero queries score every leaf 0: the order falls to the leaf ids,
    and the boundary search has to resolve the ids' bits."""
    dev = torch.device("cuda:0")
    w = _wl("tiny_4k", n=30000, h_q=4, h_kv=1, d=32, dtype="f32", r=8, b=32, L=2, centres=500, m=3, mode="chunk")
    data = _inputs(w, dev)
    data["Q"].zero_()
    data["cpu"]["Q"].zero_()
    index, desc = lsa.build_index(data["K"], data["W"], w.b, w.L, w.iters)
    torch.cuda.synchronize()
    gix = host_index(lsa.index_views(index, desc), desc)
    ref = oracle.select_flat(np32(data["cpu"]["Q"]), data["cpu"]["pos"].numpy(), gix, data["cpu"]["W"].numpy(), 777)
    sel, cnt, cut = lsa.select_flat(data["Q"], data["pos"], index, desc, data["W"], 777)
    torch.cuda.synchronize()
    assert_same_bits(cnt.cpu().numpy(), ref["count"], "sel_count")
    assert_same_bits(sel.cpu().numpy(), ref["sel"], "sel")
    assert_same_bits(cut.cpu().numpy(), ref["cutoff"], "cutoff")


@pytest.mark.parametrize("zero_q,k", [(False, 100), (False, 8192), (True, 100), (True, 8192)])
def test_flat_search_large_leaf_table(lsa, zero_q, k):
    """32768 leaves (more than fit in LDS): the sampled threshold (k = 100),
    the exact radix fallback (k = 8192: the sample weighs too little), tied
    scores that leave the order to the leaf ids, and an early row whose
    candidates weigh less than k."""
    dev = torch.device("cuda:0")
    w = _wl("tiny_4k", n=20000, h_q=4, h_kv=1, d=32, dtype="f32", r=8, b=32, L=3, centres=400, m=5, mode="chunk")
    data = _inputs(w, dev)
    data["pos"][0] = 50
    data["cpu"]["pos"][0] = 50
    if zero_q:
        data["Q"].zero_()
        data["cpu"]["Q"].zero_()
    index, desc = lsa.build_index(data["K"], data["W"], w.b, w.L, w.iters)
    torch.cuda.synchronize()
    assert desc.nodes[desc.L] == 32768
    gix = host_index(lsa.index_views(index, desc), desc)
    ref = oracle.select_flat(np32(data["cpu"]["Q"]), data["cpu"]["pos"].numpy(), gix, data["cpu"]["W"].numpy(), k)
    say("flat large table", zero_q, k)
    sel, cnt, cut = lsa.select_flat(data["Q"], data["pos"], index, desc, data["W"], k)
    torch.cuda.synchronize()
    assert_same_bits(cnt.cpu().numpy(), ref["count"], "sel_count")
    assert_same_bits(sel.cpu().numpy(), ref["sel"], "sel")
    assert_same_bits(cut.cpu().numpy(), ref["cutoff"], "cutoff")


def _check_attention(out, lse, o_ref, lse_ref, tol):
    assert np.max(np.abs(np32(out) - o_ref)) <= tol
    g = lse.cpu().numpy()
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(g), fin)
    if fin.any():
        assert np.max(np.abs(g[fin] - lse_ref[fin])) <= 1e-3


def test_positions_before_every_candidate_give_empty_rows(lsa):
    """A query whose candidate leaves only hold later keys selects nothing; its
    attention output is 0 and its lse is -inf."""
    dev = torch.device("cuda:0")
    w = _wl("tiny_4k", n=2000, h_q=2, h_kv=1, d=32, r=8, b=16, L=2, beam=1, k=4, centres=64, m=64, mode="all")
    K, V = synth.make_kv(w)
    W = synth.make_w(w)
    pos = torch.arange(0, 64, dtype=torch.int32)
    Q = synth.make_queries(w, K, pos)
    Q[:] = -K[0, 1999].float()      # aims away from early keys' clusters, mostly
    index, desc = lsa.build_index(K.to(dev), W.to(dev), w.b, w.L, 5)
    sel, cnt, cut = lsa.select(Q.to(dev), pos.to(dev), index, desc, W.to(dev), 1, 4)
    out, lse = lsa.attend(Q.to(dev), K.to(dev), V.to(dev), sel, cnt)
    torch.cuda.synchronize()
    gix = host_index(lsa.index_views(index, desc), desc)
    ref = oracle.select(Q.numpy(), pos.numpy(), gix, W.numpy(), 1, 4)
    assert_same_bits(sel.cpu().numpy(), ref["sel"], "sel")
    assert_same_bits(cnt.cpu().numpy(), ref["count"], "sel_count")
    empty = ref["count"][:, 0] == 0
    assert empty.any() and (~empty).any()
    o = out.cpu().numpy()
    assert np.all(o[empty] == 0) and np.all(np.isneginf(lse.cpu().numpy()[empty]))


@pytest.mark.parametrize("G,d,dtype,m,k", [(1, 8, torch.float32, 3, 17), (2, 64, torch.bfloat16, 1, 700),
                                           (8, 128, torch.bfloat16, 2, 2048), (16, 256, torch.float32, 2, 300),
                                           (4, 128, torch.float32, 40, 64), (8, 128, torch.bfloat16, 300, 256)])
def test_attend_random_sets(lsa, G, d, dtype, m, k):
    """Attention alone on random selections (counts from 0 to k) against the oracle."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(G * 1000 + d)
    h_kv, n = 2, 3000
    gen = torch.Generator().manual_seed(d + G)
    Q = torch.randn(m, G * h_kv, d, generator=gen).to(dtype)
    K = torch.randn(h_kv, n, d, generator=gen).to(dtype)
    V = torch.randn(h_kv, n, d, generator=gen).to(dtype)
    cnt = rng.integers(0, k + 1, size=(m, h_kv)).astype(np.int32)
    cnt[0, 0] = 0
    cnt[-1, -1] = k
    sel = np.full((m, h_kv, k), -1, np.int32)
    for i in range(m):
        for g in range(h_kv):
            sel[i, g, :cnt[i, g]] = np.sort(rng.choice(n, size=cnt[i, g], replace=False))
    say("attend_random", G, d, dtype, m, k)
    out, lse = lsa.attend(Q.to(dev), K.to(dev), V.to(dev), torch.from_numpy(sel).to(dev),
                          torch.from_numpy(cnt).to(dev))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attend(np32(Q), np32(K), np32(V), sel, cnt)
    assert np.max(np.abs(np32(out) - o_ref)) <= TOL[dtype]
    g = lse.cpu().numpy()
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(g), fin)
    assert np.max(np.abs(g[fin] - lse_ref[fin])) <= 1e-3


@pytest.mark.parametrize("b,L", [(4, 3), (16, 2), (64, 1)])
def test_dense_equivalence_on_gpu(lsa, b, L):
    """beam covering every cluster and k = n: LSA equals dense causal attention."""
    dev = torch.device("cuda:0")
    w = _wl("tiny_4k", n=1500, h_q=8, h_kv=2, d=64, dtype="f32", r=16, b=b, L=L, centres=50, m=12, mode="chunk")
    data = _inputs(w, dev)
    index, desc = lsa.build_index(data["K"], data["W"], b, L, 5)
    sel, cnt, _ = lsa.select(data["Q"], data["pos"], index, desc, data["W"], b ** (L - 1), w.n)
    out, _ = lsa.attend(data["Q"], data["K"], data["V"], sel, cnt)
    torch.cuda.synchronize()
    c = data["cpu"]
    q = c["Q"].double()[:, :, None, :]
    G = w.h_q // w.h_kv
    k = c["K"].double().repeat_interleave(G, 0)[None]
    v = c["V"].double().repeat_interleave(G, 0)[None]
    keys = torch.arange(w.n)
    mask = (keys[None, :] <= c["pos"][:, None].long())[:, None, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)[:, :, 0, :]
    assert torch.max(torch.abs(out.cpu().double() - ref)).item() <= 1e-4


# ------------------------------------------------------------------ full-size workloads
FULL = [("decode_1m", None, 1, (0, 0)), ("prefill_1m", 48, 1, (0, 0)), ("train_128k", 64, 2, (0, 0)),
        ("decode_10m", None, 0, (0, 0)), ("decode_1m", None, 0, (4, 512)), ("prefill_1m", 32, 0, (4, 512))]


@pytest.mark.parametrize("name,sample_rows,replay_depth,local", FULL,
                         ids=[f[0] + ("" if f[3] == (0, 0) else "_sinks%d_window%d" % f[3]) for f in FULL])
def test_full_size_workload(lsa, name, sample_rows, replay_depth, local):
    """The workload at its real size, in the launch configuration the benchmark
    uses: bit-exact tree on sampled nodes (the oracle re-clusters the node from
    the members the GPU gave its parent), bit-exact selection and attention on
    sampled rows."""
    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[name]
    say("generate", name)
    K, V = synth.make_kv(w, device=dev)
    W = synth.make_w(w, device=dev)
    pos = w.positions().to(dev)
    Q = synth.make_queries(w, K, pos)
    say("build", name)
    index, desc = lsa.build_index(K, W, w.b, w.L, w.iters)
    torch.cuda.synchronize()
    views = lsa.index_views(index, desc)
    gix = host_index(views, desc)
    rng = np.random.default_rng(7)
    # sampled nodes: the root of head 0 when affordable, then random parents per level
    picks = []
    if w.n <= (1 << 20) and replay_depth >= 1:
        picks.append((0, 1, 0))
    for l in range(2, w.L + 1):
        g = int(rng.integers(w.h_kv))
        nz = np.nonzero(gix.cnt(l - 1)[g])[0]
        for u in rng.choice(nz, size=min(3, len(nz)), replace=False):
            picks.append((g, l, int(u)))
    for g, l, u in picks:
        say("replay", name, g, l, u)
        replay_node(K, W, gix, g, l, u, w.iters)

    n_sink, window = local
    say("select", name, local)
    sel, cnt, cut = lsa.select(Q, pos, index, desc, W, w.beam, w.k, n_sink=n_sink, window=window)
    # with a workspace (the launch the benchmark times: the decode kernel for
    # one row, node-major batches for the prefill chunk and the training
    # layer) every row equals the one-workgroup result bit for bit
    nws = lsa.select_workspace_bytes(w.m, w.h_q, w.d, desc, w.beam, w.k, n_sink, window)
    if nws > 0:
        say("select with workspace", name, nws)
        sws = lsa.workspace(nws, dev)
        selw, cntw, cutw = lsa.select(Q, pos, index, desc, W, w.beam, w.k, n_sink=n_sink, window=window, ws=sws)
        torch.cuda.synchronize()
        assert torch.equal(cntw, cnt) and torch.equal(cutw, cut) and torch.equal(selw, sel)
        del selw, cntw, cutw, sws
    say("attend", name)
    out, lse = lsa.attend(Q, K, V, sel, cnt)
    torch.cuda.synchronize()
    # the fused call as the benchmark times it: one launch for a decode row,
    # node-major selection and attention for the prefill chunk and the
    # training layer; its outputs are checked against the oracle below
    say("select_attend", name)
    sel2, cnt2, cut2, out2, lse2 = lsa.select_attend(Q, K, V, pos, index, desc, W, w.beam, w.k,
                                                     n_sink=n_sink, window=window)
    torch.cuda.synchronize()
    assert torch.equal(sel2, sel) and torch.equal(cnt2, cnt) and torch.equal(cut2, cut)
    assert float((out2.float() - out.float()).abs().max()) <= 2 * TOL[w.torch_dtype]
    del sel2, cnt2, cut2
    # causal and count invariants on every row, on the device
    s = sel.long()
    valid = s >= 0
    assert bool(torch.all(~valid | (s <= pos[:, None, None].long())))
    assert bool(torch.all(valid.sum(-1) == cnt.long()))
    ss = torch.sort(torch.where(valid, s, torch.full_like(s, 1 << 40)), dim=-1).values
    assert bool(torch.all((ss[..., 1:] > ss[..., :-1]) | (ss[..., 1:] == (1 << 40))))   # no duplicates
    del ss

    rows = np.arange(w.m) if sample_rows is None else np.sort(rng.choice(w.m, size=sample_rows, replace=False))
    ridx = torch.from_numpy(rows).to(dev)
    Qs = np32(Q[ridx])
    say("oracle select", name, len(rows))
    ref = oracle.select(Qs, pos[ridx].cpu().numpy(), gix, np32(W), w.beam, w.k, n_sink=n_sink, window=window)
    assert_same_bits(cnt[ridx].cpu().numpy(), ref["count"], "sel_count")
    assert_same_bits(sel[ridx].cpu().numpy(), ref["sel"], "sel")
    assert_same_bits(cut[ridx].cpu().numpy(), ref["cutoff"], "cutoff")
    say("oracle attend", name, len(rows))
    Kc, Vc, selc = compact_kv(K, V, ref["sel"], ref["count"])
    o_ref, lse_ref = oracle.attend(Qs, Kc, Vc, selc, ref["count"])
    fin = np.isfinite(lse_ref)
    for label, o_gpu, l_gpu in (("attend", out, lse), ("select_attend", out2, lse2)):
        assert np.max(np.abs(np32(o_gpu[ridx]) - o_ref)) <= TOL[w.torch_dtype], label
        g = l_gpu[ridx].cpu().numpy()
        assert np.array_equal(np.isfinite(g), fin), label
        assert np.max(np.abs(g[fin] - lse_ref[fin])) <= 1e-3, label
    say("mean sel_count", name, float(cnt.float().mean()))
    del K, V, index, views, out2, lse2
    torch.cuda.empty_cache()


FLAT_FULL = [("decode_1m", None), ("prefill_1m", 16)]


@pytest.mark.parametrize("name,sample_rows", FLAT_FULL, ids=[f[0] for f in FLAT_FULL])
def test_flat_search_full_size(lsa, name, sample_rows):
    """Flat search at the workload's real size (262144 leaves per KV head),
    every row through the GPU, sampled rows against the oracle bit for bit."""
    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[name]
    say("generate", name)
    K, V = synth.make_kv(w, device=dev)
    W = synth.make_w(w, device=dev)
    pos = w.positions().to(dev)
    Q = synth.make_queries(w, K, pos)
    index, desc = lsa.build_index(K, W, w.b, w.L, w.iters)
    torch.cuda.synchronize()
    gix = host_index(lsa.index_views(index, desc), desc)
    say("flat select", name)
    sel, cnt, cut = lsa.select_flat(Q, pos, index, desc, W, w.k)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rows = np.arange(w.m) if sample_rows is None else np.sort(rng.choice(w.m, size=sample_rows, replace=False))
    ridx = torch.from_numpy(rows).to(dev)
    say("oracle flat", name, len(rows))
    ref = oracle.select_flat(np32(Q[ridx]), pos[ridx].cpu().numpy(), gix, np32(W), w.k)
    assert_same_bits(cnt[ridx].cpu().numpy(), ref["count"], "sel_count")
    assert_same_bits(sel[ridx].cpu().numpy(), ref["sel"], "sel")
    assert_same_bits(cut[ridx].cpu().numpy(), ref["cutoff"], "cutoff")
    s = sel.long()
    valid = s >= 0
    assert bool(torch.all(~valid | (s <= pos[:, None, None].long())))
    assert bool(torch.all(valid.sum(-1) == cnt.long()))
    del K, V, index
    torch.cuda.empty_cache()


PCA_CASES = [(3000, 2, 32, 12, torch.float32), (20000, 1, 128, 64, torch.bfloat16), (777, 3, 17, 17, torch.float32),
             (1 << 20, 4, 128, 64, torch.bfloat16)]


@pytest.mark.parametrize("n,h,d,r,dtype", PCA_CASES, ids=[f"n{c[0]}_h{c[1]}_d{c[2]}_r{c[3]}" for c in PCA_CASES])
def test_pca_projection_matches_oracle(lsa, n, h, d, r, dtype):
    """PCA projection of keys with a decaying spectrum (eigenvalue gaps of a few
    percent): eigenvalues within 1e-9 relative and eigenvector columns within
    2e-6 of the oracle's (double precision, then the same fp32 rounding and
    sign rule); the columns are orthonormal."""
    dev = torch.device("cuda:0")
    K = synth.make_lowrank_keys(n, h, d, dtype=dtype, seed=4100 + d, device=dev)
    say("pca", n, h, d, r, dtype)
    W, ev = lsa.pca_projection(K, r)
    torch.cuda.synchronize()
    Wr, evr = oracle.pca_projection(np32(K), r)
    np.testing.assert_allclose(ev.cpu().numpy(), evr, rtol=1e-9, atol=1e-12 * float(np.abs(evr).max()))
    Wg = W.cpu().numpy()
    assert np.abs(Wg - Wr).max() <= 2e-6
    for g in range(h):
        Wd = Wg[g].astype(np.float64)
        assert np.abs(Wd.T @ Wd - np.eye(r)).max() < 1e-5


INSERT_CASES = [("tiny_4k", [1, 7]), ("ragged_bf16_b5", [300]), ("odd_r_deep", [64, 1, 250]), ("flat_L1", [33]),
                ("multi_piece_root", [4096])]


@pytest.mark.parametrize("name,batches", INSERT_CASES, ids=[c[0] for c in INSERT_CASES])
def test_index_insert_matches_oracle(lsa, name, batches):
    """Keys appended in batches and inserted in place: after every batch the
    tree equals the oracle's insertion into the same tree bit for bit, and a
    selection over the grown index equals the oracle's."""
    dev = torch.device("cuda:0")
    w0 = _wl("tiny_4k", **dict(SMALL)[name]) if name != "tiny_4k" else _wl("tiny_4k")
    total = sum(batches)
    w = w0.replace(name=name, n=w0.n + total)
    K, V = synth.make_kv(w)
    W = synth.make_w(w)
    n = w0.n
    Kd, Wd = K.to(dev), W.to(dev)
    cap = lsa.index_layout(w.n, w.h_kv, w.r, w.b, w.L).bytes
    index = torch.zeros(cap, dtype=torch.uint8, device=dev)
    index, desc = lsa.build_index(Kd[:, :n].contiguous(), Wd, w.b, w.L, w.iters, index=index)
    torch.cuda.synchronize()
    ref = host_index(lsa.index_views(index, desc), desc)
    for mb in batches:
        say("insert", name, desc.n, mb)
        Knew = K[:, desc.n:desc.n + mb].contiguous()
        desc = lsa.index_insert(Knew.to(dev), Wd, index, desc)
        torch.cuda.synchronize()
        ref = oracle.index_insert(ref, np32(Knew), W.numpy())
        assert desc.n == ref.n
        assert_index_equal(host_index(lsa.index_views(index, desc), desc), ref)
    # select over the grown cache (decode rows at the end, chunk rows spread)
    pos = torch.tensor(sorted(np.random.default_rng(3).choice(desc.n + 1, size=6, replace=False)), dtype=torch.int32)
    Q = synth.make_queries(w, K, pos)
    sel, cnt, cut = lsa.select(Q.to(dev), pos.to(dev), index, desc, Wd, w.beam, w.k)
    torch.cuda.synchronize()
    o = oracle.select(np32(Q), pos.numpy(), ref, W.numpy(), w.beam, w.k)
    assert_same_bits(sel.cpu().numpy(), o["sel"], "sel after insertion")
    assert_same_bits(cnt.cpu().numpy(), o["count"], "sel_count after insertion")


def test_index_insert_full_size_decode(lsa):
    """The 1M-key decode index grown by 64 appended keys (one batch), then by
    one more: every array equals the oracle's insertion into the GPU-built
    tree."""
    dev = torch.device("cuda:0")
    w = synth.WORKLOADS["decode_1m"]
    n0 = w.n - 65
    K, V = synth.make_kv(w, device=dev)
    W = synth.make_w(w, device=dev)
    cap = lsa.index_layout(w.n, w.h_kv, w.r, w.b, w.L).bytes
    index = torch.zeros(cap, dtype=torch.uint8, device=dev)
    say("build", n0)
    index, desc = lsa.build_index(K[:, :n0].contiguous(), W, w.b, w.L, w.iters, index=index)
    torch.cuda.synchronize()
    ref = host_index(lsa.index_views(index, desc), desc)
    for mb in (64, 1):
        say("insert", desc.n, mb)
        Knew = K[:, desc.n:desc.n + mb].contiguous()
        desc = lsa.index_insert(Knew, W, index, desc)
        torch.cuda.synchronize()
        ref = oracle.index_insert(ref, np32(Knew), np32(W))
        assert_index_equal(host_index(lsa.index_views(index, desc), desc), ref)
    assert desc.n == w.n
    del K, V, index
    torch.cuda.empty_cache()


NM_CASES = [("nm_b64_L2", dict(n=20000, h_q=16, h_kv=2, d=128, dtype="bf16", r=64, b=64, L=2, beam=8, k=1000,
                               centres=1024, m=600, mode="chunk")),
            ("nm_b16_L3", dict(n=30000, h_q=8, h_kv=4, d=64, dtype="f32", r=64, b=16, L=3, beam=16, k=700,
                               centres=900, m=500, mode="chunk")),
            ("nm_b32_L3_all", dict(n=6000, h_q=4, h_kv=1, d=128, dtype="bf16", r=64, b=32, L=3, beam=5, k=300,
                                   centres=300, m=6000, mode="all")),
            # about 5 keys a leaf and k = 3000: rows take more than 512 of the
            # 1024 candidate leaves (the largest finish network) and more than
            # 2048 keys (the copy by leaves)
            ("nm_b64_L2_wide", dict(n=20000, h_q=8, h_kv=2, d=64, dtype="f32", r=64, b=64, L=2, beam=16, k=3000,
                                    centres=1024, m=300, mode="chunk")),
            # b = 24: two rows a level-1 sort with lanes past b masked, 384
            # packed candidates per internal level
            ("nm_b24_L3", dict(n=15000, h_q=12, h_kv=3, d=72, dtype="bf16", r=64, b=24, L=3, beam=16, k=400,
                               centres=600, m=333, mode="chunk")),
            # d = 100 (not a multiple of 8: the vector-ALU top step) and b = 4:
            # internal levels with fewer candidates than the beam
            ("nm_b4_L3_d100", dict(n=3000, h_q=4, h_kv=2, d=100, dtype="f32", r=64, b=4, L=3, beam=16, k=200,
                                   centres=64, m=257, mode="chunk"))]


@pytest.mark.parametrize("name,over", NM_CASES, ids=[c[0] for c in NM_CASES])
def test_node_major_select_matches_oracle(lsa, name, over):
    """Batches too large for the decode kernel, with a workspace: levels 2..L
    scored node by node.  Rows equal the oracle's and the one-workgroup
    kernel's bit for bit, with and without sinks and a window, in one batch and
    in one-row batches."""
    dev = torch.device("cuda:0")
    w = _wl("tiny_4k", **over).replace(name=name)
    data = _inputs(w, dev)
    index, desc = lsa.build_index(data["K"], data["W"], w.b, w.L, w.iters)
    torch.cuda.synchronize()
    gix = host_index(lsa.index_views(index, desc), desc)
    c = data["cpu"]
    nws = lsa.select_workspace_bytes(w.m, w.h_q, w.d, desc, w.beam, w.k)
    assert nws > 0
    one_row = lsa.workspace(lsa.select_workspace_bytes(1, w.h_q, w.d, desc, w.beam, w.k), dev)
    for n_sink, window in [(0, 0), (4, 64)]:
        ref = oracle.select(np32(c["Q"]), c["pos"].numpy(), gix, c["W"].numpy(), w.beam, w.k,
                            n_sink=n_sink, window=window)
        runs = [("one-workgroup", None), ("node-major", lsa.workspace(nws, dev))]
        if name != "nm_b32_L3_all":
            runs.append(("node-major one-row batches", one_row))
        for label, ws in runs:
            say("nm select", name, label, n_sink, window)
            sel, cnt, cut = lsa.select(data["Q"], data["pos"], index, desc, data["W"], w.beam, w.k, ws=ws,
                                       n_sink=n_sink, window=window)
            torch.cuda.synchronize()
            assert_same_bits(cnt.cpu().numpy(), ref["count"], f"sel_count ({label})")
            assert_same_bits(sel.cpu().numpy(), ref["sel"], f"sel ({label})")
            assert_same_bits(cut.cpu().numpy(), ref["cutoff"], f"cutoff ({label})")


# node-major attention (lsa_select_attend for batches beyond the decode
# kernel): bf16, d = 128, query heads per KV head 1, 3, 4, 8 and 16 (tiles of
# 128, 42, 32, 16 and 8 pairs), a causal all-positions layer with many pairs
# per node, several tiles per node
NMA_CASES = [("nma_G8_b64_L2", dict(n=20000, h_q=16, h_kv=2, d=128, dtype="bf16", r=64, b=64, L=2, beam=8, k=1000,
                                    centres=1024, m=600, mode="chunk")),
             ("nma_G4_b32_L3_all", dict(n=6000, h_q=4, h_kv=1, d=128, dtype="bf16", r=64, b=32, L=3, beam=5, k=300,
                                        centres=300, m=6000, mode="all")),
             ("nma_G16_b16_L3", dict(n=30000, h_q=32, h_kv=2, d=128, dtype="bf16", r=64, b=16, L=3, beam=16, k=700,
                                     centres=900, m=300, mode="chunk")),
             ("nma_G1_b64_L2", dict(n=9000, h_q=2, h_kv=2, d=128, dtype="bf16", r=64, b=64, L=2, beam=4, k=257,
                                    centres=500, m=2000, mode="chunk")),
             ("nma_G3_b8_L3", dict(n=5000, h_q=6, h_kv=2, d=128, dtype="bf16", r=64, b=8, L=3, beam=3, k=100,
                                   centres=200, m=700, mode="chunk"))]


@pytest.mark.parametrize("name,over", NMA_CASES, ids=[c[0] for c in NMA_CASES])
def test_node_major_attention_matches_oracle(lsa, name, over):
    """lsa_select_attend on batches the decode kernel does not take: the
    selection bit for bit and the attention within the bf16 tolerance against
    the oracle, every row; then the same with one-row and few-row batches (a
    workspace too small for the whole batch)."""
    dev = torch.device("cuda:0")
    w = _wl("tiny_4k", **over).replace(name=name)
    data = _inputs(w, dev)
    index, desc = lsa.build_index(data["K"], data["W"], w.b, w.L, w.iters)
    torch.cuda.synchronize()
    gix = host_index(lsa.index_views(index, desc), desc)
    c = data["cpu"]
    Qh = np32(c["Q"])
    ref = oracle.select(Qh, c["pos"].numpy(), gix, c["W"].numpy(), w.beam, w.k)
    o_ref, lse_ref = oracle.attend(Qh, np32(c["K"]), np32(c["V"]), ref["sel"], ref["count"])
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert w.m * w.h_kv * w.beam > cus                  # not the one-launch form
    full = lsa.select_attend_workspace_bytes(w.m, w.h_q, w.d, desc, w.beam, w.k)
    # the smallest batch beyond the decode kernel: the node-major form runs in
    # batches of about that many rows
    mb = cus // (w.h_kv * w.beam) + 1
    few = lsa.select_attend_workspace_bytes(mb, w.h_q, w.d, desc, w.beam, w.k)
    # a workspace for one decode row only: too small for the node-major form,
    # so the two calls run in sequence
    tiny = lsa.select_attend_workspace_bytes(1, w.h_q, w.d, desc, w.beam, w.k)
    assert few < full and tiny < few
    for label, nbytes in (("one batch", full), (f"batches of about {mb} rows", few), ("two-step form", tiny)):
        say("nm select_attend", name, label)
        ws = lsa.workspace(nbytes, dev)
        sel, cnt, cut, out, lse = lsa.select_attend(data["Q"], data["K"], data["V"], data["pos"], index, desc,
                                                    data["W"], w.beam, w.k, ws=ws)
        torch.cuda.synchronize()
        assert_same_bits(cnt.cpu().numpy(), ref["count"], f"sel_count ({label})")
        assert_same_bits(sel.cpu().numpy(), ref["sel"], f"sel ({label})")
        assert_same_bits(cut.cpu().numpy(), ref["cutoff"], f"cutoff ({label})")
        _check_attention(out, lse, o_ref, lse_ref, TOL[w.torch_dtype])

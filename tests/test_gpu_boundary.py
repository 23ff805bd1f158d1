"""GPU tests of the boundary calls around the index and the workspace:
lsa_index_import of the oracle's own tree (the GPU search run on the oracle's
index), lsa_index_export, the workspace status word, and debug mode."""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import assert_same_bits, np32, say
from _index_bytes import oracle_index_bytes

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def lsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hierarchical_key_indexing_amd as m
    m.lib()
    return m


# the tiny workload and three of the small shapes of the parity tests (20k-40k
# keys, several root pieces, one workgroup per level-1 node for the mean, the
# decode kernel's owned level-2 lists)
IMPORT_CASES = {
    "tiny_4k": {},
    "multi_piece_root": dict(n=20000, h_q=16, h_kv=2, d=128, dtype="bf16", r=64, b=64, L=2, beam=8, k=1000,
                             centres=1024, m=3, mode="decode"),
    "big_nodes_odd_r": dict(n=40000, h_q=8, h_kv=4, d=48, dtype="f32", r=33, b=16, L=3, beam=4, k=500,
                            centres=500, m=4, mode="chunk"),
    "pre_level2_b16": dict(n=30000, h_q=16, h_kv=2, d=128, dtype="bf16", r=64, b=16, L=3, beam=4, k=700,
                           centres=500, m=3, mode="decode"),
}


def _case(name):
    w = synth.WORKLOADS["tiny_4k"]
    over = IMPORT_CASES[name]
    return (w.replace(**over) if over else w).replace(name=name)


def _attn_close(out, lse, o_ref, lse_ref, tol):
    assert np.max(np.abs(np32(out) - o_ref)) <= tol
    g = lse.cpu().numpy()
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(g), fin)
    if fin.any():
        assert np.max(np.abs(g[fin] - lse_ref[fin])) <= 1e-3


@pytest.mark.parametrize("name", list(IMPORT_CASES))
def test_oracle_built_index_searched_on_gpu(lsa, name):
    """The oracle's tree, loaded with lsa_index_import: every GPU search over it
    (one workgroup per row, multi-workgroup, fused with attention, flat) equals
    the oracle's own search of the same tree bit for bit."""
    dev = torch.device("cuda:0")
    w = _case(name)
    data = synth.make_workload(w, device="cpu")
    K, V, Q, W = (np32(data[x]) for x in ("K", "V", "Q", "W"))
    pos = data["pos"].numpy()
    say("import", name)
    oix = oracle.build_index(K, W, w.b, w.L, w.iters)
    desc = lsa.index_layout(w.n, w.h_kv, w.r, w.b, w.L)
    host = oracle_index_bytes(oix, desc)
    index = lsa.index_import(torch.from_numpy(host), desc, dev)
    torch.cuda.synchronize()
    # what is read back is what was loaded (bytes between arrays aside)
    back = lsa.index_export(index, desc).numpy()
    views = lsa.index_views(torch.from_numpy(back), desc)
    assert_same_bits(views["perm"].numpy(), oix.perm.astype(np.int32), "members after the round trip")
    assert_same_bits(views["leaf_off"].numpy(), oix.leaf_off.astype(np.int32), "leaf offsets after the round trip")
    for l in range(1, w.L + 1):
        assert_same_bits(views["C"][l].numpy(), oix.C(l), f"centroids level {l} after the round trip")

    Kd, Vd, Qd, Wd = (data[x].to(dev) for x in ("K", "V", "Q", "W"))
    pd = data["pos"].to(dev)
    tol = TOL[w.torch_dtype]
    for beam, k in [(w.beam, w.k), (1, 7)]:
        ref = oracle.select(Q, pos, oix, W, beam, k)
        o_ref, lse_ref = oracle.attend(Q, K, V, ref["sel"], ref["count"])
        nws = lsa.select_workspace_bytes(w.m, w.h_q, w.d, desc, beam, k)
        for label, ws in (("single-wg", None), ("multi-wg", lsa.workspace(nws, dev))):
            if label == "multi-wg" and ws is None:
                continue
            say("select on the imported tree", name, label, beam, k)
            sel, cnt, cut = lsa.select(Qd, pd, index, desc, Wd, beam, k, ws=ws)
            torch.cuda.synchronize()
            assert_same_bits(cnt.cpu().numpy(), ref["count"], f"sel_count ({label})")
            assert_same_bits(sel.cpu().numpy(), ref["sel"], f"sel ({label})")
            assert_same_bits(cut.cpu().numpy(), ref["cutoff"], f"cutoff ({label})")
        say("select_attend on the imported tree", name, beam, k)
        fws = lsa.workspace(lsa.select_attend_workspace_bytes(w.m, w.h_q, w.d, desc, beam, k), dev)
        sel, cnt, cut, out, lse = lsa.select_attend(Qd, Kd, Vd, pd, index, desc, Wd, beam, k, ws=fws)
        torch.cuda.synchronize()
        assert_same_bits(cnt.cpu().numpy(), ref["count"], "sel_count (fused)")
        assert_same_bits(sel.cpu().numpy(), ref["sel"], "sel (fused)")
        assert_same_bits(cut.cpu().numpy(), ref["cutoff"], "cutoff (fused)")
        _attn_close(out, lse, o_ref, lse_ref, tol)
    say("select_flat on the imported tree", name)
    ref = oracle.select_flat(Q, pos, oix, W, w.k)
    sel, cnt, cut = lsa.select_flat(Qd, pd, index, desc, Wd, w.k)
    torch.cuda.synchronize()
    assert_same_bits(cnt.cpu().numpy(), ref["count"], "sel_count (flat)")
    assert_same_bits(sel.cpu().numpy(), ref["sel"], "sel (flat)")
    assert_same_bits(cut.cpu().numpy(), ref["cutoff"], "cutoff (flat)")


def test_gpu_index_export_import_round_trip(lsa):
    """A tree built on the GPU, exported, and imported into a fresh buffer:
    the arrays are those of the built tree and the searches are unchanged."""
    dev = torch.device("cuda:0")
    w = _case("pre_level2_b16")
    data = synth.make_workload(w, device=dev)
    say("export/import round trip", w.name)
    index, desc = lsa.build_index(data["K"], data["W"], w.b, w.L, w.iters)
    host = lsa.index_export(index, desc)
    views = lsa.index_views(index, desc)
    hv = lsa.index_views(host, desc)
    for key in ("perm", "leaf_off"):
        assert torch.equal(hv[key], views[key].cpu()), key
    for l in range(1, w.L + 1):
        assert torch.equal(hv["C"][l], views["C"][l].cpu()) and torch.equal(hv["cnt"][l], views["cnt"][l].cpu())
    again = lsa.index_import(host, desc, dev)
    a = lsa.select(data["Q"], data["pos"], index, desc, data["W"], w.beam, w.k)
    b = lsa.select(data["Q"], data["pos"], again, desc, data["W"], w.beam, w.k)
    torch.cuda.synchronize()
    for x, y, nm in zip(a, b, ("sel", "count", "cutoff")):
        assert torch.equal(x, y), nm


def test_wait_timeout_flag_reaches_the_status_word(lsa):
    """A group's timeout flag, set from the host before a normal one-launch
    call (so no wait is forced), is reported by the group's workgroup 0 in
    the workspace's status word and cleared in place; lsa_workspace_status
    reads and clears the status word.  Results are unaffected."""
    dev = torch.device("cuda:0")
    w = _case("multi_piece_root")
    data = synth.make_workload(w, device=dev)
    index, desc = lsa.build_index(data["K"], data["W"], w.b, w.L, w.iters)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert w.m * w.h_kv * w.beam <= cus          # the one-launch form runs
    nws = lsa.select_attend_workspace_bytes(w.m, w.h_q, w.d, desc, w.beam, w.k)
    ref = lsa.select_attend(data["Q"], data["K"], data["V"], data["pos"], index, desc, data["W"], w.beam, w.k,
                            ws=lsa.workspace(nws, dev))
    ws = lsa.workspace(nws, dev)
    assert lsa.workspace_status(ws) == 0
    # group 0's control words follow the 256-byte status header:
    # [unused, arrivals, timeout flag, unused]
    flag = slice(256 + 8, 256 + 12)
    ws[flag] = torch.tensor([1, 0, 0, 0], dtype=torch.uint8, device=dev)
    say("seeded timeout flag", w.name)
    got = lsa.select_attend(data["Q"], data["K"], data["V"], data["pos"], index, desc, data["W"], w.beam, w.k, ws=ws)
    torch.cuda.synchronize()
    assert int(ws[flag].count_nonzero()) == 0, "the group's flag was not cleared"
    assert lsa.workspace_status(ws) == lsa.LSA_STATUS_WAIT_TIMEOUT
    assert lsa.workspace_status(ws) == 0          # read and cleared
    for a, b, nm in zip(got, ref, ("sel", "count", "cutoff", "out", "lse")):
        assert torch.equal(a, b), nm
    # the next call on the same workspace reports nothing
    lsa.select_attend(data["Q"], data["K"], data["V"], data["pos"], index, desc, data["W"], w.beam, w.k, ws=ws)
    assert lsa.workspace_status(ws) == 0


def test_debug_mode(lsa):
    """LSA_DEBUG=1 (read when the library is first used, so in a process of
    its own): a good call succeeds; a reported timeout flag, an out-of-range
    sel and a damaged index are errors, the last two caught on the host
    before anything is launched."""
    env = dict(os.environ, LSA_DEBUG="1")
    say("debug mode subprocess")
    r = subprocess.run([sys.executable, os.path.join(HERE, "_debug_mode_case.py")], env=env, capture_output=True,
                       text=True, timeout=600)
    print(r.stdout[-2000:], r.stderr[-2000:])
    assert r.returncode == 0, r.stderr[-2000:]
    assert "debug mode ok" in r.stdout

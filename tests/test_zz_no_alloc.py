"""lsa_select_attend_noalloc (the library's fixed scratch instead of a
workspace) against lsa_select_attend with a caller workspace: two calls in a
row on each workload, the second with fewer rows, outputs to the parity bar
(selection bit for bit, attention within the dtype's tolerance)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from _gpu import assert_same_bits, np32, say

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}

CASES = {
    "tiny_4k": dict(m=3),
    # bf16, d = 128, r = 64, b = 64, L = 2 (the matrix-core attention step)
    "b64_L2": dict(n=20000, h_q=16, h_kv=2, d=128, dtype="bf16", r=64, b=64, L=2, beam=8, k=1000, centres=1024,
                   m=3, mode="decode"),
    # L = 3 with b <= 4 beam: level 2 scored from rows loaded before level 1
    "b16_L3": dict(n=30000, h_q=16, h_kv=2, d=128, dtype="bf16", r=64, b=16, L=3, beam=4, k=700, centres=500, m=3,
                   mode="decode"),
}


@pytest.fixture(scope="module")
def lsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hierarchical_key_indexing_amd as m
    m.lib()
    return m


def _outputs(lsa, m, w, desc, dev):
    """Preallocated outputs, so that the call under test allocates nothing."""
    h = desc.h_kv
    return dict(sel=torch.empty((m, h, w.k), dtype=torch.int32, device=dev),
                sel_count=torch.empty((m, h), dtype=torch.int32, device=dev),
                cutoff=torch.empty((m, h), dtype=torch.float32, device=dev),
                out=torch.empty((m, w.h_q, w.d), dtype=w.torch_dtype, device=dev),
                lse=torch.empty((m, w.h_q), dtype=torch.float32, device=dev))


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_matches_the_workspace_call(lsa, name):
    dev = torch.device("cuda:0")
    base = synth.WORKLOADS["tiny_4k"]
    w = base.replace(name=name, **CASES[name])
    data = synth.make_workload(w, device=dev)
    index, desc = lsa.build_index(data["K"], data["W"], w.b, w.L, w.iters)
    tol = TOL[w.torch_dtype]
    for m in (w.m, 1):          # the second call has fewer rows
        Q, pos = data["Q"][:m].contiguous(), data["pos"][:m].contiguous()
        nws = lsa.select_attend_workspace_bytes(m, w.h_q, w.d, desc, w.beam, w.k)
        ref = lsa.select_attend(Q, data["K"], data["V"], pos, index, desc, data["W"], w.beam, w.k,
                                ws=lsa.workspace(nws, dev))
        outs = _outputs(lsa, m, w, desc, dev)
        torch.cuda.synchronize()
        say("noalloc", name, "rows", m)
        before = torch.cuda.memory_stats(dev).get("allocation.all.allocated", 0)
        got = lsa.select_attend_noalloc(Q, data["K"], data["V"], pos, index, desc, data["W"], w.beam, w.k, **outs)
        after = torch.cuda.memory_stats(dev).get("allocation.all.allocated", 0)
        torch.cuda.synchronize()
        assert after == before, "the call allocated through torch"
        for nm, a, b in zip(("sel_count", "sel", "cutoff"), got[:3], ref[:3]):
            assert_same_bits(a.cpu().numpy(), b.cpu().numpy(), f"{nm} (rows {m})")
        assert np.max(np.abs(np32(got[3]) - np32(ref[3]))) <= tol
        g, r = got[4].cpu().numpy(), ref[4].cpu().numpy()
        assert np.array_equal(np.isfinite(g), np.isfinite(r))
        fin = np.isfinite(r)
        if fin.any():
            assert np.max(np.abs(g[fin] - r[fin])) <= 1e-3
    assert lsa.workspace_status(None) == 0


def test_noalloc_rejects_what_it_cannot_run(lsa):
    """A batch outside the one-launch form is refused, before anything runs."""
    dev = torch.device("cuda:0")
    w = synth.WORKLOADS["tiny_4k"].replace(name="noalloc_big", **CASES["b64_L2"])
    data = synth.make_workload(w, device=dev)
    index, desc = lsa.build_index(data["K"], data["W"], w.b, w.L, w.iters)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    m = cus // (w.h_kv * w.beam) + 1          # more workgroups than compute units
    Q = data["Q"][:1].expand(m, -1, -1).contiguous()
    pos = data["pos"][:1].expand(m).contiguous()
    with pytest.raises(lsa.LSAError) as e:
        lsa.select_attend_noalloc(Q, data["K"], data["V"], pos, index, desc, data["W"], w.beam, w.k)
    assert e.value.code == lsa.LSA_EUNSUPPORTED

"""Run by test_gpu_boundary.test_debug_mode in a process of its own with
LSA_DEBUG=1: the library's debug mode on one small decode workload."""
from __future__ import annotations

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

import torch  # noqa: E402

import hierarchical_key_indexing_amd as lsa  # noqa: E402
import synth  # noqa: E402


def expect(code, fn, what):
    try:
        fn()
    except lsa.LSAError as e:
        assert e.code == code, (what, e.code)
        print("expected error:", what, e, flush=True)
        return
    raise AssertionError(f"{what}: no error")


def main():
    assert os.environ.get("LSA_DEBUG") == "1"
    dev = torch.device("cuda:0")
    w = synth.WORKLOADS["tiny_4k"].replace(n=20000, h_q=16, h_kv=2, d=128, dtype="bf16", r=64, b=64, L=2, beam=8,
                                           k=1000, centres=1024, m=3, mode="decode", name="debug_case")
    data = synth.make_workload(w, device=dev)
    Q, K, V, W, pos = (data[x] for x in ("Q", "K", "V", "W", "pos"))
    index, desc = lsa.build_index(K, W, w.b, w.L, w.iters)
    nws = lsa.select_attend_workspace_bytes(w.m, w.h_q, w.d, desc, w.beam, w.k)
    ws = lsa.workspace(nws, dev)
    print("[case] good call", flush=True)
    sel, cnt, cut, out, lse = lsa.select_attend(Q, K, V, pos, index, desc, W, w.beam, w.k, ws=ws)
    lsa.attend(Q, K, V, sel, cnt)
    lsa.select(Q, pos, index, desc, W, w.beam, w.k)
    print("[case] reported timeout flag", flush=True)
    ws[256 + 8:256 + 12] = torch.tensor([1, 0, 0, 0], dtype=torch.uint8, device=dev)
    expect(lsa.LSA_EDEVICE, lambda: lsa.select_attend(Q, K, V, pos, index, desc, W, w.beam, w.k, ws=ws),
           "timeout flag")
    assert lsa.workspace_status(ws) == 0          # debug mode read and cleared it
    print("[case] out-of-range sel (caught before launch)", flush=True)
    bad = sel.clone()
    bad[0, 0, 0] = w.n
    expect(lsa.LSA_EINVAL, lambda: lsa.attend(Q, K, V, bad, cnt), "sel entry >= n")
    badc = cnt.clone()
    badc[0, 0] = sel.shape[2] + 1
    expect(lsa.LSA_EINVAL, lambda: lsa.attend(Q, K, V, sel, badc), "sel_count > row")
    print("[case] damaged index (caught before launch)", flush=True)
    views = lsa.index_views(index, desc)
    views["perm"][0, 0] = -1
    expect(lsa.LSA_EINVAL, lambda: lsa.select(Q, pos, index, desc, W, w.beam, w.k), "member -1")
    torch.cuda.synchronize()
    print("debug mode ok", flush=True)


if __name__ == "__main__":
    main()

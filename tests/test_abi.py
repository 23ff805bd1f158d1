"""The C ABI library loads, exports every declared entry point and rejects
bad arguments on the host (no device work is enqueued by these calls)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import hierarchical_key_indexing_amd as lsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "lsa.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(lsa_[a-z_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    L = lsa.lib()
    names = _declared()
    assert len(names) >= 11
    for nm in names:
        assert hasattr(L, nm), nm
    assert sorted(names) == sorted(lsa.EXPORTS)
    assert L.lsa_abi_version() == lsa.ABI_VERSION == 2
    assert L.lsa_strerror(-3).decode() == "buffer too small"


def test_index_layout_sizes():
    d = lsa.index_layout(1 << 20, 4, 64, 64, 3)
    assert list(d.nodes[:4]) == [1, 64, 4096, 262144]
    assert d.centroid_off[1] == 0
    for l in range(1, 4):
        assert d.centroid_off[l] % 256 == 0 and d.count_off[l] % 256 == 0
    assert d.count_off[1] >= d.centroid_off[3] + 4 * 262144 * 64 * 4
    assert d.perm_off >= d.leaf_off_off + 4 * (262144 + 1) * 4
    assert d.bytes >= d.perm_off + 4 * (1 << 20) * 4
    # the 10M-token tree: 64^4 leaves per head
    d = lsa.index_layout(10 << 20, 4, 64, 64, 4)
    assert d.nodes[4] == 64 ** 4
    assert d.bytes > 4 * 64 ** 4 * 64 * 4


@pytest.mark.parametrize("args,code", [
    ((0, 1, 8, 2, 1), lsa.LSA_EINVAL),
    ((10, 1, 8, 1, 1), lsa.LSA_EINVAL),
    ((10, 1, 65, 2, 1), lsa.LSA_EUNSUPPORTED),
    ((10, 1, 8, 65, 1), lsa.LSA_EUNSUPPORTED),
    ((10, 1, 8, 64, 7), lsa.LSA_EUNSUPPORTED),
    ((10, 1, 8, 64, 6), lsa.LSA_EUNSUPPORTED),     # 64^6 leaves overflow int32
    ((10, 0, 8, 2, 1), lsa.LSA_EINVAL),
])
def test_index_layout_rejects(args, code):
    d = lsa.IndexDesc()
    assert lsa.lib().lsa_index_layout(*args, ctypes.byref(d)) == code


def test_entry_points_validate_before_touching_the_device():
    L = lsa.lib()
    P = ctypes.c_void_p
    fake = P(0x1000)     # never dereferenced: every call below fails its host checks
    d = lsa.IndexDesc()
    # build: iters < 1, small index buffer, small workspace
    assert L.lsa_build_index(fake, 0, 100, 1, 16, fake, 8, 4, 2, 0, fake, 1 << 30, fake, 1 << 30,
                             ctypes.byref(d), None) == lsa.LSA_EINVAL
    assert L.lsa_build_index(fake, 0, 100, 1, 16, fake, 8, 4, 2, 5, fake, 16, fake, 1 << 30,
                             ctypes.byref(d), None) == lsa.LSA_ENOSPC
    assert L.lsa_build_index(fake, 0, 100, 1, 16, fake, 8, 4, 2, 5, fake, 1 << 30, fake, 16,
                             ctypes.byref(d), None) == lsa.LSA_ENOSPC
    assert L.lsa_build_index(fake, 7, 100, 1, 16, fake, 8, 4, 2, 5, fake, 1 << 30, fake, 1 << 30,
                             ctypes.byref(d), None) == lsa.LSA_EUNSUPPORTED
    assert L.lsa_build_index(fake, 0, 100, 1, 300, fake, 8, 4, 2, 5, fake, 1 << 30, fake, 1 << 30,
                             ctypes.byref(d), None) == lsa.LSA_EUNSUPPORTED
    # select: descriptor must be one lsa_index_layout produced
    d = lsa.index_layout(100, 2, 8, 4, 2)
    bad = lsa.IndexDesc.from_buffer_copy(d)
    bad.bytes += 1
    assert L.lsa_select(fake, 0, 1, 4, 16, fake, ctypes.byref(bad), fake, fake, 2, 8, 0, 0, fake, fake, None, None, 0,
                        None) == lsa.LSA_EINVAL
    assert L.lsa_select(fake, 0, 1, 3, 16, fake, ctypes.byref(d), fake, fake, 2, 8, 0, 0, fake, fake, None, None, 0,
                        None) == lsa.LSA_EINVAL          # h_q % h_kv != 0
    assert L.lsa_select(fake, 0, 1, 4, 16, fake, ctypes.byref(d), fake, fake, 2000, 8, 0, 0, fake, fake, None, None, 0,
                        None) == lsa.LSA_EUNSUPPORTED    # beam * b > 4096
    assert L.lsa_select(fake, 0, 1, 4, 16, fake, ctypes.byref(d), fake, fake, 2, 9000, 0, 0, fake, fake, None, None, 0,
                        None) == lsa.LSA_EUNSUPPORTED    # k > 8192
    assert L.lsa_select(fake, 0, 0, 4, 16, fake, ctypes.byref(d), fake, fake, 2, 8, 0, 0, fake, fake, None, None, 0,
                        None) == lsa.LSA_OK              # m = 0: nothing to do
    assert L.lsa_select(fake, 0, 1, 4, 16, fake, ctypes.byref(d), fake, fake, 2, 8, -1, 0, fake, fake, None, None, 0,
                        None) == lsa.LSA_EINVAL          # negative sink count
    assert L.lsa_select(fake, 0, 1, 4, 16, fake, ctypes.byref(d), fake, fake, 2, 8, 0, -5, fake, fake, None, None, 0,
                        None) == lsa.LSA_EINVAL          # negative window
    assert L.lsa_select(fake, 0, 1, 4, 16, fake, ctypes.byref(d), fake, fake, 2, 8, 1 << 23, 1 << 23, fake, fake,
                        None, None, 0, None) == lsa.LSA_EUNSUPPORTED    # row longer than 2^24
    # flat search: workspace required and sized per row
    one = lsa.select_flat_workspace_bytes(1, 4, d)
    assert one >= 2 * 4 ** 2 * 6 and lsa.select_flat_workspace_bytes(1000, 4, d) > one
    assert L.lsa_select_flat(fake, 0, 1, 4, 16, fake, ctypes.byref(d), fake, fake, 8, 0, 0, fake, fake, None, None, 0,
                             None) == lsa.LSA_ENOSPC      # no workspace
    assert L.lsa_select_flat(fake, 0, 1, 4, 16, fake, ctypes.byref(d), fake, fake, 8, 0, 0, fake, fake, None, fake,
                             one - 1, None) == lsa.LSA_ENOSPC
    assert L.lsa_select_flat(fake, 0, 1, 4, 16, fake, ctypes.byref(d), fake, fake, 9000, 0, 0, fake, fake, None, fake,
                             one, None) == lsa.LSA_EUNSUPPORTED    # k > 8192
    assert L.lsa_select_flat(fake, 0, 1, 4, 16, fake, ctypes.byref(bad), fake, fake, 8, 0, 0, fake, fake, None, fake,
                             one, None) == lsa.LSA_EINVAL
    # insertion: batch size, capacity and workspace checked on the host
    di = lsa.index_layout(100, 2, 8, 4, 2)
    assert L.lsa_index_insert(fake, 0, 0, 16, fake, ctypes.byref(di), fake, 1 << 30, fake, 1 << 30,
                              None) == lsa.LSA_EINVAL
    assert L.lsa_index_insert(fake, 0, 5000, 16, fake, ctypes.byref(di), fake, 1 << 30, fake, 1 << 30,
                              None) == lsa.LSA_EUNSUPPORTED
    assert lsa.index_layout(300, 2, 8, 4, 2).bytes > di.bytes
    assert L.lsa_index_insert(fake, 0, 200, 16, fake, ctypes.byref(di), fake, di.bytes, fake, 1 << 30,
                              None) == lsa.LSA_ENOSPC          # no room for 300 keys
    assert L.lsa_index_insert(fake, 0, 3, 16, fake, ctypes.byref(di), fake, 1 << 30, fake, 8,
                              None) == lsa.LSA_ENOSPC          # workspace too small
    assert di.n == 100                                          # unchanged on error
    # PCA projection
    assert L.lsa_pca_projection(fake, 0, 100, 2, 129, 8, fake, None, fake, 1 << 40, None) == lsa.LSA_EUNSUPPORTED
    assert L.lsa_pca_projection(fake, 0, 100, 2, 64, 65, fake, None, fake, 1 << 40, None) == lsa.LSA_EINVAL
    assert L.lsa_pca_projection(fake, 0, 100, 2, 64, 8, fake, None, fake, 16, None) == lsa.LSA_ENOSPC
    assert lsa.pca_workspace_bytes(1 << 20, 4, 128) >= 4 * 128 * 128 * 8 * 128
    # attend
    f = ctypes.c_float
    assert L.lsa_attend(fake, fake, fake, 0, 1, 4, 3, 100, 64, fake, fake, 8, f(0), fake, None, None, 0,
                        None) == lsa.LSA_EINVAL          # h_q % h_kv
    assert L.lsa_attend(fake, fake, fake, 0, 1, 34, 2, 100, 64, fake, fake, 8, f(0), fake, None, None, 0,
                        None) == lsa.LSA_EUNSUPPORTED    # G = 17
    assert L.lsa_attend(fake, fake, fake, 0, 1, 4, 2, 100, 60, fake, fake, 8, f(0), fake, None, None, 0,
                        None) == lsa.LSA_EUNSUPPORTED    # d % 8
    assert L.lsa_attend(fake, fake, fake, 0, 1, 4, 2, 100, 64, fake, fake, 8, f(-1), fake, None, None, 0,
                        None) == lsa.LSA_EINVAL          # negative scale
    nws = lsa.attend_workspace_bytes(1, 32, 4, 128, 2048)
    assert nws > 0
    assert L.lsa_attend(fake, fake, fake, 1, 1, 32, 4, 100, 128, fake, fake, 2048, f(0), fake, None, None, 0,
                        None) == lsa.LSA_ENOSPC
    assert lsa.build_workspace_bytes(1 << 20, 4, 128, 64, 64, 3) > 4 * (1 << 20) * 64 * 4


def _small_oracle_tree():
    import numpy as np
    import oracle
    import synth
    w = synth.WORKLOADS["tiny_4k"].replace(n=600, b=4, L=3, r=8, d=16, centres=20)
    data = synth.make_workload(w, device="cpu")
    K = data["K"].float().numpy()
    oix = oracle.build_index(K, data["W"].numpy(), w.b, w.L, w.iters)
    desc = lsa.index_layout(w.n, w.h_kv, w.r, w.b, w.L)
    return oix, desc


def _corruptions(desc, oix):
    """(name, function that damages a copy of host index memory)."""
    import numpy as np
    from _index_bytes import view
    L = desc.L
    cL = oix.cnt(L)[0]
    big = int(np.argmax(cL))                       # a leaf with >= 2 members
    assert cL[big] >= 2
    nonempty = int(np.nonzero(oix.cnt(1)[0])[0][0])

    def first_off(buf):
        view(buf, desc, "leaf_off")[0, 0] = 1

    def last_off(buf):
        view(buf, desc, "leaf_off")[0, -1] -= 1

    def leaf_count(buf):
        view(buf, desc, "cnt", L)[0, big] += 1

    def inner_count(buf):
        view(buf, desc, "cnt", 1)[0, nonempty] += 1

    def duplicate_member(buf):
        p = view(buf, desc, "perm")
        s = int(view(buf, desc, "leaf_off")[0, big])
        p[0, s + 1] = p[0, s]

    def unsorted_leaf(buf):
        p = view(buf, desc, "perm")
        s = int(view(buf, desc, "leaf_off")[0, big])
        p[0, s], p[0, s + 1] = p[0, s + 1], p[0, s]

    def member_out_of_range(buf):
        p = view(buf, desc, "perm")
        s = int(view(buf, desc, "leaf_off")[0, big])
        p[0, s] = desc.n

    def negative_member(buf):
        view(buf, desc, "perm")[0, 0] = -1

    def nan_centroid(buf):
        view(buf, desc, "C", 1)[0, nonempty, 3] = np.nan

    def decreasing_offsets(buf):
        lo = view(buf, desc, "leaf_off")
        lo[0, big + 1] = lo[0, big] - 1

    return [first_off, last_off, leaf_count, inner_count, duplicate_member, unsorted_leaf,
            member_out_of_range, negative_member, nan_centroid, decreasing_offsets]


def test_index_import_rejects_an_inconsistent_tree_before_any_copy():
    """lsa_index_import checks the tree on the host and returns EINVAL without
    touching the device (the destination pointer below is never dereferenced)."""
    oix, desc = _small_oracle_tree()
    from _index_bytes import oracle_index_bytes
    L = lsa.lib()
    fake = ctypes.c_void_p(0x1000)
    good = oracle_index_bytes(oix, desc)
    ptr = lambda a: ctypes.c_void_p(a.ctypes.data)
    assert L.lsa_index_import(ctypes.byref(desc), ptr(good), good.size - 1, fake, desc.bytes,
                              None) == lsa.LSA_ENOSPC
    assert L.lsa_index_import(ctypes.byref(desc), ptr(good), good.size, fake, desc.bytes - 1,
                              None) == lsa.LSA_ENOSPC
    assert L.lsa_index_import(ctypes.byref(desc), None, good.size, fake, desc.bytes, None) == lsa.LSA_EINVAL
    assert L.lsa_index_export(ctypes.byref(desc), fake, ptr(good), good.size - 1, None) == lsa.LSA_ENOSPC
    for damage in _corruptions(desc, oix):
        buf = good.copy()
        damage(buf)
        assert L.lsa_index_import(ctypes.byref(desc), ptr(buf), buf.size, fake, desc.bytes,
                                  None) == lsa.LSA_EINVAL, damage.__name__


def test_workspace_status_rejects_bad_arguments():
    L = lsa.lib()
    v = ctypes.c_int32()
    fake = ctypes.c_void_p(0x1000)
    assert L.lsa_workspace_status(fake, 255, ctypes.byref(v), None) == lsa.LSA_EINVAL
    assert L.lsa_workspace_status(fake, 4096, None, None) == lsa.LSA_EINVAL
    assert L.lsa_strerror(lsa.LSA_EDEVICE).decode().startswith("a kernel reported")

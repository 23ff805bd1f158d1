"""Index memory assembled on the host from the oracle's tree, in the layout an
IndexDesc gives (for lsa_index_import): the same arrays the library's build
writes, placed at the descriptor's byte offsets."""
from __future__ import annotations

import numpy as np


def oracle_index_bytes(oix, desc) -> np.ndarray:
    """oix: oracle.Index; desc: the IndexDesc of lsa_index_layout for the same
    (n, h_kv, r, b, L).  Returns a uint8 array of desc.bytes bytes."""
    assert (oix.n, oix.h_kv, oix.r, oix.b, oix.L) == (desc.n, desc.h_kv, desc.r, desc.b, desc.L)
    buf = np.zeros(desc.bytes, np.uint8)

    def put(off, arr):
        raw = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
        buf[off:off + raw.size] = raw

    for l in range(1, desc.L + 1):
        put(desc.centroid_off[l], oix.C(l).astype(np.float32))
        put(desc.count_off[l], oix.cnt(l).astype(np.int32))
    put(desc.leaf_off_off, oix.leaf_off.astype(np.int32))
    put(desc.perm_off, oix.perm.astype(np.int32))
    return buf


def view(buf: np.ndarray, desc, what: str, l: int = 0) -> np.ndarray:
    """A writable typed view of one array inside host index memory."""
    h, r, n, L = desc.h_kv, desc.r, desc.n, desc.L
    if what == "C":
        o, cnt, dt, shape = desc.centroid_off[l], h * desc.nodes[l] * r, np.float32, (h, desc.nodes[l], r)
    elif what == "cnt":
        o, cnt, dt, shape = desc.count_off[l], h * desc.nodes[l], np.int32, (h, desc.nodes[l])
    elif what == "leaf_off":
        o, cnt, dt, shape = desc.leaf_off_off, h * (desc.nodes[L] + 1), np.int32, (h, desc.nodes[L] + 1)
    elif what == "perm":
        o, cnt, dt, shape = desc.perm_off, h * n, np.int32, (h, n)
    else:
        raise ValueError(what)
    return buf[o:o + cnt * 4].view(dt).reshape(shape)

"""Latent sparse attention (LSA) layer for MI355X: Python binding of liblsa.so.

A thin ctypes layer over the C ABI declared in include/lsa.h.  Every step of
the layer runs in the HIP library; this module only allocates outputs with
torch (device memory) and passes pointers and the current stream.

    index, desc = build_index(K, W, b, L, iters)      # lsa_build_index
    sel, count, cutoff = select(Q, q_pos, index, desc, W, beam, k)   # lsa_select
    out, lse = attend(Q, K, V, sel, count)            # lsa_attend

Importing works without a GPU; calling a device entry point without the built
library raises (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from ._build import LIB as _LIB_PATH

LSA_OK, LSA_EINVAL, LSA_EUNSUPPORTED, LSA_ENOSPC, LSA_EHIP = 0, -1, -2, -3, -4
LSA_EDEVICE, LSA_ESCRATCH = -5, -6
LSA_STATUS_WAIT_TIMEOUT = 1
LSA_F32, LSA_BF16 = 0, 1
MAX_LEVELS = 6
ABI_VERSION = 2

EXPORTS = ["lsa_abi_version", "lsa_strerror", "lsa_index_layout", "lsa_index_export", "lsa_index_import",
           "lsa_workspace_status", "lsa_build_workspace_bytes",
           "lsa_build_index", "lsa_select_workspace_bytes", "lsa_select", "lsa_attend_workspace_bytes",
           "lsa_attend", "lsa_select_attend_workspace_bytes", "lsa_select_attend", "lsa_select_flat_workspace_bytes",
           "lsa_select_flat", "lsa_pca_workspace_bytes", "lsa_pca_projection",
           "lsa_index_insert_workspace_bytes", "lsa_index_insert", "lsa_select_attend_noalloc"]


class IndexDesc(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("h_kv", ctypes.c_int32), ("r", ctypes.c_int32),
                ("b", ctypes.c_int32), ("L", ctypes.c_int32),
                ("nodes", ctypes.c_int64 * (MAX_LEVELS + 1)),
                ("centroid_off", ctypes.c_int64 * (MAX_LEVELS + 1)),
                ("count_off", ctypes.c_int64 * (MAX_LEVELS + 1)),
                ("leaf_off_off", ctypes.c_int64), ("perm_off", ctypes.c_int64), ("bytes", ctypes.c_int64)]


class LSAError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {lib().lsa_strerror(code).decode()} ({code})")
        self.code = code


_lib = None


def lib():
    """Load liblsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"HIP library {_LIB_PATH} is not built; run __graft_entry__.build() "
                               "or python -m hierarchical_key_indexing_amd._build")
        L = ctypes.CDLL(_LIB_PATH)
        P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        D = ctypes.POINTER(IndexDesc)
        L.lsa_abi_version.restype = i32
        L.lsa_strerror.argtypes = [i32]
        L.lsa_strerror.restype = ctypes.c_char_p
        L.lsa_index_layout.argtypes = [i64, i32, i32, i32, i32, D]
        L.lsa_index_export.argtypes = [D, P, P, i64, P]
        L.lsa_index_import.argtypes = [D, P, i64, P, i64, P]
        L.lsa_workspace_status.argtypes = [P, i64, ctypes.POINTER(ctypes.c_int32), P]
        L.lsa_build_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, i32, ctypes.POINTER(i64)]
        L.lsa_build_index.argtypes = [P, i32, i64, i32, i32, P, i32, i32, i32, i32, P, i64, P, i64, D, P]
        L.lsa_select_workspace_bytes.argtypes = [i64, i32, i32, D, i32, i32, i32, i32, ctypes.POINTER(i64)]
        L.lsa_select_attend_workspace_bytes.argtypes = [i64, i32, i32, D, i32, i32, i32, i32, ctypes.POINTER(i64)]
        L.lsa_select_attend.argtypes = [P, P, P, i32, i64, i32, i32, P, D, P, P, i32, i32, i32, i32, ctypes.c_float,
                                        P, P, P, P, P, P, i64, P]
        L.lsa_select_attend_noalloc.argtypes = [P, P, P, i32, i64, i32, i32, P, D, P, P, i32, i32, i32, i32,
                                                ctypes.c_float, P, P, P, P, P, P]
        L.lsa_select.argtypes = [P, i32, i64, i32, i32, P, D, P, P, i32, i32, i32, i32, P, P, P, P, i64, P]
        L.lsa_select_flat_workspace_bytes.argtypes = [i64, i32, D, ctypes.POINTER(i64)]
        L.lsa_select_flat.argtypes = [P, i32, i64, i32, i32, P, D, P, P, i32, i32, i32, P, P, P, P, i64, P]
        L.lsa_index_insert_workspace_bytes.argtypes = [i64, D, ctypes.POINTER(i64)]
        L.lsa_index_insert.argtypes = [P, i32, i64, i32, P, D, P, i64, P, i64, P]
        L.lsa_pca_workspace_bytes.argtypes = [i64, i32, i32, ctypes.POINTER(i64)]
        L.lsa_pca_projection.argtypes = [P, i32, i64, i32, i32, i32, P, P, P, i64, P]
        L.lsa_attend_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, ctypes.POINTER(i64)]
        L.lsa_attend.argtypes = [P, P, P, i32, i64, i32, i32, i64, i32, P, P, i32, ctypes.c_float,
                                 P, P, P, i64, P]
        for name in EXPORTS:
            if name not in ("lsa_abi_version", "lsa_strerror"):
                getattr(L, name).restype = i32
        _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc != LSA_OK:
        raise LSAError(rc, what)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return LSA_F32
    if t.dtype == torch.bfloat16:
        return LSA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_out(t: Optional[torch.Tensor], name: str, shape, dtype):
    """A caller-provided output: device, contiguous, of exactly this shape and dtype."""
    if t is None:
        return
    _need(t, name)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")


# ------------------------------------------------------------------ layout
def index_layout(n: int, h_kv: int, r: int, b: int, L: int) -> IndexDesc:
    d = IndexDesc()
    _check(lib().lsa_index_layout(n, h_kv, r, b, L, ctypes.byref(d)), "lsa_index_layout")
    return d


def build_workspace_bytes(n: int, h_kv: int, d: int, r: int, b: int, L: int) -> int:
    v = ctypes.c_int64()
    _check(lib().lsa_build_workspace_bytes(n, h_kv, d, r, b, L, ctypes.byref(v)), "lsa_build_workspace_bytes")
    return v.value


def select_workspace_bytes(m: int, h_q: int, d: int, desc: IndexDesc, beam: int, k: int,
                           n_sink: int = 0, window: int = 0) -> int:
    v = ctypes.c_int64()
    _check(lib().lsa_select_workspace_bytes(m, h_q, d, ctypes.byref(desc), beam, k, n_sink, window,
                                            ctypes.byref(v)),
           "lsa_select_workspace_bytes")
    return v.value


def select_attend_workspace_bytes(m: int, h_q: int, d: int, desc: IndexDesc, beam: int, k: int,
                                  n_sink: int = 0, window: int = 0) -> int:
    v = ctypes.c_int64()
    _check(lib().lsa_select_attend_workspace_bytes(m, h_q, d, ctypes.byref(desc), beam, k, n_sink, window,
                                                   ctypes.byref(v)),
           "lsa_select_attend_workspace_bytes")
    return v.value


def workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    """A zero-filled workspace (the multi-workgroup kernels need zeroed counters
    on first use and leave them zeroed)."""
    return torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=device) if nbytes > 0 else None


def attend_workspace_bytes(m: int, h_q: int, h_kv: int, d: int, k: int) -> int:
    v = ctypes.c_int64()
    _check(lib().lsa_attend_workspace_bytes(m, h_q, h_kv, d, k, ctypes.byref(v)), "lsa_attend_workspace_bytes")
    return v.value


def index_views(index: torch.Tensor, desc: IndexDesc) -> dict:
    """Typed views of the arrays inside index memory (no copy)."""
    h, r, L, n = desc.h_kv, desc.r, desc.L, desc.n
    out = {"C": {}, "cnt": {}}
    for l in range(1, L + 1):
        nodes = desc.nodes[l]
        o = desc.centroid_off[l]
        out["C"][l] = index[o:o + h * nodes * r * 4].view(torch.float32).view(h, nodes, r)
        o = desc.count_off[l]
        out["cnt"][l] = index[o:o + h * nodes * 4].view(torch.int32).view(h, nodes)
    nl = desc.nodes[L]
    o = desc.leaf_off_off
    out["leaf_off"] = index[o:o + h * (nl + 1) * 4].view(torch.int32).view(h, nl + 1)
    o = desc.perm_off
    out["perm"] = index[o:o + h * n * 4].view(torch.int32).view(h, n)
    return out


def index_export(index: torch.Tensor, desc: IndexDesc, stream=None) -> torch.Tensor:
    """Copy index memory to a host uint8 tensor of desc.bytes bytes (lsa_index_export)."""
    _need(index, "index")
    host = torch.empty(desc.bytes, dtype=torch.uint8)
    _check(lib().lsa_index_export(ctypes.byref(desc), _ptr(index), ctypes.c_void_p(host.data_ptr()), host.numel(),
                                  _stream(stream)),
           "lsa_index_export")
    return host


def index_import(host, desc: IndexDesc, device, index: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Load host index memory (uint8, desc's layout; checked on the host first)
    into a device tensor (lsa_index_import)."""
    host = torch.as_tensor(host)
    if host.dtype != torch.uint8 or host.device.type != "cpu" or not host.is_contiguous():
        raise ValueError("host index memory must be a contiguous uint8 host buffer")
    if index is None:
        index = torch.empty(desc.bytes, dtype=torch.uint8, device=device)
    _need(index, "index")
    _check(lib().lsa_index_import(ctypes.byref(desc), ctypes.c_void_p(host.data_ptr()), host.numel(), _ptr(index),
                                  index.numel(), _stream(stream)),
           "lsa_index_import")
    return index


def workspace_status(ws: Optional[torch.Tensor], stream=None) -> int:
    """Read and clear a workspace's status word (LSA_STATUS_* bits;
    lsa_workspace_status); ws None reads the no-alloc entry point's scratch."""
    if ws is not None:
        _need(ws, "ws")
    v = ctypes.c_int32()
    _check(lib().lsa_workspace_status(_ptr(ws), 0 if ws is None else ws.numel(), ctypes.byref(v), _stream(stream)),
           "lsa_workspace_status")
    return v.value


def _need_kv(K: torch.Tensor, V: torch.Tensor, Q: torch.Tensor, h_kv: int, n: Optional[int]):
    """K and V: the same [h_kv, n, d] shape and Q's dtype."""
    d = Q.shape[2]
    want = (h_kv, K.shape[1] if n is None else n, d)
    for t, nm in ((K, "K"), (V, "V")):
        if tuple(t.shape) != want or t.dtype != Q.dtype:
            raise ValueError(f"{nm} must be {Q.dtype} of shape {want}, got {t.dtype} {tuple(t.shape)}")


# ------------------------------------------------------------------ entry points
def build_index(K: torch.Tensor, W: torch.Tensor, b: int, L: int, iters: int = 5,
                index: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None):
    """K [h_kv, n, d] (f32/bf16), W [h_kv, d, r] f32 -> (index uint8 tensor, IndexDesc)."""
    _need(K, "K"); _need(W, "W")
    h, n, d = K.shape
    r = W.shape[2]
    if W.dtype != torch.float32 or tuple(W.shape) != (h, d, r):
        raise ValueError("W must be float32 [h_kv, d, r]")
    desc = index_layout(n, h, r, b, L)
    if index is None:
        index = torch.empty(desc.bytes, dtype=torch.uint8, device=K.device)
    nws = build_workspace_bytes(n, h, d, r, b, L)
    if ws is None:
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=K.device)
    out = IndexDesc()
    _check(lib().lsa_build_index(_ptr(K), _dtype_code(K), n, h, d, _ptr(W), r, b, L, iters, _ptr(index),
                                 index.numel(), _ptr(ws), ws.numel(), ctypes.byref(out), _stream(stream)),
           "lsa_build_index")
    return index, out


_NO_WS = object()


def select(Q: torch.Tensor, q_pos: torch.Tensor, index: torch.Tensor, desc: IndexDesc, W: torch.Tensor,
           beam: int, k: int, sel: Optional[torch.Tensor] = None, sel_count: Optional[torch.Tensor] = None,
           cutoff: Optional[torch.Tensor] = None, want_cutoff: bool = True, ws=_NO_WS, stream=None,
           n_sink: int = 0, window: int = 0):
    """Q [m, h_q, d], q_pos int32 [m] -> (sel int32 [m, h_kv, k + n_sink + window], count int32 [m, h_kv],
    cutoff f32 [m, h_kv]).  A row of sel: retrieved keys, then the sinks and the window.

    ws: None runs one workgroup per (row, KV head); a zero-filled workspace of
    select_workspace_bytes lets small batches use the multi-workgroup kernel
    (allocated per call when omitted)."""
    _need(Q, "Q"); _need(q_pos, "q_pos"); _need(W, "W")
    m, h_q, d = Q.shape
    h = desc.h_kv
    dev = Q.device
    if sel is None:
        sel = torch.empty((m, h, k + n_sink + window), dtype=torch.int32, device=dev)
    if sel_count is None:
        sel_count = torch.empty((m, h), dtype=torch.int32, device=dev)
    if cutoff is None and want_cutoff:
        cutoff = torch.empty((m, h), dtype=torch.float32, device=dev)
    _need_out(sel, "sel", (m, h, k + n_sink + window), torch.int32)
    _need_out(sel_count, "sel_count", (m, h), torch.int32)
    _need_out(cutoff, "cutoff", (m, h), torch.float32)
    if ws is _NO_WS:
        ws = workspace(select_workspace_bytes(m, h_q, d, desc, beam, k, n_sink, window), dev)
    _check(lib().lsa_select(_ptr(Q), _dtype_code(Q), m, h_q, d, _ptr(q_pos), ctypes.byref(desc), _ptr(index),
                            _ptr(W), beam, k, n_sink, window, _ptr(sel), _ptr(sel_count), _ptr(cutoff), _ptr(ws),
                            0 if ws is None else ws.numel(), _stream(stream)),
           "lsa_select")
    return sel, sel_count, cutoff


def select_flat_workspace_bytes(m: int, h_q: int, desc: IndexDesc) -> int:
    v = ctypes.c_int64()
    _check(lib().lsa_select_flat_workspace_bytes(m, h_q, ctypes.byref(desc), ctypes.byref(v)),
           "lsa_select_flat_workspace_bytes")
    return v.value


def select_flat(Q: torch.Tensor, q_pos: torch.Tensor, index: torch.Tensor, desc: IndexDesc, W: torch.Tensor,
                k: int, sel: Optional[torch.Tensor] = None, sel_count: Optional[torch.Tensor] = None,
                cutoff: Optional[torch.Tensor] = None, want_cutoff: bool = True, ws: Optional[torch.Tensor] = None,
                stream=None, n_sink: int = 0, window: int = 0):
    """Flat search (every leaf scored) -> (sel, count, cutoff) as select()."""
    _need(Q, "Q"); _need(q_pos, "q_pos"); _need(W, "W")
    m, h_q, d = Q.shape
    h = desc.h_kv
    dev = Q.device
    if sel is None:
        sel = torch.empty((m, h, k + n_sink + window), dtype=torch.int32, device=dev)
    if sel_count is None:
        sel_count = torch.empty((m, h), dtype=torch.int32, device=dev)
    if cutoff is None and want_cutoff:
        cutoff = torch.empty((m, h), dtype=torch.float32, device=dev)
    _need_out(sel, "sel", (m, h, k + n_sink + window), torch.int32)
    _need_out(sel_count, "sel_count", (m, h), torch.int32)
    _need_out(cutoff, "cutoff", (m, h), torch.float32)
    if ws is None:
        ws = torch.empty(max(select_flat_workspace_bytes(m, h_q, desc), 1), dtype=torch.uint8, device=dev)
    _check(lib().lsa_select_flat(_ptr(Q), _dtype_code(Q), m, h_q, d, _ptr(q_pos), ctypes.byref(desc), _ptr(index),
                                 _ptr(W), k, n_sink, window, _ptr(sel), _ptr(sel_count), _ptr(cutoff), _ptr(ws),
                                 ws.numel(), _stream(stream)),
           "lsa_select_flat")
    return sel, sel_count, cutoff


def select_attend(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, q_pos: torch.Tensor, index: torch.Tensor,
                  desc: IndexDesc, W: torch.Tensor, beam: int, k: int, scale: float = 0.0,
                  sel: Optional[torch.Tensor] = None, sel_count: Optional[torch.Tensor] = None,
                  cutoff: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                  lse: Optional[torch.Tensor] = None, want_cutoff: bool = True, want_lse: bool = True,
                  ws: Optional[torch.Tensor] = None, stream=None, n_sink: int = 0, window: int = 0):
    """lsa_select + lsa_attend (one launch for small batches) -> (sel, count, cutoff, out, lse)."""
    for t, nm in ((Q, "Q"), (K, "K"), (V, "V"), (q_pos, "q_pos"), (W, "W")):
        _need(t, nm)
    m, h_q, d = Q.shape
    h = desc.h_kv
    _need_kv(K, V, Q, h, desc.n)
    dev = Q.device
    if sel is None:
        sel = torch.empty((m, h, k + n_sink + window), dtype=torch.int32, device=dev)
    if sel_count is None:
        sel_count = torch.empty((m, h), dtype=torch.int32, device=dev)
    if cutoff is None and want_cutoff:
        cutoff = torch.empty((m, h), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty_like(Q)
    if lse is None and want_lse:
        lse = torch.empty((m, h_q), dtype=torch.float32, device=dev)
    _need_out(sel, "sel", (m, h, k + n_sink + window), torch.int32)
    _need_out(sel_count, "sel_count", (m, h), torch.int32)
    _need_out(cutoff, "cutoff", (m, h), torch.float32)
    _need_out(out, "out", (m, h_q, d), Q.dtype)
    _need_out(lse, "lse", (m, h_q), torch.float32)
    if ws is None:
        ws = workspace(select_attend_workspace_bytes(m, h_q, d, desc, beam, k, n_sink, window), dev)
    _check(lib().lsa_select_attend(_ptr(Q), _ptr(K), _ptr(V), _dtype_code(Q), m, h_q, d, _ptr(q_pos),
                                   ctypes.byref(desc), _ptr(index), _ptr(W), beam, k, n_sink, window, float(scale),
                                   _ptr(sel),
                                   _ptr(sel_count), _ptr(cutoff), _ptr(out), _ptr(lse), _ptr(ws),
                                   0 if ws is None else ws.numel(), _stream(stream)),
           "lsa_select_attend")
    return sel, sel_count, cutoff, out, lse


def select_attend_noalloc(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, q_pos: torch.Tensor,
                          index: torch.Tensor, desc: IndexDesc, W: torch.Tensor, beam: int, k: int,
                          scale: float = 0.0, sel: Optional[torch.Tensor] = None,
                          sel_count: Optional[torch.Tensor] = None, cutoff: Optional[torch.Tensor] = None,
                          out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                          want_cutoff: bool = True, want_lse: bool = True, stream=None, n_sink: int = 0,
                          window: int = 0):
    """lsa_select_attend_noalloc: the one-launch select + attend on the
    library's fixed scratch (no workspace).  Pass every output to make the
    call allocate nothing at all.  -> (sel, count, cutoff, out, lse)"""
    for t, nm in ((Q, "Q"), (K, "K"), (V, "V"), (q_pos, "q_pos"), (W, "W")):
        _need(t, nm)
    m, h_q, d = Q.shape
    h = desc.h_kv
    _need_kv(K, V, Q, h, desc.n)
    dev = Q.device
    if sel is None:
        sel = torch.empty((m, h, k + n_sink + window), dtype=torch.int32, device=dev)
    if sel_count is None:
        sel_count = torch.empty((m, h), dtype=torch.int32, device=dev)
    if cutoff is None and want_cutoff:
        cutoff = torch.empty((m, h), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty_like(Q)
    if lse is None and want_lse:
        lse = torch.empty((m, h_q), dtype=torch.float32, device=dev)
    _need_out(sel, "sel", (m, h, k + n_sink + window), torch.int32)
    _need_out(sel_count, "sel_count", (m, h), torch.int32)
    _need_out(cutoff, "cutoff", (m, h), torch.float32)
    _need_out(out, "out", (m, h_q, d), Q.dtype)
    _need_out(lse, "lse", (m, h_q), torch.float32)
    _check(lib().lsa_select_attend_noalloc(_ptr(Q), _ptr(K), _ptr(V), _dtype_code(Q), m, h_q, d, _ptr(q_pos),
                                           ctypes.byref(desc), _ptr(index), _ptr(W), beam, k, n_sink, window,
                                           float(scale), _ptr(sel), _ptr(sel_count), _ptr(cutoff), _ptr(out),
                                           _ptr(lse), _stream(stream)),
           "lsa_select_attend_noalloc")
    return sel, sel_count, cutoff, out, lse


def attend(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, sel: torch.Tensor, sel_count: torch.Tensor,
           scale: float = 0.0, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
           want_lse: bool = True, ws: Optional[torch.Tensor] = None, stream=None):
    """-> (out [m, h_q, d] in Q's dtype, lse f32 [m, h_q])."""
    for t, nm in ((Q, "Q"), (K, "K"), (V, "V"), (sel, "sel"), (sel_count, "sel_count")):
        _need(t, nm)
    m, h_q, d = Q.shape
    h_kv, n, _ = K.shape
    _need_kv(K, V, Q, h_kv, None)
    k = sel.shape[2]
    if out is None:
        out = torch.empty_like(Q)
    if lse is None and want_lse:
        lse = torch.empty((m, h_q), dtype=torch.float32, device=Q.device)
    _need_out(sel_count, "sel_count", (m, h_kv), torch.int32)
    if tuple(sel.shape[:2]) != (m, h_kv):
        raise ValueError(f"sel must be [m, h_kv, row] = [{m}, {h_kv}, row], got {tuple(sel.shape)}")
    _need_out(out, "out", (m, h_q, d), Q.dtype)
    _need_out(lse, "lse", (m, h_q), torch.float32)
    nws = attend_workspace_bytes(m, h_q, h_kv, d, k)
    if ws is None and nws > 0:
        ws = torch.empty(nws, dtype=torch.uint8, device=Q.device)
    _check(lib().lsa_attend(_ptr(Q), _ptr(K), _ptr(V), _dtype_code(Q), m, h_q, h_kv, n, d, _ptr(sel),
                            _ptr(sel_count), k, float(scale), _ptr(out), _ptr(lse), _ptr(ws),
                            0 if ws is None else ws.numel(), _stream(stream)),
           "lsa_attend")
    return out, lse


def pca_workspace_bytes(n: int, h_kv: int, d: int) -> int:
    v = ctypes.c_int64()
    _check(lib().lsa_pca_workspace_bytes(n, h_kv, d, ctypes.byref(v)), "lsa_pca_workspace_bytes")
    return v.value


def pca_projection(K: torch.Tensor, r: int, W: Optional[torch.Tensor] = None, want_eigenvalues: bool = True,
                   ws: Optional[torch.Tensor] = None, stream=None):
    """K [h_kv, n, d] (f32/bf16) -> (W f32 [h_kv, d, r], eigenvalues f64 [h_kv, r] or None)."""
    _need(K, "K")
    h, n, d = K.shape
    if W is None:
        W = torch.empty((h, d, r), dtype=torch.float32, device=K.device)
    _need_out(W, "W", (h, d, r), torch.float32)
    ev = torch.empty((h, r), dtype=torch.float64, device=K.device) if want_eigenvalues else None
    if ws is None:
        ws = torch.empty(pca_workspace_bytes(n, h, d), dtype=torch.uint8, device=K.device)
    _check(lib().lsa_pca_projection(_ptr(K), _dtype_code(K), n, h, d, r, _ptr(W), _ptr(ev), _ptr(ws), ws.numel(),
                                    _stream(stream)),
           "lsa_pca_projection")
    return W, ev


def index_insert_workspace_bytes(m: int, desc: IndexDesc) -> int:
    v = ctypes.c_int64()
    _check(lib().lsa_index_insert_workspace_bytes(m, ctypes.byref(desc), ctypes.byref(v)),
           "lsa_index_insert_workspace_bytes")
    return v.value


def index_insert(K_new: torch.Tensor, W: torch.Tensor, index: torch.Tensor, desc: IndexDesc,
                 ws: Optional[torch.Tensor] = None, stream=None) -> IndexDesc:
    """Insert the keys K_new [h_kv, m, d] (positions desc.n ..) into `index` in
    place; `index` must hold the layout for desc.n + m keys.  Returns the new
    descriptor (desc itself is left unchanged)."""
    _need(K_new, "K_new"); _need(W, "W"); _need(index, "index")
    h, m, d = K_new.shape
    if h != desc.h_kv:
        raise ValueError("K_new must have one row block per KV head of the index")
    out = IndexDesc.from_buffer_copy(desc)
    if ws is None:
        ws = torch.empty(index_insert_workspace_bytes(m, desc), dtype=torch.uint8, device=K_new.device)
    _check(lib().lsa_index_insert(_ptr(K_new), _dtype_code(K_new), m, d, _ptr(W), ctypes.byref(out), _ptr(index),
                                  index.numel(), _ptr(ws), ws.numel(), _stream(stream)),
           "lsa_index_insert")
    return out

"""Python binding of libdt.so (include/dt.h): argument marshalling only.

Every step of the path runs in the library's HIP kernels.  torch supplies
device memory, the stream and (optionally) the profiling events; the
functions below only turn tensors into the plain pointers and sizes the C
ABI takes.  If the library is missing the import fails loudly: there is no
CPU fallback.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdt.so")

DT_OK, DT_ERR_INVALID_ARG, DT_ERR_UNSUPPORTED, DT_ERR_WORKSPACE, DT_ERR_HIP = 0, 1, 2, 3, 4
DT_DTYPE_F32, DT_DTYPE_BF16 = 0, 1
DT_MODE_DART, DT_MODE_DARTREE, DT_MODE_DARTREE_FULL = 0, 1, 2
DT_NGRAM_NONE, DT_NGRAM_DENSE_BIGRAM, DT_NGRAM_CSR_BIGRAM, DT_NGRAM_HASH_TRIGRAM = 0, 1, 2, 3


class DtError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {dt_status_string(status)}")


class _NGram(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("min_logp", ctypes.c_float),
        ("dense_logp", ctypes.c_void_p),
        ("row_ptr", ctypes.c_void_p),
        ("col", ctypes.c_void_p),
        ("csr_logp", ctypes.c_void_p),
        ("nnz", ctypes.c_int64),
        ("keys", ctypes.c_void_p),
        ("succ", ctypes.c_void_p),
        ("hash_logp", ctypes.c_void_p),
        ("cap", ctypes.c_int64),
        ("S", ctypes.c_int32),
    ]


class _Params(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("V", ctypes.c_int32), ("d", ctypes.c_int32), ("k", ctypes.c_int32),
        ("W", ctypes.c_int32), ("budget", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("mode", ctypes.c_int32), ("ctx", ctypes.c_void_p), ("E", ctypes.c_void_p),
        ("F", ctypes.c_void_p), ("R", ctypes.c_int32), ("sweep_chunks", ctypes.c_int32),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p), ("prof_event_start", ctypes.c_void_p),
        ("prof_event_stop", ctypes.c_void_p),
    ]


class _TreeOut(ctypes.Structure):
    _fields_ = [("n_nodes", ctypes.c_void_p), ("tokens", ctypes.c_void_p),
                ("parents", ctypes.c_void_p), ("depths", ctypes.c_void_p),
                ("scores", ctypes.c_void_p), ("mask", ctypes.c_void_p)]


EXPORTED = ("dt_build_tree", "dt_build_tree_noalloc", "dt_workspace_size", "dt_status_string", "dt_position_topk",
            "dt_ngram_update", "dt_verify_length")
DT_NOALLOC_SCRATCH_BYTES = 32 << 20

_lib = None


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                              "(python -m draft_tree_construction_dt_amd.build)")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.dt_build_tree.restype = ctypes.c_int
        lib.dt_build_tree.argtypes = [ctypes.c_void_p, ctypes.POINTER(_NGram), ctypes.POINTER(_Params),
                                      ctypes.POINTER(_TreeOut)]
        lib.dt_build_tree_noalloc.restype = ctypes.c_int
        lib.dt_build_tree_noalloc.argtypes = lib.dt_build_tree.argtypes
        lib.dt_workspace_size.restype = ctypes.c_size_t
        lib.dt_workspace_size.argtypes = [ctypes.POINTER(_Params)]
        lib.dt_status_string.restype = ctypes.c_char_p
        lib.dt_status_string.argtypes = [ctypes.c_int]
        lib.dt_position_topk.restype = ctypes.c_int
        lib.dt_position_topk.argtypes = [ctypes.c_void_p, ctypes.POINTER(_Params), ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p]
        lib.dt_ngram_update.restype = ctypes.c_int
        lib.dt_ngram_update.argtypes = [ctypes.POINTER(_NGram), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p,
                                        ctypes.c_void_p]
        lib.dt_verify_length.restype = ctypes.c_int
        lib.dt_verify_length.argtypes = [ctypes.POINTER(_TreeOut), ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
                                         ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        _lib = lib
    return _lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


# ---------------------------------------------------------------------------
# Python mirrors of the C structs (fields hold torch tensors or plain values)
# ---------------------------------------------------------------------------

@dataclass
class NGram:
    kind: int = DT_NGRAM_NONE
    min_logp: float = float("-inf")
    dense_logp: Optional[torch.Tensor] = None
    row_ptr: Optional[torch.Tensor] = None
    col: Optional[torch.Tensor] = None
    csr_logp: Optional[torch.Tensor] = None
    keys: Optional[torch.Tensor] = None      # int64 view of the uint64 keys
    succ: Optional[torch.Tensor] = None
    hash_logp: Optional[torch.Tensor] = None
    cap: int = 0
    S: int = 0

    def _c(self) -> _NGram:
        nnz = int(self.col.numel()) if isinstance(self.col, torch.Tensor) else 0
        return _NGram(int(self.kind), float(self.min_logp), _ptr(self.dense_logp), _ptr(self.row_ptr),
                      _ptr(self.col), _ptr(self.csr_logp), nnz, _ptr(self.keys), _ptr(self.succ),
                      _ptr(self.hash_logp), int(self.cap), int(self.S))


@dataclass
class Params:
    B: int
    V: int
    d: int
    k: int
    W: int
    budget: int
    dtype: int
    mode: int = DT_MODE_DART
    ctx: Optional[torch.Tensor] = None
    E: Optional[torch.Tensor] = None
    F: Optional[torch.Tensor] = None
    R: int = 0
    sweep_chunks: int = 0
    workspace: Optional[torch.Tensor] = None
    stream: Optional[object] = None           # torch.cuda.Stream, raw handle (int) or None = current
    prof_event_start: Optional[object] = None  # torch.cuda.Event or raw handle
    prof_event_stop: Optional[object] = None

    def _c(self) -> _Params:
        if self.stream is None:
            stream = torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else 0
        elif isinstance(self.stream, int):
            stream = self.stream
        else:
            stream = self.stream.cuda_stream

        def ev(e):
            if e is None:
                return None
            return e if isinstance(e, int) else e.cuda_event

        ws = self.workspace
        return _Params(int(self.B), int(self.V), int(self.d), int(self.k), int(self.W), int(self.budget),
                       int(self.dtype), int(self.mode), _ptr(self.ctx), _ptr(self.E), _ptr(self.F),
                       int(self.R), int(self.sweep_chunks), _ptr(ws),
                       int(ws.numel() * ws.element_size()) if ws is not None else 0,
                       stream, ev(self.prof_event_start), ev(self.prof_event_stop))


@dataclass
class TreeOut:
    n_nodes: torch.Tensor
    tokens: torch.Tensor
    parents: torch.Tensor
    depths: torch.Tensor
    scores: torch.Tensor
    mask: torch.Tensor

    def _c(self) -> _TreeOut:
        return _TreeOut(_ptr(self.n_nodes), _ptr(self.tokens), _ptr(self.parents), _ptr(self.depths),
                        _ptr(self.scores), _ptr(self.mask))

    def numpy(self) -> dict:
        return dict(n_nodes=self.n_nodes.cpu().numpy(), tokens=self.tokens.cpu().numpy(),
                    parents=self.parents.cpu().numpy(), depths=self.depths.cpu().numpy(),
                    scores=self.scores.cpu().numpy(),
                    mask=self.mask.cpu().numpy().view(np.uint32))


# ---------------------------------------------------------------------------
# the C entry points, same names
# ---------------------------------------------------------------------------

def dt_status_string(status: int) -> str:
    return _load().dt_status_string(int(status)).decode()


def dt_workspace_size(params: Params) -> int:
    p = params._c()
    return int(_load().dt_workspace_size(ctypes.byref(p)))


def dt_build_tree(logits: torch.Tensor, ngram: NGram, params: Params, out: TreeOut) -> None:
    g, p, o = ngram._c(), params._c(), out._c()
    st = _load().dt_build_tree(_ptr(logits), ctypes.byref(g), ctypes.byref(p), ctypes.byref(o))
    if st != DT_OK:
        raise DtError(st, "dt_build_tree")


def dt_build_tree_noalloc(logits: torch.Tensor, ngram: NGram, params: Params, out: TreeOut) -> None:
    """dt_build_tree on the library's own per-GPU scratch array (params.workspace
    is ignored): for callers that cannot allocate."""
    g, p, o = ngram._c(), params._c(), out._c()
    st = _load().dt_build_tree_noalloc(_ptr(logits), ctypes.byref(g), ctypes.byref(p), ctypes.byref(o))
    if st != DT_OK:
        raise DtError(st, "dt_build_tree_noalloc")


def dt_ngram_update(ngram: "NGram", ctx: torch.Tensor, tokens: torch.Tensor, lengths: torch.Tensor,
                    new_logp: float = 0.0, counts: Optional[torch.Tensor] = None, stream=None) -> None:
    """Add the trigrams of the accepted tokens to a device trigram table in
    place (see dt_ngram_update in dt.h).  ctx int32 [B][2], tokens int32
    [B][L], lengths int32 [B], counts int32 [3] or None; all on the device."""
    g = ngram._c()
    B, L = (int(tokens.shape[0]), int(tokens.shape[1])) if tokens.dim() == 2 else (0, 0)
    if stream is None:
        h = torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else 0
    elif isinstance(stream, int):
        h = stream
    else:
        h = stream.cuda_stream
    st = _load().dt_ngram_update(ctypes.byref(g), _ptr(ctx), _ptr(tokens), _ptr(lengths), B, L,
                                 float(new_logp), _ptr(counts), h)
    if st != DT_OK:
        raise DtError(st, "dt_ngram_update")


def dt_verify_length(tree: "TreeOut", budget: int, cost_fixed: float, cost_per_token: float,
                     n_verify: torch.Tensor, rank: torch.Tensor, stream=None) -> None:
    """How many best-first nodes of each tree to verify, and every node's
    best-first position (see dt_verify_length in dt.h); all on the device."""
    t = tree._c()
    B = int(tree.n_nodes.shape[0])
    if stream is None:
        h = torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else 0
    elif isinstance(stream, int):
        h = stream
    else:
        h = stream.cuda_stream
    st = _load().dt_verify_length(ctypes.byref(t), B, int(budget), float(cost_fixed), float(cost_per_token),
                                  _ptr(n_verify), _ptr(rank), h)
    if st != DT_OK:
        raise DtError(st, "dt_verify_length")


def dt_position_topk(logits: torch.Tensor, params: Params, lse: torch.Tensor, topk_tok: torch.Tensor,
                     topk_val: torch.Tensor) -> None:
    p = params._c()
    st = _load().dt_position_topk(_ptr(logits), ctypes.byref(p), _ptr(lse), _ptr(topk_tok), _ptr(topk_val))
    if st != DT_OK:
        raise DtError(st, "dt_position_topk")


# ---------------------------------------------------------------------------
# plumbing: move a generated problem to the device and allocate outputs
# ---------------------------------------------------------------------------

def _dev(a, device, dtype=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint64:
        a = a.view(np.int64)
    elif a.dtype == np.uint16:
        a = a.view(np.int16)
    t = torch.from_numpy(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


def upload_ngram(ng, device) -> NGram:
    return NGram(kind=int(ng.kind), min_logp=float(ng.min_logp),
                 dense_logp=_dev(ng.dense_logp, device), row_ptr=_dev(ng.row_ptr, device),
                 col=_dev(ng.col, device), csr_logp=_dev(ng.csr_logp, device),
                 keys=_dev(ng.keys, device), succ=_dev(ng.succ, device),
                 hash_logp=_dev(ng.hash_logp, device), cap=int(ng.cap or 0), S=int(ng.S or 0))


def alloc_tree_out(B: int, budget: int, device) -> TreeOut:
    words = (budget + 31) // 32
    i32 = dict(dtype=torch.int32, device=device)
    return TreeOut(n_nodes=torch.empty(B, **i32), tokens=torch.empty(B, budget, **i32),
                   parents=torch.empty(B, budget, **i32), depths=torch.empty(B, budget, **i32),
                   scores=torch.empty(B, budget, dtype=torch.float32, device=device),
                   mask=torch.empty(B, budget, words, **i32))


def logits_tensor(p, device) -> torch.Tensor:
    if p.logits.dtype == np.uint16:
        return _dev(p.logits, device).view(torch.bfloat16)
    return _dev(p.logits, device, torch.float32)


@dataclass
class DeviceProblem:
    logits: torch.Tensor
    ngram: NGram
    params: Params
    out: TreeOut
    extra_logits: list = field(default_factory=list)


def upload_problem(p, device, *, sweep_chunks: int = 0, W=None, budget=None) -> DeviceProblem:
    """Copy a generated problem to ``device`` and size the workspace and outputs."""
    W = p.W if W is None else W
    budget = p.budget if budget is None else budget
    dtype = DT_DTYPE_BF16 if p.logits.dtype == np.uint16 else DT_DTYPE_F32
    params = Params(B=p.B, V=p.V, d=p.d, k=p.k, W=W, budget=budget, dtype=dtype, mode=int(p.mode),
                    ctx=_dev(p.ctx, device, torch.int32), E=_dev(p.E, device), F=_dev(p.F, device),
                    R=int(p.R or 0), sweep_chunks=sweep_chunks)
    nbytes = dt_workspace_size(params)
    params.workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    return DeviceProblem(logits=logits_tensor(p, device), ngram=upload_ngram(p.ngram, device),
                         params=params, out=alloc_tree_out(p.B, budget, device))

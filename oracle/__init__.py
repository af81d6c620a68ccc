"""CPU oracle for draft-tree construction -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it, and it
imports nothing from the HIP package: inputs are passed as plain numpy arrays
(or any object carrying the same attributes as a generated problem).

The arithmetic lives in ``oracle.c`` (plain C, double precision, full sorts);
this module only marshals arguments.  What it computes and the readings it
takes are stated in ``oracle.h``.  Parity status: every function here is
pinned by ``tests/test_oracle_*.py`` (closed forms, library routines, brute
force over all paths, textbook special cases, per-depth top-W checks that
rescore every candidate from the logits, and a hand-derived worked example
under ``tests/golden/``).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

# enumerations as oracle.h defines them (kept here, not imported, on purpose)
NGRAM_NONE, NGRAM_DENSE_BIGRAM, NGRAM_CSR_BIGRAM, NGRAM_HASH_TRIGRAM = 0, 1, 2, 3
MODE_DART, MODE_DARTREE, MODE_DARTREE_FULL = 0, 1, 2
DTYPE_F32, DTYPE_BF16 = 0, 1


def build(force: bool = True) -> str:
    """Compile liboracle.so with plain gcc (no fast-math, no contraction)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
             "-Wall", "-Wextra", "-o", tmp, os.path.join(HERE, "oracle.c"), "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class _NGram(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("min_logp", ctypes.c_float),
        ("dense_logp", ctypes.c_void_p),
        ("row_ptr", ctypes.c_void_p),
        ("col", ctypes.c_void_p),
        ("csr_logp", ctypes.c_void_p),
        ("keys", ctypes.c_void_p),
        ("succ", ctypes.c_void_p),
        ("hash_logp", ctypes.c_void_p),
        ("cap", ctypes.c_int64),
        ("S", ctypes.c_int32),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(LIB_PATH)
        lib.oracle_row_lse.restype = ctypes.c_double
        lib.oracle_row_lse.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64]
        lib.oracle_row_topk.restype = None
        lib.oracle_row_topk.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_continuity.restype = ctypes.c_int
        lib.oracle_continuity.argtypes = [ctypes.POINTER(_NGram), ctypes.c_int64, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32]
        lib.oracle_ngram_update.restype = ctypes.c_int
        lib.oracle_ngram_update.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                            ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_void_p]
        lib.oracle_verify_length.restype = ctypes.c_int
        lib.oracle_verify_length.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                             ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_build_tree.restype = ctypes.c_int
        lib.oracle_build_tree.argtypes = [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(_NGram),
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


class _Held:
    """Keeps the contiguous copies alive while C reads them."""

    def __init__(self, ng):
        self.dense = _c(getattr(ng, "dense_logp", None), np.float32)
        self.row_ptr = _c(getattr(ng, "row_ptr", None), np.int32)
        self.col = _c(getattr(ng, "col", None), np.int32)
        self.csr_logp = _c(getattr(ng, "csr_logp", None), np.float32)
        self.keys = _c(getattr(ng, "keys", None), np.uint64)
        self.succ = _c(getattr(ng, "succ", None), np.int32)
        self.hash_logp = _c(getattr(ng, "hash_logp", None), np.float32)
        self.s = _NGram(int(ng.kind), float(ng.min_logp), _ptr(self.dense), _ptr(self.row_ptr),
                        _ptr(self.col), _ptr(self.csr_logp), _ptr(self.keys), _ptr(self.succ),
                        _ptr(self.hash_logp), int(getattr(ng, "cap", 0) or 0),
                        int(getattr(ng, "S", 0) or 0))


def _row(row):
    row = np.ascontiguousarray(row)
    if row.dtype == np.uint16:
        return row, 1
    return np.ascontiguousarray(row, dtype=np.float32), 0


def row_lse(row) -> float:
    """Log-softmax normaliser of one logit row (uint16 = bf16 bits, else fp32)."""
    r, bf = _row(row)
    return float(_load().oracle_row_lse(r.ctypes.data, bf, r.size))


def row_topk(row, k: int):
    """(ids int32[k], values float64[k]) of the k largest entries, lower id first on ties."""
    r, bf = _row(row)
    tok = np.empty(k, dtype=np.int32)
    val = np.empty(k, dtype=np.float64)
    _load().oracle_row_topk(r.ctypes.data, bf, r.size, int(k), tok.ctypes.data, val.ctypes.data)
    return tok, val


def continuity(ngram, V: int, t2: int, t1: int, c: int) -> bool:
    h = _Held(ngram)
    return bool(_load().oracle_continuity(ctypes.byref(h.s), int(V), int(t2), int(t1), int(c)))


def build_tree(p, *, W=None, budget=None, ngram=None) -> dict:
    """Run the whole path for problem ``p`` (attributes as a generated problem).

    ``W``, ``budget`` and ``ngram`` override the problem's values.  Returns
    a dict of numpy arrays: n_nodes [B], tokens/parents/depths [B][budget],
    scores f32 [B][budget], mask u32 [B][budget][ceil(budget/32)], lookups [B].
    """
    W = p.W if W is None else W
    budget = p.budget if budget is None else budget
    ng = p.ngram if ngram is None else ngram
    B, d, V = p.logits.shape
    bf = 1 if p.logits.dtype == np.uint16 else 0
    logits = np.ascontiguousarray(p.logits)
    ctx = np.ascontiguousarray(p.ctx, dtype=np.int32)
    E = _c(p.E, np.float32)
    F = _c(p.F, np.float32)
    h = _Held(ng)
    words = (budget + 31) // 32
    out = dict(
        n_nodes=np.zeros(B, dtype=np.int32),
        tokens=np.zeros((B, budget), dtype=np.int32),
        parents=np.zeros((B, budget), dtype=np.int32),
        depths=np.zeros((B, budget), dtype=np.int32),
        scores=np.zeros((B, budget), dtype=np.float32),
        mask=np.zeros((B, budget, words), dtype=np.uint32),
        lookups=np.zeros(B, dtype=np.int64),
    )
    rc = _load().oracle_build_tree(
        logits.ctypes.data, bf, B, V, d, int(p.k), int(W), int(budget), int(p.mode), ctx.ctypes.data,
        _ptr(E), _ptr(F), int(p.R or 0), ctypes.byref(h.s),
        out["n_nodes"].ctypes.data, out["tokens"].ctypes.data, out["parents"].ctypes.data,
        out["depths"].ctypes.data, out["scores"].ctypes.data, out["mask"].ctypes.data,
        out["lookups"].ctypes.data)
    if rc != 0:
        raise ValueError("oracle_build_tree rejected its arguments")
    return out


def ngram_update(ngram, ctx, tokens, lengths, new_logp: float = 0.0):
    """Apply the accepted tokens to a trigram table in place (numpy arrays
    ngram.keys, ngram.succ and, if present, ngram.hash_logp), sequentially in
    stream order.  ctx int32[B][2], tokens int32[B][L], lengths int32[B].
    Returns (keys added, successors added, trigrams dropped)."""
    keys = ngram.keys
    succ = ngram.succ
    lp = getattr(ngram, "hash_logp", None)
    for a, dt in ((keys, np.uint64), (succ, np.int32)):
        if a.dtype != dt or not a.flags.c_contiguous:
            raise ValueError("table arrays must be contiguous uint64 keys and int32 succ")
    if lp is not None and (lp.dtype != np.float32 or not lp.flags.c_contiguous):
        raise ValueError("hash_logp must be contiguous float32")
    ctx = np.ascontiguousarray(ctx, dtype=np.int32)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    lengths = np.ascontiguousarray(lengths, dtype=np.int32)
    B, L = tokens.shape
    counts = np.zeros(3, dtype=np.int64)
    rc = _load().oracle_ngram_update(keys.ctypes.data, succ.ctypes.data, _ptr(lp), int(ngram.cap), int(ngram.S),
                                     ctx.ctypes.data, tokens.ctypes.data, lengths.ctypes.data, int(B), int(L),
                                     float(new_logp), counts.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_ngram_update: invalid arguments")
    return tuple(int(x) for x in counts)


def verify_length(tree: dict, cost_fixed: float, cost_per_token: float):
    """How many best-first nodes of each tree to verify, and every node's
    best-first position (see oracle_verify_length).  ``tree`` holds the
    arrays build_tree returns.  Returns (n_verify int32[B], rank int32[B][budget])."""
    n_nodes = np.ascontiguousarray(tree["n_nodes"], dtype=np.int32)
    parents = np.ascontiguousarray(tree["parents"], dtype=np.int32)
    depths = np.ascontiguousarray(tree["depths"], dtype=np.int32)
    scores = np.ascontiguousarray(tree["scores"], dtype=np.float32)
    B, budget = parents.shape
    n_verify = np.zeros(B, dtype=np.int32)
    rank = np.zeros((B, budget), dtype=np.int32)
    rc = _load().oracle_verify_length(n_nodes.ctypes.data, parents.ctypes.data, depths.ctypes.data,
                                      scores.ctypes.data, int(B), int(budget), float(cost_fixed),
                                      float(cost_per_token), n_verify.ctypes.data, rank.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_verify_length: invalid arguments")
    return n_verify, rank

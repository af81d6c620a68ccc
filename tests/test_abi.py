"""The C ABI on a machine without a GPU: the library loads, exports every
function include/dt.h declares, and rejects invalid arguments on the host
before anything is enqueued (no compute call is made here)."""

import ctypes
import math
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dt.h")

bd = pytest.importorskip("draft_tree_construction_dt_amd.binding")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dt_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert _declared() == sorted(bd.EXPORTED)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", bd.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (dt_\w+)", out))
    assert set(_declared()) <= exported
    lib = ctypes.CDLL(bd.library_path())
    for name in _declared():
        assert hasattr(lib, name)


def test_header_compiles_as_c():
    src = '#include "dt.h"\nint main(void){dt_params p={0}; (void)p; return (int)dt_workspace_size(0);}\n'
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-I" + os.path.dirname(HEADER),
                        "-x", "c", "-"], input=src, text=True, capture_output=True)
    assert r.returncode == 0, r.stderr


def test_status_strings():
    for s in range(5):
        assert bd.dt_status_string(s).startswith("DT_")
    assert "unknown" in bd.dt_status_string(99)


FAKE = 0x100000          # a 16-byte aligned non-null address never dereferenced by validation


def _params(**kw):
    base = dict(B=2, V=1000, d=4, k=5, W=4, budget=10, dtype=bd.DT_DTYPE_BF16, mode=bd.DT_MODE_DART)
    base.update(kw)
    return bd.Params(**base)


def _call(params, ngram=None, logits=FAKE, out=None, workspace=True):
    p = params._c()
    p.ctx = FAKE
    if workspace:
        p.workspace = FAKE
        p.workspace_bytes = 1 << 30
    g = (ngram or bd.NGram())._c()
    o = out or bd._TreeOut(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    return bd._load().dt_build_tree(logits, ctypes.byref(g), ctypes.byref(p), ctypes.byref(o))


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), bd.DT_ERR_INVALID_ARG),
    (dict(d=0), bd.DT_ERR_INVALID_ARG),
    (dict(k=0), bd.DT_ERR_INVALID_ARG),
    (dict(k=1001), bd.DT_ERR_INVALID_ARG),
    (dict(W=0), bd.DT_ERR_INVALID_ARG),
    (dict(budget=0), bd.DT_ERR_INVALID_ARG),
    (dict(dtype=7), bd.DT_ERR_INVALID_ARG),
    (dict(mode=3), bd.DT_ERR_INVALID_ARG),
    (dict(sweep_chunks=-2), bd.DT_ERR_INVALID_ARG),
    (dict(k=33), bd.DT_ERR_UNSUPPORTED),
    (dict(W=65), bd.DT_ERR_UNSUPPORTED),
    (dict(W=64, k=17), bd.DT_ERR_UNSUPPORTED),
    (dict(d=33), bd.DT_ERR_UNSUPPORTED),
    (dict(budget=1025), bd.DT_ERR_UNSUPPORTED),
    (dict(V=1 << 26), bd.DT_ERR_UNSUPPORTED),
    (dict(sweep_chunks=200, k=5), bd.DT_ERR_UNSUPPORTED),
    (dict(mode=bd.DT_MODE_DARTREE), bd.DT_ERR_INVALID_ARG),             # E, F missing
    (dict(mode=bd.DT_MODE_DARTREE, E=FAKE, F=FAKE, R=6), bd.DT_ERR_UNSUPPORTED),
    (dict(mode=bd.DT_MODE_DARTREE, E=FAKE, F=FAKE, R=8, d=32, W=32, k=32),
     bd.DT_ERR_UNSUPPORTED),                                             # shared-memory plan over 160 KiB
])
def test_invalid_parameters(kw, status):
    assert _call(_params(**kw)) == status


class _Csr:
    """A CSR table descriptor with explicit pointers and entry count."""

    def __init__(self, row_ptr, col, nnz, min_logp=-math.inf):
        self.row_ptr, self.col, self.nnz, self.min_logp = row_ptr, col, nnz, min_logp

    def _c(self):
        g = bd.NGram(kind=bd.DT_NGRAM_CSR_BIGRAM, min_logp=self.min_logp)._c()
        g.row_ptr, g.col, g.nnz = self.row_ptr or None, self.col or None, self.nnz
        return g


def test_invalid_tables_and_buffers():
    P = _params()
    assert _call(P, bd.NGram(kind=9)) == bd.DT_ERR_INVALID_ARG
    assert _call(P, bd.NGram(kind=bd.DT_NGRAM_DENSE_BIGRAM)) == bd.DT_ERR_INVALID_ARG
    assert _call(P, _Csr(row_ptr=0, col=FAKE, nnz=5)) == bd.DT_ERR_INVALID_ARG
    assert _call(P, _Csr(row_ptr=FAKE, col=0, nnz=5)) == bd.DT_ERR_INVALID_ARG        # entries, no array
    assert _call(P, _Csr(row_ptr=FAKE, col=FAKE, nnz=-1)) == bd.DT_ERR_INVALID_ARG
    assert _call(P, _Csr(row_ptr=FAKE, col=FAKE, nnz=5, min_logp=-2.0)) == \
        bd.DT_ERR_INVALID_ARG                                            # finite threshold needs logp
    hk = dict(kind=bd.DT_NGRAM_HASH_TRIGRAM, keys=FAKE, succ=FAKE, S=16)
    assert _call(P, bd.NGram(cap=1000, **hk)) == bd.DT_ERR_INVALID_ARG      # not a power of two
    assert _call(P, bd.NGram(cap=1024, **dict(hk, S=65))) == bd.DT_ERR_UNSUPPORTED
    assert _call(P, bd.NGram(min_logp=math.nan)) == bd.DT_ERR_INVALID_ARG
    assert _call(P, logits=FAKE + 4) == bd.DT_ERR_INVALID_ARG               # misaligned logits
    assert _call(P, logits=0) == bd.DT_ERR_INVALID_ARG
    assert _call(P, out=bd._TreeOut(FAKE, 0, FAKE, FAKE, FAKE, FAKE)) == bd.DT_ERR_INVALID_ARG
    assert _call(P, workspace=False) == bd.DT_ERR_WORKSPACE


def test_workspace_size_depends_on_shape_only():
    a = bd.dt_workspace_size(_params(B=64, V=151936, d=8, k=10))
    b = bd.dt_workspace_size(_params(B=64, V=151936, d=8, k=10, W=2, budget=3))
    assert a == b > 0
    assert bd.dt_workspace_size(_params(k=0)) == 0
    assert bd.dt_workspace_size(_params(B=0)) == 0


def test_position_topk_validation():
    p = _params()._c()
    p.workspace = FAKE
    p.workspace_bytes = 1 << 30
    f = bd._load().dt_position_topk
    assert f(FAKE, ctypes.byref(p), 0, FAKE, FAKE) == bd.DT_ERR_INVALID_ARG
    p.k = 40
    assert f(FAKE, ctypes.byref(p), FAKE, FAKE, FAKE) == bd.DT_ERR_UNSUPPORTED
    p.k = 5
    p.workspace_bytes = 8
    assert f(FAKE, ctypes.byref(p), FAKE, FAKE, FAKE) == bd.DT_ERR_WORKSPACE


def test_ngram_update_validation():
    f = bd._load().dt_ngram_update
    hk = dict(kind=bd.DT_NGRAM_HASH_TRIGRAM, keys=FAKE, succ=FAKE, cap=1024, S=16)

    def call(ng, B=2, L=3, logp=0.0, ctx=FAKE, tok=FAKE, lens=FAKE):
        g = ng._c()
        return f(ctypes.byref(g), ctx, tok, lens, B, L, logp, 0, 0)

    assert f(None, FAKE, FAKE, FAKE, 1, 1, 0.0, 0, 0) == bd.DT_ERR_INVALID_ARG
    assert call(bd.NGram(**dict(hk, kind=bd.DT_NGRAM_CSR_BIGRAM))) == bd.DT_ERR_INVALID_ARG
    assert call(bd.NGram(**dict(hk, cap=1000))) == bd.DT_ERR_INVALID_ARG     # not a power of two
    assert call(bd.NGram(**dict(hk, cap=1))) == bd.DT_ERR_INVALID_ARG
    assert call(bd.NGram(**dict(hk, keys=FAKE + 4))) == bd.DT_ERR_INVALID_ARG  # keys not 8-byte aligned
    assert call(bd.NGram(**dict(hk, hash_logp=FAKE + 2))) == bd.DT_ERR_INVALID_ARG
    assert call(bd.NGram(**dict(hk, succ=0))) == bd.DT_ERR_INVALID_ARG
    assert call(bd.NGram(**dict(hk, S=0))) == bd.DT_ERR_UNSUPPORTED
    assert call(bd.NGram(**hk), B=-1) == bd.DT_ERR_INVALID_ARG
    assert call(bd.NGram(**hk), logp=math.nan) == bd.DT_ERR_INVALID_ARG
    assert call(bd.NGram(**hk), tok=0) == bd.DT_ERR_INVALID_ARG
    assert call(bd.NGram(**hk), B=0) == bd.DT_OK                             # nothing to add: no launch
    assert call(bd.NGram(**hk), L=0, tok=0) == bd.DT_OK


def test_verify_length_validation():
    f = bd._load().dt_verify_length
    t = bd._TreeOut(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)

    def call(B=2, budget=8, c0=1.0, c1=1.0, nv=FAKE, rk=FAKE, tree=t):
        return f(ctypes.byref(tree) if tree is not None else None, B, budget, c0, c1, nv, rk, 0)

    assert call(tree=None) == bd.DT_ERR_INVALID_ARG
    assert call(B=-1) == bd.DT_ERR_INVALID_ARG
    assert call(budget=0) == bd.DT_ERR_INVALID_ARG
    assert call(c0=0.0) == bd.DT_ERR_INVALID_ARG
    assert call(c0=math.inf) == bd.DT_ERR_INVALID_ARG
    assert call(c1=-0.5) == bd.DT_ERR_INVALID_ARG
    assert call(c1=math.nan) == bd.DT_ERR_INVALID_ARG
    assert call(nv=0) == bd.DT_ERR_INVALID_ARG
    assert call(tree=bd._TreeOut(FAKE, FAKE, 0, FAKE, FAKE, FAKE)) == bd.DT_ERR_INVALID_ARG
    assert call(budget=2048) == bd.DT_ERR_UNSUPPORTED
    assert call(B=0) == bd.DT_OK                                            # nothing to do: no launch


def _noalloc(params, **kw):
    p = params._c()
    p.ctx = FAKE
    g = bd.NGram()._c()
    o = bd._TreeOut(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    return bd._load().dt_build_tree_noalloc(kw.get("logits", FAKE), ctypes.byref(g), ctypes.byref(p), ctypes.byref(o))


def test_noalloc_validation_before_any_device_call():
    """dt_build_tree_noalloc validates like dt_build_tree, ignores the
    caller's workspace fields, and refuses parameters whose workspace would
    not fit its scratch array, all before touching a device (this machine
    has none)."""
    assert _noalloc(_params(B=-1)) == bd.DT_ERR_INVALID_ARG
    assert _noalloc(_params(k=33)) == bd.DT_ERR_UNSUPPORTED
    assert _noalloc(_params(), logits=FAKE + 4) == bd.DT_ERR_INVALID_ARG
    assert _noalloc(_params(B=0)) == bd.DT_OK
    big = _params(B=1024, V=1000, d=32, k=32, W=32, budget=1024)     # room for 30,753 trigram contexts each
    assert bd.dt_workspace_size(big) > bd.DT_NOALLOC_SCRATCH_BYTES
    assert _noalloc(big) == bd.DT_ERR_WORKSPACE

"""Seeded synthetic inputs shaped like the draft-tree workloads.

This module only draws random numbers and lays them out in the formats the
tree builder consumes: per-position draft logit rows, N-gram continuity tables
(dense bigram, CSR bigram, open-addressing trigram) and the two low-rank
embedding tables of the parent-conditioned score.  It contains no part of the
tree-construction arithmetic (no normaliser, no top-k, no expansion, pruning
or mask packing), so the CPU oracle and the HIP path can both be fed from it
without sharing any of the method.

Workloads (DART, arXiv 2601.19278, Fig. 3 "Continuity-Aware Tree Pruning";
DARTree, "Tree Construction"):

=======  ===  ======  ==  ==  ==  ======  =====================================
name      B     V     d   k   W  budget  notes
=======  ===  ======  ==  ==  ==  ======  =====================================
c1        1      64   4   3   4     16   fp32 N(0,2); dense bigram, keep logp>-4
c2        1   32000   8   8   8     60   bf16 N(0,3) + one token/position +8;
                                         CSR bigram, 32 uniform successors
c3        1  151936   8  10   8     64   bf16 N(0,3) + log Zipf(1.1) prior;
                                         trigram hash 2^22 slots, 16 successors
c4       64  151936   8  10   8     64   c3's generator per request, shared
                                         trigram table (the batched metric case)
c4L      64   32000   8   8   8     60   c2's logits per request, shared
                                         trigram table over 32000 ids
c5        8  151936  16  16  16    256   DARTree: bf16 N(0,3), E,F fp32 [V][64]
                                         ~N(0,0.1), no N-gram
=======  ===  ======  ==  ==  ==  ======  =====================================

A trailing ``p`` (``c2p``, ``c3p``, ``c4p``, ``c4Lp``) adds *coherence
planting*: per request and position i a few token ids P_i are drawn and their
logits raised by ``plant_boost``; the N-gram table is then edited so that
every planted context leading into position i lists all of P_i as
successors.  Uniform random tables almost never contain the drafted tokens,
so without planting the continuity filter leaves near-empty trees.  Planting
only needs the ids the generator itself drew; it never looks at which tokens
end up in a position's top-k.
"""

from __future__ import annotations

import dataclasses
import zlib
from dataclasses import dataclass, field
from functools import lru_cache
from typing import Optional

import numpy as np

# ---- enumerations shared by the C ABI (include/dt.h) and the oracle ----
NGRAM_NONE, NGRAM_DENSE_BIGRAM, NGRAM_CSR_BIGRAM, NGRAM_HASH_TRIGRAM = 0, 1, 2, 3
DTYPE_F32, DTYPE_BF16 = 0, 1
MODE_DART, MODE_DARTREE, MODE_DARTREE_FULL = 0, 1, 2
EMPTY_KEY = np.uint64(0xFFFFFFFFFFFFFFFF)

_M64 = np.uint64(0xFFFFFFFFFFFFFFFF)


# ----------------------------------------------------------------------------
# formats
# ----------------------------------------------------------------------------

def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  Inputs are finite or -inf.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    finite = (u & np.uint32(0x7F800000)) != np.uint32(0x7F800000)
    r = np.where(finite, u + rounding, u)
    return (r >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def splitmix64_finalizer(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output mixing function (Steele, Lea, Flood 2014; Vigna's
    public-domain reference), used as the hash of a trigram key."""
    z = np.asarray(z, dtype=np.uint64).copy()
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= np.uint64(0xBF58476D1CE4E5B9)
        z ^= z >> np.uint64(27)
        z *= np.uint64(0x94D049BB133111EB)
        z ^= z >> np.uint64(31)
    return z


def trigram_key(t2, t1) -> np.ndarray:
    """Key of the context (t_{-2}, t_{-1}): t_{-2} in the high word."""
    return (np.asarray(t2, dtype=np.uint64) << np.uint64(32)) | (
        np.asarray(t1, dtype=np.int64).astype(np.uint64) & np.uint64(0xFFFFFFFF))


# ----------------------------------------------------------------------------
# containers
# ----------------------------------------------------------------------------

@dataclass
class NGramTable:
    kind: int = NGRAM_NONE
    min_logp: float = float("-inf")
    dense_logp: Optional[np.ndarray] = None   # f32 [V][V]
    row_ptr: Optional[np.ndarray] = None      # i32 [V+1]
    col: Optional[np.ndarray] = None          # i32 [nnz], ascending per row
    csr_logp: Optional[np.ndarray] = None     # f32 [nnz]
    keys: Optional[np.ndarray] = None         # u64 [cap], EMPTY_KEY = free
    succ: Optional[np.ndarray] = None         # i32 [cap][S], -1 = no successor
    hash_logp: Optional[np.ndarray] = None    # f32 [cap][S]
    cap: int = 0
    S: int = 0


@dataclass
class Problem:
    name: str
    seed: int
    B: int
    V: int
    d: int
    k: int
    W: int
    budget: int
    dtype: int
    mode: int
    logits: np.ndarray            # uint16 bf16 bits or float32, [B][d][V]
    ctx: np.ndarray               # int32 [B][2]: (t_{-2}, t_{-1}); ctx[b][1] is the root
    ngram: NGramTable
    E: Optional[np.ndarray] = None  # f32 [V][R]
    F: Optional[np.ndarray] = None  # f32 [V][R]
    R: int = 0
    planted: list = field(default_factory=list)  # per request: list of d id arrays

    @property
    def logits_f32(self) -> np.ndarray:
        if self.dtype == DTYPE_BF16:
            return f32_from_bf16_bits(self.logits)
        return self.logits

    @property
    def mask_words(self) -> int:
        return (self.budget + 31) // 32

    def logit_bytes(self) -> int:
        return int(self.logits.nbytes)


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    V: int
    d: int
    k: int
    W: int
    budget: int
    dtype: int = DTYPE_BF16
    mode: int = MODE_DART
    sigma: float = 3.0
    zipf_prior: Optional[float] = None   # exponent of a Zipf prior added to logits
    plus8: bool = False                  # one uniform token per position raised by +8
    ngram: int = NGRAM_NONE
    min_logp: float = float("-inf")
    ngram_ids: str = "uniform"           # "uniform" or "zipf" ids in N-gram tables
    zipf_s: float = 1.1
    csr_deg: int = 32
    hash_cap_log2: int = 22
    hash_keys_log2: int = 21
    hash_S: int = 16
    plant: int = 0                       # max planted ids per position (0 = literal)
    plant_boost: float = 24.0
    R: int = 64
    ef_sigma: float = 0.1


_BASE = {
    "c1": Config("c1", B=1, V=64, d=4, k=3, W=4, budget=16, dtype=DTYPE_F32, sigma=2.0,
                 ngram=NGRAM_DENSE_BIGRAM, min_logp=-4.0),
    "c2": Config("c2", B=1, V=32000, d=8, k=8, W=8, budget=60, plus8=True,
                 ngram=NGRAM_CSR_BIGRAM, ngram_ids="uniform"),
    "c3": Config("c3", B=1, V=151936, d=8, k=10, W=8, budget=64, zipf_prior=1.1,
                 ngram=NGRAM_HASH_TRIGRAM, ngram_ids="zipf"),
    "c4": Config("c4", B=64, V=151936, d=8, k=10, W=8, budget=64, zipf_prior=1.1,
                 ngram=NGRAM_HASH_TRIGRAM, ngram_ids="zipf"),
    "c4L": Config("c4L", B=64, V=32000, d=8, k=8, W=8, budget=60, plus8=True,
                  ngram=NGRAM_HASH_TRIGRAM, ngram_ids="uniform"),
    "c5": Config("c5", B=8, V=151936, d=16, k=16, W=16, budget=256, mode=MODE_DARTREE),
    # c5 with every node proposing its own W tokens from the whole vocabulary
    "c5f": Config("c5f", B=8, V=151936, d=16, k=16, W=16, budget=256, mode=MODE_DARTREE_FULL),
}

CONFIGS = dict(_BASE)
for _n in ("c2", "c3", "c4", "c4L"):
    CONFIGS[_n + "p"] = dataclasses.replace(_BASE[_n], name=_n + "p", plant=6)


def config(name: str, **overrides) -> Config:
    cfg = CONFIGS[name]
    if overrides:
        cfg = dataclasses.replace(cfg, **overrides)
    return cfg


# ----------------------------------------------------------------------------
# random building blocks
# ----------------------------------------------------------------------------

def _zipf_cdf(V: int, s: float) -> np.ndarray:
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    c = np.cumsum(w)
    return c / c[-1]


def _zipf_log_pmf(V: int, s: float) -> np.ndarray:
    w = np.arange(1, V + 1, dtype=np.float64)
    lw = -s * np.log(w)
    return lw - np.log(np.sum(np.exp(lw)))


class _Ids:
    """Draws token ids, uniform or Zipf(s) with id 0 the most frequent."""

    def __init__(self, V: int, kind: str, s: float):
        self.V, self.kind = V, kind
        self.cdf = _zipf_cdf(V, s) if kind == "zipf" else None

    def draw(self, rng: np.random.Generator, size) -> np.ndarray:
        if self.kind == "zipf":
            u = rng.random(size)
            return np.minimum(np.searchsorted(self.cdf, u, side="right"), self.V - 1).astype(np.int64)
        return rng.integers(0, self.V, size=size, dtype=np.int64)

    def draw_distinct(self, rng: np.random.Generator, n: int) -> np.ndarray:
        out: list = []
        seen = set()
        while len(out) < n:
            for v in self.draw(rng, 2 * n).tolist():
                if v not in seen:
                    seen.add(v)
                    out.append(v)
                    if len(out) == n:
                        break
        return np.array(out, dtype=np.int64)


def _distinct_rows(rng: np.random.Generator, ids: _Ids, n: int, S: int) -> np.ndarray:
    """n rows of S distinct ids each (ascending within a row): duplicates are
    redrawn until none remain."""
    rows = np.sort(ids.draw(rng, (n, S)), axis=1)
    todo = np.arange(n)
    while todo.size:
        sub = rows[todo]
        dup = np.zeros_like(sub, dtype=bool)
        dup[:, 1:] = sub[:, 1:] == sub[:, :-1]
        bad = dup.any(axis=1)
        if not bad.any():
            break
        todo = todo[bad]
        sub, dup = sub[bad], dup[bad]
        sub[dup] = ids.draw(rng, int(dup.sum()))
        rows[todo] = np.sort(sub, axis=1)
    return rows


def _log_softmax_rows(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.float64)
    m = z.max(axis=1, keepdims=True)
    return z - (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))


# ----------------------------------------------------------------------------
# open-addressing table construction (linear probing from splitmix64 & (cap-1))
# ----------------------------------------------------------------------------

def hash_place(keys: np.ndarray, cap: int) -> tuple:
    """Place distinct keys into a table of ``cap`` slots by linear probing.

    Rounds of first-come-first-served: every pending key targets its current
    probe slot; the lowest-numbered key wins a free slot, everyone else moves
    one slot on.  A key only moves past slots that are occupied, which is the
    linear-probing invariant lookups rely on.
    """
    n = keys.size
    assert cap & (cap - 1) == 0 and n < cap
    mask = np.uint64(cap - 1)
    table = np.full(cap, EMPTY_KEY, dtype=np.uint64)
    slot_of = np.full(n, -1, dtype=np.int64)
    pos = (splitmix64_finalizer(keys) & mask).astype(np.int64)
    pending = np.arange(n)
    while pending.size:
        p = pos[pending]
        free = table[p] == EMPTY_KEY
        cand, tp = pending[free], p[free]
        if cand.size:
            uniq, first = np.unique(tp, return_index=True)
            winners = cand[first]
            table[uniq] = keys[winners]
            slot_of[winners] = uniq
            won = np.zeros(n, dtype=bool)
            won[winners] = True
            pending = pending[~won[pending]]
        pos[pending] = (pos[pending] + 1) & (cap - 1)
    return table, slot_of


def hash_find_or_insert(table: np.ndarray, key: int, cap: int) -> tuple:
    """Return (slot, inserted) for one key, inserting it if absent."""
    key = np.uint64(key)
    s = int(splitmix64_finalizer(np.array([key]))[0] & np.uint64(cap - 1))
    for _ in range(cap):
        cur = table[s]
        if cur == key:
            return s, False
        if cur == EMPTY_KEY:
            table[s] = key
            return s, True
        s = (s + 1) & (cap - 1)
    raise RuntimeError("hash table full")


# ----------------------------------------------------------------------------
# tables
# ----------------------------------------------------------------------------

def _dense_bigram(rng, V: int) -> np.ndarray:
    return _log_softmax_rows(rng.standard_normal((V, V))).astype(np.float32)


def _csr_bigram(rng, V: int, deg: int, ids: _Ids):
    col = _distinct_rows(rng, ids, V, deg)            # sorted per row
    logp = _log_softmax_rows(rng.standard_normal((V, deg))).astype(np.float32)
    row_ptr = (np.arange(V + 1, dtype=np.int64) * deg).astype(np.int32)
    return row_ptr, col.astype(np.int32).ravel(), logp.ravel()


def _hash_trigram(rng, cfg: Config, ids: _Ids):
    cap = 1 << cfg.hash_cap_log2
    n = 1 << cfg.hash_keys_log2
    S = cfg.hash_S
    got = np.empty(0, dtype=np.uint64)
    draw = max(n, 1024)
    while got.size < n:
        a = ids.draw(rng, 3 * draw)
        b = ids.draw(rng, 3 * draw)
        k = trigram_key(a, b)
        allk = np.concatenate([got, k])
        _, idx = np.unique(allk, return_index=True)
        got = allk[np.sort(idx)]
        draw *= 2
    keys = got[:n]
    succ_rows = _distinct_rows(rng, ids, n, S)
    perm = rng.permuted(succ_rows, axis=1)           # successor order carries no meaning
    logp_rows = _log_softmax_rows(rng.standard_normal((n, S))).astype(np.float32)
    table, slot_of = hash_place(keys, cap)
    succ = np.full((cap, S), -1, dtype=np.int32)
    logp = np.zeros((cap, S), dtype=np.float32)
    succ[slot_of] = perm.astype(np.int32)
    logp[slot_of] = logp_rows
    return table, succ, logp, cap, S


# ----------------------------------------------------------------------------
# coherence planting (edits tables so planted contexts list the planted ids)
# ----------------------------------------------------------------------------

class _RowPlanter:
    """Puts ids into fixed-length successor rows; planted entries occupy the
    lowest slots of a row, earlier plantings are never overwritten."""

    def __init__(self, succ: np.ndarray, logp: np.ndarray):
        self.succ, self.logp = succ, logp
        self.n_planted: dict = {}

    def plant(self, row: int, tok: int) -> None:
        r = self.succ[row]
        n = self.n_planted.get(row, 0)
        hit = np.nonzero(r == tok)[0]
        if hit.size:
            q = int(hit[0])
            if q < n:
                return
            if q != n:
                r[[n, q]] = r[[q, n]]
                lp = self.logp[row]
                lp[[n, q]] = lp[[q, n]]
            self.n_planted[row] = n + 1
            return
        if n >= r.size:
            return                       # row full of planted ids: dropped
        r[n] = tok
        self.n_planted[row] = n + 1


def _plant_csr(ng: NGramTable, plans: list) -> None:
    deg = int(ng.row_ptr[1] - ng.row_ptr[0])
    succ = ng.col.reshape(-1, deg)
    logp = ng.csr_logp.reshape(-1, deg)
    pl = _RowPlanter(succ, logp)
    touched = set()
    for ctx, P in plans:
        A = [np.array([ctx[1]])] + [P[i] for i in range(len(P))]
        for i in range(len(P)):
            for a1 in A[i].tolist():
                for c in P[i].tolist():
                    pl.plant(a1, c)
                    touched.add(a1)
    for row in touched:                  # keep every row ascending
        o = np.argsort(succ[row], kind="stable")
        succ[row] = succ[row][o]
        logp[row] = logp[row][o]


def _plant_hash(ng: NGramTable, plans: list) -> None:
    pl = _RowPlanter(ng.succ, ng.hash_logp)
    for ctx, P in plans:
        A = [np.array([ctx[0]]), np.array([ctx[1]])] + [P[i] for i in range(len(P))]
        for i in range(len(P)):
            for a2 in A[i].tolist():
                for a1 in A[i + 1].tolist():
                    slot, new = hash_find_or_insert(ng.keys, int(trigram_key(a2, a1)), ng.cap)
                    if new:
                        ng.succ[slot, :] = -1
                        ng.hash_logp[slot, :] = -1.0
                    for c in P[i].tolist():
                        pl.plant(slot, c)


# ----------------------------------------------------------------------------
# problem generation
# ----------------------------------------------------------------------------

def _streams(cfg: Config, seed: int):
    """Independent streams: one per request (request b's stream does not
    depend on B), one for the table, one for the embedding tables."""
    root = np.random.SeedSequence([int(seed), zlib.crc32(cfg.name.encode())])
    req_root, tab, ef = root.spawn(3)
    return req_root.spawn(cfg.B), tab, ef


def make_logits(cfg: Config, seed: int, ids_for_plant: Optional[_Ids] = None):
    """Per-request logits [B][d][V] (+ context tokens and planted ids)."""
    req_ss, _, _ = _streams(cfg, seed)
    prior = _zipf_log_pmf(cfg.V, cfg.zipf_s).astype(np.float32) if cfg.zipf_prior else None
    ids = ids_for_plant or _Ids(cfg.V, cfg.ngram_ids, cfg.zipf_s)
    out = np.empty((cfg.B, cfg.d, cfg.V),
                   dtype=np.uint16 if cfg.dtype == DTYPE_BF16 else np.float32)
    ctx = np.empty((cfg.B, 2), dtype=np.int32)
    planted = []
    for b in range(cfg.B):
        rng = np.random.default_rng(req_ss[b])
        x = (rng.standard_normal((cfg.d, cfg.V), dtype=np.float32) * np.float32(cfg.sigma))
        if prior is not None:
            x += prior[None, :]
        if cfg.plus8:
            pid = rng.integers(0, cfg.V, size=cfg.d)
            x[np.arange(cfg.d), pid] += np.float32(8.0)
        ctx[b] = rng.integers(0, cfg.V, size=2)
        P = []
        if cfg.plant:
            lo = max(1, cfg.plant - 2)
            for i in range(cfg.d):
                m = int(rng.integers(lo, cfg.plant + 1))
                p = ids.draw_distinct(rng, m)
                x[i, p] += np.float32(cfg.plant_boost)
                P.append(p)
        planted.append(P)
        out[b] = bf16_bits_from_f32(x) if cfg.dtype == DTYPE_BF16 else x
    return out, ctx, planted


@lru_cache(maxsize=4)
def _random_table(cfg: Config, seed: int) -> NGramTable:
    _, tab_ss, _ = _streams(cfg, seed)
    rng = np.random.default_rng(tab_ss)
    ids = _Ids(cfg.V, cfg.ngram_ids, cfg.zipf_s)
    if cfg.ngram == NGRAM_NONE:
        return NGramTable(NGRAM_NONE, cfg.min_logp)
    if cfg.ngram == NGRAM_DENSE_BIGRAM:
        return NGramTable(NGRAM_DENSE_BIGRAM, cfg.min_logp, dense_logp=_dense_bigram(rng, cfg.V))
    if cfg.ngram == NGRAM_CSR_BIGRAM:
        rp, col, lp = _csr_bigram(rng, cfg.V, cfg.csr_deg, ids)
        return NGramTable(NGRAM_CSR_BIGRAM, cfg.min_logp, row_ptr=rp, col=col, csr_logp=lp)
    keys, succ, logp, cap, S = _hash_trigram(rng, cfg, ids)
    return NGramTable(NGRAM_HASH_TRIGRAM, cfg.min_logp, keys=keys, succ=succ,
                      hash_logp=logp, cap=cap, S=S)


def _copy_table(t: NGramTable) -> NGramTable:
    return NGramTable(**{f.name: (getattr(t, f.name).copy() if isinstance(getattr(t, f.name), np.ndarray)
                                  else getattr(t, f.name)) for f in dataclasses.fields(t)})


def make_problem(name: str, seed: int = 0, **overrides) -> Problem:
    """Build the seeded problem ``name`` (see the module docstring)."""
    cfg = config(name, **overrides)
    logits, ctx, planted = make_logits(cfg, seed)
    # planted variants share the literal table's random part, then edit a copy
    base_cfg = dataclasses.replace(cfg, plant=0, name=cfg.name.rstrip("p") if cfg.plant else cfg.name)
    table = _random_table(base_cfg, seed)
    if cfg.plant and cfg.ngram in (NGRAM_CSR_BIGRAM, NGRAM_HASH_TRIGRAM):
        table = _copy_table(table)
        plans = [(ctx[b], planted[b]) for b in range(cfg.B)]
        if cfg.ngram == NGRAM_CSR_BIGRAM:
            _plant_csr(table, plans)
        else:
            _plant_hash(table, plans)
    E = F = None
    R = 0
    if cfg.mode != MODE_DART:
        _, _, ef_ss = _streams(cfg, seed)
        rng = np.random.default_rng(ef_ss)
        E = (rng.standard_normal((cfg.V, cfg.R), dtype=np.float32) * np.float32(cfg.ef_sigma))
        F = (rng.standard_normal((cfg.V, cfg.R), dtype=np.float32) * np.float32(cfg.ef_sigma))
        R = cfg.R
    return Problem(name=cfg.name, seed=seed, B=cfg.B, V=cfg.V, d=cfg.d, k=cfg.k, W=cfg.W,
                   budget=cfg.budget, dtype=cfg.dtype, mode=cfg.mode, logits=logits, ctx=ctx,
                   ngram=table, E=E, F=F, R=R, planted=planted)


def random_problem(rng: np.random.Generator, *, B: int, V: int, d: int, k: int, W: int,
                   budget: int, dtype: int = DTYPE_F32, mode: int = MODE_DART,
                   ngram: int = NGRAM_NONE, min_logp: float = float("-inf"),
                   sigma: float = 2.0, R: int = 8, hash_cap: int = 256, hash_S: int = 4,
                   csr_deg: int = 3, density: float = 0.5, neg_inf_frac: float = 0.0,
                   integer_logits: bool = False) -> Problem:
    """Small arbitrary problems for property tests and brute force.

    ``density`` is the fraction of (context, token) pairs the table admits;
    ``neg_inf_frac`` sets that fraction of logits to -inf; ``integer_logits``
    draws small integers, which makes exact score ties common.
    """
    if integer_logits:
        x = rng.integers(-3, 4, size=(B, d, V)).astype(np.float32)
    else:
        x = (rng.standard_normal((B, d, V)) * sigma).astype(np.float32)
    if neg_inf_frac > 0:
        x[rng.random(x.shape) < neg_inf_frac] = -np.inf
    logits = bf16_bits_from_f32(x) if dtype == DTYPE_BF16 else x
    ctx = rng.integers(0, V, size=(B, 2)).astype(np.int32)
    ng = NGramTable(ngram, min_logp)
    if ngram == NGRAM_DENSE_BIGRAM:
        t = _log_softmax_rows(rng.standard_normal((V, V))).astype(np.float32)
        t[rng.random((V, V)) >= density] = -np.inf
        ng.dense_logp = t
    elif ngram == NGRAM_CSR_BIGRAM:
        deg = min(csr_deg, V)
        rows = [np.sort(rng.choice(V, size=int(rng.integers(0, deg + 1)), replace=False))
                for _ in range(V)]
        rp = np.zeros(V + 1, dtype=np.int64)
        rp[1:] = np.cumsum([r.size for r in rows])
        ng.row_ptr = rp.astype(np.int32)
        ng.col = (np.concatenate(rows) if rp[-1] else np.zeros(0)).astype(np.int32)
        ng.csr_logp = (rng.standard_normal(int(rp[-1])) - 1.0).astype(np.float32)
    elif ngram == NGRAM_HASH_TRIGRAM:
        S = hash_S
        pairs = [(a, b) for a in range(V) for b in range(V) if rng.random() < density]
        pairs = pairs[: hash_cap // 2]
        keys = np.array([int(trigram_key(a, b)) for a, b in pairs], dtype=np.uint64)
        table, slot_of = hash_place(keys, hash_cap) if keys.size else (
            np.full(hash_cap, EMPTY_KEY, dtype=np.uint64), np.zeros(0, dtype=np.int64))
        succ = np.full((hash_cap, S), -1, dtype=np.int32)
        logp = np.zeros((hash_cap, S), dtype=np.float32)
        for i in range(len(pairs)):
            m = int(rng.integers(0, min(S, V) + 1))
            succ[slot_of[i], :m] = rng.choice(V, size=m, replace=False)
            logp[slot_of[i], :m] = rng.standard_normal(m) - 1.0
        ng.keys, ng.succ, ng.hash_logp, ng.cap, ng.S = table, succ, logp, hash_cap, S
    E = F = None
    if mode != MODE_DART:
        E = (rng.standard_normal((V, R)) * 0.5).astype(np.float32)
        F = (rng.standard_normal((V, R)) * 0.5).astype(np.float32)
    return Problem(name="random", seed=-1, B=B, V=V, d=d, k=k, W=W, budget=budget,
                   dtype=dtype, mode=mode, logits=logits, ctx=ctx, ngram=ng, E=E, F=F,
                   R=R if mode != MODE_DART else 0)

"""Independent checks used by the tests.

Nothing here is shared with the oracle or the HIP library: continuity is
re-derived from the table arrays without the hash function, scores are
re-summed from per-position normalisers computed with numpy, and the checks
below only restate what the pages fix about a draft tree:

* DART (arXiv 2601.19278) Fig. 3: depth-t tokens come from position t-1's
  own top candidates; an N-gram keeps expansions continuous; the tree is
  verified with tree attention, so each node's mask row is its ancestor set.
* DARTree (llmdb "Tree Construction"): at most W nodes survive per depth,
  chosen across the whole frontier.
"""

from __future__ import annotations

import itertools
import math

import numpy as np

NGRAM_NONE, NGRAM_DENSE_BIGRAM, NGRAM_CSR_BIGRAM, NGRAM_HASH_TRIGRAM = 0, 1, 2, 3
MODE_DART, MODE_DARTREE, MODE_DARTREE_FULL = 0, 1, 2


def logits_f64(p) -> np.ndarray:
    if p.logits.dtype == np.uint16:
        return (p.logits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return p.logits.astype(np.float64)


def lse_np(row: np.ndarray) -> float:
    return float(np.logaddexp.reduce(row.astype(np.float64)))


def topk_np(row: np.ndarray, k: int) -> np.ndarray:
    return np.argsort(-row, kind="stable")[:k]


class Continuity:
    """N-gram membership from the raw table arrays (no hashing: the trigram
    keys are indexed by a dict built from the occupied slots)."""

    def __init__(self, ng, V: int):
        self.ng, self.V = ng, V
        self.kind = int(ng.kind)
        self.tau = float(ng.min_logp)
        if self.kind == NGRAM_HASH_TRIGRAM:
            keys = np.asarray(ng.keys, dtype=np.uint64)
            occ = np.nonzero(keys != np.uint64(0xFFFFFFFFFFFFFFFF))[0]
            self.slot = dict(zip(keys[occ].tolist(), occ.tolist()))

    def __call__(self, t2: int, t1: int, c: int) -> bool:
        ng, tau = self.ng, self.tau
        if self.kind == NGRAM_NONE:
            return True
        if self.kind == NGRAM_DENSE_BIGRAM:
            return float(ng.dense_logp[t1, c]) > tau
        if self.kind == NGRAM_CSR_BIGRAM:
            lo, hi = int(ng.row_ptr[t1]), int(ng.row_ptr[t1 + 1])
            hit = np.nonzero(ng.col[lo:hi] == c)[0]
            if hit.size == 0:
                return False
            return tau == -math.inf or ng.csr_logp is None or float(ng.csr_logp[lo + hit[0]]) > tau
        key = (int(t2) << 32) | (int(t1) & 0xFFFFFFFF)
        s = self.slot.get(key)
        if s is None:
            return False
        hit = np.nonzero(ng.succ[s] == c)[0]
        if hit.size == 0:
            return False
        return tau == -math.inf or ng.hash_logp is None or float(ng.hash_logp[s, hit[0]]) > tau


def mask_closure(parents: np.ndarray, n: int, budget: int) -> np.ndarray:
    """Warshall transitive closure of the parent relation plus the identity,
    packed LSB-first into ceil(budget/32) words per row."""
    words = (budget + 31) // 32
    reach = np.zeros((budget, budget), dtype=bool)
    for i in range(n):
        reach[i, i] = True
        if parents[i] >= 0:
            reach[i, parents[i]] = True
    for m in range(n):
        reach[:n, :n] |= reach[:n, m:m + 1] & reach[m:m + 1, :n]
    out = np.zeros((budget, words), dtype=np.uint32)
    for i in range(n):
        for j in np.nonzero(reach[i])[0]:
            out[i, j >> 5] |= np.uint32(1 << (j & 31))
    return out


def paths_of(tree: dict, b: int) -> dict:
    """token path (tuple) -> index, for request b of a tree output."""
    n = int(tree["n_nodes"][b])
    tok, par = tree["tokens"][b], tree["parents"][b]
    out = {}
    path = {}
    for i in range(n):
        pth = (path[par[i]] if par[i] >= 0 else ()) + (int(tok[i]),)
        path[i] = pth
        out[pth] = i
    return out


def check_invariants(p, tree: dict, *, W=None, budget=None, score_tol=1e-4, lse=None, topk=None):
    """Everything a correct tree satisfies, whatever the tie-breaks.

    Returns the list of violated properties (empty when all hold)."""
    W = p.W if W is None else W
    budget = p.budget if budget is None else budget
    X = logits_f64(p)
    cont = Continuity(p.ngram, p.V)
    errs = []
    for b in range(p.B):
        if lse is None:
            L = [lse_np(X[b, i]) for i in range(p.d)]
        else:
            L = lse[b]
        if p.mode == MODE_DARTREE_FULL:
            T = None                       # children come from the whole vocabulary
        elif topk is None:
            T = [set(topk_np(X[b, i], p.k).tolist()) for i in range(p.d)]
        else:
            T = [set(topk[b][i]) for i in range(p.d)]
        n = int(tree["n_nodes"][b])
        tok, par, dep = tree["tokens"][b], tree["parents"][b], tree["depths"][b]
        sc = tree["scores"][b]
        if not 0 <= n <= budget:
            errs.append(f"b{b}: n_nodes {n} outside [0,{budget}]")
            continue
        per_depth = {}
        seen = set()
        S = {}
        for i in range(n):
            pi = int(par[i])
            if not (pi == -1 or 0 <= pi < i):
                errs.append(f"b{b} n{i}: parent {pi} not earlier")
                continue
            want_depth = 1 if pi < 0 else int(dep[pi]) + 1
            if int(dep[i]) != want_depth:
                errs.append(f"b{b} n{i}: depth {dep[i]} != {want_depth}")
            t = int(dep[i])
            if not 1 <= t <= p.d:
                errs.append(f"b{b} n{i}: depth {t} out of range")
                continue
            if i > 0 and int(dep[i]) < int(dep[i - 1]):
                errs.append(f"b{b} n{i}: not in BFS order")
            c = int(tok[i])
            if p.mode != MODE_DARTREE_FULL and c not in T[t - 1]:
                errs.append(f"b{b} n{i}: token {c} not in position {t - 1}'s top-k")
            x = X[b, t - 1, c]
            if x == -math.inf:
                errs.append(f"b{b} n{i}: zero-probability token drafted")
            ptok = int(p.ctx[b, 1]) if pi < 0 else int(tok[pi])
            pprev = int(p.ctx[b, 0]) if pi < 0 else (int(p.ctx[b, 1]) if par[pi] < 0 else int(tok[par[pi]]))
            if not cont(pprev, ptok, c):
                errs.append(f"b{b} n{i}: continuity broken ({pprev},{ptok})->{c}")
            if (pi, c) in seen:
                errs.append(f"b{b} n{i}: duplicate child")
            seen.add((pi, c))
            per_depth[t] = per_depth.get(t, 0) + 1
            g = 0.0
            if p.mode != MODE_DART:
                g = float(np.dot(p.E[ptok].astype(np.float64), p.F[c].astype(np.float64)))
            S[i] = (S[pi] if pi >= 0 else 0.0) + (x - L[t - 1]) + g
            if abs(float(sc[i]) - S[i]) > score_tol:
                errs.append(f"b{b} n{i}: score {sc[i]} vs {S[i]}")
        for t, cnt in per_depth.items():
            if cnt > W:
                errs.append(f"b{b}: depth {t} has {cnt} > W nodes")
        want = mask_closure(np.asarray(par[:n]), n, budget)
        if not np.array_equal(tree["mask"][b], want):
            errs.append(f"b{b}: mask is not the ancestor closure")
        if n < budget:
            if (np.any(tok[n:] != -1) or np.any(par[n:] != -1) or np.any(dep[n:] != 0)
                    or not np.all(np.isneginf(sc[n:]))):
                errs.append(f"b{b}: padding rows not cleared")
    return errs


# ---------------------------------------------------------------------------
# brute force over all paths (tiny V, d)
# ---------------------------------------------------------------------------

def all_valid_paths(p, b: int):
    """Every token path of length 1..d whose edges are all admissible:
    child in its position's top-k, finite logit, continuity with its two
    predecessors (root context included).  Returns {path: (S, Rk)} with
    S and Rk summed in float64 in path order."""
    X = logits_f64(p)
    cont = Continuity(p.ngram, p.V)
    L = [lse_np(X[b, i]) for i in range(p.d)]
    full = p.mode == MODE_DARTREE_FULL
    T = None if full else [set(topk_np(X[b, i], p.k).tolist()) for i in range(p.d)]
    out = {}
    frontier = {(): (0.0, 0.0)}
    ctx2, ctx1 = int(p.ctx[b, 0]), int(p.ctx[b, 1])
    for t in range(1, p.d + 1):
        nxt = {}
        for path, (s, rk) in frontier.items():
            ptok = path[-1] if path else ctx1
            pprev = (path[-2] if len(path) >= 2 else ctx1) if path else ctx2
            for c in range(p.V):
                x = X[b, t - 1, c]
                if (not full and c not in T[t - 1]) or x == -math.inf or not cont(pprev, ptok, c):
                    continue
                g = 0.0
                if p.mode != MODE_DART:
                    g = float(np.dot(p.E[ptok].astype(np.float64), p.F[c].astype(np.float64)))
                nxt[path + (c,)] = ((s + (x - L[t - 1])) + g, (rk + x) + g)
        out.update(nxt)
        frontier = nxt
    return out


def sketch_build(p, b: int, W: int):
    """The DARTree page's implementation sketch restated with paths as tuples:
    every frontier path proposes its position's top-W tokens, all candidates
    are scored in one batch by their cumulative score, and the best ``width``
    are kept across the whole frontier.  The sketch's unstable argsort is
    replaced by a stable order (score desc, token asc, parent position asc).
    Returns {depth: [paths]} as the sketch does (no N-gram, no budget)."""
    X = logits_f64(p)
    ctx1 = int(p.ctx[b, 1])
    nodes = {0: [()]}
    score = {(): 0.0}
    full = p.mode == MODE_DARTREE_FULL
    for t in range(1, p.d + 1):
        shared = None if full else topk_np(X[b, t - 1], p.k).tolist()
        cands = []
        for r, path in enumerate(nodes[t - 1]):
            ptok = path[-1] if path else ctx1
            if full:
                # batch_propose(path, num_drafts=W): this path's own W best
                # tokens under x + E[ptok] . F[v] over the whole vocabulary
                g_all = p.F.astype(np.float64) @ p.E[ptok].astype(np.float64)
                cond = X[b, t - 1] + g_all
                order = np.lexsort((np.arange(p.V), -cond))
                props = [int(v) for v in order if X[b, t - 1, v] != -math.inf][:W]
            else:
                props = shared
            for tok in props:
                x = X[b, t - 1, tok]
                if x == -math.inf:
                    continue
                g = 0.0
                if p.mode != MODE_DART:
                    g = float(np.dot(p.E[ptok].astype(np.float64), p.F[tok].astype(np.float64)))
                cands.append(((score[path] + x) + g, tok, r, path + (tok,)))
        cands.sort(key=lambda c: (-c[0], c[1], c[2]))
        nodes[t] = []
        for rk, tok, r, pth in cands[:W]:
            score[pth] = rk
            nodes[t].append(pth)
        if not nodes[t]:
            break
    return nodes


def has_near_ties(values, tol: float) -> bool:
    v = np.sort(np.asarray(list(values), dtype=np.float64))
    return bool(v.size > 1 and np.min(np.diff(v)) < tol)


def product_count(k: int, d: int) -> int:
    return sum(k ** t for t in range(1, d + 1))


__all__ = [n for n in dir() if not n.startswith("_")] + ["itertools"]

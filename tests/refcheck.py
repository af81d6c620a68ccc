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


def tree_paths(tree: dict, b: int) -> list:
    """Token path (tuple) of every node of request b, in node order."""
    n = int(tree["n_nodes"][b])
    tok, par = tree["tokens"][b], tree["parents"][b]
    out = []
    for i in range(n):
        out.append((out[int(par[i])] if par[i] >= 0 else ()) + (int(tok[i]),))
    return out


class PathScorer:
    """fp64 keys of token paths of request b, summed from the logits in path
    order, parent term first: Rk = (Rk_parent + x) + g (the lse-free key the
    per-depth selection ranks) and S = (S_parent + (x - lse)) + g (the
    cumulative log-score the verification budget ranks).  g = E[parent token]
    . F[child] outside DART mode (the DARTree page's P_AR equation, low-rank
    stand-in)."""

    def __init__(self, p, b: int):
        self.p, self.b = p, b
        self.X = logits_f64(p)[b]
        self.L = [lse_np(self.X[i]) for i in range(p.d)]
        self.ctx = (int(p.ctx[b, 0]), int(p.ctx[b, 1]))
        self.memo = {(): (0.0, 0.0)}
        if p.mode != MODE_DART:
            self.E = p.E.astype(np.float64)
            self.F = p.F.astype(np.float64)

    def parent_tokens(self, path):
        """(grandparent token, parent token) of a child appended to ``path``."""
        if not path:
            return self.ctx
        if len(path) == 1:
            return self.ctx[1], path[0]
        return path[-2], path[-1]

    def g(self, ptok: int, c: int) -> float:
        if self.p.mode == MODE_DART:
            return 0.0
        return float(np.dot(self.E[ptok], self.F[c]))

    def keys(self, path):
        """(Rk, S) of a path."""
        got = self.memo.get(path)
        if got is None:
            rk_p, s_p = self.keys(path[:-1])
            t, c = len(path), path[-1]
            x = self.X[t - 1, c]
            g = self.g(self.parent_tokens(path[:-1])[1], c)
            got = ((rk_p + x) + g, (s_p + (x - self.L[t - 1])) + g)
            self.memo[path] = got
        return got


def depth_candidates(p, sc: PathScorer, cont, frontier: list, t: int) -> list:
    """Every admissible child of the depth t-1 frontier (a list of paths in
    rank order), per parent rank r: (child tokens ascending, their Rk).
    Children come from position t-1's top-k (DART Fig. 3), or from the whole
    vocabulary in DARTREE_FULL mode, with a finite logit and N-gram
    continuity after the parent's context."""
    X = sc.X[t - 1]
    full = p.mode == MODE_DARTREE_FULL
    finite = np.nonzero(np.isfinite(X))[0]
    pool = finite if full else np.sort(np.array([c for c in topk_np(X, p.k) if np.isfinite(X[c])], dtype=np.int64))
    out = []
    for path in frontier:
        a2, a1 = sc.parent_tokens(path)
        if cont.kind != NGRAM_NONE:
            toks = np.array([c for c in pool.tolist() if cont(a2, a1, c)], dtype=np.int64)
        else:
            toks = pool
        rk_p = sc.keys(path)[0]
        if p.mode == MODE_DART:
            g = np.zeros(len(toks))
        elif 0 <= a1 < p.V:
            g = sc.F[toks] @ sc.E[a1]
        else:
            g = np.zeros(len(toks))
        out.append((toks, (rk_p + X[toks]) + g))
    return out


def check_depth_selection(p, tree: dict, b: int, *, W=None, tol: float = 1e-4, exact: bool = False) -> list:
    """Step-wise check of the per-depth selection of an unpruned candidate
    tree (DARTree page, "Tree Construction": after each depth the top-W
    scored nodes across the entire frontier are kept).  Taking the tree's
    own depth t-1 as the frontier, depth t must hold min(W, #admissible)
    admissible children, none of them below an unselected one by more than
    tol, in key order up to inversions smaller than tol.  Exact keys give a
    unique answer (ties: token, then parent rank); the band admits the
    choices an fp64 rounding difference below tol could flip.  With
    ``exact`` the depth must instead equal the first min(W, #admissible)
    children in the total order (Rk desc, token asc, parent rank asc).
    Returns the violated properties (empty when the tree passes)."""
    W = p.W if W is None else W
    sc = PathScorer(p, b)
    cont = Continuity(p.ngram, p.V)
    paths = tree_paths(tree, b)
    by_depth = {}
    for q in paths:
        by_depth.setdefault(len(q), []).append(q)
    errs = []
    frontier = [()]
    seen = 0
    for t in range(1, p.d + 1):
        cand = depth_candidates(p, sc, cont, frontier, t)
        n_cand = sum(len(toks) for toks, _ in cand)
        sel = by_depth.get(t, [])
        want = min(W, n_cand)
        if len(sel) != want:
            errs.append(f"b{b} depth {t}: {len(sel)} nodes, expected {want}")
            return errs
        if not sel:
            break
        seen += len(sel)
        rank = {q: r for r, q in enumerate(frontier)}
        ks = []
        taken = [np.zeros(len(toks), dtype=bool) for toks, _ in cand]
        for q in sel:
            r = rank.get(q[:-1])
            toks, rk = cand[r] if r is not None else (np.zeros(0, dtype=np.int64), None)
            j = int(np.searchsorted(toks, q[-1]))
            if r is None or j >= len(toks) or toks[j] != q[-1]:
                errs.append(f"b{b} depth {t}: {q} is not an admissible child of the frontier")
                return errs
            taken[r][j] = True
            ks.append(float(rk[j]))
        if exact:
            order = sorted(((-float(v), int(c), r) for r, (toks, rk) in enumerate(cand) for c, v in zip(toks, rk)))
            best = [frontier[r] + (c,) for _, c, r in order[:want]]
            if best != sel:
                errs.append(f"b{b} depth {t}: {sel} is not the exact top-{W} {best}")
                return errs
        rest = max((float(np.max(rk[~tk])) for (_, rk), tk in zip(cand, taken) if np.any(~tk)), default=None)
        if rest is not None and min(ks) < rest - tol:
            errs.append(f"b{b} depth {t}: selected key {min(ks)} below unselected {rest}")
        for i in range(len(ks) - 1):
            if ks[i] < ks[i + 1] - tol:
                errs.append(f"b{b} depth {t}: nodes {i},{i + 1} out of key order")
                break
        frontier = sel
    if seen != len(paths):
        errs.append(f"b{b}: {len(paths) - seen} node(s) below the last selected depth")
    return errs


def check_budget_selection(p, tree: dict, cand_tree: dict, b: int, *, budget=None, tol: float = 1e-4,
                           ref_tree=None) -> list:
    """Step-wise check of the verification budget (DARTree abstract: best-
    first pruning selects the verification tree from the fixed-width
    candidate tree).  ``cand_tree`` is the unpruned candidate tree.  Best-
    first is replayed over it: at every step the tree's next node must be
    available (its parent already taken, or depth 1) and its cumulative score
    S within tol of the best available one; the node taken is the tree's best
    available node.  With ``ref_tree`` (the exact selection) given in DART
    mode, where S never rises along a path and the selection is the global
    top-budget by S, every node in which the two sets differ must also lie
    within tol of the cut (the budget-th best S).  Returns the violated
    properties."""
    budget = p.budget if budget is None else budget
    sc = PathScorer(p, b)
    cand = tree_paths(cand_tree, b)
    kids = {}
    for q in cand:
        kids.setdefault(q[:-1], []).append(q)
    got = tree_paths(tree, b)
    G = set(got)
    errs = []
    if len(cand) <= budget:
        if G != set(cand):
            errs.append(f"b{b}: budget does not bind but the node set differs from the candidate tree")
        return errs
    if len(got) != budget or len(G) != budget:
        return [f"b{b}: {len(got)} nodes, expected {budget}"]
    outside = [q for q in got if q not in set(cand)]
    if outside:
        return [f"b{b}: {outside[0]} is not in the candidate tree"]
    S = {q: sc.keys(q)[1] for q in cand}
    avail = set(kids.get((), []))
    for step in range(budget):
        best = max(S[a] for a in avail)
        mine = [a for a in avail if a in G]
        if not mine:
            errs.append(f"b{b} step {step}: no selected node is available")
            break
        pick = max(mine, key=lambda a: S[a])
        if S[pick] < best - tol:
            errs.append(f"b{b} step {step}: took S={S[pick]} with {best} available")
            break
        avail.discard(pick)
        avail.update(kids.get(pick, []))
    if ref_tree is not None and p.mode == MODE_DART:
        O = set(tree_paths(ref_tree, b))
        cut = min(S[q] for q in O)
        off = [q for q in G ^ O if abs(S[q] - cut) > tol]
        if off:
            errs.append(f"b{b}: {off[0]} differs from the exact selection {S[off[0]] - cut:+.3g} from the cut")
    return errs


def has_near_ties(values, tol: float) -> bool:
    v = np.sort(np.asarray(list(values), dtype=np.float64))
    return bool(v.size > 1 and np.min(np.diff(v)) < tol)


def product_count(k: int, d: int) -> int:
    return sum(k ** t for t in range(1, d + 1))


__all__ = [n for n in dir() if not n.startswith("_")] + ["itertools"]

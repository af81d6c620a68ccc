"""Helpers for the GPU tests: run the HIP path through the C ABI and compare
it with the oracle element by element."""

from __future__ import annotations

import math

import numpy as np

from refcheck import check_budget_selection, check_depth_selection, check_invariants, logits_f64

SCORE_TOL = 1e-4   # absolute, fp32 scores (the stated parity tolerance)


def run_gpu(p, device, *, W=None, budget=None, sweep_chunks=0, stream=None):
    import torch
    from draft_tree_construction_dt_amd import binding as bd
    dp = bd.upload_problem(p, device, sweep_chunks=sweep_chunks, W=W, budget=budget)
    if stream is not None:
        dp.params.stream = stream
    bd.dt_build_tree(dp.logits, dp.ngram, dp.params, dp.out)
    torch.cuda.synchronize()
    return dp.out.numpy()


def run_gpu_topk(p, device, *, sweep_chunks=0):
    import torch
    from draft_tree_construction_dt_amd import binding as bd
    dp = bd.upload_problem(p, device, sweep_chunks=sweep_chunks)
    rows = p.B * p.d
    lse = torch.empty(rows, dtype=torch.float64, device=device)
    tok = torch.empty(rows, p.k, dtype=torch.int32, device=device)
    val = torch.empty(rows, p.k, dtype=torch.float32, device=device)
    bd.dt_position_topk(dp.logits, dp.params, lse, tok, val)
    torch.cuda.synchronize()
    return lse.cpu().numpy(), tok.cpu().numpy(), val.cpu().numpy()


def tree_diff(gpu: dict, ora: dict, b: int) -> list:
    """Differences of request b: exact on structure and mask, SCORE_TOL on scores."""
    out = []
    if gpu["n_nodes"][b] != ora["n_nodes"][b]:
        out.append(f"n_nodes {gpu['n_nodes'][b]} != {ora['n_nodes'][b]}")
    for key in ("tokens", "parents", "depths", "mask"):
        if not np.array_equal(gpu[key][b], ora[key][b]):
            idx = np.argwhere(gpu[key][b] != ora[key][b])[:3].tolist()
            out.append(f"{key} differ at {idx}")
    g, o = gpu["scores"][b], ora["scores"][b]
    fin = np.isfinite(o)
    if not np.array_equal(np.isfinite(g), fin) or (fin.any() and np.max(np.abs(g[fin] - o[fin])) > SCORE_TOL):
        out.append("scores differ beyond tolerance")
    return out


NEAR_TIE_TOTAL = {"requests": 0, "accepted": 0}


def near_tie_errors(p, gpu: dict, b: int, *, ora: dict, ora_full=None, tol: float = SCORE_TOL) -> list:
    """Why request b of ``gpu`` is not an acceptable answer, given that it
    differs from the oracle's.  It must satisfy every invariant, and:
    * when the oracle's candidate tree does not exceed the budget (no node is
      pruned), the GPU tree is its own candidate tree and every depth must be
      a top-W selection of its own previous depth up to tol
      (check_depth_selection);
    * otherwise the GPU's nodes must come from the oracle's candidate tree
      and be a best-first selection of it up to tol, and in DART mode every
      node in which it differs from the oracle's selection must lie within
      tol of the oracle's cut (check_budget_selection).
    Empty list: accepted."""
    sub = _slice(gpu, b)
    q = _one(p, b)
    errs = check_invariants(q, sub)
    if errs:
        return errs
    cand = ora_full if ora_full is not None else ora
    full_budget = cand["tokens"].shape[1]
    cand_b = _slice(cand, b)
    n_cand = int(cand["n_nodes"][b])
    if n_cand <= p.budget:
        if ora_full is None and n_cand == full_budget and full_budget < p.d * p.W:
            return ["the oracle tree may be pruned and no candidate tree was given"]
        return check_depth_selection(q, sub, 0, tol=tol)
    return check_budget_selection(q, sub, cand_b, 0, tol=tol, ref_tree=_slice(ora, b))


def assert_parity(p, gpu: dict, ora: dict, *, ora_full=None, label="", say=print):
    """Bit-exact tokens/parents/depths/mask and n_nodes, scores within
    SCORE_TOL.  A request that differs is accepted only when the step-wise
    validator (near_tie_errors) shows that its choices differ from the
    oracle's at keys closer than SCORE_TOL; how many requests took that path
    is printed and returned."""
    bad = []
    near = 0
    for b in range(p.B):
        diff = tree_diff(gpu, ora, b)
        if not diff:
            continue
        errs = near_tie_errors(p, gpu, b, ora=ora, ora_full=ora_full)
        if errs:
            bad.append((b, diff, errs[:2]))
        else:
            near += 1
    NEAR_TIE_TOTAL["requests"] += p.B
    NEAR_TIE_TOTAL["accepted"] += near
    if near:
        say(f"[near-tie] {label}: {near} of {p.B} request(s) differ from the oracle within the "
            f"{SCORE_TOL:g} band (step-wise validator)")
    assert not bad, f"{label}: {len(bad)} request(s) differ, first: {bad[:2]}"
    return near


def _slice(t: dict, b: int) -> dict:
    return {k: v[b:b + 1] for k, v in t.items()}


def _one(p, b: int):
    import copy
    q = copy.copy(p)
    q.B = 1
    q.logits = p.logits[b:b + 1]
    q.ctx = p.ctx[b:b + 1]
    return q


def lse_rows(p) -> np.ndarray:
    X = logits_f64(p)
    out = np.empty((p.B, p.d))
    for b in range(p.B):
        for i in range(p.d):
            m = np.max(X[b, i])
            out[b, i] = -math.inf if m == -math.inf else m + math.log(np.sum(np.exp(X[b, i] - m)))
    return out

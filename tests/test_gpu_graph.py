"""dt_build_tree captured in a HIP graph (through torch.cuda.graph) and
replayed: every replay must reproduce the eager result exactly, with eager
work between replays, and a replay over new input contents must equal the
eager call on those contents.  The library enqueues kernels only (no
allocation, no memset, no synchronisation), so the whole call is
capturable; this is what a serving loop that replays one graph per step
relies on.
"""

import sys

import numpy as np
import pytest

from draft_tree_construction_dt_amd import synth
from refcheck import MODE_DARTREE_FULL

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _same(a: dict, b: dict, label: str):
    for key in ("n_nodes", "tokens", "parents", "depths", "scores", "mask"):
        assert np.array_equal(a[key], b[key]), f"{label}: {key} differs"


def _problems():
    rng = np.random.default_rng(12)
    full = synth.random_problem(rng, B=3, V=900, d=4, k=8, W=8, budget=20, mode=MODE_DARTREE_FULL, R=16)
    return [
        ("c3p B=1", synth.make_problem("c3p", 3, hash_cap_log2=16, hash_keys_log2=14)),
        ("c4p B=64", synth.make_problem("c4p", 4, hash_cap_log2=16, hash_keys_log2=14)),
        ("full-vocabulary", full),
    ]


@pytest.mark.parametrize("which", range(3))
def test_graph_replay_matches_eager(device, which):
    import torch
    from draft_tree_construction_dt_amd import binding as bd
    label, p = _problems()[which]
    _say(f"[case] graph {label}")
    dp = bd.upload_problem(p, device)
    bd.dt_build_tree(dp.logits, dp.ngram, dp.params, dp.out)
    torch.cuda.synchronize()
    ref = dp.out.numpy()

    # unrelated eager work between replays: another problem into other buffers
    rng = np.random.default_rng(99)
    other = synth.random_problem(rng, B=2, V=500, d=3, k=4, W=4, budget=8)
    do = bd.upload_problem(other, device)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dp.params.stream = torch.cuda.current_stream()
        bd.dt_build_tree(dp.logits, dp.ngram, dp.params, dp.out)
    dp.params.stream = None
    for rep in range(3):
        for t in (dp.out.tokens, dp.out.parents, dp.out.depths, dp.out.n_nodes, dp.out.mask):
            t.fill_(-7)
        dp.out.scores.fill_(float("nan"))
        bd.dt_build_tree(do.logits, do.ngram, do.params, do.out)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(dp.out.numpy(), ref, f"{label} replay {rep}")

    # new contents in the captured input buffer: the replay computes the new tree
    q = synth.make_problem("c3p", 5, hash_cap_log2=16, hash_keys_log2=14) if which == 0 else None
    if q is not None:
        dp.logits.copy_(bd.logits_tensor(q, device))
        g.replay()
        torch.cuda.synchronize()
        got = dp.out.numpy()
        dq = bd.upload_problem(q, device)
        dq.ngram = dp.ngram                      # the same table and context as captured
        dq.params.ctx = dp.params.ctx
        bd.dt_build_tree(dq.logits, dq.ngram, dq.params, dq.out)
        torch.cuda.synchronize()
        _same(got, dq.out.numpy(), f"{label} new logits")

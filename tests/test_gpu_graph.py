"""dt_build_tree captured in a HIP graph (through torch.cuda.graph) and
replayed: every replay must match the oracle (and reproduce the eager result
exactly), with eager work between replays, and a replay over new input
contents must match the oracle on those contents.  The library enqueues
kernels only (no allocation, no memset, no synchronisation), so the whole
call is capturable; this is what a serving loop that replays one graph per
step relies on.  The single-request workloads run at their full sizes.
"""

import copy
import sys

import numpy as np
import pytest

from draft_tree_construction_dt_amd import synth
from gpu_util import assert_parity
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
        ("c3 B=1 full size", lambda: synth.make_problem("c3", 3)),
        ("c3p B=1 full size", lambda: synth.make_problem("c3p", 3)),
        ("c4p B=64", lambda: synth.make_problem("c4p", 4, hash_cap_log2=16, hash_keys_log2=14)),
        ("full-vocabulary", lambda: full),
    ]


def _check(p, got, oracle_lib, label):
    ora = oracle_lib.build_tree(p)
    full = oracle_lib.build_tree(p, budget=p.d * p.W) if p.budget < p.d * p.W else None
    assert_parity(p, got, ora, ora_full=full, label=label, say=_say)


@pytest.mark.parametrize("which", range(4))
def test_graph_replay_matches_oracle(device, oracle_lib, which):
    import torch
    from draft_tree_construction_dt_amd import binding as bd
    label, make = _problems()[which]
    p = make()
    _say(f"[case] graph {label}")
    dp = bd.upload_problem(p, device)
    bd.dt_build_tree(dp.logits, dp.ngram, dp.params, dp.out)
    torch.cuda.synchronize()
    ref = dp.out.numpy()
    _check(p, ref, oracle_lib, f"{label} eager")

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
        got = dp.out.numpy()
        _same(got, ref, f"{label} replay {rep}")
        _check(p, got, oracle_lib, f"{label} replay {rep}")

    # new contents in the captured input buffer: the replay computes the tree
    # of the new logits (with the table and context that were captured)
    if which <= 1:
        q = synth.make_problem("c3p", 5)
        dp.logits.copy_(bd.logits_tensor(q, device))
        g.replay()
        torch.cuda.synchronize()
        qq = copy.copy(p)
        qq.logits = q.logits
        _check(qq, dp.out.numpy(), oracle_lib, f"{label} new logits")

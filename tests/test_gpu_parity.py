"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bar: n_nodes, tokens, parents, depths and mask bit-exact; scores within
1e-4 absolute; node choices may differ only where the oracle's own budget
cut is a near tie below that tolerance.  Every size used here spans several
sweep chunks and a ragged tail somewhere; the named workloads run at their
full sizes in the launch configuration the benchmark uses.
"""

import math
import sys

import numpy as np
import pytest

from draft_tree_construction_dt_amd import synth
from gpu_util import assert_parity, lse_rows, run_gpu, run_gpu_topk
from refcheck import (MODE_DART, MODE_DARTREE, NGRAM_CSR_BIGRAM, NGRAM_DENSE_BIGRAM,
                      NGRAM_HASH_TRIGRAM, NGRAM_NONE, check_invariants, logits_f64, topk_np)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _parity(p, device, oracle, *, sweep_chunks=0, label=None):
    label = label or f"{p.name}/seed{p.seed}"
    _say(f"[case] {label} B={p.B} V={p.V} d={p.d} k={p.k} W={p.W} budget={p.budget} chunks={sweep_chunks}")
    gpu = run_gpu(p, device, sweep_chunks=sweep_chunks)
    ora = oracle.build_tree(p)
    full = oracle.build_tree(p, budget=p.d * p.W) if p.budget < p.d * p.W else None
    assert_parity(p, gpu, ora, ora_full=full, label=label)
    return gpu, ora


# --------------------------------------------------------------------------
# step 1 alone: per-position normaliser and top-k
# --------------------------------------------------------------------------

TOPK_CASES = [
    ("c1", {}, 0), ("c1", {}, 3), ("c2", {}, 0), ("c2", {}, 1), ("c3", {}, 0),
    ("c5", dict(B=2), 0), ("c2", dict(V=1003), 5), ("c2", dict(V=37, k=8), 0),
    ("c1", dict(V=7, k=7), 0), ("c4L", dict(B=3, V=8191), 7),
]


@pytest.mark.parametrize("name,ov,chunks", TOPK_CASES, ids=[f"{n}-{o}-{c}" for n, o, c in TOPK_CASES])
def test_position_topk(device, oracle_lib, name, ov, chunks):
    ov = dict(ov)
    if synth.config(name).ngram == NGRAM_HASH_TRIGRAM:
        ov.update(hash_cap_log2=10, hash_keys_log2=8)
    p = synth.make_problem(name, 1, **ov)
    _say(f"[case] topk {name} {ov} chunks={chunks}")
    lse, tok, val = run_gpu_topk(p, device, sweep_chunks=chunks)
    X = logits_f64(p).reshape(p.B * p.d, p.V)
    ref = lse_rows(p).reshape(-1)
    np.testing.assert_allclose(lse, ref, rtol=0, atol=1e-5)
    for r in range(p.B * p.d):
        want = topk_np(X[r], p.k)
        assert tok[r].tolist() == want.tolist(), f"row {r}"
        assert np.array_equal(val[r].astype(np.float64), X[r][want])


def test_position_topk_neg_inf_and_ties(device):
    rng = np.random.default_rng(5)
    V = 5000
    x = rng.integers(-3, 4, size=(1, 4, V)).astype(np.float32)     # heavy ties
    x[0, 1, :] = -np.inf                                            # an all -inf row
    x[0, 2, rng.random(V) < 0.9] = -np.inf
    x[0, 3, 17] = 0.0
    x[0, 3, 18] = -0.0                                              # -0 ties +0 by id
    p = synth.random_problem(rng, B=1, V=V, d=4, k=12, W=2, budget=4)
    p.logits = x
    lse, tok, val = run_gpu_topk(p, device, sweep_chunks=3)
    X = x.reshape(4, V).astype(np.float64)
    for r in range(4):
        assert tok[r].tolist() == topk_np(X[r], 12).tolist(), f"row {r}"
    assert lse[1] == -np.inf
    ref = lse_rows(p).reshape(-1)
    np.testing.assert_allclose(lse[[0, 2, 3]], ref[[0, 2, 3]], rtol=0, atol=1e-5)


# --------------------------------------------------------------------------
# whole path on the named workloads
# --------------------------------------------------------------------------

def test_c1_many_seeds(device, oracle_lib):
    sizes = set()
    for seed in range(300):
        p = synth.make_problem("c1", seed)
        gpu = run_gpu(p, device)
        ora = oracle_lib.build_tree(p)
        assert_parity(p, gpu, ora, label=f"c1/seed{seed}")
        sizes.add(int(gpu["n_nodes"][0]))
    _say(f"c1 tree sizes seen: {sorted(sizes)}")
    assert 0 in sizes and max(sizes) >= 10


@pytest.mark.parametrize("name", ["c2", "c2p", "c3", "c3p"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_single_request_workloads(device, oracle_lib, name, seed):
    p = synth.make_problem(name, seed)
    gpu, ora = _parity(p, device, oracle_lib)
    if name.endswith("p"):
        assert gpu["n_nodes"][0] >= 20


@pytest.mark.parametrize("name", ["c4p", "c4", "c4Lp", "c4L"])
def test_batched_workloads(device, oracle_lib, name):
    p = synth.make_problem(name, 0)
    gpu, _ = _parity(p, device, oracle_lib)
    _say(f"{name}: mean nodes {gpu['n_nodes'].mean():.1f} min {gpu['n_nodes'].min()} max {gpu['n_nodes'].max()}")


def test_dartree_workload(device, oracle_lib):
    p = synth.make_problem("c5", 0)
    gpu, _ = _parity(p, device, oracle_lib)
    assert np.all(gpu["n_nodes"] == p.d * p.W)


# --------------------------------------------------------------------------
# random problems over every table kind, both modes, both dtypes
# --------------------------------------------------------------------------

KINDS = [NGRAM_NONE, NGRAM_DENSE_BIGRAM, NGRAM_CSR_BIGRAM, NGRAM_HASH_TRIGRAM]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("mode", [MODE_DART, MODE_DARTREE])
def test_random_problems(device, oracle_lib, kind, mode):
    rng = np.random.default_rng(100 * kind + mode)
    for trial in range(12):
        V = int(rng.integers(8, 40))
        k = int(rng.integers(1, min(V, 12) + 1))
        W = int(rng.integers(1, 10))
        d = int(rng.integers(1, 7))
        budget = int(rng.integers(1, d * W + 3))
        p = synth.random_problem(
            rng, B=int(rng.integers(1, 5)), V=V, d=d, k=k, W=W, budget=budget, ngram=kind, mode=mode,
            dtype=synth.DTYPE_BF16 if trial % 2 else synth.DTYPE_F32, density=0.6,
            # dense rows are log-softmaxes over V: a threshold near -log V admits about half
            min_logp=(-math.log(V) - 0.5) if kind == NGRAM_DENSE_BIGRAM else (-1.0 if trial % 3 == 0 else -math.inf),
            hash_cap=256, hash_S=int(rng.integers(1, 9)), csr_deg=int(rng.integers(1, 12)),
            neg_inf_frac=0.05 if trial % 4 == 0 else 0.0, integer_logits=trial % 5 == 0, R=8)
        _parity(p, device, oracle_lib, sweep_chunks=int(rng.integers(0, 4)),
                label=f"random kind={kind} mode={mode} trial={trial}")


# --------------------------------------------------------------------------
# edge cases
# --------------------------------------------------------------------------

def test_budget_one_and_chain_widths(device, oracle_lib):
    for W, budget in [(1, 1), (1, 8), (8, 1), (3, 5)]:
        p = synth.make_problem("c2p", 0, budget=budget, W=W)
        _parity(p, device, oracle_lib, label=f"c2p W={W} budget={budget}")


def test_k_equals_v_and_k1(device, oracle_lib):
    rng = np.random.default_rng(3)
    p = synth.random_problem(rng, B=2, V=9, d=3, k=9, W=20, budget=200, R=4)
    _parity(p, device, oracle_lib, label="k=V")
    p = synth.random_problem(rng, B=2, V=300, d=6, k=1, W=4, budget=6, ngram=NGRAM_HASH_TRIGRAM,
                             density=0.02, hash_cap=1 << 16, hash_S=8)
    _parity(p, device, oracle_lib, label="k=1")


def test_ragged_vocab_multi_chunk(device, oracle_lib):
    for V, chunks in [(1003, 3), (4099, 7), (77777, 0), (77777, 8)]:
        p = synth.make_problem("c2p", 4, V=V)
        _parity(p, device, oracle_lib, sweep_chunks=chunks, label=f"c2p V={V} chunks={chunks}")


def test_empty_trees(device, oracle_lib):
    p = synth.make_problem("c3", 0, hash_cap_log2=8, hash_keys_log2=2)   # nothing admitted
    gpu, _ = _parity(p, device, oracle_lib)
    assert gpu["n_nodes"][0] == 0 and np.all(gpu["mask"] == 0) and np.all(gpu["tokens"] == -1)


def test_neg_inf_logits(device, oracle_lib):
    rng = np.random.default_rng(11)
    p = synth.random_problem(rng, B=3, V=500, d=5, k=8, W=4, budget=12, neg_inf_frac=0.97)
    p.logits[1, 2, :] = -np.inf
    _parity(p, device, oracle_lib, sweep_chunks=2, label="neg inf")


def test_csr_long_rows_and_threshold(device, oracle_lib):
    rng = np.random.default_rng(21)
    p = synth.random_problem(rng, B=2, V=400, d=5, k=10, W=6, budget=20, ngram=NGRAM_CSR_BIGRAM,
                             csr_deg=200, min_logp=-0.5)
    _parity(p, device, oracle_lib, label="csr long rows")


def test_dartree_budget_binding(device, oracle_lib):
    rng = np.random.default_rng(8)
    for trial in range(6):
        p = synth.random_problem(rng, B=3, V=60, d=5, k=6, W=6, budget=7, mode=MODE_DARTREE, R=8)
        p.E *= 3
        _parity(p, device, oracle_lib, label=f"dartree budget trial {trial}")


def test_hash_wide_rows_large_k_and_many_survivors(device, oracle_lib):
    """Trigram rows longer than 16 successors (several chunks per lookup),
    row lengths that are not a multiple of four, a 4-slot table whose probe
    window wraps, k up to 32 (the children's token table full to its bound,
    contexts split over several workgroups) and frontiers whose survivors
    exceed 32 (the streamed ranking)."""
    rng = np.random.default_rng(31)
    cases = [(20, 17, 1024, 64), (32, 24, 512, 64), (32, 64, 2048, 64), (12, 33, 4, 40), (17, 5, 64, 48)]
    for i, (k, S, cap, V) in enumerate(cases):
        W = int(rng.integers(4, 1024 // k + 1))
        W = min(W, 32)
        d = int(rng.integers(3, 6))
        p = synth.random_problem(
            rng, B=2, V=V, d=d, k=k, W=W, budget=d * W, ngram=NGRAM_HASH_TRIGRAM, density=0.5,
            hash_cap=cap, hash_S=S, min_logp=-1.0 if i % 2 else -math.inf,
            dtype=synth.DTYPE_BF16 if i % 2 else synth.DTYPE_F32)
        _parity(p, device, oracle_lib, label=f"hash k={k} S={S} cap={cap} W={W}")
    for W, k in [(32, 32), (64, 16)]:
        p = synth.random_problem(rng, B=2, V=300, d=4, k=k, W=W, budget=min(4 * W, 1024),
                                 integer_logits=True)
        _parity(p, device, oracle_lib, label=f"no table W={W} k={k}")


def test_tight_bound_many_candidates(device, oracle_lib):
    """Depths where more than 32 candidates reach the first-valid-child
    bound (no table, and in DARTree mode a strong parent term that reorders
    each parent's children): the depth loop then bounds the W-th key by the
    W-th largest of the lanes' best keys rounded down to fp32.  Continuous
    and bf16 logits, up to eight candidate slots per lane."""
    rng = np.random.default_rng(41)
    cases = [(MODE_DART, 16, 16), (MODE_DARTREE, 16, 16), (MODE_DARTREE, 8, 32), (MODE_DART, 24, 20)]
    for trial, (mode, W, k) in enumerate(cases):
        p = synth.random_problem(rng, B=3, V=700, d=5, k=k, W=W, budget=5 * W, mode=mode, R=8,
                                 dtype=synth.DTYPE_BF16 if trial % 2 else synth.DTYPE_F32)
        if mode == MODE_DARTREE:
            p.E *= 4
        _parity(p, device, oracle_lib, label=f"many candidates mode={mode} W={W} k={k}")


def test_fp32_logits_full_vocabulary(device, oracle_lib):
    """fp32 logits at the Qwen3 vocabulary (the sweep's four-element vectors
    and a ragged row length), trigram table and coherence planting, in the
    launch plan of a small batch and of a forced chunk count."""
    for V, chunks in [(151936, 0), (151937, 3)]:
        p = synth.make_problem("c3p", 1, B=3, V=V, dtype=synth.DTYPE_F32, hash_cap_log2=16, hash_keys_log2=15)
        _parity(p, device, oracle_lib, sweep_chunks=chunks, label=f"fp32 V={V} chunks={chunks}")


def test_empty_csr_table(device, oracle_lib):
    """A CSR table with no successors at all (nnz = 0, no successor arrays):
    nothing is admitted."""
    rng = np.random.default_rng(71)
    p = synth.random_problem(rng, B=2, V=40, d=4, k=4, W=4, budget=16, ngram=NGRAM_CSR_BIGRAM, csr_deg=1)
    p.ngram.row_ptr[:] = 0
    p.ngram.col = np.zeros(0, dtype=np.int32)
    p.ngram.csr_logp = np.zeros(0, dtype=np.float32)
    gpu, _ = _parity(p, device, oracle_lib, label="empty csr")
    assert np.all(gpu["n_nodes"] == 0)


def test_large_shared_plans(device, oracle_lib):
    """Tree-kernel shared-memory plans between 64 and 160 KiB: many
    candidates per depth with long trees, a wide trigram context table, and
    DARTree terms for deep trees."""
    rng = np.random.default_rng(61)
    cases = [
        dict(B=4, V=694, d=10, k=16, W=57, budget=427, ngram=NGRAM_NONE, mode=MODE_DART),
        dict(B=3, V=114, d=10, k=28, W=32, budget=222, ngram=NGRAM_HASH_TRIGRAM, mode=MODE_DART,
             hash_cap=1024, hash_S=12, density=0.5),
        dict(B=3, V=427, d=9, k=22, W=42, budget=268, ngram=NGRAM_NONE, mode=MODE_DARTREE, R=16),
    ]
    for i, c in enumerate(cases):
        p = synth.random_problem(rng, dtype=synth.DTYPE_BF16 if i % 2 else synth.DTYPE_F32, **c)
        _parity(p, device, oracle_lib, label=f"large plan {i}")


def test_random_campaign(device, oracle_lib):
    """Four hundred random problems over every mode, table kind, dtype and
    launch plan (V up to 5000, k up to 32, W up to 64, d up to 10, budgets
    from 1 past d*W, integer logits for exact ties, -inf logits, strong
    parent terms).  Parameters outside the library's limits must be refused
    with DT_ERR_UNSUPPORTED; every other problem must match the oracle."""
    from draft_tree_construction_dt_amd import binding as bd
    from refcheck import MODE_DARTREE_FULL
    rng = np.random.default_rng(2024)
    refused = 0
    for n in range(400):
        mode = [MODE_DART, MODE_DART, MODE_DARTREE, MODE_DARTREE_FULL][int(rng.integers(0, 4))]
        kind = NGRAM_NONE if mode == MODE_DARTREE_FULL else int(rng.choice(KINDS))
        vmax = {NGRAM_HASH_TRIGRAM: 250, NGRAM_DENSE_BIGRAM: 1500}.get(kind, 5000)
        V = int(rng.integers(2, vmax))
        if mode == MODE_DARTREE_FULL:
            W = int(rng.integers(1, 17))
            k = min(W, V)
            R = int(rng.choice([16, 32, 64]))
        else:
            k = int(rng.integers(1, min(V, 32) + 1))
            W = int(rng.integers(1, min(64, 1024 // k) + 1))
            R = int(rng.choice([4, 8, 16, 64]))
        d = int(rng.integers(1, 11))
        budget = min(int(rng.integers(1, d * W + 3)), 1024)
        p = synth.random_problem(
            rng, B=int(rng.integers(1, 7)), V=V, d=d, k=k, W=W, budget=budget, ngram=kind, mode=mode,
            dtype=synth.DTYPE_BF16 if rng.random() < 0.5 else synth.DTYPE_F32,
            density=float(rng.uniform(0.05, 0.9)),
            min_logp=-1.0 if (kind != NGRAM_NONE and rng.random() < 0.3) else -math.inf,
            hash_cap=int(2 ** rng.integers(4, 12)), hash_S=int(rng.integers(1, 20)),
            csr_deg=int(rng.integers(1, 40)), neg_inf_frac=0.05 if rng.random() < 0.2 else 0.0,
            integer_logits=bool(rng.random() < 0.15), R=R, sigma=float(rng.choice([0.5, 2.0, 6.0])))
        if mode == MODE_DARTREE and rng.random() < 0.3:
            p.E *= 4
        chunks = int(rng.integers(0, 5)) if mode != MODE_DARTREE_FULL else 0
        try:
            _parity(p, device, oracle_lib, sweep_chunks=chunks, label=f"campaign {n} mode={mode} kind={kind}")
        except bd.DtError as e:
            assert e.status == bd.DT_ERR_UNSUPPORTED, str(e)
            refused += 1
    _say(f"[campaign] {400 - refused} problems matched, {refused} refused as unsupported")
    assert refused < 60


def test_zero_requests(device):
    import torch
    from draft_tree_construction_dt_amd import binding as bd
    p = synth.make_problem("c1", 0)
    dp = bd.upload_problem(p, device)
    dp.params.B = 0
    bd.dt_build_tree(dp.logits, dp.ngram, dp.params, dp.out)
    torch.cuda.synchronize()


def test_deterministic_across_calls_and_streams(device, oracle_lib):
    import torch
    p = synth.make_problem("c5", 2, B=2)
    a = run_gpu(p, device)
    s = torch.cuda.Stream(device=device)
    b = run_gpu(p, device, stream=s)
    for key in a:
        assert np.array_equal(a[key], b[key]), key
    assert not check_invariants(p, a)


def test_calls_in_flight_on_four_streams(device):
    """Batched calls (B=64, so the sweeps take turns on the compute units)
    in flight together on four streams, each with its own workspace and
    outputs, repeated so that sweeps and tails of different calls overlap:
    every call's tree equals the same call made alone."""
    import copy
    import bench
    import torch
    from draft_tree_construction_dt_amd import binding as bd
    prob = bench.make_workload(2, 0)
    subs = []
    for s in (0, 1):
        sub = copy.copy(prob)
        sub.B = bench.BATCH
        sub.logits = prob.logits[s * bench.BATCH:(s + 1) * bench.BATCH]
        sub.ctx = prob.ctx[s * bench.BATCH:(s + 1) * bench.BATCH]
        subs.append(sub)
    alone = [run_gpu(sub, device) for sub in subs]
    streams = [torch.cuda.Stream(device=device) for _ in range(4)]
    ups = []
    for i in range(4):
        dp = bd.upload_problem(subs[i % 2], device)
        dp.params.stream = streams[i]
        ups.append(dp)
    torch.cuda.synchronize()
    _say("[case] 4 streams x 6 rounds of B=64 calls")
    for _ in range(6):
        for dp in ups:
            bd.dt_build_tree(dp.logits, dp.ngram, dp.params, dp.out)
    torch.cuda.synchronize()
    for i, dp in enumerate(ups):
        got = dp.out.numpy()
        for key, want in alone[i % 2].items():
            assert np.array_equal(got[key], want), (i, key)


def test_bench_workload_sampled(device, oracle_lib):
    """The benchmark's own inputs in its launch configuration (B=64 per call,
    automatic chunking): sampled requests of two sets against the oracle."""
    import copy
    import bench
    from draft_tree_construction_dt_amd import binding as bd
    import torch
    prob = bench.make_workload(2, 0)
    for s in (0, 1):
        sub = copy.copy(prob)
        sub.B = bench.BATCH
        sub.logits = prob.logits[s * bench.BATCH:(s + 1) * bench.BATCH]
        sub.ctx = prob.ctx[s * bench.BATCH:(s + 1) * bench.BATCH]
        _say(f"[case] bench workload set {s}")
        gpu = run_gpu(sub, device)
        pick = [0, 7, 13, 29, 31, 42, 58, 63]
        samp = copy.copy(sub)
        samp.B = len(pick)
        samp.logits = sub.logits[pick]
        samp.ctx = sub.ctx[pick]
        ora = oracle_lib.build_tree(samp)
        g = {k: v[pick] for k, v in gpu.items()}
        assert_parity(samp, g, ora, label=f"bench set {s}")
        assert not check_invariants(sub, gpu)

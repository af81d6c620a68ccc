"""Driver for tests/test_sanitizers.py (run in a child process, not collected
by pytest).

    python sanitize_run.py oracle LIB OUT.npz   # the oracle on a fixed problem set
    python sanitize_run.py abi LIB               # tests/test_abi.py against LIB

``oracle``: loads the oracle library LIB (a plain or a sanitizer build of
oracle.c) and runs every entry point on a deterministic set of problems: the
brute-force pins' tiny instances of every table kind and mode, random
problems with -inf logits, integer logits and every table kind, the
full-vocabulary mode, the trigram update and the verification length; all
outputs go to OUT.npz so that the parent can compare the two builds.

``abi``: points the binding at LIB (a build whose host code is instrumented)
and runs the ABI tests, which only exercise host-side validation and
planning (no GPU call).
"""

import math
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)


def run_oracle(lib: str, out_path: str) -> None:
    import numpy as np

    import oracle
    from draft_tree_construction_dt_amd import synth

    oracle.LIB_PATH = lib
    results = {}

    def keep(tag, tree):
        for key, v in tree.items():
            results[f"{tag}/{key}"] = np.asarray(v)

    n = 0
    for kind in range(4):
        for mode in (synth.MODE_DART, synth.MODE_DARTREE):
            for seed in range(6):
                rng = np.random.default_rng([seed, kind, mode])
                V = int(rng.integers(6, 60))
                d = int(rng.integers(1, 6))
                k = int(rng.integers(1, min(V, 9) + 1))
                W = int(rng.integers(1, 9))
                p = synth.random_problem(
                    rng, B=2, V=V, d=d, k=k, W=W, budget=int(rng.integers(1, d * W + 3)), ngram=kind,
                    mode=mode, R=4, density=0.6,
                    min_logp=(-math.log(V) - 0.5) if kind == synth.NGRAM_DENSE_BIGRAM else
                    (-1.0 if seed % 2 else -math.inf),
                    hash_cap=256, hash_S=int(rng.integers(1, 9)), csr_deg=int(rng.integers(1, 12)),
                    neg_inf_frac=0.1 if seed % 3 == 0 else 0.0, integer_logits=seed % 2 == 0,
                    dtype=synth.DTYPE_BF16 if seed % 2 else synth.DTYPE_F32)
                keep(f"random{n}", oracle.build_tree(p))
                keep(f"random{n}full", oracle.build_tree(p, budget=p.d * p.W))
                n += 1
    for seed in range(4):
        rng = np.random.default_rng(50 + seed)
        p = synth.random_problem(rng, B=2, V=30, d=4, k=4, W=3, budget=7, mode=synth.MODE_DARTREE_FULL, R=4,
                                 neg_inf_frac=0.1 * seed)
        keep(f"fullvocab{seed}", oracle.build_tree(p))
    for name in ("c1", "c2p"):
        p = synth.make_problem(name, 0)
        keep(name, oracle.build_tree(p))
    p = synth.make_problem("c4p", 0, B=4, hash_cap_log2=12, hash_keys_log2=10)
    tree = oracle.build_tree(p)
    keep("c4p_small", tree)
    nv, rank = oracle.verify_length(tree, 16.0, 1.0)
    results["verify/n"], results["verify/rank"] = nv, rank
    ng = synth.make_problem("c3", 0, hash_cap_log2=8, hash_keys_log2=6).ngram
    rng = np.random.default_rng(9)
    ctx = rng.integers(0, 50, size=(6, 2)).astype(np.int32)
    toks = rng.integers(0, 50, size=(6, 9)).astype(np.int32)
    lens = rng.integers(0, 10, size=6).astype(np.int32)
    counts = oracle.ngram_update(ng, ctx, toks, lens, -0.5)
    results["update/counts"] = np.array(counts)
    results["update/keys"], results["update/succ"] = ng.keys, ng.succ
    np.savez(out_path, **results)
    print(f"oracle: {len(results)} arrays written", flush=True)


def run_abi(lib: str) -> int:
    import pytest

    from draft_tree_construction_dt_amd import binding
    binding._LIB_PATH = lib
    return pytest.main([os.path.join(HERE, "test_abi.py"), "-q", "-p", "no:cacheprovider", "-x"])


if __name__ == "__main__":
    what = sys.argv[1]
    if what == "oracle":
        run_oracle(sys.argv[2], sys.argv[3])
    elif what == "abi":
        sys.exit(run_abi(sys.argv[2]))
    else:
        sys.exit(f"unknown driver {what}")

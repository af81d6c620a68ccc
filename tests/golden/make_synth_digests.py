"""Writes synth_digests.json: SHA-256 digests of every array the seeded
generator produces for scaled-down versions of the named workloads.

Run from the repository root:  python tests/golden/make_synth_digests.py
It calls only the input generator (no oracle, no HIP library); the digests
pin the generator's determinism so benchmark inputs cannot drift silently.
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from draft_tree_construction_dt_amd import synth  # noqa: E402

# scaled-down shapes: same recipes, sizes that generate in well under a second
CASES = {
    "c1": {},
    "c2": dict(V=4096),
    "c2p": dict(V=4096),
    "c3": dict(V=8192, hash_cap_log2=14, hash_keys_log2=13),
    "c3p": dict(V=8192, hash_cap_log2=14, hash_keys_log2=13),
    "c4p": dict(B=4, V=8192, hash_cap_log2=14, hash_keys_log2=13),
    "c4Lp": dict(B=4, V=4096, hash_cap_log2=14, hash_keys_log2=13),
    "c5": dict(B=2, V=4096, d=4),
}


def digest(p):
    out = {}
    arrays = dict(logits=p.logits, ctx=p.ctx, E=p.E, F=p.F)
    for f in ("dense_logp", "row_ptr", "col", "csr_logp", "keys", "succ", "hash_logp"):
        arrays["ngram." + f] = getattr(p.ngram, f)
    for name, a in arrays.items():
        if a is not None:
            a = np.ascontiguousarray(a)
            out[name] = hashlib.sha256(a.tobytes() + str(a.dtype).encode() + str(a.shape).encode()).hexdigest()
    return out


def main():
    res = {name: digest(synth.make_problem(name, 0, **ov)) for name, ov in CASES.items()}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "synth_digests.json")
    with open(path, "w") as f:
        json.dump({"cases": CASES, "digests": res}, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main()

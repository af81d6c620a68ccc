#!/usr/bin/env python3
"""Throughput of draft-tree construction on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one dt_build_tree call on the batched Qwen3-vocab workload: B=64
independent requests, V=151936, d=8 draft positions, top-k 10, width 8,
budget 64, bf16 logits (N(0,3) plus a log Zipf(1.1) prior, coherence-planted),
a shared open-addressing trigram table of 2^22 slots with 16 successors.
Inputs rotate over several distinct sets totalling more than three times
the 256 MB Infinity Cache, all resident in HBM before timing starts.
Consecutive calls alternate over --streams HIP streams (default 4, the
hardware queues a process gets), each
with its own workspace and outputs, so the latency-bound tree kernels of one
batch overlap the bandwidth-bound sweep of the next, as a serving loop would
run them; the one-stream figures are reported as well ("single_stream").
The single-request case (B=1, same shape) is timed the same two ways and
reported under "b1".  Prints one JSON line.

Roofline: the vocabulary sweep kernel dominates; its duration is measured
live with HIP events that the library records around that kernel on the
launch stream (every n-th launch of the one-stream timed loop, where no other
kernel shares the GPU with it, so that the events time the kernel itself),
and its algorithmic bytes are the logits it must read (B*d*V*2 per launch).
"""

import argparse
import copy
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "draft trees/sec and µs/tree (B=1, B=64) at V=151936, d=8; % HBM roofline"
HBM_PEAK_GBS = 8000.0
BATCH = 64
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sweep_traffic.json")
SWEEP_SOURCES = [os.path.join(ROOT, "draft_tree_construction_dt_amd", "csrc", f)
                 for f in ("sweep.hip", "sweep_dev.h", "common.h", "wave.h")]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--sets", type=int, default=5, help="distinct B=64 input sets to rotate over")
    ap.add_argument("--b1-steps", type=int, default=2000, help="timed single-request calls")
    ap.add_argument("--cpu-sample", type=int, default=128,
                    help="requests the oracle builds for cpu_baseline (about 12 s of one core)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--streams", type=int, default=4,
                    help="HIP streams the calls alternate over (consecutive batches in flight together)")
    ap.add_argument("--event-every", type=int, default=1,
                    help="bracket every n-th B=64 sweep launch of the one-stream pass with timing events")
    ap.add_argument("--one-stream-calls", type=int, default=200,
                    help="least number of calls in the one-stream pass (its sweep launches are the roofline "
                         "samples), whatever --steps is")
    ap.add_argument("--cpu-procs", type=int, default=0,
                    help="worker processes of the multi-process oracle run (0 = the host's cores, at most 16)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--update-steps", type=int, default=2000, help="timed trigram-table update calls")
    ap.add_argument("--sweep-chunks", type=int, default=0, help="0 = the library's automatic plan")
    ap.add_argument("--workload", default="c4p",
                    help="c4p (the default JSON contract) or another named configuration, timed per call "
                         "(c1, c2, c2p, c3, c3p, c4, c4L, c4Lp, c5, c5f)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this size (counter calibration)")
    ap.add_argument("--traffic-from", default="",
                    help="only write the sweep's HBM traffic file from rocprofv3 counter runs under this "
                         "directory (subdirectories fetch, write, cfetch, cwrite; no GPU needed)")
    return ap.parse_args()


def make_workload(n_sets: int, seed: int = 0):
    """The benchmark's inputs: n_sets * 64 coherence-planted Qwen3-vocab
    requests sharing one trigram table; set s is requests [64 s, 64 s + 64)."""
    from draft_tree_construction_dt_amd import synth
    return synth.make_problem("c4p", seed, B=BATCH * n_sets)


def kernel_sources_hash() -> str:
    h = hashlib.sha256()
    for f in SWEEP_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic():
    """HBM bytes per sweep launch from committed rocprofv3 counter runs, or
    None when absent or taken on a different version of the kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sources_sha256") != kernel_sources_hash():
        return None
    return t.get("bytes_per_launch")


class TimingEvents:
    """HIP events for timing only, created with hipEventDisableSystemFence.

    An ordinary event record ends with a system-scope release: the caches are
    written back and invalidated between the kernels it separates, which costs
    several microseconds per record and lengthens the bracketed interval.
    These events skip that fence, so the interval between a start and a stop
    record is the kernel's own duration.  They come from the HIP runtime that
    torch has already loaded (the one libdt.so binds to as well)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD)
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        e = ctypes.c_void_p()
        rc = self.lib.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        return e.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def destroy(self, e: int) -> None:
        self.lib.hipEventDestroy(e)

    def record(self, e: int, stream: int) -> None:
        rc = self.lib.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")


def _counter_rows(d: str, counter: str):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") == counter:
                    rows.append((r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"no {counter} rows under {d}")
    return rows


def write_traffic(root: str, commands: list) -> None:
    """HBM bytes per B=64 sweep launch from two counter runs of the bench
    (FETCH_SIZE, WRITE_SIZE: KiB per dispatch) and the same counters over a
    plain device copy of known size, whose readings give each counter's
    scale to bytes."""
    import statistics
    grid = BATCH * 8 * 256                       # B=64 rows x 1 chunk x 256 threads
    def sweep_avg(sub, counter):
        v = [x for n, g, x in _counter_rows(os.path.join(root, sub), counter) if "sweep_kernel" in n and g == grid]
        if not v:
            raise SystemExit(f"no B=64 sweep dispatches in {sub}")
        return statistics.mean(v)
    def copy_max(sub, counter):
        v = [(g, x) for n, g, x in _counter_rows(os.path.join(root, sub), counter) if "copyBuffer" in n]
        g = max(g for g, _ in v)
        return statistics.mean(x for gg, x in v if gg == g)
    copy_bytes = None
    with open(os.path.join(root, "copy.json")) as fh:
        for line in fh:
            if line.startswith("{") and "copy_probe_bytes_read" in line:
                copy_bytes = json.loads(line)["copy_probe_bytes_read"]
    if copy_bytes is None:
        raise SystemExit("copy.json holds no copy probe line")
    fetch_kib, write_kib = sweep_avg("fetch", "FETCH_SIZE"), sweep_avg("write", "WRITE_SIZE")
    fscale = copy_bytes / (copy_max("cfetch", "FETCH_SIZE") * 1024)
    wscale = copy_bytes / (copy_max("cwrite", "WRITE_SIZE") * 1024)
    t = {
        "kernel": "sweep_kernel<bf16>", "workload": "B=64, V=151936, d=8, bf16",
        "kernel_sources_sha256": kernel_sources_hash(),
        "fetch_size_kib": fetch_kib, "write_size_kib": write_kib,
        "fetch_scale": fscale, "write_scale": wscale,
        "bytes_per_launch": fetch_kib * 1024 * fscale + write_kib * 1024 * wscale,
        "fetched_bytes": fetch_kib * 1024 * fscale, "written_bytes": write_kib * 1024 * wscale,
        "commands": commands,
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(t, f, indent=1)
    print(json.dumps(t))


def copy_probe(mib: int) -> None:
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 5}))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_slice(args):
    """Worker of the multi-process oracle run: build the trees of requests
    [lo, hi) of the shared problem (inherited from the parent by fork)."""
    lo, hi = args
    import oracle
    p = _CPU_PROB
    sub = copy.copy(p)
    sub.B = hi - lo
    sub.logits = p.logits[lo:hi]
    sub.ctx = p.ctx[lo:hi]
    oracle.build_tree(sub)
    return hi - lo


_CPU_PROB = None


def cpu_baseline(prob, sample: int, procs: int) -> dict:
    """The oracle as it stands, on this host's cores: the first ``sample``
    requests on one thread, and every request of the input sets spread over
    worker processes (one slice of requests each; the oracle is
    single-threaded C).  Runs before the GPU is initialised."""
    import multiprocessing as mp
    import oracle
    global _CPU_PROB
    n = max(1, min(sample, prob.B))
    sub = copy.copy(prob)
    sub.B = n
    sub.logits = prob.logits[:n]
    sub.ctx = prob.ctx[:n]
    tc = time.perf_counter()
    oracle.build_tree(sub)
    one_s = time.perf_counter() - tc
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    nproc = max(1, min(procs or cores, 16, prob.B))
    _CPU_PROB = prob
    per = -(-prob.B // nproc)
    slices = [(lo, min(prob.B, lo + per)) for lo in range(0, prob.B, per)]
    ctx = mp.get_context("fork")
    tm = time.perf_counter()
    with ctx.Pool(nproc) as pool:
        done = sum(pool.map(_oracle_slice, slices))
    multi_s = time.perf_counter() - tm
    _CPU_PROB = None
    print(f"[bench] oracle: {n} trees on 1 thread in {one_s:.1f}s, {done} trees on {nproc} processes in "
          f"{multi_s:.1f}s", file=sys.stderr, flush=True)
    return {
        "value": n / one_s,
        "unit": "trees/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"the first {n} requests of the input sets (whole path: normaliser, top-k, trigram expansion, "
                  f"top-W, budget, mask), single-threaded C, {one_s:.1f}s",
        "cpu_model": cpu_model(),
        "host_cores": cores,
        "multi": {
            "value": done / multi_s, "unit": "trees/s", "cores": nproc, "kind": "oracle",
            "sample": f"all {done} requests of the input sets over {nproc} worker processes (one slice of "
                      f"requests each, process start-up included), {multi_s:.1f}s",
        },
    }


def run_workload(args) -> None:
    """Per-call latency of one named configuration: calls on one stream, each
    bracketed by fence-free events, inputs rotated over enough distinct sets
    to exceed the Infinity Cache where the generator allows it (small
    configurations stay cache-resident and are latency-bound anyway)."""
    import statistics
    import numpy as np
    import torch
    from draft_tree_construction_dt_amd import binding as bd, synth

    cfg = synth.config(args.workload)
    bpe = 2 if cfg.dtype == synth.DTYPE_BF16 else 4
    per_call = cfg.B * cfg.d * cfg.V * bpe
    sets = max(1, min(-(-(800 << 20) // per_call), 1600 // cfg.B))
    dev = torch.device("cuda:0")
    t0 = time.time()
    prob = synth.make_problem(args.workload, args.seed, B=cfg.B * sets)
    print(f"[bench] {args.workload}: generated {sets} input sets in {time.time() - t0:.1f}s",
          file=sys.stderr, flush=True)
    logits = bd.logits_tensor(prob, dev)
    ctx = torch.from_numpy(prob.ctx).to(dev)
    ngram = bd.upload_ngram(prob.ngram, dev)
    E = F = None
    if prob.mode != bd.DT_MODE_DART:
        E = torch.from_numpy(prob.E).to(dev)
        F = torch.from_numpy(prob.F).to(dev)
    stream = torch.cuda.current_stream()
    pcs, keep = [], []
    for sidx in range(sets):
        q = bd.Params(B=cfg.B, V=prob.V, d=prob.d, k=prob.k, W=prob.W, budget=prob.budget,
                      dtype=bd.DT_DTYPE_BF16 if bpe == 2 else bd.DT_DTYPE_F32, mode=prob.mode,
                      ctx=ctx[sidx * cfg.B:(sidx + 1) * cfg.B], stream=stream, E=E, F=F,
                      R=prob.E.shape[1] if E is not None else 0)
        q.workspace = torch.empty(max(bd.dt_workspace_size(q), 16), dtype=torch.uint8, device=dev)
        keep.append(q)
        pcs.append(q._c())
    out = bd.alloc_tree_out(cfg.B, prob.budget, dev)
    out_c, ng_c = out._c(), ngram._c()
    ptrs = [logits[sidx * cfg.B].data_ptr() for sidx in range(sets)]
    fn = bd._load().dt_build_tree
    tev = TimingEvents()
    for i in range(args.warmup):
        fn(ptrs[i % sets], ctypes.byref(ng_c), ctypes.byref(pcs[i % sets]), ctypes.byref(out_c))
    torch.cuda.synchronize()
    K = args.steps
    ev = [(tev.create(), tev.create()) for _ in range(K)]
    h = stream.cuda_stream
    t1 = time.perf_counter()
    for i in range(K):
        tev.record(ev[i][0], h)
        st = fn(ptrs[i % sets], ctypes.byref(ng_c), ctypes.byref(pcs[i % sets]), ctypes.byref(out_c))
        tev.record(ev[i][1], h)
        if st != 0:
            raise bd.DtError(st, "dt_build_tree")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t1
    us = sorted(tev.elapsed_ms(a, b) * 1e3 for a, b in ev)
    for a, b in ev:
        tev.destroy(a)
        tev.destroy(b)
    med = statistics.median(us)
    full = None
    if prob.mode == bd.DT_MODE_DARTREE_FULL:
        # the depth loop alone (d vocabulary launches + d frontier merges),
        # timed by events the library records around it on its stream
        evs = [(tev.create(), tev.create()) for _ in range(K)]
        for i in range(K):
            pc = pcs[i % sets]
            pc.prof_event_start, pc.prof_event_stop = evs[i]
            fn(ptrs[i % sets], ctypes.byref(ng_c), ctypes.byref(pc), ctypes.byref(out_c))
        torch.cuda.synchronize()
        loop_us = sorted(tev.elapsed_ms(a, b) * 1e3 for a, b in evs)
        for pc in pcs:
            pc.prof_event_start = pc.prof_event_stop = None
        for a, b in evs:
            tev.destroy(a)
            tev.destroy(b)
        # algorithmic MFMA work: 2 R V flops per (frontier node, depth); the
        # last call's tree (budget = d W keeps every node) gives the frontier
        # sizes; 16-row tiles padded past the frontier are not counted
        o = out.numpy()
        R = prob.E.shape[1]
        rows = 0
        for b in range(cfg.B):
            dep = o["depths"][b][: int(o["n_nodes"][b])]
            rows += 1 + int(np.sum(dep < prob.d))
        flops = 2.0 * R * prob.V * rows
        lmed = statistics.median(loop_us)
        full = {
            "bound": "mfma", "kernel": "vocab_kernel + frontier_kernel, the whole depth loop",
            "achieved": flops / lmed / 1e6, "peak": 2500.0, "unit": "TFLOP/s",
            "frac": flops / lmed / 1e6 / 2500.0, "traffic": None,
            "depth_loop_us_median": lmed, "algorithmic_flops_per_call": flops,
            "timing": "HIP events recorded by the library around the depth loop, one stream",
            "dtype": "bf16 MFMA for the screen (dense bf16 peak), fp64 exact rescoring of the survivors",
        }
    if prob.mode == bd.DT_MODE_DARTREE:
        # the parent-conditioned contraction g = E[parent] . F[child] on fp64
        # matrix cores: per request 2 R k (1 + (d - 1) k) flops (the root row at
        # depth 1, k parents after); its kernel (prep_kernel, which also merges
        # rows) is not timed apart live, so the whole call's median bounds its
        # duration and the fraction below is a lower bound
        R = prob.E.shape[1]
        flops = 2.0 * R * prob.k * (1 + (prob.d - 1) * prob.k) * cfg.B
        full = {
            "bound": "mfma", "kernel": "prep_kernel: G = E[parents] F[children]^T, fp64 MFMA 16x16x4",
            "achieved": flops / med / 1e6, "peak": 78.6, "unit": "TFLOP/s",
            "frac": flops / med / 1e6 / 78.6, "traffic": None, "algorithmic_flops_per_call": flops,
            "timing": "the whole call's median (events) as the contraction's duration: a lower bound on the "
                      "fraction; rocprofv3 MFMA counters are in profiles/",
        }
    res = {
        "metric": METRIC, "workload": args.workload, "value": cfg.B / med * 1e6, "unit": "trees/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "B": cfg.B,
        "us_per_call_median": med, "us_per_call_p10": us[len(us) // 10], "us_per_call_p90": us[(9 * len(us)) // 10],
        "us_per_tree": med / cfg.B, "wall_us_per_call": wall / K * 1e6,
        "logit_bytes_per_call": per_call, "gb_per_s": per_call / med / 1e3,
        "frac_of_8tbs": per_call / med / 1e3 / HBM_PEAK_GBS,
        "input_sets": sets, "input_bytes_rotated": per_call * sets,
        "cache_resident": per_call * sets < (256 << 20),
        "data": "synthetic", "dtype": "f32",
    }
    if full is not None:
        res["roofline"] = full
    if not args.no_cpu:
        import oracle
        n = min(prob.B, {synth.MODE_DART: 64, synth.MODE_DARTREE: 16}.get(prob.mode, 2))
        sample = copy.copy(prob)
        sample.B = n
        sample.logits = prob.logits[:n]
        sample.ctx = prob.ctx[:n]
        tc = time.perf_counter()
        oracle.build_tree(sample)
        cpu_s = time.perf_counter() - tc
        res["cpu_baseline"] = {"value": n / cpu_s, "unit": "trees/s", "cores": 1, "kind": "oracle",
                               "sample": f"the first {n} requests, single-threaded C, {cpu_s:.2f}s",
                               "cpu_model": cpu_model()}
    print(json.dumps(res), flush=True)


def time_ngram_update(lib, ngram, prob, dev, K: int, warmup: int, seed: int) -> dict:
    """Back-to-back dt_ngram_update calls on one stream, each adding the
    accepted tokens of B=64 requests (d+1 each: the d drafted positions and the
    bonus token) to a copy of the trigram table.  Every call gets a batch of
    its own with uniform ids, so nearly every trigram is a new key: the
    insertion path, not the lookup of trigrams already present."""
    import dataclasses
    import numpy as np
    import torch
    from draft_tree_construction_dt_amd import binding as bd
    tab = dataclasses.replace(ngram, keys=ngram.keys.clone(), succ=ngram.succ.clone(),
                              hash_logp=None if ngram.hash_logp is None else ngram.hash_logp.clone())
    g = tab._c()
    L = prob.d + 1
    n = warmup + K
    rng = np.random.default_rng(seed + 991)
    tokens = torch.from_numpy(rng.integers(0, prob.V, size=(n, BATCH, L), dtype=np.int32)).to(dev)
    ctx = torch.from_numpy(rng.integers(0, prob.V, size=(n, BATCH, 2), dtype=np.int32)).to(dev)
    lengths = torch.full((BATCH,), L, dtype=torch.int32, device=dev)
    counts = torch.zeros(3, dtype=torch.int32, device=dev)
    h = torch.cuda.current_stream().cuda_stream
    occupied0 = int((tab.keys != -1).sum())
    fn = lib.dt_ngram_update

    def call(i):
        st = fn(ctypes.byref(g), ctypes.c_void_p(ctx[i].data_ptr()), ctypes.c_void_p(tokens[i].data_ptr()),
                ctypes.c_void_p(lengths.data_ptr()), BATCH, L, 0.0, ctypes.c_void_p(counts.data_ptr()), h)
        if st != 0:
            raise bd.DtError(st, "dt_ngram_update")

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    c0 = counts.cpu().tolist()
    t0 = time.perf_counter()
    for i in range(warmup, n):
        call(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    c1 = counts.cpu().tolist()
    tri = K * BATCH * L
    return {
        "workload": f"B={BATCH} requests x {L} accepted tokens per call (uniform ids) into a copy of the "
                    f"trigram table ({tab.cap} slots x {tab.S}, {occupied0} keys before)",
        "us_per_call": wall / K * 1e6,
        "trigrams_per_s": tri / wall,
        "steps": K,
        "keys_added": c1[0] - c0[0],
        "successors_added": c1[1] - c0[1],
        "dropped": c1[2] - c0[2],
        "timing": "wall clock of back-to-back calls on one stream",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures the single-GPU path only; --gpus must be 1 "
              "(requests shard across GPUs with no exchange)", file=sys.stderr)
        sys.exit(2)
    if args.traffic_from:
        r = "$R/" + os.path.relpath(args.traffic_from, ROOT)
        write_traffic(args.traffic_from, [
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {r}/fetch -o bench -- python3 $R/bench.py "
            "--steps 20 --warmup 5 --b1-steps 10 --update-steps 20 --no-cpu --streams 1",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {r}/write -o bench -- python3 $R/bench.py "
            "--steps 20 --warmup 5 --b1-steps 10 --update-steps 20 --no-cpu --streams 1",
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {r}/cfetch -o copy -- python3 $R/bench.py "
            f"--copy-probe-mib 1024 > {r}/copy.json",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {r}/cwrite -o copy -- python3 $R/bench.py "
            "--copy-probe-mib 1024"])
        return
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    if args.workload != "c4p":
        run_workload(args)
        return

    t0 = time.time()
    prob = make_workload(args.sets, args.seed)
    gen_s = time.time() - t0
    print(f"[bench] generated {args.sets} input sets in {gen_s:.1f}s", file=sys.stderr, flush=True)
    # the oracle's timing runs first, before anything touches the GPU (its
    # worker processes are forked from this one)
    cpu = None if args.no_cpu else cpu_baseline(prob, args.cpu_sample, args.cpu_procs)

    import statistics
    import torch
    from draft_tree_construction_dt_amd import binding as bd

    dev = torch.device("cuda:0")

    logits = bd.logits_tensor(prob, dev)                      # [sets*64][d][V] bf16
    ctx = torch.from_numpy(prob.ctx).to(dev)
    ngram = bd.upload_ngram(prob.ngram, dev)
    lib = bd._load()
    fn = lib.dt_build_tree
    nstream = max(1, args.streams)
    streams = [torch.cuda.current_stream()] + [torch.cuda.Stream(device=dev) for _ in range(nstream - 1)]

    def params(B, first, stream):
        p = bd.Params(B=B, V=prob.V, d=prob.d, k=prob.k, W=prob.W, budget=prob.budget,
                      dtype=bd.DT_DTYPE_BF16, mode=bd.DT_MODE_DART, ctx=ctx[first:first + B], stream=stream,
                      sweep_chunks=args.sweep_chunks if B > 1 else 0)
        p.workspace = torch.empty(max(bd.dt_workspace_size(p), 16), dtype=torch.uint8, device=dev)
        return p

    ng_c = ngram._c()
    tev = TimingEvents()

    def run(B, inputs, K, warmup, S, events_every=0):
        """K calls of dt_build_tree; call i takes input i % len(inputs) on stream
        i % S, with a workspace and output buffers of its own per (input, stream)
        so that calls in flight on different streams share nothing.  Returns
        the wall time of the K calls and, if events_every, the sweep durations
        of every events_every-th call."""
        keep = []
        pcs = []
        for si in range(S):
            row = []
            for first in inputs:
                q = params(B, first, streams[si])
                keep.append(q)
                row.append(q._c())
            pcs.append(row)
        outs = [bd.alloc_tree_out(B, prob.budget, dev) for _ in range(S)]
        outs_c = [o._c() for o in outs]
        ptrs = [logits[first].data_ptr() for first in inputs]
        n = len(inputs)

        def call(i):
            st = fn(ptrs[i % n], ctypes.byref(ng_c), ctypes.byref(pcs[i % S][i % n]), ctypes.byref(outs_c[i % S]))
            if st != 0:
                raise bd.DtError(st, "dt_build_tree")

        for i in range(warmup):
            call(i)
        torch.cuda.synchronize()
        raw = {}
        if events_every:
            raw = {i: (tev.create(), tev.create()) for i in range(0, K, events_every)}
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            pc = pcs[i % S][i % n]
            pc.prof_event_start, pc.prof_event_stop = raw.get(i, (None, None))
            call(i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = [tev.elapsed_ms(x, y) for x, y in raw.values()]
        for x, y in raw.values():
            tev.destroy(x)
            tev.destroy(y)
        return wall, ms

    # ---- B = 64: rotate over the sets; the timed run brackets every
    #      event_every-th sweep launch with events (the roofline figure)
    logit_bytes = BATCH * prob.d * prob.V * 2
    set_first = [s * BATCH for s in range(args.sets)]
    K = args.steps
    every = max(1, args.event_every)
    t_total, _ = run(BATCH, set_first, K, args.warmup, nstream)
    ms_per_step = t_total / K * 1e3
    trees_per_s = BATCH * K / t_total
    # one stream: the kernels run alone, so the sweep events time the kernel
    # itself; at least --one-stream-calls calls, so the roofline figure does
    # not hang on a handful of launches
    K_one = max(K, args.one_stream_calls)
    t_one, sweep_ms = run(BATCH, set_first, K_one, args.warmup, 1, events_every=every)
    sweep_avg_s = sum(sweep_ms) / len(sweep_ms) / 1e3
    sweep_sorted = sorted(sweep_ms)

    # ---- B = 1: one request per call, rotating over every request of every set
    nreq = BATCH * args.sets
    K1 = args.b1_steps
    b1_wall, _ = run(1, list(range(nreq)), K1, min(200, K1), nstream)
    b1_one, _ = run(1, list(range(nreq)), K1, min(200, K1), 1)

    # ---- how many of each B=64 tree's nodes to verify (expected-speedup rule)
    qv = params(BATCH, 0, None)
    out_v = bd.alloc_tree_out(BATCH, prob.budget, dev)
    ov = out_v._c()
    qvc = qv._c()
    if fn(logits[0].data_ptr(), ctypes.byref(ng_c), ctypes.byref(qvc), ctypes.byref(ov)) != 0:
        raise RuntimeError("dt_build_tree")
    nv = torch.empty(BATCH, dtype=torch.int32, device=dev)
    rank = torch.empty(BATCH, prob.budget, dtype=torch.int32, device=dev)
    vfn = lib.dt_verify_length
    hv = torch.cuda.current_stream().cuda_stream
    cost_fixed, cost_per_token = 16.0, 1.0
    for _ in range(20):
        vfn(ctypes.byref(ov), BATCH, prob.budget, cost_fixed, cost_per_token, ctypes.c_void_p(nv.data_ptr()),
            ctypes.c_void_p(rank.data_ptr()), hv)
    torch.cuda.synchronize()
    tv = time.perf_counter()
    KV = 1000
    for _ in range(KV):
        vfn(ctypes.byref(ov), BATCH, prob.budget, cost_fixed, cost_per_token, ctypes.c_void_p(nv.data_ptr()),
            ctypes.c_void_p(rank.data_ptr()), hv)
    torch.cuda.synchronize()
    verify_us = (time.perf_counter() - tv) / KV * 1e6
    nv_host = nv.cpu().numpy()

    upd = time_ngram_update(lib, ngram, prob, dev, args.update_steps, 100, args.seed)

    achieved = logit_bytes / sweep_avg_s / 1e9
    traffic = stored_traffic()
    res = {
        "metric": METRIC,
        "value": trees_per_s,
        "unit": "trees/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "batched Qwen3-vocab draft trees: B=64, V=151936, d=8, k=10, W=8, budget=64, "
                        "bf16 logits N(0,3)+log Zipf(1.1) prior with coherence planting, shared "
                        "trigram table 2^22 slots x 16 successors (DART mode)",
            "B": BATCH, "V": prob.V, "d": prob.d, "k": prob.k, "W": prob.W, "budget": prob.budget,
            "logits": "bf16", "input_sets": args.sets,
            "input_bytes_rotated": logit_bytes * args.sets,
        },
        "us_per_tree": t_total / (BATCH * K) * 1e6,
        "streams": nstream,
        "single_stream": {
            "trees_per_s": BATCH * K_one / t_one,
            "ms_per_step": t_one / K_one * 1e3,
            "us_per_tree": t_one / (BATCH * K_one) * 1e6,
            "steps": K_one,
            "hbm_frac_whole_call": logit_bytes / (t_one / K_one) / 1e9 / HBM_PEAK_GBS,
        },
        "b1": {
            "workload": "same shape, B=1 (one request per call)",
            "us_per_tree": b1_one / K1 * 1e6,
            "trees_per_s": K1 / b1_one,
            "timing": "one stream, calls back to back: the latency of one request",
            "trees_per_s_streams": K1 / b1_wall,
            "streams": nstream,
            "steps": K1,
        },
        "ngram_update": upd,
        "verify_length": {
            "workload": f"the {BATCH} trees of input set 0, cost_fixed={cost_fixed}, cost_per_token={cost_per_token} "
                        "(a round's fixed cost as 16 verified tokens)",
            "us_per_call": verify_us,
            "n_verify_mean": float(nv_host.mean()),
            "timing": "wall clock of back-to-back calls on one stream",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "sweep_kernel<bf16>",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "avg_launch_us": sweep_avg_s * 1e6,
            "median_launch_us": statistics.median(sweep_ms) * 1e3,
            "p10_launch_us": sweep_sorted[len(sweep_sorted) // 10] * 1e3,
            "p90_launch_us": sweep_sorted[(9 * len(sweep_sorted)) // 10] * 1e3,
            "samples": len(sweep_ms),
            "timing": f"HIP events recorded by the library around every {every}-th sweep launch of the "
                      f"one-stream timed loop ({len(sweep_ms)} launches) on its stream, created with "
                      f"hipEventDisableSystemFence; achieved = algorithmic bytes / the mean duration",
            "algorithmic_bytes_per_launch": logit_bytes,
        },
    }

    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the batched gapped-extension hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one whole fz_extend_batch call (every phase of the path) over the
workload's batch, inputs already resident in device memory; the reported
step time is the median over the timed steps.  Prints one JSON line: GCUPS
(canonical cells / step time), seed extensions per second, the roofline of
the dominant kernel (integer VALU bound) and of the whole call against the
same peak (roofline.end_to_end), the int32 VALU rate measured by a probe
kernel beside the peak from unit counts, and the CPU oracle timed on a
bounded sample of the same batch on this host's cores.

Workloads (seeded, synthetic; see smith_waterman_dp_amd/workloads.py):
  skewed          one million 19-mer seeds on a 10 Mbp pair (default)
  local           4,096 full-matrix local alignments of 2048 x 2048
  tiny, executor_heavy, chromosome
  chromosome_rc   the chromosome pair searched on the query's reverse strand
  skewed_matrix   the skewed batch scored with a 4x4 matrix, runs of N planted
  chromosome_rounds  the chromosome pair's seeds in random order through
                  fz_extend_rounds (covered-seed suppression, --round-size)
  seeds           the seed stage (fz_find_seeds) on the 20 Mbp chromosome pair,
                  both strands per step; reported in Mbp/s of target + query
  pipeline        the whole chain on the 20 Mbp chromosome pair: per strand,
                  the seed stage, then the seeds in a seeded random order
                  through fz_extend_rounds; Mbp/s of target + query
"""
import argparse
import concurrent.futures as concurrent_futures
import contextlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GCUPS and seed extensions/sec on 1M-seed skewed batch, 1 MI355X"

# Integer VALU peak of MI355X: 256 CUs x 4 SIMD x 16 lanes (64 lane-ops per
# clock per CU) x 2.4 GHz peak engine clock; packed 16-bit instructions do
# two operations per lane, so the extension's packed layouts have twice that.
N_CU, LANE_OPS_PER_CLK_PER_CU, CLOCK_HZ = 256, 64, 2.4e9
VALU_PEAK_OPS = N_CU * LANE_OPS_PER_CLK_PER_CU * CLOCK_HZ
VALU_PEAK_OPS_PK16 = 2 * VALU_PEAK_OPS

# Algorithmic integer operations per cell (fixed, independent of the code):
#   extension: 5 adds + 4 compares of the three-state cell (FastZ section 2.2,
#   observation (1)), 1 substitution lookup, 2 for the y-drop test and kill,
#   1 running maximum = 13;
#   local: 5 adds + 5 max (zero clamp included), 1 substitution, 1 running
#   maximum = 12.
OPS_PER_CELL = {"extend": 13, "local": 12}


def extension_kernels(cells, onepass_cells, inspector_ms, onepass_ms, peak):
    """Rooflines of the two kernels that sweep the extension's cells: the
    inspector (the cells of every side it finished: all but the one-pass
    sides') and the one-pass executor (its sides' cells, each swept once with
    its pointers).  Returns (dominant, [both]); a kernel that did not run
    (0 ms) is left out."""
    ops = OPS_PER_CELL["extend"]
    ks = []
    for name, c, ms in (("extend_kernel (inspector)", cells - onepass_cells, inspector_ms),
                        ("extend_kernel (one-pass executor)", onepass_cells, onepass_ms)):
        if ms > 0 and c > 0:
            ach = ops * c / (ms / 1e3) / 1e12
            ks.append({"kernel": name, "cells": int(c), "ms": round(ms, 3), "achieved": round(ach, 3),
                       "frac": round(ach / peak, 4)})
    dom = max(ks, key=lambda k: k["ms"]) if ks else None
    return dom, ks


# HBM traffic of one launch of each extension kernel on the 1M-seed skewed
# batch, from two rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE, KiB)
# scaled by what the same counters read for a plain 1 GiB device copy in the
# same run (FETCH_SIZE reads 0.5 GiB for it, WRITE_SIZE 1.0 GiB).  Valid only
# for the kernel sources it was taken on (hash of fz_extend.hpp,
# fz_device.hpp and fz_packed.hpp); reported as null otherwise.
TRAFFIC_SRC_HASH = "1269baeb08c0dd35"
TRAFFIC = {"extend_kernel (inspector)": (4.681e6 * 1024 / 0.5, 7.593e6 * 1024 / 1.0),
           "extend_kernel (one-pass executor)": (3.756e6 * 1024 / 0.5, 1.676e8 * 1024 / 1.0)}


# The same for one join_count_kernel launch of the seed stage on the 20 Mbp
# chromosome pair (mean of the forward and reverse-strand launches), valid
# for the sources hashed from fz_seeds.hpp.
SEED_TRAFFIC_SRC_HASH = "1c0d0bf8ec6f018d"
SEED_TRAFFIC_FETCH_BYTES = 1.910e6 * 1024 / 0.5
SEED_TRAFFIC_WRITE_BYTES = 2.344e5 * 1024 / 1.0


def kernel_src_hash(files=("fz_extend.hpp", "fz_device.hpp", "fz_packed.hpp")):
    """sha256 over the files' sha256 hex digests, first 16 hex digits."""
    import hashlib
    d = os.path.join(ROOT, "smith_waterman_dp_amd", "csrc")
    digests = "".join(hashlib.sha256(open(os.path.join(d, f), "rb").read()).hexdigest()
                      for f in files)
    return hashlib.sha256(digests.encode()).hexdigest()[:16]


def measured_traffic(fetch, write, seconds):
    tot = fetch + write
    return {"bytes_per_launch": int(tot), "fetch_bytes": int(fetch), "write_bytes": int(write),
            "gb_per_s": round(tot / seconds / 1e9, 2), "hbm_frac": round(tot / seconds / 8e12, 5)}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="skewed",
                    choices=["skewed", "local", "tiny", "executor_heavy", "chromosome", "chromosome_rc",
                             "skewed_matrix", "chromosome_rounds", "seeds", "pipeline"])
    ap.add_argument("--round-size", type=int, default=2048,
                    help="chromosome_rounds, pipeline: seeds per round of covered-seed suppression (with the "
                         "doubling schedule, of the first round)")
    ap.add_argument("--round-schedule", choices=["doubling", "fixed"], default="doubling",
                    help="doubling: each round twice the size of the one before; fixed: all rounds alike")
    ap.add_argument("--strands", choices=["concurrent", "serial"], default="concurrent",
                    help="pipeline: the two strands on two contexts and streams from two host threads, "
                         "or one after the other on one context")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU-oracle sample time")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--two-pass", action="store_true",
                    help="every side through the inspector and the two-pass executor (FZ_TWO_PASS)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="after the timed steps, one plain device-to-device copy of this many MiB "
                         "(a known-size reference for HBM traffic counters)")
    a = ap.parse_args()
    a.round_doubling = a.round_schedule == "doubling"
    return a


def make_workload(name):
    from smith_waterman_dp_amd import workloads as W
    return W.WORKLOADS[name]()


def cpu_baseline(w, target_seconds, local):
    """The oracle, as it stands, on a seeded sample of the batch, on the host
    cores this process may use (at most 16)."""
    import numpy as np

    import oracle
    threads = oracle.default_threads()
    rng = np.random.default_rng(123)
    seeds = w["seeds"]
    query = oracle.revcomp(w["query"]) if w.get("query_rc") else w["query"]
    n = seeds.shape[0]
    order = rng.permutation(n)
    done_cells = 0
    done = 0
    t0 = time.time()
    chunk = max(threads, 8)
    while done < n and time.time() - t0 < target_seconds:
        idx = order[done:done + chunk]
        hits, _, _ = oracle.run(w["target"], query, seeds[idx], w["scoring"],
                                oracle.YDROP_INF if local else w["ydrop"], min_tb=w.get("min_tb"),
                                traceback=not local and w.get("traceback", True), local=local, threads=threads)
        done_cells += int(hits["cells_r"].sum() + (0 if local else hits["cells_l"].sum()))
        done += len(idx)
        chunk = min(chunk * 2, 4096)
    dt = time.time() - t0
    return {"value": round(done_cells / dt / 1e9, 4), "unit": "GCUPS", "cores": threads, "kind": "oracle",
            "sample": "%d of %d records (seeded draw), %.1f s, %.3g cells, extensions/s %.1f"
                      % (done, n, dt, done_cells, done / dt)}


def copy_probe(mib, dev):
    """One plain device-to-device copy of `mib` MiB (a known-size reference
    for the HBM traffic counters), or nothing for 0."""
    if mib <= 0:
        return
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()


SEED_PHASES = ("pack", "keys", "sort_keys", "index", "join", "scan", "emit", "sort_hits", "runs", "write")


def cpu_seed_baseline(w, target_seconds):
    """The oracle's seed stage, as it stands, on growing prefixes of the pair
    (both strands each), until one run passes half the target time."""
    import oracle
    L = 1 << 20
    full = min(w["target"].size, w["query"].size)
    while True:
        L = min(L, full)
        t0 = time.time()
        for rc in (False, True):
            oracle.find_seeds(w["target"][:L], w["query"][:L], w["k"], w["flank"], query_rc=rc)
        dt = time.time() - t0
        if dt > target_seconds / 2 or L == full:
            break
        L *= 2
    return {"value": round(2 * L / dt / 1e6, 3), "unit": "Mbp/s", "cores": 1, "kind": "oracle",
            "sample": "first %d bases of target and query, both strands, %.1f s (numpy, one thread)" % (L, dt)}


def bench_seeds(a):
    import numpy as np
    import torch

    from smith_waterman_dp_amd import fz
    from smith_waterman_dp_amd import workloads as W

    steps = a.steps if a.steps is not None else 10
    print("[bench] generating the 20 Mbp chromosome pair", file=sys.stderr, flush=True)
    w = W.chromosome_seed_stage()
    dev = torch.device("cuda:0")
    T = torch.from_numpy(w["target"]).to(dev)
    Q = torch.from_numpy(w["query"]).to(dev)
    ctx = fz.Context(0)

    def step():
        # the reverse strand reuses the target index the forward call built
        out = []
        for rc in (False, True):
            out.append(ctx.find_seeds(T, Q, w["k"], w["flank"], query_rc=rc, want_stats=True, reuse_index=rc))
        return out

    for k in range(a.warmup):
        step()
        print("[bench] warmup %d done" % k, file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    phases = {p: [] for p in SEED_PHASES}
    t0 = time.perf_counter()
    res = None
    for k in range(steps):
        res = step()
        for _, _, st in res:
            for p in SEED_PHASES:
                phases[p].append(st["ms_" + p])
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    copy_probe(a.copy_probe, dev)
    ms_per_step = dt / steps * 1e3
    bases = int(w["target"].size + w["query"].size)
    nt = w["target"].size - w["k"] + 1
    nq = w["query"].size - w["k"] + 1
    hits = [h for _, h, _ in res]
    n_seeds = [int(s.shape[0]) for s, _, _ in res]
    mean = {p: float(np.mean(v)) for p, v in phases.items()}
    # HBM roofline of the join kernel, the longest single launch of the
    # stage: per query position it reads the position's code (1 B; its k-1
    # neighbours are shared with the next positions) and writes the range
    # start (4 B) and the count (8 B); the bucket table (4 B per bucket) and
    # the sorted target keys (8 B each) are counted once, the least any
    # lookup of every query key must read.
    nb_bits = 1
    while nb_bits < 30 and (1 << nb_bits) < nt:
        nb_bits += 1
    nb = 1 << min(nb_bits, 2 * w["k"])
    join_bytes = 13 * nq + 4 * (nb + 1) + 8 * nt
    achieved = join_bytes / (mean["join"] / 1e3) / 1e9
    traffic = None
    if kernel_src_hash(("fz_seeds.hpp",)) == SEED_TRAFFIC_SRC_HASH:
        traffic = measured_traffic(SEED_TRAFFIC_FETCH_BYTES, SEED_TRAFFIC_WRITE_BYTES, mean["join"] / 1e3)
    cfg = {"workload": "chromosome_seed_stage", "target_bp": int(w["target"].size), "query_bp": int(w["query"].size),
           "k": w["k"], "flank": w["flank"], "strands": 2, "hits": hits, "seeds": n_seeds,
           "phase_ms": {p: round(v, 3) for p, v in mean.items()}}
    out = {"metric": "seed stage throughput on a 20 Mbp chromosome pair, both strands, 1 MI355X",
           "value": round(bases / (ms_per_step / 1e3) / 1e6, 3), "unit": "Mbp/s", "n_gpus": 1, "steps": steps,
           "warmup": a.warmup, "ms_per_step": round(ms_per_step, 3), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "u64", "data": "synthetic", "config": cfg,
           "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": 8000.0, "unit": "GB/s",
                        "frac": round(achieved / 8000.0, 4), "traffic": traffic, "kernel": "join_count_kernel",
                        "bytes_per_launch": join_bytes}}
    if not a.no_cpu:
        print("[bench] CPU oracle sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_seed_baseline(w, a.cpu_seconds)
    ctx.close()
    print(json.dumps(out), flush=True)


def cpu_pipeline_baseline(w, target_seconds, round_size, doubling):
    """The oracle's seed stage and rounds, as they stand, on growing prefixes
    of the pair (both strands), until one run passes half the target time."""
    import numpy as np

    import oracle
    threads = oracle.default_threads()
    L = 1 << 12
    full = min(w["target"].size, w["query"].size)
    while True:
        L = min(L, full)
        T, Q = w["target"][:L], w["query"][:L]
        t0 = time.time()
        for rc in (False, True):
            s, _ = oracle.find_seeds(T, Q, w["k"], w["flank"], query_rc=rc)
            s = s[np.random.default_rng(7).permutation(len(s))]
            oracle.extend_rounds(T, oracle.revcomp(Q) if rc else Q, s, w["scoring"], w["ydrop"], 3000, round_size,
                                 threads=threads, doubling=doubling)
        dt = time.time() - t0
        if dt > target_seconds / 2 or L == full:
            break
        L *= 2
    return {"value": round(2 * L / dt / 1e6, 4), "unit": "Mbp/s", "cores": threads, "kind": "oracle",
            "sample": "first %d bases of target and query, both strands, %.1f s" % (L, dt)}


def bench_pipeline(a):
    import numpy as np
    import torch

    from smith_waterman_dp_amd import fz
    from smith_waterman_dp_amd import workloads as W

    steps = a.steps if a.steps is not None else 3
    print("[bench] generating the 20 Mbp chromosome pair", file=sys.stderr, flush=True)
    w = dict(W.chromosome_seed_stage(), scoring=dict(W.DEFAULT_SCORING), ydrop=W.DEFAULT_YDROP)
    dev = torch.device("cuda:0")
    T = torch.from_numpy(w["target"]).to(dev)
    Q = torch.from_numpy(w["query"]).to(dev)
    concurrent = a.strands == "concurrent"
    ctxs = [fz.Context(0), fz.Context(0)] if concurrent else [fz.Context(0)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()] if concurrent else [None]
    torch.cuda.synchronize()

    def strand(rc):
        # one strand: the seed stage, a seeded order, the rounds
        k = 1 if (rc and concurrent) else 0
        ctx, strm = ctxs[k], streams[k]
        with torch.cuda.stream(strm) if strm is not None else contextlib.nullcontext():
            seeds, _ = ctx.find_seeds(T, Q, w["k"], w["flank"], query_rc=rc, reuse_index=rc and not concurrent,
                                      stream=strm)
            perm = torch.randperm(seeds.shape[0], generator=torch.Generator().manual_seed(7)).to(dev)
            h, c, st = ctx.extend_rounds(T, Q, seeds[perm], w["scoring"], w["ydrop"], 3000, a.round_size,
                                         want_stats=True, query_rc=rc, doubling=a.round_doubling, stream=strm)
            if strm is not None:
                strm.synchronize()
        return seeds.shape[0], h, st

    pool = concurrent_futures.ThreadPoolExecutor(2) if concurrent else None

    def step():
        if concurrent:
            return list(pool.map(strand, (False, True)))
        return [strand(False), strand(True)]

    for k in range(a.warmup):
        step()
        print("[bench] warmup %d done" % k, file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    res, main_ms, op_ms = None, [], []
    for k in range(steps):
        res = step()
        main_ms.append(sum(st["ms_main"] for _, _, st in res))
        op_ms.append(sum(st["ms_onepass"] for _, _, st in res))
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_per_step = dt / steps * 1e3
    cells = 0
    per_strand = []
    for n, h, st in res:
        hh = h.cpu().numpy()
        cells += int(hh[:, 8].sum())
        per_strand.append({"seeds": int(n), "covered": int(((hh[:, 1] & fz.FZ_HIT_COVERED) != 0).sum()),
                           "traced": int(((hh[:, 1] & fz.FZ_HIT_TRACED) != 0).sum())})
    kern_s = float(np.mean(main_ms)) / 1e3
    packed = all(int(st["n_packed"]) > 0 for _, _, st in res)
    peak = (VALU_PEAK_OPS_PK16 if packed else VALU_PEAK_OPS) / 1e12
    op_cells = sum(int(st["onepass_cells"]) for _, _, st in res)
    dom, kernels = extension_kernels(cells, op_cells, kern_s * 1e3, float(np.mean(op_ms)), peak)
    bases = int(w["target"].size + w["query"].size)
    out = {"metric": "whole-pair alignment (seed stage + covered-seed rounds, both strands) on a 20 Mbp "
                     "chromosome pair, 1 MI355X",
           "value": round(bases / (ms_per_step / 1e3) / 1e6, 3), "unit": "Mbp/s", "n_gpus": 1, "steps": steps,
           "warmup": a.warmup, "ms_per_step": round(ms_per_step, 3), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "int16x2" if packed else "int32", "data": "synthetic",
           "config": {"workload": "chromosome_pipeline", "target_bp": int(w["target"].size),
                      "query_bp": int(w["query"].size), "k": w["k"], "flank": w["flank"], "round_size": a.round_size,
                      "round_doubling": bool(a.round_doubling), "strands_run": a.strands,
                      "min_traceback_score": 3000, "cells_per_step": cells, "strands": per_strand,
                      "inspector_ms": round(kern_s * 1e3, 3)},
           "roofline": {"bound": "alu", "achieved": dom["achieved"], "peak": round(peak, 3), "unit": "TOP/s",
                        "frac": dom["frac"], "traffic": None, "kernel": dom["kernel"] + ", all rounds",
                        "ops_per_cell": OPS_PER_CELL["extend"], "kernels": kernels}}
    if not a.no_cpu:
        print("[bench] CPU oracle sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_pipeline_baseline(w, a.cpu_seconds, a.round_size, a.round_doubling)
    if pool is not None:
        pool.shutdown()
    for c in ctxs:
        c.close()
    print(json.dumps(out), flush=True)


def call_overhead_ms(ctx, T, Q, S, w, min_tb, calls=20):
    """Median wall time of a one-seed call: the fixed cost of the call's
    launches and its host read-backs of sizes."""
    import numpy as np
    import torch
    one = S[:1].contiguous()
    times = []
    for _ in range(calls):
        torch.cuda.synchronize()
        t = time.perf_counter()
        ctx.extend(T, Q, one, w["scoring"], w["ydrop"], min_tb, traceback=w.get("traceback", True))
        torch.cuda.synchronize()
        times.append((time.perf_counter() - t) * 1e3)
    return float(np.median(times))


def measured_valu_peak(packed=False):
    """int32 add/max issue rate measured by libfz_probe.so (TOP/s of lane
    operations; packed: v_pk_add_u16 / v_pk_max_i16, TOP/s of 16-bit
    operations), or None when the probe is not built."""
    import ctypes
    path = os.path.join(ROOT, "smith_waterman_dp_amd", "libfz_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    fn = lib.fz_probe_valu_pk16 if packed else lib.fz_probe_valu
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_float),
                   ctypes.POINTER(ctypes.c_double)]
    ms, ops = ctypes.c_float(0), ctypes.c_double(0)
    if fn(0, 8, 1 << 14, ctypes.byref(ms), ctypes.byref(ops)) != 0 or ms.value <= 0:
        return None
    return round(ops.value / (ms.value / 1e3) / 1e12, 3)


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (--gpus %d refused)" % a.gpus,
              file=sys.stderr)
        sys.exit(2)
    if a.workload == "seeds":
        return bench_seeds(a)
    if a.workload == "pipeline":
        return bench_pipeline(a)
    import numpy as np
    import torch

    from smith_waterman_dp_amd import fz

    local = a.workload == "local"
    steps = a.steps if a.steps is not None else (20 if local else 5)
    print("[bench] generating workload %s" % a.workload, file=sys.stderr, flush=True)
    t = time.time()
    w = make_workload(a.workload)
    print("[bench] generated in %.1fs: %d records" % (time.time() - t, len(w["seeds"])), file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    T = torch.from_numpy(w["target"]).to(dev)
    Q = torch.from_numpy(w["query"]).to(dev)
    S = torch.from_numpy(w["seeds"]).to(dev)
    ctx = fz.Context(0)
    min_tb = w.get("min_tb")
    min_tb = -(1 << 62) if min_tb is None else min_tb

    rounds = a.workload == "chromosome_rounds"

    def step():
        rc = bool(w.get("query_rc"))
        if local:
            return ctx.local(T, Q, S, w["scoring"], want_stats=True, query_rc=rc)
        if rounds:
            return ctx.extend_rounds(T, Q, S, w["scoring"], w["ydrop"], min_tb, a.round_size, want_stats=True,
                                     query_rc=rc, doubling=a.round_doubling, two_pass=a.two_pass)
        return ctx.extend(T, Q, S, w["scoring"], w["ydrop"], min_tb, traceback=w.get("traceback", True),
                          want_stats=True, query_rc=rc, two_pass=a.two_pass)

    for k in range(a.warmup):
        step()
        print("[bench] warmup %d done" % k, file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    main_ms, step_ms, op_ms = [], [], []
    t0 = time.perf_counter()
    hits = None
    st = None
    for k in range(steps):
        ts = time.perf_counter()
        hits, cig, st = step()
        torch.cuda.synchronize()
        step_ms.append((time.perf_counter() - ts) * 1e3)
        main_ms.append(st["ms_main"])
        op_ms.append(0.0 if local else st["ms_onepass"])
        print("[bench] step %d: %.1f ms (dominant kernel %.1f ms%s)" % (
            k, step_ms[-1], st["ms_main"], "" if local else ", one-pass %.1f ms, exec %.1f ms" % (
                st["ms_onepass"], st["ms_exec"])), file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    call_ms = None if local or rounds else call_overhead_ms(ctx, T, Q, S, w, min_tb)
    plain_ms = None
    if rounds:
        # the same seeds as one ordinary batch, for comparison (not timed above)
        t1 = time.perf_counter()
        ctx.extend(T, Q, S, w["scoring"], w["ydrop"], min_tb)
        torch.cuda.synchronize()
        plain_ms = (time.perf_counter() - t1) * 1e3
    copy_probe(a.copy_probe, dev)
    h = hits.cpu().numpy()
    cells = int(h[:, 8].sum())
    n = len(w["seeds"])
    # the median step (every step is one call, synchronised at its end)
    ms_per_step = float(np.median(step_ms))
    gcups = cells / (ms_per_step / 1e3) / 1e9
    ops = OPS_PER_CELL["local" if local else "extend"]
    kern_s = float(np.median(main_ms)) / 1e3
    # the extension's cells run in packed 16-bit layouts when the scoring
    # allows it (every side after its first 34 anti-diagonals): their peak
    # is the packed rate
    packed = (not local) and int(st["n_packed"]) > 0
    peak = (VALU_PEAK_OPS_PK16 if packed else VALU_PEAK_OPS) / 1e12
    if local:
        dom = {"kernel": "local_kernel", "cells": cells, "ms": round(kern_s * 1e3, 3),
               "achieved": round(ops * cells / kern_s / 1e12, 3)}
        dom["frac"] = round(dom["achieved"] / peak, 4)
        kernels = [dom]
    else:
        dom, kernels = extension_kernels(cells, int(st["onepass_cells"]), kern_s * 1e3, float(np.median(op_ms)), peak)
    traffic = None
    if a.workload == "skewed" and kernel_src_hash() == TRAFFIC_SRC_HASH:
        for k in kernels:
            if k["kernel"] in TRAFFIC:
                k["traffic"] = measured_traffic(*TRAFFIC[k["kernel"]], k["ms"] / 1e3)
        traffic = dom.get("traffic")
    cfg = {"workload": a.workload, "records": n, "target_bp": int(w["target"].size), "query_bp": int(w["query"].size),
           "cells_per_step": cells, "scoring": w["scoring"], "ydrop": None if local else w["ydrop"],
           "min_traceback_score": w.get("min_tb"), "main_kernel_ms": round(kern_s * 1e3, 3),
           "timing": "median of %d steps after %d warm-up; mean %.3f ms" % (steps, a.warmup, dt / steps * 1e3)}
    if call_ms is not None:
        cfg["call_ms"] = round(call_ms, 3)
    if not local:
        cfg["extensions_per_sec"] = round(n / (ms_per_step / 1e3), 1)
        # last step's statistics (phase times are stream-event spans; "exec"
        # covers the executor batches with their walks)
        cfg["executor_cells"] = int(st["executor_cells"])
        cfg["pointer_bytes"] = int(st["pointer_bytes"])
        cfg["executor_sides"] = int(st["n_executor"])
        cfg["executor_batches"] = int(st["n_batches"])
        cfg["onepass_sides"] = int(st["n_onepass"])
        cfg["onepass_cells"] = int(st["onepass_cells"])
        cfg["onepass_pool_bytes"] = int(st["onepass_bytes"])
        cfg["tail_walked_sides"] = int(st["n_tail_walked"])
        cfg["phase_ms"] = {k[3:]: round(float(st[k]), 1) for k in
                           ("ms_pack", "ms_inspect", "ms_onepass", "ms_bin", "ms_exec", "ms_walk", "ms_gather")}
        cfg["max_band"] = int(st["max_band"])
    if rounds:
        from smith_waterman_dp_amd import fz as _fz
        cfg["round_size"] = a.round_size
        cfg["round_doubling"] = bool(a.round_doubling)
        r0, size, nr = 0, a.round_size, 0
        while r0 < n:
            r0, nr = r0 + size, nr + 1
            size *= 2 if a.round_doubling else 1
        cfg["rounds"] = nr
        cfg["covered_seeds"] = int(((h[:, 1] & _fz.FZ_HIT_COVERED) != 0).sum())
        cfg["plain_batch_ms"] = round(plain_ms, 1)
    out = {"metric": METRIC if a.workload == "skewed" else "GCUPS on the %s batch, 1 MI355X" % a.workload,
           "value": round(gcups, 3), "unit": "GCUPS", "n_gpus": 1, "steps": steps, "warmup": a.warmup,
           "ms_per_step": round(ms_per_step, 3), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "int16x2" if packed else "int32", "data": "synthetic", "config": cfg,
           "roofline": {"bound": "alu", "achieved": dom["achieved"], "peak": round(peak, 3), "unit": "TOP/s",
                        "frac": dom["frac"], "traffic": traffic, "kernel": dom["kernel"],
                        "ops_per_cell": ops, "kernels": kernels,
                        # the whole call against the same peak: ops_per_cell x GCUPS
                        "end_to_end": {"achieved": round(ops * gcups / 1e3, 3),
                                       "frac": round(ops * gcups / 1e3 / peak, 4),
                                       "frac_of_int32_peak": round(ops * gcups / 1e3 / (VALU_PEAK_OPS / 1e12), 4)}}}
    if packed:
        # for comparison with 32-bit builds: the same figure against the
        # int32 lane rate
        out["roofline"]["frac_of_int32_peak"] = round(dom["achieved"] / (VALU_PEAK_OPS / 1e12), 4)
        out["roofline"]["arith"] = "packed int16 pairs after anti-diagonal 33, int32 before"
    probe = measured_valu_peak(packed)
    if probe is not None:
        out["roofline"]["peak_measured"] = probe
    if not a.no_cpu:
        print("[bench] CPU oracle sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, a.cpu_seconds, local)
    ctx.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

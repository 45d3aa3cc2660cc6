"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer work, so the bar is bit-exact: scores, coordinates, canonical cell
counts, per-side scores and CIGAR words.  Full batches are compared where
the oracle finishes in seconds; at full workload sizes a seeded sample of
seeds is compared one by one and the rest is checked through invariants
that hold at any size (CIGAR rescoring, spans).
"""
import os
import random

import numpy as np
import pytest

import oracle
from smith_waterman_dp_amd import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from smith_waterman_dp_amd import fz  # noqa: E402

SC = dict(W.DEFAULT_SCORING)

# The first design of the extension kernel (a persistent grid pulling sides
# from an atomic work queue) went silent on the first extension call it was
# given, test_tiny_full's batch.  The cause is in its compiled code: at the
# end of a side lanes 1..63 took the loop's back edge without lane 0, read
# side index 0 from lane 1 through readfirstlane and re-ran side 0 forever
# (the exit mask on that path held lane 0 only).  Every wave of every batch
# hung after its first side; the batch itself was not special.  The current
# kernels take their side from blockIdx and have no per-lane loop exit
# (tests/test_kernel_isa.py checks the compiled code for it).
OK_BITS = (fz.FZ_HIT_TRACED | fz.FZ_HIT_EAGER_LEFT | fz.FZ_HIT_EAGER_RIGHT | fz.FZ_HIT_BELOW_MIN
           | fz.FZ_HIT_WIDE)


def log(msg):
    print("[gpu] " + msg, flush=True)


@pytest.fixture(scope="module")
def ctx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    log("torch device init")
    torch.zeros(1, device="cuda:0").add_(1)
    torch.cuda.synchronize()
    log("torch device ready; creating libfz context")
    c = fz.Context(0)
    yield c
    c.close()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def run_gpu(ctx, w, seeds=None, local=False, ydrop=None, min_tb=None, traceback=True, scoring=None,
            two_pass=False):
    seeds = w["seeds"] if seeds is None else seeds
    sc = scoring or w["scoring"]
    T, Q, S = dev(w["target"]), dev(w["query"]), dev(seeds)
    log("call %s: %d records, target %d, query %d" % ("local" if local else "extend", len(seeds),
                                                      T.numel(), Q.numel()))
    rc = bool(w.get("query_rc"))
    if local:
        hits, cig, st = ctx.local(T, Q, S, sc, want_stats=True, query_rc=rc)
    else:
        yd = w["ydrop"] if ydrop is None else ydrop
        mt = -(1 << 62) if min_tb is None else min_tb
        hits, cig, st = ctx.extend(T, Q, S, sc, yd, mt, traceback=traceback, want_stats=True, query_rc=rc,
                                   two_pass=two_pass)
    torch.cuda.synchronize()
    log("call done")
    return hits.cpu().numpy(), cig.cpu().numpy().view(np.uint32), st


def oracle_query(w):
    """The query as the oracle sees it: with query_rc, its reverse complement."""
    return oracle.revcomp(w["query"]) if w.get("query_rc") else w["query"]


def run_oracle(w, seeds=None, local=False, ydrop=None, min_tb=None, traceback=True, scoring=None):
    seeds = w["seeds"] if seeds is None else seeds
    yd = w["ydrop"] if ydrop is None else ydrop
    return oracle.run(w["target"], oracle_query(w), seeds, scoring or w["scoring"], yd, min_tb=min_tb,
                      traceback=traceback, local=local)


def compare(gh, gc, oh, ow, oo, idx=None, local=False, label=""):
    """Element-by-element comparison; idx maps oracle rows to GPU rows."""
    n = len(oh)
    idx = np.arange(n) if idx is None else idx
    bad = []
    for k in range(n):
        g = dict(zip(fz.HIT_FIELDS, gh[idx[k]].tolist()))
        o = oh[k]
        if o["status"] != 0:
            if o["status"] & oracle.STATUS_ESEED:
                if not g["status"] & fz.FZ_HIT_ESEED:
                    bad.append((k, "status", g["status"], int(o["status"])))
            continue
        if g["status"] & ~OK_BITS:
            bad.append((k, "status", g["status"], 0))
            continue
        fields = [("score", "score"), ("t_begin", "t_begin"), ("t_end", "t_end"), ("q_begin", "q_begin"),
                  ("q_end", "q_end")]
        if not local:
            fields += [("score_left", "score_l"), ("score_right", "score_r")]
        for gf, of in fields:
            if g[gf] != int(o[of]):
                bad.append((k, gf, g[gf], int(o[of])))
        cells = int(o["cells_r"]) if local else int(o["cells_l"] + o["cells_r"])
        if g["cells"] != cells:
            bad.append((k, "cells", g["cells"], cells))
        if not local:
            got = gc[g["cigar_off"]:g["cigar_off"] + g["cigar_len"]]
            exp = ow[oo[k]:oo[k] + o["n_runs"]]
            if not np.array_equal(got, exp):
                bad.append((k, "cigar", oracle.cigar_string(got)[:80], oracle.cigar_string(exp)[:80]))
    if bad:
        print("%s: %d mismatching fields, first ones:" % (label, len(bad)))
        for b in bad[:12]:
            print("   ", b)
    assert not bad, "%s: %d mismatches, first %s" % (label, len(bad), bad[:3])


# ---------------------------------------------------------------- tiny --

def test_tiny_full(ctx):
    """1,000 seeds, 256-bp flanks: the whole batch, every field."""
    w = W.tiny()
    gh, gc, st = run_gpu(ctx, w)
    oh, ow, oo = run_oracle(w)
    compare(gh, gc, oh, ow, oo, label="tiny")
    assert st["cells"] == int((oh["cells_l"] + oh["cells_r"]).sum())


def test_deterministic(ctx):
    """The same batch twice gives the same hits and CIGAR words bit for bit."""
    w = W.tiny(n_seeds=200, seed=5)
    a = run_gpu(ctx, w)
    b = run_gpu(ctx, w)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def random_case_workload(rng, n):
    """P3's recipe: many small random cases with random scoring, windows
    from 0 to 70 bases per side, related and unrelated flanks."""
    tp, qp, rows = [], [], []
    to = qo = 0
    for _ in range(n):
        L = rng.choice([0, 1, 5, 19])
        ml, mr = rng.randint(0, 70), rng.randint(0, 70)
        t = "".join(rng.choice("ACGT") for _ in range(ml + L + mr))
        if rng.random() < 0.6:
            q = list(t)
            for _ in range(rng.randint(0, 8)):
                p = rng.randrange(len(q)) if q else 0
                r = rng.random()
                if r < 0.3 and q:
                    del q[p]
                elif r < 0.6:
                    q.insert(p, rng.choice("ACGT"))
                elif q:
                    q[p] = rng.choice("ACGT")
            q = "".join(q)
            # keep the seed columns exact
            q = q[:ml] + t[ml:ml + L] + q[ml + L:] if len(q) >= ml + L else t
        else:
            q = "".join(rng.choice("ACGT") for _ in range(rng.randint(0, 70))) + t[ml:ml + L] + \
                "".join(rng.choice("ACGT") for _ in range(rng.randint(0, 70)))
        qpos = q.find(t[ml:ml + L]) if L else rng.randint(0, len(q))
        if qpos < 0:
            q, qpos = t, ml
        tp.append(t)
        qp.append(q)
        rows.append((to + ml, qo + qpos, L, to, to + len(t), qo, qo + len(q)))
        to += len(t)
        qo += len(q)
    T = np.frombuffer("".join(tp).encode(), dtype=np.uint8).copy()
    Q = np.frombuffer("".join(qp).encode(), dtype=np.uint8).copy()
    return dict(target=T, query=Q, seeds=np.array(rows, dtype=np.int64).reshape(-1, 7), scoring=dict(SC),
                ydrop=9400)


@pytest.mark.parametrize("case", range(6))
def test_random_small_batches(ctx, case):
    rng = random.Random(40 + case)
    w = random_case_workload(rng, 100)
    if case % 2:
        w["scoring"] = dict(match=rng.randint(1, 120), transition=rng.randint(-150, 40),
                            transversion=rng.randint(-200, 0), gap_open=rng.randint(0, 500),
                            gap_extend=rng.randint(1, 80))
    if case == 5:   # scores outside int8: the general substitution path
        w["scoring"] = dict(match=300, transition=-200, transversion=-400, gap_open=700, gap_extend=90)
    for ydrop in (0, 150, 1000, 9400, fz.FZ_YDROP_INF):
        gh, gc, _ = run_gpu(ctx, w, ydrop=ydrop)
        oh, ow, oo = run_oracle(w, ydrop=ydrop)
        compare(gh, gc, oh, ow, oo, label="random case %d ydrop %d" % (case, ydrop))


def test_min_traceback_gating(ctx):
    w = W.tiny(n_seeds=100, seed=9)
    thr = int(np.median(run_oracle(w, traceback=False)[0]["score"]))
    gh, gc, _ = run_gpu(ctx, w, min_tb=thr)
    oh, ow, oo = run_oracle(w, min_tb=thr)
    compare(gh, gc, oh, ow, oo, label="min_tb")
    traced = (gh[:, 1] & fz.FZ_HIT_TRACED) != 0
    assert np.array_equal(traced, oh["score"] > thr)
    assert np.array_equal((gh[:, 1] & fz.FZ_HIT_BELOW_MIN) != 0, oh["score"] <= thr)


def test_no_traceback_flag(ctx):
    w = W.tiny(n_seeds=50, seed=12)
    gh, gc, _ = run_gpu(ctx, w, traceback=False)
    oh, _, _ = run_oracle(w, traceback=False)
    assert np.array_equal(gh[:, 0], oh["score"])
    assert (gh[:, 7] == 0).all() and gc.size == 0


# --------------------------------------------------------------- edges --

def one_seed(t, q, t_pos, q_pos, L, t_lo=0, t_hi=None, q_lo=0, q_hi=None):
    t_hi = len(t) if t_hi is None else t_hi
    q_hi = len(q) if q_hi is None else q_hi
    return dict(target=np.frombuffer(t.encode(), dtype=np.uint8).copy(),
                query=np.frombuffer(q.encode(), dtype=np.uint8).copy(),
                seeds=np.array([[t_pos, q_pos, L, t_lo, t_hi, q_lo, q_hi]], dtype=np.int64),
                scoring=dict(SC), ydrop=9400)


def test_edge_seeds(ctx):
    rng = random.Random(3)
    s = "".join(rng.choice("ACGT") for _ in range(300))
    cases = [
        one_seed(s, s, 0, 0, 19),                     # empty left flank
        one_seed(s, s, 281, 281, 19),                 # empty right flank
        one_seed(s, s, 100, 100, 0),                  # zero-length seed
        one_seed(s, s, 140, 140, 19, 140, 159, 140, 159),   # both windows = the seed
        one_seed(s, s[:150] + "A" * 40 + s[150:], 50, 50, 19),   # 40-base insertion
        one_seed(s, s[:150] + s[190:], 50, 50, 19),   # 40-base deletion
        one_seed(s.lower(), s, 10, 10, 19),           # lower-case target
    ]
    for w in cases:
        gh, gc, _ = run_gpu(ctx, w)
        oh, ow, oo = run_oracle(w)
        compare(gh, gc, oh, ow, oo, label="edge")


def test_invalid_seed_status(ctx):
    s = "ACGT" * 50
    w = one_seed(s, s, 10, 10, 19)
    w["seeds"] = np.array([[10, 10, 19, 0, 200, 0, 200], [5, 5, 19, 10, 200, 0, 200],
                           [190, 10, 19, 0, 200, 0, 200], [10, 10, 19, 0, 400, 0, 200]], dtype=np.int64)
    gh, gc, _ = run_gpu(ctx, w)
    st = gh[:, 1]
    assert not st[0] & fz.FZ_HIT_ESEED
    assert all(st[k] & fz.FZ_HIT_ESEED for k in (1, 2, 3))
    oh, ow, oo = run_oracle(w)
    compare(gh, gc, oh, ow, oo, label="invalid seeds")


def test_non_acgt_rejected(ctx):
    w = one_seed("ACGTNACGT" * 10, "ACGTACGT" * 10, 0, 0, 4)
    with pytest.raises(fz.FzError) as e:
        run_gpu(ctx, w)
    assert e.value.code == fz.FZ_EINVAL


def test_empty_batch(ctx):
    w = one_seed("ACGT" * 10, "ACGT" * 10, 0, 0, 4)
    w["seeds"] = np.zeros((0, 7), dtype=np.int64)
    gh, gc, _ = run_gpu(ctx, w)
    assert gh.shape == (0, 12) and gc.size == 0


def test_wide_band_and_overflow(ctx):
    """No pruning on identical 700-base flanks: the band (701 wide) outgrows
    the standard window and is redone by the wide one; at 1,300 bases it
    outgrows that too and the seed reports FZ_HIT_EBAND."""
    rng = random.Random(8)
    s = "".join(rng.choice("ACGT") for _ in range(1419))
    w = one_seed(s[:719], s[:719], 0, 0, 19)
    gh, gc, st = run_gpu(ctx, w, ydrop=fz.FZ_YDROP_INF)
    oh, ow, oo = run_oracle(w, ydrop=oracle.YDROP_INF)
    compare(gh, gc, oh, ow, oo, label="wide")
    assert st["n_overflow"] >= 1 and gh[0, 1] & fz.FZ_HIT_WIDE
    w2 = one_seed(s, s, 0, 0, 19)
    gh2, _, _ = run_gpu(ctx, w2, ydrop=fz.FZ_YDROP_INF)
    assert gh2[0, 1] & fz.FZ_HIT_EBAND


def test_pointer_workspace_batches(ctx):
    """A tiny pointer workspace forces many executor batches; results equal.
    (Two-pass: the cap would otherwise serve most sides in one-pass rounds.)"""
    w = W.executor_heavy(n_pairs=60, len_min=300, len_max=3000, seed=4)
    ref = run_gpu(ctx, w)
    fz.fz_set_pointer_workspace(ctx.h, 4 << 20)
    try:
        gh, gc, st = run_gpu(ctx, w, two_pass=True)
    finally:
        fz.fz_set_pointer_workspace(ctx.h, 0)
    assert st["n_batches"] > 1
    assert np.array_equal(gh, ref[0]) and np.array_equal(gc, ref[1])
    oh, ow, oo = run_oracle(w)
    compare(gh, gc, oh, ow, oo, label="executor batches")


def test_workspace_cap_at_create():
    """fz_create's workspace_bytes caps the pointer workspace as
    fz_set_pointer_workspace does: many batches, the same results."""
    w = W.executor_heavy(n_pairs=40, len_min=300, len_max=3000, seed=6)
    c0 = fz.Context(0)
    c1 = fz.Context(0, workspace_bytes=4 << 20)
    try:
        ref = run_gpu(c0, w)
        gh, gc, st = run_gpu(c1, w, two_pass=True)
    finally:
        c0.close()
        c1.close()
    assert st["n_batches"] > 1
    assert np.array_equal(gh, ref[0]) and np.array_equal(gc, ref[1])


def test_executor_mismatch_is_reported(ctx):
    """A forced disagreement between executor and inspector (every executor
    side gets one pointer-row word fewer than the inspector sized, so the
    executor's row-capacity check trips) comes back as FZ_HIT_EEXEC on the
    affected seeds, without a CIGAR, while scores and coordinates stay the
    oracle's; seeds traced wholly in the inspector are untouched."""
    w = W.tiny(n_seeds=150, seed=12)
    oh, ow, oo = run_oracle(w)
    fz.fz_debug_set(ctx.h, fz.FZ_DEBUG_SHRINK_ROWS, 1)
    try:
        gh, gc, st = run_gpu(ctx, w)
    finally:
        fz.fz_debug_set(ctx.h, fz.FZ_DEBUG_SHRINK_ROWS, 0)
    assert st["n_executor"] > 0
    eager_both = fz.FZ_HIT_EAGER_LEFT | fz.FZ_HIT_EAGER_RIGHT
    n_flagged = 0
    for k in range(len(oh)):
        g = dict(zip(fz.HIT_FIELDS, gh[k].tolist()))
        for gf, of in (("score", "score"), ("t_begin", "t_begin"), ("t_end", "t_end"), ("q_begin", "q_begin"),
                       ("q_end", "q_end")):
            assert g[gf] == int(oh[of][k]), (k, gf)
        if (g["status"] & eager_both) == eager_both:
            assert g["status"] & fz.FZ_HIT_TRACED and not g["status"] & fz.FZ_HIT_EEXEC, k
        else:
            assert g["status"] & fz.FZ_HIT_EEXEC and not g["status"] & fz.FZ_HIT_TRACED, k
            assert g["cigar_len"] == 0
            n_flagged += 1
    assert n_flagged > 0
    # normal sizing again: every field matches
    gh, gc, st = run_gpu(ctx, w)
    compare(gh, gc, oh, ow, oo, label="after shrink")
    assert st["max_band"] > 0 and st["ms_walk"] > 0
    with pytest.raises(fz.FzError):
        fz.fz_debug_set(ctx.h, 99, 1)


# --------------------------------------------------------------- local --

def test_local_small_full(ctx):
    w = W.local_pairs(n_pairs=96, length=300, seed=2)
    gh, _, _ = run_gpu(ctx, w, local=True)
    oh, ow, oo = run_oracle(w, local=True, traceback=False)
    compare(gh, None, oh, ow, oo, local=True, label="local 300")


def test_local_ragged_and_strips(ctx):
    """Windows of many shapes, including ones taller than one 2,048-row strip
    and empty ones."""
    rng = np.random.default_rng(6)
    shapes = [(0, 5), (5, 0), (1, 1), (63, 64), (2048, 100), (2049, 77), (3000, 500), (4500, 260), (129, 2500)]
    tp, qp, rows = [], [], []
    to = qo = 0
    for (m, n) in shapes:
        tp.append(W.random_codes(rng, m))
        q = W.random_codes(rng, n)
        if m and n:   # plant a shared stretch so scores are not tiny
            L = min(m, n, 60)
            q[:L] = tp[-1][:L]
        qp.append(q)
        rows.append((to, qo, 0, to, to + m, qo, qo + n))
        to += m
        qo += n
    w = dict(target=W.to_ascii(np.concatenate(tp)), query=W.to_ascii(np.concatenate(qp)),
             seeds=np.array(rows, dtype=np.int64), scoring=dict(SC), ydrop=0)
    gh, _, _ = run_gpu(ctx, w, local=True)
    oh, ow, oo = run_oracle(w, local=True, traceback=False)
    compare(gh, None, oh, ow, oo, local=True, label="local ragged")


def test_local_identical_closed_form(ctx):
    rng = np.random.default_rng(1)
    a = W.to_ascii(W.random_codes(rng, 2048))
    w = dict(target=a, query=a.copy(), seeds=np.array([[0, 0, 0, 0, 2048, 0, 2048]], dtype=np.int64),
             scoring=dict(SC), ydrop=0)
    gh, _, _ = run_gpu(ctx, w, local=True)
    assert (gh[0, 0], gh[0, 3], gh[0, 5]) == (91 * 2048, 2048, 2048)


def test_local_full_size_all(ctx):
    """The 4,096 x 2048^2 batch in the benchmark's launch configuration:
    every pair against the oracle."""
    w = W.local_pairs()
    gh, _, _ = run_gpu(ctx, w, local=True)
    log("local full: oracle on all %d pairs" % len(w["seeds"]))
    oh, ow, oo = run_oracle(w, local=True, traceback=False)
    compare(gh, None, oh, ow, oo, local=True, label="local full")
    assert (gh[:, 0] >= 0).all()


# ------------------------------------------------------- larger batches --

def check_invariants(w, gh, gc, label):
    """Every traced seed's CIGAR, laid on the sequences from its begin
    coordinates, rescores to its score and ends at its end coordinates
    (oracle.rescore, any batch size).  Returns the number checked."""
    traced = np.nonzero(gh[:, 1] & fz.FZ_HIT_TRACED)[0]
    if traced.size == 0:
        return 0
    s, te, qe, bad = oracle.rescore(w["target"], oracle_query(w), gh[traced, 2], gh[traced, 4], gh[traced, 6],
                                    gh[traced, 7], gc, w["scoring"])
    assert bad == 0, (label, bad)
    wrong = np.nonzero((s != gh[traced, 0]) | (te != gh[traced, 3]) | (qe != gh[traced, 5]))[0]
    assert wrong.size == 0, (label, "seed", int(traced[wrong[0]]), int(s[wrong[0]]), gh[traced[wrong[0]]].tolist())
    log("%s: %d traced alignments rescored" % (label, traced.size))
    return traced.size


def sample_compare(ctx, w, n_sample, label, seed=0, extra_idx=None):
    gh, gc, st = run_gpu(ctx, w, min_tb=w.get("min_tb"))
    rng = np.random.default_rng(seed)
    n = len(w["seeds"])
    idx = rng.choice(n, min(n_sample, n), replace=False)
    if extra_idx is not None:
        idx = np.concatenate([idx, extra_idx])
    idx = np.unique(idx)
    oh, ow, oo = run_oracle(w, seeds=w["seeds"][idx], min_tb=w.get("min_tb"))
    compare(gh, gc, oh, ow, oo, idx=idx, label=label)
    assert not (gh[:, 1] & (fz.FZ_HIT_EBAND | fz.FZ_HIT_ERANGE)).any(), label
    return gh, gc, st


def test_skewed_reduced(ctx):
    w = W.skewed(target_len=1_000_000, n_seeds=20_000, n_short=30, n_long=10, seed=1)
    gh, gc, st = sample_compare(ctx, w, 400, "skewed reduced")
    check_invariants(w, gh, gc, "skewed reduced")


def test_executor_heavy_reduced(ctx):
    w = W.executor_heavy(n_pairs=400, seed=2)
    gh, gc, st = sample_compare(ctx, w, 120, "executor heavy reduced")
    check_invariants(w, gh, gc, "executor heavy reduced")


def test_chromosome_reduced(ctx):
    w = W.chromosome(length=600_000, inv_min=5_000, inv_max=20_000, seed=3)
    gh, gc, st = sample_compare(ctx, w, 40, "chromosome reduced")
    check_invariants(w, gh, gc, "chromosome reduced")


def stratified(gh, rng, n_uniform, per_bin, n_wide, n_eager, n_below, n_longest):
    """Seed indices for a full-size comparison: a uniform draw, then up to
    per_bin seeds of every executor length bin, the sides redone in the wide
    window, seeds traced wholly (or half) in the inspector, seeds below the
    traceback threshold, and the longest alignments."""
    n = len(gh)
    parts = [rng.choice(n, min(n_uniform, n), replace=False)]

    def some(mask, k):
        cand = np.nonzero(mask)[0]
        return rng.choice(cand, min(k, cand.size), replace=False) if cand.size else cand

    st = gh[:, 1]
    for b in range(8):
        parts.append(some(gh[:, 11] == b, per_bin))
    parts.append(some((st & fz.FZ_HIT_WIDE) != 0, n_wide))
    both = fz.FZ_HIT_EAGER_LEFT | fz.FZ_HIT_EAGER_RIGHT
    parts.append(some((st & both) == both, n_eager))
    parts.append(some(((st & both) != 0) & ((st & both) != both), n_eager))
    parts.append(some((st & fz.FZ_HIT_BELOW_MIN) != 0, n_below))
    span = gh[:, 3] - gh[:, 2]
    parts.append(np.argsort(span)[-n_longest:])
    return np.unique(np.concatenate(parts))


@pytest.mark.skipif(os.environ.get("FZ_FULL_SIZE", "1") == "0", reason="full-size runs disabled")
def test_skewed_full_size_stratified(ctx):
    """The one-million-seed skewed batch as the benchmark runs it: over
    10,000 seeds against the oracle field by field (a uniform draw plus
    every stratum: each executor length bin, wide-window retries, eager
    sides, untraced seeds, the longest alignments), and every traced
    alignment rescored."""
    w = W.skewed()
    gh, gc, st = run_gpu(ctx, w, min_tb=w["min_tb"])
    idx = stratified(gh, np.random.default_rng(0), 7200, 400, 600, 600, 400, 40)
    log("skewed full: oracle on %d seeds (%.3g cells)" % (len(idx), float(gh[idx, 8].sum())))
    assert len(idx) >= 10000
    oh, ow, oo = run_oracle(w, seeds=w["seeds"][idx], min_tb=w["min_tb"])
    compare(gh, gc, oh, ow, oo, idx=idx, label="skewed full")
    assert not (gh[:, 1] & (fz.FZ_HIT_EBAND | fz.FZ_HIT_ERANGE | fz.FZ_HIT_ESEED | fz.FZ_HIT_EEXEC)).any()
    assert check_invariants(w, gh, gc, "skewed full") == int(((gh[:, 1] & fz.FZ_HIT_TRACED) != 0).sum())


def _full_size_sampled(ctx, w, n_uniform, per_bin, n_longest, label):
    log("%s: %d records, target %d bp" % (label, len(w["seeds"]), w["target"].size))
    gh, gc, st = run_gpu(ctx, w, min_tb=w.get("min_tb"))
    log("%s: %d executor sides, %d batches, %.3g pointer bytes" % (label, st["n_executor"], st["n_batches"],
                                                                   st["pointer_bytes"]))
    idx = stratified(gh, np.random.default_rng(0), n_uniform, per_bin, per_bin, per_bin, per_bin, n_longest)
    oh, ow, oo = run_oracle(w, seeds=w["seeds"][idx], min_tb=w.get("min_tb"))
    log("%s: oracle done on %d records" % (label, len(idx)))
    compare(gh, gc, oh, ow, oo, idx=idx, label=label)
    assert not (gh[:, 1] & (fz.FZ_HIT_EBAND | fz.FZ_HIT_ERANGE | fz.FZ_HIT_ESEED | fz.FZ_HIT_EEXEC)).any(), label
    assert check_invariants(w, gh, gc, label) == int(((gh[:, 1] & fz.FZ_HIT_TRACED) != 0).sum())
    return idx


@pytest.mark.skipif(os.environ.get("FZ_FULL_SIZE", "1") == "0", reason="full-size runs disabled")
def test_executor_heavy_full_size_sampled(ctx):
    """100,000 pairs of 1-20 kb homology, every seed traced: 1,500 seeds by
    a seeded draw, up to 100 per executor length bin and the 20 longest
    alignments against the oracle; every traced alignment rescored."""
    log("generating the executor-heavy batch")
    _full_size_sampled(ctx, W.executor_heavy(), 1500, 100, 20, "executor heavy full")


@pytest.mark.skipif(os.environ.get("FZ_FULL_SIZE", "1") == "0", reason="full-size runs disabled")
def test_chromosome_full_size_sampled(ctx):
    """Two 20 Mbp chromosomes, all forward shared 19-mers after diagonal
    dedup: 600 seeds by a seeded draw, up to 40 per stratum and the 10
    longest alignments against the oracle; every traced alignment
    rescored."""
    log("generating the chromosome pair")
    _full_size_sampled(ctx, W.chromosome(), 600, 40, 10, "chromosome full")


# ------------------------------------------------------ reverse strand --

def on_reverse_strand(w):
    """The same alignments asked on the other strand: the query handed in is
    the reverse complement of w's query (built by the input generator), so
    with query_rc the library must see w's query again."""
    r = dict(w)
    r["query"] = W.to_ascii(W.revcomp_codes(np.searchsorted(np.frombuffer(b"ACGT", np.uint8),
                                                              np.asarray(w["query"], np.uint8))))
    r["query_rc"] = True
    return r


def test_query_rc_tiny_full(ctx):
    """A 200-seed tiny batch through FZ_QUERY_RC: every field against the
    oracle on the reverse complement, and identical to the forward call."""
    w = W.tiny(n_seeds=200, seed=21)
    r = on_reverse_strand(w)
    gh, gc, st = run_gpu(ctx, r)
    oh, ow, oo = run_oracle(r)
    compare(gh, gc, oh, ow, oo, label="query_rc tiny")
    fh, fc, _ = run_gpu(ctx, w)
    assert np.array_equal(fh, gh) and np.array_equal(fc, gc)


def test_query_rc_local(ctx):
    w = W.local_pairs(n_pairs=24, length=300, seed=22)
    r = on_reverse_strand(w)
    gh, gc, st = run_gpu(ctx, r, local=True)
    oh, ow, oo = run_oracle(r, local=True)
    compare(gh, gc, oh, ow, oo, local=True, label="query_rc local")


def test_chromosome_rc_reduced(ctx):
    """Reverse-strand seeds of a 600 kb chromosome pair (the inversions)."""
    w = W.chromosome_rc(length=600_000, inv_min=5_000, inv_max=20_000, seed=3)
    gh, gc, st = sample_compare(ctx, w, 40, "chromosome rc reduced")
    check_invariants(w, gh, gc, "chromosome rc reduced")


@pytest.mark.skipif(os.environ.get("FZ_FULL_SIZE", "1") == "0", reason="full-size runs disabled")
def test_chromosome_rc_full_size_sampled(ctx):
    """The 20 Mbp chromosome pair searched on the reverse strand (seeds in
    the five inversions and chance hits): 400 seeds by a seeded draw, up to
    30 per stratum and the 6 longest alignments against the oracle; every
    traced alignment rescored."""
    log("generating the chromosome pair, reverse-strand seeds")
    _full_size_sampled(ctx, W.chromosome_rc(), 400, 30, 6, "chromosome rc full")


# ------------------------------------------------ 4x4 matrix and N ---

def sprinkle_n(rng, seq, rate):
    a = np.array(seq, dtype=np.uint8, copy=True)
    hit = np.array([rng.random() < rate for _ in range(a.size)], dtype=bool)
    a[hit] = ord("N") if rng.random() < 0.5 else ord("n")
    return a


def rand_matrix(rng):
    return [[rng.randint(-128, 127) for _ in range(4)] for _ in range(4)]


@pytest.mark.parametrize("case", range(4))
def test_matrix_random_small_batches(ctx, case):
    """Random cases, random asymmetric int8 matrices and N scores, N in
    both sequences (seed columns included), every field against the
    oracle at several y-drops."""
    rng = random.Random(90 + case)
    w = random_case_workload(rng, 100)
    w["target"] = sprinkle_n(rng, w["target"], 0.03)
    w["query"] = sprinkle_n(rng, w["query"], 0.03)
    mat = rand_matrix(rng)
    for a in range(4):       # matches positive so extensions run
        mat[a][a] = rng.randint(20, 127)
    w["scoring"] = dict(matrix=mat, n_score=rng.randint(-128, 127), gap_open=rng.randint(0, 400),
                        gap_extend=rng.randint(1, 60))
    for ydrop in (0, 150, 1000, fz.FZ_YDROP_INF):
        gh, gc, _ = run_gpu(ctx, w, ydrop=ydrop)
        oh, ow, oo = run_oracle(w, ydrop=ydrop)
        compare(gh, gc, oh, ow, oo, label="matrix case %d ydrop %d" % (case, ydrop))


def test_matrix_of_triple_equals_triple(ctx):
    """The triple written as a matrix runs the matrix kernels and gives the
    triple kernels' results bit for bit."""
    w = W.tiny(n_seeds=400, seed=31)
    sc = w["scoring"]
    cls = {0: "match", 2: "transition"}
    mat = [[sc[cls.get(x ^ y, "transversion")] for y in range(4)] for x in range(4)]
    wm = dict(w, scoring=dict(matrix=mat, n_score=-128, gap_open=sc["gap_open"], gap_extend=sc["gap_extend"]))
    h1, c1, _ = run_gpu(ctx, w)
    h2, c2, _ = run_gpu(ctx, wm)
    assert np.array_equal(h1, h2) and np.array_equal(c1, c2)


def test_matrix_tiny_with_n(ctx):
    rng = np.random.default_rng(4)
    w = W.with_matrix_and_n(W.tiny(n_seeds=500, seed=32), 60, 1, 40, seed=5)
    assert (w["target"] == ord("N")).any() and (w["query"] == ord("N")).any()
    gh, gc, _ = run_gpu(ctx, w)
    oh, ow, oo = run_oracle(w)
    compare(gh, gc, oh, ow, oo, label="matrix tiny with N")
    check_invariants(w, gh, gc, "matrix tiny with N")


def test_matrix_reverse_strand(ctx):
    w = W.with_matrix_and_n(W.chromosome_rc(length=300_000, inv_min=5_000, inv_max=20_000, seed=6), 30, 5, 200,
                            seed=7)
    gh, gc, st = sample_compare(ctx, w, 60, "matrix chromosome rc reduced")
    check_invariants(w, gh, gc, "matrix chromosome rc reduced")


def test_matrix_local(ctx):
    rng = random.Random(12)
    w = W.local_pairs(n_pairs=48, length=300, seed=8)
    w["target"] = sprinkle_n(rng, w["target"], 0.02)
    w["query"] = sprinkle_n(rng, w["query"], 0.02)
    w["scoring"] = W.matrix_scoring()
    gh, gc, _ = run_gpu(ctx, w, local=True)
    oh, ow, oo = run_oracle(w, local=True)
    compare(gh, gc, oh, ow, oo, local=True, label="matrix local")


def test_matrix_skewed_reduced(ctx):
    w = W.with_matrix_and_n(W.skewed(target_len=1_000_000, n_seeds=20_000, n_short=30, n_long=10, seed=1),
                            60, 10, 1000, seed=9)
    gh, gc, st = sample_compare(ctx, w, 300, "matrix skewed reduced")
    check_invariants(w, gh, gc, "matrix skewed reduced")


def test_matrix_errors(ctx):
    w = W.tiny(n_seeds=4, seed=33)
    T = w["target"].copy()
    T[300] = ord("N")
    with pytest.raises(fz.FzError):                       # N without a matrix
        run_gpu(ctx, dict(w, target=T))
    bad = W.matrix_scoring()
    bad["matrix"][1][2] = 128
    with pytest.raises(fz.FzError):                       # entry outside int8
        run_gpu(ctx, dict(w, scoring=bad))
    bad = W.matrix_scoring(n_score=-129)
    with pytest.raises(fz.FzError):
        run_gpu(ctx, dict(w, scoring=bad))
    T[300] = ord("R")                                      # other letters stay invalid
    with pytest.raises(fz.FzError):
        run_gpu(ctx, dict(w, target=T, scoring=W.matrix_scoring()))


@pytest.mark.skipif(os.environ.get("FZ_FULL_SIZE", "1") == "0", reason="full-size runs disabled")
def test_skewed_matrix_full_size_sampled(ctx):
    """The matrix benchmark batch (one million seeds, runs of N): 1,500
    seeds by a seeded draw, up to 150 per stratum and the 20 longest
    alignments against the oracle; every traced alignment rescored."""
    w = W.skewed_matrix()
    _full_size_sampled(ctx, w, 1500, 150, 20, "skewed matrix full")


def test_matrix_wide_band(ctx):
    """The 1024-position retry in matrix mode: no pruning on 700-base flanks
    that hold N and an asymmetric matrix; every field against the oracle,
    and the reverse strand of the same pair."""
    rng = random.Random(18)
    s = list("".join(rng.choice("ACGT") for _ in range(719)))
    q = list(s)
    for p in rng.sample(range(30, 719), 40):
        q[p] = rng.choice("ACGTN")
    s, q = "".join(s), "".join(q)
    w = one_seed(s, q, 0, 0, 19)
    w["scoring"] = W.matrix_scoring()
    gh, gc, st = run_gpu(ctx, w, ydrop=fz.FZ_YDROP_INF)
    oh, ow, oo = run_oracle(w, ydrop=oracle.YDROP_INF)
    compare(gh, gc, oh, ow, oo, label="matrix wide")
    assert st["n_overflow"] >= 1
    wr = dict(w, query=np.frombuffer(oracle.revcomp(q).tobytes(), dtype=np.uint8).copy(), query_rc=True)
    gh2, gc2, _ = run_gpu(ctx, wr, ydrop=fz.FZ_YDROP_INF)
    oh2, ow2, oo2 = run_oracle(wr, ydrop=oracle.YDROP_INF)
    compare(gh2, gc2, oh2, ow2, oo2, label="matrix wide rc")


def test_matrix_local_strips(ctx):
    """Local mode in matrix mode on windows taller than one strip (2,048
    rows), so that the strip's last row is spilled and read back, with N."""
    rng = random.Random(19)
    w = W.local_pairs(n_pairs=6, length=2600, seed=20)
    w["target"] = sprinkle_n(rng, w["target"], 0.01)
    w["query"] = sprinkle_n(rng, w["query"], 0.01)
    w["scoring"] = W.matrix_scoring()
    gh, gc, _ = run_gpu(ctx, w, local=True)
    oh, ow, oo = run_oracle(w, local=True)
    compare(gh, gc, oh, ow, oo, local=True, label="matrix local strips")


WIDE_SC = dict(match=300, transition=-200, transversion=-400, gap_open=700, gap_extend=90)


def test_wide_scores_wide_band_and_strips(ctx):
    """Scores outside int8 (the general substitution path) in the
    1024-position retry and in local mode across strips."""
    rng = random.Random(21)
    s = list("".join(rng.choice("ACGT") for _ in range(719)))
    q = list(s)
    for p in rng.sample(range(30, 719), 40):
        q[p] = rng.choice("ACGT")
    w = one_seed("".join(s), "".join(q), 0, 0, 19)
    w["scoring"] = dict(WIDE_SC)
    gh, gc, st = run_gpu(ctx, w, ydrop=fz.FZ_YDROP_INF)
    oh, ow, oo = run_oracle(w, ydrop=oracle.YDROP_INF)
    compare(gh, gc, oh, ow, oo, label="wide scores, wide band")
    assert st["n_overflow"] >= 1
    wl = W.local_pairs(n_pairs=4, length=2300, seed=22)
    wl["scoring"] = dict(WIDE_SC)
    gh, gc, _ = run_gpu(ctx, wl, local=True)
    oh, ow, oo = run_oracle(wl, local=True)
    compare(gh, gc, oh, ow, oo, local=True, label="wide scores, local strips")

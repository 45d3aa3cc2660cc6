"""The one-pass executor against the two-pass inspector / executor scheme
(FZ_TWO_PASS) and the oracle.

A side whose best score at anti-diagonal 256 already makes its seed traced
(whatever the other side scores) and is still growing leaves the inspector
there; the one-pass executor extends it again from the start to its end,
finds its best cell and writes its pointer rows in the same pass, into
blocks of 64 anti-diagonals carved from a pool.  Every result -- hits, CIGAR
words, canonical cell counts -- must equal the two-pass run's.  The cases
cover batches of long homologous sides (most of them one-pass), thresholds
that make the hand-over test decide either way, pools too small for all
one-pass sides at once (served in rounds, walking each round's sides before
the next, and giving back sides that never fit), the pool turned
off, the pointer-workspace cap (which bounds the pool too), covered-seed
rounds, and the reverse strand.
"""
import numpy as np
import pytest

import oracle
from smith_waterman_dp_amd import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from smith_waterman_dp_amd import fz  # noqa: E402


def log(msg):
    print("[gpu] " + msg, flush=True)


@pytest.fixture(scope="module")
def ctx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.zeros(1, device="cuda:0").add_(1)
    torch.cuda.synchronize()
    c = fz.Context(0)
    yield c
    c.close()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def run(ctx, w, two_pass, min_tb=None, label=""):
    mt = w.get("min_tb") if min_tb is None else min_tb
    mt = -(1 << 62) if mt is None else mt
    log("%s: extend two_pass=%d, %d seeds, min_tb %d" % (label, two_pass, len(w["seeds"]), mt))
    hits, cig, st = ctx.extend(dev(w["target"]), dev(w["query"]), dev(w["seeds"]), w["scoring"], w["ydrop"], mt,
                               want_stats=True, two_pass=two_pass, query_rc=bool(w.get("query_rc")))
    torch.cuda.synchronize()
    log("%s: done, %d one-pass sides, %d executor sides" % (label, st["n_onepass"], st["n_executor"]))
    return hits.cpu().numpy(), cig.cpu().numpy().view(np.uint32), st


def same(a, b, label):
    ha, ca, sa = a
    hb, cb, sb = b
    diff = np.nonzero((ha != hb).any(axis=1))[0]
    assert diff.size == 0, "%s: %d seeds differ, first %d: %s vs %s" % (
        label, diff.size, diff[0], ha[diff[0]].tolist(), hb[diff[0]].tolist())
    assert np.array_equal(ca, cb), label + ": CIGAR words differ"
    assert sa["cells"] == sb["cells"], label
    assert sa["max_band"] == sb["max_band"], label


def against_oracle(w, got, min_tb=None, label=""):
    mt = w.get("min_tb") if min_tb is None else min_tb
    q = oracle.revcomp(w["query"]) if w.get("query_rc") else w["query"]
    oh, ow, oo = oracle.run(w["target"], q, w["seeds"], w["scoring"], w["ydrop"], min_tb=mt)
    gh, gc, _ = got
    bad = []
    for k in range(len(oh)):
        g = dict(zip(fz.HIT_FIELDS, gh[k].tolist()))
        if oh["status"][k] != 0:
            continue
        for gf, of in (("score", "score"), ("t_begin", "t_begin"), ("t_end", "t_end"), ("q_begin", "q_begin"),
                       ("q_end", "q_end"), ("score_left", "score_l"), ("score_right", "score_r")):
            if g[gf] != int(oh[of][k]):
                bad.append((k, gf, g[gf], int(oh[of][k])))
        if g["cells"] != int(oh["cells_l"][k] + oh["cells_r"][k]):
            bad.append((k, "cells"))
        if not np.array_equal(gc[g["cigar_off"]:g["cigar_off"] + g["cigar_len"]], ow[oo[k]:oo[k] + oh["n_runs"][k]]):
            bad.append((k, "cigar"))
    assert not bad, "%s: %d mismatches, first %s" % (label, len(bad), bad[:3])


@pytest.fixture(scope="module")
def heavy():
    # pairs of 1-6 kb homology (15% substitutions, indels): long traced
    # sides, most of which pass the hand-over test
    return W.executor_heavy(n_pairs=400, len_min=1000, len_max=6000, seed=11)


def test_onepass_equals_two_pass_and_oracle(ctx, heavy):
    a = run(ctx, heavy, False, label="heavy one-pass")
    b = run(ctx, heavy, True, label="heavy two-pass")
    # (the seeds sit at the pairs' starts: one side each)
    assert a[2]["n_onepass"] > len(heavy["seeds"]) // 2, "the one-pass executor should take most sides"
    assert b[2]["n_onepass"] == 0
    assert a[2]["onepass_cells"] > 0 and a[2]["onepass_bytes"] > 0
    assert a[2]["n_executor"] < b[2]["n_executor"]
    same(a, b, "heavy")
    against_oracle(heavy, a, label="heavy one-pass")


@pytest.mark.parametrize("delta", [-2000, -300, 0, 300, 2000])
def test_onepass_thresholds(ctx, heavy, delta):
    """Traceback thresholds around the scores the sides reach by
    anti-diagonal 256, so that the hand-over test passes for some sides and
    fails for others; every seed's result equals the two-pass run's."""
    w = dict(heavy)
    w["seeds"] = heavy["seeds"][:120]
    mt = 1729 + 9000 + delta
    a = run(ctx, w, False, min_tb=mt, label="threshold %d" % delta)
    b = run(ctx, w, True, min_tb=mt, label="threshold %d" % delta)
    same(a, b, "threshold %d" % delta)


def test_onepass_pool_rounds(ctx, heavy):
    """Pools smaller than the one-pass sides need: at half of what the
    default run took, and at 3 MiB (a handful of sides at a time), the sides
    a round finishes are walked at once and the pool serves the next round;
    sides that never fit go back to the inspector and the two-pass
    executor.  The results are the same every time."""
    ref = run(ctx, heavy, True, label="pool ref")
    full = run(ctx, heavy, False, label="pool default")
    same(full, ref, "pool default")
    half = max(full[2]["onepass_bytes"] // 2, 1 << 20)
    for pool in (half, 3 << 20):
        fz.fz_debug_set(ctx.h, fz.FZ_DEBUG_ONEPASS_POOL, pool)
        try:
            a = run(ctx, heavy, False, label="pool %d" % pool)
        finally:
            fz.fz_debug_set(ctx.h, fz.FZ_DEBUG_ONEPASS_POOL, -1)
        assert a[2]["n_onepass"] <= full[2]["n_onepass"]
        if pool == half:
            assert a[2]["n_onepass"] > full[2]["n_onepass"] // 2
            assert a[2]["onepass_bytes"] > pool        # (more than one round)
        same(a, ref, "pool %d" % pool)


def test_onepass_pool_off(ctx, heavy):
    fz.fz_debug_set(ctx.h, fz.FZ_DEBUG_ONEPASS_POOL, 0)
    try:
        a = run(ctx, heavy, False, label="pool off")
    finally:
        fz.fz_debug_set(ctx.h, fz.FZ_DEBUG_ONEPASS_POOL, -1)
    b = run(ctx, heavy, True, label="pool off ref")
    assert a[2]["n_onepass"] == 0
    same(a, b, "pool off")


def test_onepass_launch_order(ctx, heavy):
    """The one-pass sides go longest first by a predicted length; in the
    order the inspector handed them over the results are the same."""
    a = run(ctx, heavy, False, label="order predicted")
    fz.fz_debug_set(ctx.h, fz.FZ_DEBUG_ONEPASS_ORDER, 0)
    try:
        b = run(ctx, heavy, False, label="order as handed over")
    finally:
        fz.fz_debug_set(ctx.h, fz.FZ_DEBUG_ONEPASS_ORDER, 1)
    assert a[2]["n_onepass"] == b[2]["n_onepass"] > 0
    same(a, b, "launch order")


def tail_mode(ctx, mode):
    fz.fz_debug_set(ctx.h, fz.FZ_DEBUG_TAIL_WALK, mode)


@pytest.mark.parametrize("mode", [0, 2, 3000])
def test_onepass_tail_walk(ctx, heavy, mode):
    """The tail walk (one-pass sides walked while the one-pass executor's
    last waves still run) changes no result: off, after the executor (every
    side whose runs fit is walked there), and after it within 3,000 run words
    (a few sides fit, the rest fall back to the walk after the executor)."""
    ref = run(ctx, heavy, False, label="tail default")
    assert ref[2]["n_tail_walked"] <= ref[2]["n_onepass"]
    tail_mode(ctx, mode)
    try:
        a = run(ctx, heavy, False, label="tail mode %d" % mode)
    finally:
        tail_mode(ctx, 1)
    log("tail mode %d: %d of %d one-pass sides walked in the tail" % (mode, a[2]["n_tail_walked"], a[2]["n_onepass"]))
    if mode == 0:
        assert a[2]["n_tail_walked"] == 0
    elif mode == 2:
        assert a[2]["n_tail_walked"] >= 0.9 * a[2]["n_onepass"]
    else:
        assert 0 < a[2]["n_tail_walked"] < a[2]["n_onepass"]
    same(a, ref, "tail mode %d" % mode)
    if mode == 2:
        against_oracle(heavy, a, label="tail after the executor")


def test_onepass_tail_walk_pool_rounds(ctx, heavy):
    """Pool rounds with the tail walk taking every finished side: each
    round's tail-walked runs are packed with the round's other walked sides
    before the next round reuses the tail buffer."""
    ref = run(ctx, heavy, True, label="tail rounds ref")
    full = run(ctx, heavy, False, label="tail rounds default")
    pool = max(full[2]["onepass_bytes"] // 2, 1 << 20)
    fz.fz_debug_set(ctx.h, fz.FZ_DEBUG_ONEPASS_POOL, pool)
    tail_mode(ctx, 2)
    try:
        a = run(ctx, heavy, False, label="tail rounds, pool %d" % pool)
    finally:
        tail_mode(ctx, 1)
        fz.fz_debug_set(ctx.h, fz.FZ_DEBUG_ONEPASS_POOL, -1)
    assert a[2]["onepass_bytes"] > pool        # (more than one round)
    assert a[2]["n_tail_walked"] > a[2]["n_onepass"] // 2
    same(a, ref, "tail rounds")


def test_onepass_under_workspace_cap(ctx, heavy):
    """A 4 MiB pointer-memory cap bounds the pool too (many rounds), the
    same results."""
    ref = run(ctx, heavy, True, label="cap ref")
    fz.fz_set_pointer_workspace(ctx.h, 4 << 20)
    try:
        a = run(ctx, heavy, False, label="cap 4 MiB")
    finally:
        fz.fz_set_pointer_workspace(ctx.h, 0)
    same(a, ref, "cap 4 MiB")


def test_onepass_skewed_sample(ctx):
    w = W.skewed(target_len=1_000_000, n_seeds=4000, n_short=30, n_long=10, seed=2)
    a = run(ctx, w, False, label="skewed one-pass")
    b = run(ctx, w, True, label="skewed two-pass")
    assert a[2]["n_onepass"] > 0
    same(a, b, "skewed")
    against_oracle(w, a, label="skewed one-pass")


def test_onepass_reverse_strand(ctx):
    w = W.chromosome_rc(length=300_000, inv_min=20_000, inv_max=60_000, seed=5)
    a = run(ctx, w, False, label="rc one-pass")
    b = run(ctx, w, True, label="rc two-pass")
    same(a, b, "reverse strand")


def test_onepass_rounds(ctx):
    """Covered-seed rounds (each round an extension batch) take the same
    decisions with and without the one-pass executor."""
    w = W.homolog_rounds(length=12_000, block=4000, gap=1000, flank=1500, seed=3)
    T, Q, S = dev(w["target"]), dev(w["query"]), dev(w["seeds"])
    log("rounds: %d seeds" % len(w["seeds"]))
    ra = ctx.extend_rounds(T, Q, S, w["scoring"], w["ydrop"], w["min_tb"], 64, want_stats=True)
    rb = ctx.extend_rounds(T, Q, S, w["scoring"], w["ydrop"], w["min_tb"], 64, two_pass=True)
    torch.cuda.synchronize()
    log("rounds: done")
    assert ra[2]["n_onepass"] > 0
    assert np.array_equal(ra[0].cpu().numpy(), rb[0].cpu().numpy())
    assert np.array_equal(ra[1].cpu().numpy(), rb[1].cpu().numpy())

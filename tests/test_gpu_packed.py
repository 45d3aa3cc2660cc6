"""The packed 16-bit layouts (two cells per lane register) against the
32-bit layouts (FZ_EXACT32) and the oracle.

Both layouts make the same y-drop kills, the same best-cell choices and the
same traceback pointers, so hits, CIGAR words and canonical cell counts
agree bit for bit.  The cases reach the limits of the packed range (ydrop
16,000; int8 substitution scores at +-127 / -128; gap_open + 2 * gap_extend
= 4,000), bands that move a side between the 256- and 384-position packed
windows and past them into the wide retry, the executor's eager-block
hand-over (sides whose best cell lies before anti-diagonal 34 but outside
the eager corner), and scorings just outside the range (run in 32 bits).
"""
import random

import numpy as np
import pytest

import oracle
from smith_waterman_dp_amd import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from smith_waterman_dp_amd import fz  # noqa: E402

# every hit column but the executor length bin (a scheduling detail)
COLS = [k for k, f in enumerate(fz.HIT_FIELDS) if f != "bin"]


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


def run(ctx, w, exact32, ydrop=None, scoring=None, traceback=True, two_pass=True):
    """(two-pass by default: these cases compare the packed executor's rows
    and counts with the 32-bit one's)"""
    yd = w["ydrop"] if ydrop is None else ydrop
    sc = scoring or w["scoring"]
    log("call extend exact32=%d two_pass=%d: %d seeds, ydrop %d, scoring %s" % (exact32, two_pass, len(w["seeds"]),
                                                                             yd, sc))
    hits, cig, st = ctx.extend(dev(w["target"]), dev(w["query"]), dev(w["seeds"]), sc, yd, traceback=traceback,
                               want_stats=True, exact32=exact32, two_pass=two_pass)
    torch.cuda.synchronize()
    log("call done")
    return hits.cpu().numpy(), cig.cpu().numpy().view(np.uint32), st


def same(a, b, label):
    """Equal results.  Which sides go to the 1024-position retry (the
    FZ_HIT_WIDE bit) may differ: the packed and 32-bit 384-position windows
    slide on different lane grids, so a band of about 384 positions fits one
    and not the other; the retry's results are the same."""
    ha, ca, sa = a
    hb, cb, sb = b
    ha, hb = ha.copy(), hb.copy()
    ha[:, 1] &= ~fz.FZ_HIT_WIDE
    hb[:, 1] &= ~fz.FZ_HIT_WIDE
    diff = np.nonzero((ha[:, COLS] != hb[:, COLS]).any(axis=1))[0]
    assert diff.size == 0, "%s: %d seeds differ, first %d: %s vs %s" % (
        label, diff.size, diff[0], ha[diff[0]].tolist(), hb[diff[0]].tolist())
    assert np.array_equal(ca, cb), label + ": CIGAR words differ"
    assert sa["cells"] == sb["cells"], label
    assert sa["executor_cells"] == sb["executor_cells"], label


def against_oracle(w, got, ydrop=None, scoring=None, label=""):
    yd = w["ydrop"] if ydrop is None else ydrop
    oh, ow, oo = oracle.run(w["target"], w["query"], w["seeds"], scoring or w["scoring"], yd)
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
            bad.append((k, "cells", g["cells"], int(oh["cells_l"][k] + oh["cells_r"][k])))
        got_c = gc[g["cigar_off"]:g["cigar_off"] + g["cigar_len"]]
        exp_c = ow[oo[k]:oo[k] + oh["n_runs"][k]]
        if not np.array_equal(got_c, exp_c):
            bad.append((k, "cigar"))
    assert not bad, "%s: %d mismatches, first %s" % (label, len(bad), bad[:3])


def one_seed(t, q, t_pos, q_pos, L):
    return dict(target=np.frombuffer(t.encode(), dtype=np.uint8).copy(),
                query=np.frombuffer(q.encode(), dtype=np.uint8).copy(),
                seeds=np.array([[t_pos, q_pos, L, 0, len(t), 0, len(q)]], dtype=np.int64),
                scoring=dict(W.DEFAULT_SCORING), ydrop=9400)


def test_packed_tiny_equals_exact32(ctx):
    """1,000 seeds with 256-base flanks: the packed run equals the 32-bit
    one, and writes fewer pointer bytes (eight cells per pointer word in
    the 256-position layout, six in the 32-bit 192-position one)."""
    w = W.tiny()
    a = run(ctx, w, False)
    b = run(ctx, w, True)
    same(a, b, "tiny")
    assert a[2]["n_executor"] > 0
    assert a[2]["pointer_bytes"] < b[2]["pointer_bytes"]
    assert a[2]["n_packed"] == 2 * len(w["seeds"]) and b[2]["n_packed"] == 0


# cheap gaps widen the band: a cell k diagonals off the main one on
# identical flanks scores about k * (match / 2 + gap_extend) below the best,
# so the live range holds about ydrop / 6 positions
CHEAP = dict(match=10, transition=-10, transversion=-10, gap_open=0, gap_extend=1)


@pytest.mark.parametrize("length", [300, 700, 1000])
def test_packed_identical_flanks(ctx, length):
    """Identical flanks: with the default scoring the band stays in the
    256-position packed window; with cheap gaps it passes the 232 positions
    that move a packed side to the 384-position window (ydrop 1,800) and at
    ydrop 16,000 outgrows that, so the side is redone by the wide 32-bit
    retry."""
    rng = random.Random(length)
    s = "".join(rng.choice("ACGT") for _ in range(2 * length + 19))
    w = one_seed(s, s, length, length, 19)
    for sc, ydrop in ((None, 3000), (None, 9400), (None, 16000), (CHEAP, 1000), (CHEAP, 1800), (CHEAP, 16000)):
        label = "identical %d ydrop %d %s" % (length, ydrop, "cheap" if sc else "default")
        a = run(ctx, w, False, ydrop=ydrop, scoring=sc)
        b = run(ctx, w, True, ydrop=ydrop, scoring=sc)
        same(a, b, label)
        against_oracle(w, a, ydrop=ydrop, scoring=sc, label=label)
        if sc is CHEAP and length >= 700:
            if ydrop == 1800:
                assert 232 < a[2]["max_band"] <= 384, (label, a[2]["max_band"])
                assert a[2]["n_overflow"] == 0, label
            if ydrop == 16000:
                assert a[2]["n_overflow"] >= 1, label


# (scoring, ydrop, packed)
LIMIT_SCORINGS = [
    # the packed range's edges
    (dict(match=127, transition=-128, transversion=-128, gap_open=3940, gap_extend=30), 16000, True),
    (dict(match=127, transition=-1, transversion=-2, gap_open=0, gap_extend=1), 16000, True),
    (dict(match=1, transition=-1, transversion=-1, gap_open=0, gap_extend=1), 0, True),
    (dict(match=1, transition=-1, transversion=-1, gap_open=0, gap_extend=1), 1, True),
    (dict(match=91, transition=-31, transversion=-123, gap_open=2000, gap_extend=1000), 16000, True),
    # just outside it: the 32-bit layouts
    (dict(match=91, transition=-31, transversion=-123, gap_open=400, gap_extend=30), 16001, False),
    (dict(match=91, transition=-31, transversion=-123, gap_open=3942, gap_extend=30), 9400, False),
    (dict(match=128, transition=-31, transversion=-123, gap_open=400, gap_extend=30), 9400, False),
]


@pytest.mark.parametrize("case", range(len(LIMIT_SCORINGS)))
def test_packed_limit_scorings(ctx, case):
    sc, ydrop, packed = LIMIT_SCORINGS[case]
    w = W.tiny(n_seeds=300, flank=400, seed=20 + case)
    a = run(ctx, w, False, ydrop=ydrop, scoring=sc)
    b = run(ctx, w, True, ydrop=ydrop, scoring=sc)
    same(a, b, "limit scoring %d" % case)
    assert (a[2]["n_packed"] > 0) == packed and b[2]["n_packed"] == 0
    against_oracle(w, a, ydrop=ydrop, scoring=sc, label="limit scoring %d" % case)


def test_packed_short_executor_sides(ctx):
    """Sides whose best cell lies before anti-diagonal 34 but outside the
    eager corner go to the executor, which then stops inside its 32-bit
    start: left flanks of p matching bases, a g-base deletion in the query,
    r matching bases, then mismatches (p = 7..9, g = 2..4, r = 6..8)."""
    rng = random.Random(77)
    rows, tp, qp = [], [], []
    to = qo = 0
    for k in range(64):
        p, g, r = 7 + k % 3, 2 + (k // 3) % 3, 6 + (k // 9) % 3
        core, P, G, R = ("".join(rng.choice("ACGT") for _ in range(n)) for n in (19, p, g, r))
        t = "T" * 12 + R + G + P + core
        q = "G" * 12 + R + P + core
        rows.append((to + len(t) - 19, qo + len(q) - 19, 19, to, to + len(t), qo, qo + len(q)))
        tp.append(t)
        qp.append(q)
        to += len(t)
        qo += len(q)
    w = dict(target=np.frombuffer("".join(tp).encode(), dtype=np.uint8).copy(),
             query=np.frombuffer("".join(qp).encode(), dtype=np.uint8).copy(),
             seeds=np.array(rows, dtype=np.int64), scoring=dict(W.DEFAULT_SCORING), ydrop=9400)
    oh, _, _ = oracle.run(w["target"], w["query"], w["seeds"], w["scoring"], w["ydrop"])
    i = w["seeds"][:, 0] - oh["t_begin"]
    j = w["seeds"][:, 1] - oh["q_begin"]
    assert ((i + j < 34) & (np.maximum(i, j) > 16)).sum() >= 10
    a = run(ctx, w, False)
    b = run(ctx, w, True)
    same(a, b, "short executor sides")
    against_oracle(w, a, label="short executor sides")
    assert a[2]["n_executor"] > 0


def test_packed_executor_heavy(ctx):
    """Long homologous sides (300..3,000 bases): many layout moves, pointer
    rows in both packed formats, executor batches."""
    w = W.executor_heavy(n_pairs=60, len_min=300, len_max=3000, seed=9)
    a = run(ctx, w, False)
    b = run(ctx, w, True)
    same(a, b, "executor heavy")
    against_oracle(w, a, label="executor heavy")
    assert a[2]["pointer_bytes"] < b[2]["pointer_bytes"]


def test_packed_rounds(ctx):
    """Covered-seed rounds take the same decisions in both layouts."""
    w = W.homolog_rounds(length=12_000, block=4000, gap=1000, flank=1500, seed=3)
    S = dev(w["seeds"])
    T, Q = dev(w["target"]), dev(w["query"])
    ra = ctx.extend_rounds(T, Q, S, w["scoring"], w["ydrop"], w["min_tb"], 64)
    rb = ctx.extend_rounds(T, Q, S, w["scoring"], w["ydrop"], w["min_tb"], 64, exact32=True)
    torch.cuda.synchronize()
    ha, ca = ra[0].cpu().numpy(), ra[1].cpu().numpy()
    hb, cb = rb[0].cpu().numpy(), rb[1].cpu().numpy()
    assert np.array_equal(ha[:, COLS], hb[:, COLS])
    assert np.array_equal(ca, cb)

"""GPU parity of covered-seed suppression by rounds (fz_extend_rounds)
against the oracle's extend_rounds: the covered set exactly, and every
field and CIGAR of every extended seed; one round against fz_extend_batch;
at chromosome scale, the covered set recomputed from the GPU's own CIGARs
and sampled extended seeds against the oracle."""
import os

import numpy as np
import pytest

import oracle
from smith_waterman_dp_amd import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from smith_waterman_dp_amd import fz  # noqa: E402

from test_gpu_parity import compare, oracle_query  # noqa: E402


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


def run_rounds(ctx, w, round_size, seeds=None, doubling=False):
    S = w["seeds"] if seeds is None else seeds
    log("rounds: %d seeds, round size %d, doubling %d" % (len(S), round_size, doubling))
    h, c, st = ctx.extend_rounds(dev(w["target"]), dev(w["query"]), dev(S), w["scoring"], w["ydrop"], w["min_tb"],
                                 round_size, want_stats=True, query_rc=bool(w.get("query_rc")), doubling=doubling)
    torch.cuda.synchronize()
    log("rounds done")
    return h.cpu().numpy(), c.cpu().numpy().view(np.uint32), st


def check_against_oracle(ctx, w, round_size, label, doubling=False):
    gh, gc, _ = run_rounds(ctx, w, round_size, doubling=doubling)
    oh, ow, oo = oracle.extend_rounds(w["target"], oracle_query(w), w["seeds"], w["scoring"], w["ydrop"],
                                      w["min_tb"], round_size, doubling=doubling)
    gcov = (gh[:, 1] & fz.FZ_HIT_COVERED) != 0
    ocov = (oh["status"] & oracle.STATUS_COVERED) != 0
    assert np.array_equal(gcov, ocov), (label, np.nonzero(gcov != ocov)[0][:10])
    # covered records: status only, bin -1
    cov = gh[gcov]
    assert (cov[:, 1] == fz.FZ_HIT_COVERED).all() and (cov[:, 11] == -1).all()
    assert (np.delete(cov, [1, 11], axis=1) == 0).all()
    idx = np.nonzero(~gcov)[0]
    compare(gh, gc, oh[idx], ow, oo[idx], idx=idx, label=label)
    return gh, gcov


@pytest.mark.parametrize("round_size", [1, 3, 10, 40])
def test_rounds_homolog_vs_oracle(ctx, round_size):
    w = W.homolog_rounds(length=16_000, seed=4)
    gh, gcov = check_against_oracle(ctx, w, round_size, "homolog rounds %d" % round_size)
    assert gcov.any() or round_size >= len(w["seeds"])


@pytest.mark.parametrize("round_size", [1, 5])
def test_rounds_doubling_vs_oracle(ctx, round_size):
    w = W.homolog_rounds(length=16_000, seed=4)
    gh, gcov = check_against_oracle(ctx, w, round_size, "homolog doubling %d" % round_size, doubling=True)
    assert gcov.any()


def test_rounds_doubling_chromosome_reduced(ctx):
    w = W.chromosome_rounds(length=400_000, inv_min=5_000, inv_max=20_000, seed=3)
    gh, gcov = check_against_oracle(ctx, w, 64, "chromosome doubling reduced", doubling=True)
    log("covered %d of %d" % (gcov.sum(), len(gcov)))


def test_rounds_one_round_is_the_batch(ctx):
    w = W.homolog_rounds(length=30_000, seed=5)
    n = len(w["seeds"])
    gh, gc, _ = run_rounds(ctx, w, n + 7)
    h, c, _ = ctx.extend(dev(w["target"]), dev(w["query"]), dev(w["seeds"]), w["scoring"], w["ydrop"], w["min_tb"])
    assert np.array_equal(gh, h.cpu().numpy())
    assert np.array_equal(gc, c.cpu().numpy().view(np.uint32))


def test_rounds_matrix_reverse_strand(ctx):
    base = W.chromosome_rc(length=200_000, inv_min=20_000, inv_max=60_000, seed=6)
    w = W.with_matrix_and_n(base, 20, 5, 100, seed=8)
    rng = np.random.default_rng(3)
    w = dict(w, seeds=w["seeds"][rng.permutation(len(w["seeds"]))], min_tb=3000)
    gh, gcov = check_against_oracle(ctx, w, 16, "rounds matrix rc")
    assert gcov.any()


def test_rounds_chromosome_reduced(ctx):
    w = W.chromosome_rounds(length=400_000, inv_min=5_000, inv_max=20_000, seed=3)
    gh, gcov = check_against_oracle(ctx, w, 512, "chromosome rounds reduced")
    log("covered %d of %d" % (gcov.sum(), len(gcov)))
    assert gcov.sum() > len(gcov) // 2


def test_rounds_errors(ctx):
    w = W.homolog_rounds(length=5_000, seed=9)
    T, Q, S = dev(w["target"]), dev(w["query"]), dev(w["seeds"])
    with pytest.raises(fz.FzError):
        ctx.extend_rounds(T, Q, S, w["scoring"], w["ydrop"], 0, 0)                  # round size 0
    with pytest.raises(fz.FzError):                                                  # no traceback
        fz.fz_extend_batch(ctx.h, T, Q, S, w["scoring"], w["ydrop"], 0, 0, round_size=4)
    with pytest.raises(fz.FzError):                                                  # local mode
        fz.fz_extend_batch(ctx.h, T, Q, S, w["scoring"], w["ydrop"], 0, fz.FZ_LOCAL | fz.FZ_TRACEBACK,
                           round_size=4)
    h, c, _ = ctx.extend_rounds(T, Q, S[:0], w["scoring"], w["ydrop"], 0, 4)         # empty batch
    assert h.shape[0] == 0 and c.numel() == 0


def segments_of(gh, gc, rows):
    """Aligned (M) runs of the given traced rows as arrays (diagonal, t0, t1),
    each CIGAR walked from (t_begin, q_begin)."""
    rows = np.asarray(rows, dtype=np.int64)
    if rows.size == 0:
        z = np.zeros(0, dtype=np.int64)
        return z, z, z
    offs, lens = gh[rows, 6], gh[rows, 7]
    first = np.cumsum(lens) - lens
    pos = np.repeat(offs - first, lens) + np.arange(int(lens.sum()))
    wd = gc[pos].astype(np.int64)
    n, op = wd >> 4, wd & 15
    dt = np.where(op != 1, n, 0)
    dq = np.where(op != 2, n, 0)
    ct = np.cumsum(dt) - dt
    cq = np.cumsum(dq) - dq
    t = np.repeat(gh[rows, 2] - ct[first], lens) + ct
    q = np.repeat(gh[rows, 4] - cq[first], lens) + cq
    m = op == 0
    return t[m] - q[m], t[m], t[m] + n[m]


@pytest.fixture(scope="module")
def chromosome_rounds_full():
    log("generating the chromosome pair")
    return W.chromosome_rounds()


@pytest.mark.skipif(os.environ.get("FZ_FULL_SIZE", "1") == "0", reason="full-size runs disabled")
@pytest.mark.parametrize("B,doubling", [(16384, False), (256, True)])
def test_rounds_chromosome_full_size(ctx, chromosome_rounds_full, B, doubling):
    """The 20 Mbp pair's 144,179 seeds in rounds (fixed, or doubling from a
    small first round): the covered set recomputed from the call's own
    alignments, round by round, and a sample of extended seeds against the
    oracle's plain extension."""
    w = chromosome_rounds_full
    S = w["seeds"]
    gh, gc, st = run_rounds(ctx, w, B, doubling=doubling)
    gcov = (gh[:, 1] & fz.FZ_HIT_COVERED) != 0
    log("covered %d of %d, %d cells" % (gcov.sum(), len(S), st["cells"]))
    tlen, qlen = w["target"].size, w["query"].size
    D = np.zeros(0, dtype=np.int64)
    A = np.zeros(0, dtype=np.int64)
    Bn = np.zeros(0, dtype=np.int64)
    for r0, r1 in oracle.round_bounds(len(S), B, doubling):
        rows = np.arange(r0, r1)
        order = np.argsort(D, kind="stable")
        Ds, As, Bs = D[order], A[order], Bn[order]
        for k in rows:
            t, q, L = (int(x) for x in S[k, :3])
            inside = L >= 1 and t >= 0 and q >= 0 and t + L <= tlen and q + L <= qlen
            lo, hi = np.searchsorted(Ds, [t - q, t - q + 1])
            cov = inside and bool(np.any((As[lo:hi] < t + L) & (Bs[lo:hi] > t)))
            assert bool(gcov[k]) == cov, k
        traced = rows[(gh[rows, 1] & fz.FZ_HIT_TRACED) != 0]
        d, a, b = segments_of(gh, gc, traced)
        D, A, Bn = np.concatenate([D, d]), np.concatenate([A, a]), np.concatenate([Bn, b])
        log("round at %d checked, %d segments" % (r0, D.size))
    rng = np.random.default_rng(0)
    ext = np.nonzero(~gcov)[0]
    idx = np.sort(rng.choice(ext, min(40, ext.size), replace=False))
    oh, ow, oo = oracle.run(w["target"], w["query"], S[idx], w["scoring"], w["ydrop"], min_tb=w["min_tb"])
    compare(gh, gc, oh, ow, oo, idx=idx, label="chromosome rounds full")


def test_rounds_with_invalid_and_empty_seeds(ctx):
    """Seeds with no columns are never covered; seeds outside their windows
    are covered like any other (coverage looks at the columns only) or, when
    not, report FZ_HIT_ESEED as in a plain batch."""
    w = W.homolog_rounds(length=12_000, seed=11)
    S = w["seeds"].copy()
    bad = S[:6].copy()
    bad[:3, 3] = bad[:3, 0] + 1          # t_lo past the seed: invalid
    bad[3:, 2] = 0                       # no columns
    w = dict(w, seeds=np.concatenate([S[:4], bad, S[4:]]))
    gh, gcov = check_against_oracle(ctx, w, 3, "rounds with invalid seeds", doubling=True)
    assert not gcov[7:10].any()
    assert (gh[4:7, 1] & (fz.FZ_HIT_ESEED | fz.FZ_HIT_COVERED)).all()

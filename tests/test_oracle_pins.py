"""Pins for the CPU oracle: it is checked against things other than itself.

- exhaustive path enumeration (tests/bruteforce.py) for the recurrence,
  the y-drop rule, the end-cell rule and the traceback tie rules;
- hand-derived closed forms (tests/golden/closed_forms.tsv);
- the linear-gap special case of local mode against a textbook one-matrix
  Smith-Waterman (DPX article, section 1.1);
- invariants: the CIGAR rescored from the sequences equals the score, spans
  match the coordinates, the left side equals the right side on reversed
  strings, local >= any seeded extension in the same window.
"""
import os
import random

import numpy as np
import pytest

import bruteforce as bf
import oracle
from smith_waterman_dp_amd import workloads as W

SC = dict(W.DEFAULT_SCORING)
HERE = os.path.dirname(os.path.abspath(__file__))


def rand_seq(rng, n, alphabet="ACGT"):
    return "".join(rng.choice(alphabet) for _ in range(n))


def rand_scoring(rng):
    return dict(match=rng.randint(1, 120), transition=rng.randint(-150, 40),
                transversion=rng.randint(-200, 0), gap_open=rng.randint(1, 500),
                gap_extend=rng.randint(1, 80))


def check_against_brute(a, b, sc, ydrop):
    ob = oracle.side(a, b, sc, oracle.YDROP_INF if ydrop is None else ydrop, matrices=True)
    assert ob["status"] == 0
    br = bf.extension_brute(a, b, sc, ydrop)
    ctx = (a, b, sc, ydrop)
    assert ob["score"] == br["score"], ctx
    assert (ob["ie"], ob["je"]) == (br["ie"], br["je"]), ctx
    assert ob["ops"] == br["ops"][::-1], ctx
    # live set and every live value
    live_o = {(i, j) for i in range(len(a) + 1) for j in range(len(b) + 1) if ob["S"][i, j] is not None}
    assert live_o == br["live"], ctx
    for c in live_o:
        assert ob["S"][c] == br["V"][c], (ctx, c)


@pytest.mark.parametrize("case", range(150))
def test_bruteforce_unpruned(case):
    """No pruning: the oracle's maximum is the maximum over every path."""
    rng = random.Random(1000 + case)
    alphabet = ["ACGT", "AC", "AG", "A"][case % 4]
    a = rand_seq(rng, rng.randint(0, 5), alphabet)
    b = rand_seq(rng, rng.randint(0, 5), alphabet)
    sc = SC if case % 3 == 0 else rand_scoring(rng)
    check_against_brute(a, b, sc, None)


@pytest.mark.parametrize("case", range(200))
def test_bruteforce_ydrop(case):
    """Anti-diagonal y-drop: live set, values, end cell and path all match
    the enumeration with the same kill rule."""
    rng = random.Random(5000 + case)
    alphabet = ["ACGT", "AC", "AG", "AT", "A"][case % 5]
    a = rand_seq(rng, rng.randint(1, 6), alphabet)
    b = rand_seq(rng, rng.randint(1, 6), alphabet)
    sc = SC if case % 2 == 0 else rand_scoring(rng)
    ydrop = rng.choice([0, 1, 30, 100, 150, 300, 500, 900])
    check_against_brute(a, b, sc, ydrop)


@pytest.mark.parametrize("a,b", [("AAAAA", "AAAA"), ("ACACAC", "ACAC"), ("AAAA", "AAAAAA"),
                                 ("ACGACG", "ACG"), ("AGAGAG", "AG"), ("TTTTT", "TT")])
def test_bruteforce_repeat_ties(a, b):
    """Homopolymer and short-repeat indels: many equal-scoring gap places;
    the traceback picks the tie-ruled one."""
    sc = dict(match=91, transition=-31, transversion=-123, gap_open=40, gap_extend=30)
    for ydrop in (None, 200, 1000):
        check_against_brute(a, b, sc, ydrop)
        check_against_brute(b, a, sc, ydrop)


def load_closed_forms():
    rows = []
    with open(os.path.join(HERE, "golden", "closed_forms.tsv")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            p = line.rstrip("\n").split("\t")
            rows.append((p[0], p[1], p[2], int(p[3]), int(p[4]), int(p[5]), int(p[6]), p[7] if len(p) > 7 else ""))
    return rows


@pytest.mark.parametrize("row", load_closed_forms(), ids=lambda r: r[0])
def test_closed_forms(row):
    name, a, b, ydrop, score, ie, je, ops = row
    r = oracle.side(a, b, SC, ydrop)
    assert (r["score"], r["ie"], r["je"], r["ops"]) == (score, ie, je, ops)


@pytest.mark.parametrize("ell", [1, 7, 64, 300])
def test_identical_flanks_closed_form(ell):
    rng = random.Random(ell)
    a = rand_seq(rng, ell)
    r = oracle.side(a, a, SC, W.DEFAULT_YDROP)
    assert (r["score"], r["ie"], r["je"], r["ops"]) == (91 * ell, ell, ell, "M" * ell)


@pytest.mark.parametrize("g,kind", [(1, "D"), (5, "D"), (40, "I"), (200, "I")])
def test_single_gap_closed_form(g, kind):
    """One gap of g bases inside long identical flanks costs open + g*extend."""
    rng = random.Random(g)
    left, right = rand_seq(rng, 400), rand_seq(rng, 400)
    ins = rand_seq(rng, g)
    # guard against the inserted bases extending a neighbouring identical run
    while ins[0] == right[0] or ins[-1] == left[-1]:
        ins = rand_seq(rng, g)
    a = left + right
    b = left + ins + right
    if kind == "D":
        a, b = b, a
    r = oracle.side(a, b, SC, W.DEFAULT_YDROP)
    assert r["score"] == 91 * 800 - (400 + 30 * g)
    assert r["ops"].count(kind) == g and set(r["ops"]) == {"M", kind}


@pytest.mark.parametrize("k", [0, 1, 9, 50])
def test_ydrop_zero_closed_form(k):
    rng = random.Random(k)
    a = rand_seq(rng, k) + "A" + rand_seq(rng, 30)
    b = a[:k] + "C" + a[k + 1:]
    r = oracle.side(a, b, SC, 0)
    assert (r["score"], r["ie"], r["je"]) == (91 * k, k, k)


def test_infinite_ydrop_equals_unpruned_bruteforce_medium():
    """ydrop = inf on medium random pairs equals an unpruned full-matrix
    maximum computed by a separate path-free route: the best path score to
    each cell by the three-state recurrence written over the whole matrix."""
    rng = random.Random(7)
    for _ in range(20):
        a = rand_seq(rng, rng.randint(5, 40))
        b = rand_seq(rng, rng.randint(5, 40))
        r = oracle.side(a, b, SC, oracle.YDROP_INF, matrices=True)
        m, n = len(a), len(b)
        assert r["cells"] == (m + 1) * (n + 1)
        assert r["score"] == bf.path_score(r["ops"][::-1], a, b, SC)


def full_matrix_ydrop(a, b, sc, ydrop):
    """Unbanded y-drop: every cell of the matrix, anti-diagonal order, the
    kill rule applied cell by cell with no range bookkeeping."""
    m, n = len(a), len(b)
    NEG = None
    S = [[NEG] * (n + 1) for _ in range(m + 1)]
    I = [[NEG] * (n + 1) for _ in range(m + 1)]
    D = [[NEG] * (n + 1) for _ in range(m + 1)]
    S[0][0] = 0
    best = 0
    OE = sc["gap_open"] + sc["gap_extend"]
    E = sc["gap_extend"]

    def mx(*xs):
        xs = [x for x in xs if x is not None]
        return max(xs) if xs else None

    def sub_(x, y):
        return None if x is None else x + y

    for d in range(1, m + n + 1):
        thr = best - ydrop
        dbest = None
        for i in range(max(0, d - n), min(m, d) + 1):
            j = d - i
            Iv = mx(sub_(I[i][j - 1], -E), sub_(S[i][j - 1], -OE)) if j >= 1 else None
            Dv = mx(sub_(D[i - 1][j], -E), sub_(S[i - 1][j], -OE)) if i >= 1 else None
            H = sub_(S[i - 1][j - 1], bf.sub(a[i - 1], b[j - 1], sc)) if i >= 1 and j >= 1 else None
            Sv = mx(H, Iv, Dv)
            if Sv is None or Sv < thr:
                continue
            S[i][j], I[i][j], D[i][j] = Sv, Iv, Dv
            dbest = Sv if dbest is None else max(dbest, Sv)
        if dbest is not None:
            best = max(best, dbest)
    return S


@pytest.mark.parametrize("case", range(12))
def test_band_bookkeeping_vs_full_matrix(case):
    """The oracle's range rule (hull of cells with a live predecessor) loses
    nothing: same live set and values as evaluating the whole matrix."""
    rng = random.Random(900 + case)
    m, n = rng.randint(20, 70), rng.randint(20, 70)
    a = rand_seq(rng, m)
    # half the cases: b is a mutated a, so the band wanders
    if case % 2:
        b = list(a)
        for _ in range(rng.randint(1, 6)):
            p = rng.randrange(len(b))
            op = rng.random()
            if op < 0.4:
                b.insert(p, rng.choice("ACGT"))
            elif op < 0.8 and len(b) > 1:
                del b[p]
            else:
                b[p] = rng.choice("ACGT")
        b = "".join(b)
    else:
        b = rand_seq(rng, n)
    ydrop = rng.choice([100, 400, 900, 2000])
    r = oracle.side(a, b, SC, ydrop, matrices=True)
    S = full_matrix_ydrop(a, b, SC, ydrop)
    for i in range(len(a) + 1):
        for j in range(len(b) + 1):
            assert r["S"][i, j] == S[i][j], (i, j)


def canonical_cells_from_live(live, m, n):
    """Sum of |R_d| rebuilt from a live set alone (FastZ section 2.1, Fig. 3a,
    in the completed-scores form of section 3.4): R_0 = {(0,0)}; for d >= 1,
    R_d is the hull of the cells of diagonal d, inside the matrix, that have
    a live predecessor -- (i, j-1) or (i-1, j) on d-1, (i-1, j-1) on d-2;
    the run ends at the first empty R_d.  No band bookkeeping: every cell of
    every diagonal is tested against the live set."""
    total = 1
    for d in range(1, m + n + 2):
        cand = [i for i in range(max(0, d - n), min(m, d) + 1)
                if (i, d - i - 1) in live or (i - 1, d - i) in live or (i - 1, d - i - 1) in live]
        if not cand:
            break
        total += max(cand) - min(cand) + 1
    return total


def _mutated(rng, a, edits):
    b = list(a)
    for _ in range(edits):
        p = rng.randrange(len(b))
        op = rng.random()
        if op < 0.4:
            b.insert(p, rng.choice("ACGT"))
        elif op < 0.8 and len(b) > 1:
            del b[p]
        else:
            b[p] = rng.choice("ACGT")
    return "".join(b)


@pytest.mark.parametrize("case", range(40))
def test_cell_count_vs_full_matrix_live_set(case):
    """The oracle's canonical cell count (the GCUPS numerator) equals the
    count rebuilt from the live set of the unbanded full-matrix y-drop DP."""
    rng = random.Random(4200 + case)
    m, n = rng.randint(1, 60), rng.randint(1, 60)
    a = rand_seq(rng, m)
    b = _mutated(rng, a, rng.randint(1, 8)) if case % 2 else rand_seq(rng, n)
    ydrop = [0, 30, 120, 500, 900, 2000, 9400][case % 7]
    sc = SC if case % 3 else rand_scoring(rng)
    r = oracle.side(a, b, sc, ydrop)
    S = full_matrix_ydrop(a, b, sc, ydrop)
    live = {(i, j) for i in range(len(a) + 1) for j in range(len(b) + 1) if S[i][j] is not None}
    assert r["cells"] == canonical_cells_from_live(live, len(a), len(b)), (a, b, sc, ydrop)


@pytest.mark.parametrize("case", range(60))
def test_cell_count_vs_enumeration(case):
    """The same count from the live set of exhaustive path enumeration
    (tiny pairs, several y-drops)."""
    rng = random.Random(5100 + case)
    alphabet = ["ACGT", "AC", "AG", "A"][case % 4]
    a = rand_seq(rng, rng.randint(0, 5), alphabet)
    b = rand_seq(rng, rng.randint(0, 5), alphabet)
    sc = SC if case % 2 == 0 else rand_scoring(rng)
    ydrop = [0, 100, 300, 600, 1500][case % 5]
    r = oracle.side(a, b, sc, ydrop)
    br = bf.extension_brute(a, b, sc, ydrop)
    assert r["cells"] == canonical_cells_from_live(br["live"], len(a), len(b)), (a, b, sc, ydrop)


def load_cell_counts():
    rows = []
    with open(os.path.join(HERE, "golden", "cell_counts.tsv")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            p = line.rstrip("\n").split("\t")
            rows.append((p[0], p[1], p[2], int(p[3]), int(p[4]), int(p[5]), int(p[6]), int(p[7])))
    return rows


@pytest.mark.parametrize("row", load_cell_counts(), ids=lambda r: r[0])
def test_cell_count_closed_forms(row):
    """Hand-derived counts (tests/golden/cell_counts.tsv, derivations there)."""
    name, a, b, ydrop, cells, score, ie, je = row
    r = oracle.side(a, b, SC, ydrop)
    assert (r["cells"], r["score"], r["ie"], r["je"]) == (cells, score, ie, je)
    assert canonical_cells_from_live_of(a, b, ydrop) == cells


def canonical_cells_from_live_of(a, b, ydrop):
    S = full_matrix_ydrop(a, b, SC, ydrop)
    live = {(i, j) for i in range(len(a) + 1) for j in range(len(b) + 1) if S[i][j] is not None}
    return canonical_cells_from_live(live, len(a), len(b))


@pytest.mark.parametrize("ell", [0, 1, 2, 17, 200])
def test_cell_count_identical_ydrop0(ell):
    """Identical flanks with ydrop 0: 1 + 3 * ell cells (derivation in
    tests/golden/cell_counts.tsv)."""
    rng = random.Random(ell)
    a = rand_seq(rng, ell)
    r = oracle.side(a, a, SC, 0)
    assert (r["cells"], r["score"]) == (1 + 3 * ell, 91 * ell)


# ------------------------------------------------------------- local mode --

def textbook_sw_linear(a, b, sc):
    """One-matrix local alignment with a linear gap penalty g per base:
    H = max(0, diag + s, up - g, left - g) (DPX article, section 1.1)."""
    m, n = len(a), len(b)
    g = sc["gap_extend"]
    H = np.zeros((m + 1, n + 1), dtype=np.int64)
    for i in range(1, m + 1):
        for j in range(1, n + 1):
            H[i, j] = max(0, H[i - 1, j - 1] + bf.sub(a[i - 1], b[j - 1], sc), H[i - 1, j] - g, H[i, j - 1] - g)
    top = int(H.max())
    cells = [(i + j, i) for i in range(m + 1) for j in range(n + 1) if H[i, j] == top]
    d, i = min(cells)
    return top, i, d - i


def run_local(a, b, sc):
    seeds = np.array([[0, 0, 0, 0, len(a), 0, len(b)]], dtype=np.int64)
    hits, _, _ = oracle.run(a, b, seeds, sc, oracle.YDROP_INF, local=True, traceback=False, threads=1)
    h = hits[0]
    assert h["status"] == 0
    return int(h["score"]), int(h["t_end"]), int(h["q_end"]), int(h["cells_r"])


@pytest.mark.parametrize("case", range(30))
def test_local_linear_gap_equals_textbook(case):
    rng = random.Random(300 + case)
    a = rand_seq(rng, rng.randint(1, 60), "ACGT" if case % 2 else "AC")
    b = rand_seq(rng, rng.randint(1, 60), "ACGT" if case % 2 else "AC")
    sc = dict(SC, gap_open=0) if case % 3 else dict(rand_scoring(rng), gap_open=0)
    assert run_local(a, b, sc)[:3] == textbook_sw_linear(a, b, sc)


@pytest.mark.parametrize("case", range(60))
def test_local_bruteforce(case):
    rng = random.Random(700 + case)
    a = rand_seq(rng, rng.randint(0, 5), ["ACGT", "AC", "A"][case % 3])
    b = rand_seq(rng, rng.randint(0, 5), ["ACGT", "AC", "A"][case % 3])
    sc = SC if case % 2 else rand_scoring(rng)
    br = bf.local_brute(a, b, sc)
    s, ie, je, cells = run_local(a, b, sc)
    assert (s, ie, je) == (br["score"], br["ie"], br["je"])
    assert cells == len(a) * len(b)


def test_local_identical_2048():
    rng = random.Random(2048)
    a = rand_seq(rng, 2048)
    assert run_local(a, a, SC)[:3] == (91 * 2048, 2048, 2048)


# ------------------------------------------------------------- invariants --

def rescore_cigar(T, Q, t0, q0, words, sc):
    t, q, total = t0, q0, 0
    for w in words:
        n, op = int(w) >> 4, int(w) & 15
        if op == 0:
            for k in range(n):
                total += bf.sub(chr(T[t + k]), chr(Q[q + k]), sc)
            t += n
            q += n
        else:
            total -= sc["gap_open"] + n * sc["gap_extend"]
            if op == 1:
                q += n
            else:
                t += n
    return total, t, q


@pytest.fixture(scope="module")
def tiny_small():
    return W.tiny(n_seeds=60, seed=3)


def test_tiny_invariants(tiny_small):
    w = tiny_small
    hits, words, offs = oracle.run(w["target"], w["query"], w["seeds"], w["scoring"], w["ydrop"], threads=4)
    assert (hits["status"] == 0).all()
    for k, h in enumerate(hits):
        cw = words[offs[k]:offs[k] + h["n_runs"]]
        total, t_end, q_end = rescore_cigar(w["target"], w["query"], h["t_begin"], h["q_begin"], cw, w["scoring"])
        assert total == h["score"]
        assert (t_end, q_end) == (h["t_end"], h["q_end"])
        ops = [int(x) & 15 for x in cw]
        assert all(ops[i] != ops[i + 1] for i in range(len(ops) - 1)), "runs must be maximal"


def test_left_equals_right_on_reversed(tiny_small):
    w = tiny_small
    T, Q = bytes(w["target"]), bytes(w["query"])
    for s in w["seeds"][:20]:
        t_pos, q_pos, L, t_lo, t_hi, q_lo, q_hi = [int(x) for x in s]
        left_a = T[t_lo:t_pos][::-1]
        left_b = Q[q_lo:q_pos][::-1]
        hits, _, _ = oracle.run(w["target"], w["query"], s.reshape(1, 7), w["scoring"], w["ydrop"], threads=1)
        r = oracle.side(left_a, left_b, w["scoring"], w["ydrop"])
        h = hits[0]
        assert (r["score"], r["ie"], r["je"], r["cells"]) == (h["score_l"], h["i_l"], h["j_l"], h["cells_l"])


def test_local_at_least_seeded_extension(tiny_small):
    w = tiny_small
    seeds = w["seeds"][:8]
    hits, _, _ = oracle.run(w["target"], w["query"], seeds, w["scoring"], w["ydrop"], traceback=False, threads=4)
    loc = seeds.copy()
    loc[:, 2] = 0
    lh, _, _ = oracle.run(w["target"], w["query"], loc, w["scoring"], oracle.YDROP_INF, local=True,
                          traceback=False, threads=4)
    assert (lh["score"] >= hits["score"]).all()


def test_seed_validation():
    T = "ACGT" * 10
    bad = np.array([[5, 5, 19, 10, 40, 0, 40]], dtype=np.int64)   # seed before its window
    hits, _, _ = oracle.run(T, T, bad, SC, 9400, threads=1)
    assert hits[0]["status"] == oracle.STATUS_ESEED


def test_empty_flanks():
    """Seed flush with both window ends: both sides empty, total = seed."""
    T = "ACGTACGTACGTACGTACG"
    s = np.array([[0, 0, 19, 0, 19, 0, 19]], dtype=np.int64)
    hits, words, _ = oracle.run(T, T, s, SC, 9400, threads=1)
    h = hits[0]
    assert (h["score"], h["t_begin"], h["t_end"], h["cells_l"], h["cells_r"]) == (19 * 91, 0, 19, 1, 1)
    assert oracle.cigar_string(words) == "19M"


# ------------------------------------------------------ reverse strand --

def test_revcomp_hand_examples():
    """Complement A<->T, C<->G (either case), then reverse; other bytes kept."""
    assert oracle.revcomp(b"AACGTTTGCA").tobytes() == b"TGCAAACGTT"
    assert oracle.revcomp(b"acgT").tobytes() == b"Acgt"
    assert oracle.revcomp(b"ANC").tobytes() == b"GNT"
    assert oracle.revcomp(b"").tobytes() == b""


def test_revcomp_involution():
    rng = np.random.default_rng(5)
    for n in (1, 2, 19, 1000):
        s = W.to_ascii(W.random_codes(rng, n))
        r = oracle.revcomp(s)
        assert r.size == n
        assert np.array_equal(oracle.revcomp(r), s)
        # no base is its own complement, so every position changes
        assert (oracle.revcomp(s)[::-1] != s).all()


def _strand_case(seed):
    """T random; R = mut(T) holds the homology; the query handed in is the
    reverse complement of R, so the seeds (shared 19-mers of T and R) lie on
    the query's reverse strand."""
    rng = np.random.default_rng(seed)
    T = W.random_codes(rng, 1500)
    R = W.mutate(rng, T, 0.08, 0.01, 0.5)
    t, q = W.shared_kmers(T, R)
    keep = np.unique(t - q, return_index=True)[1][:12]
    t, q = t[keep], q[keep]
    lo_t = np.maximum(t - 400, 0)
    hi_t = np.minimum(t + 19 + 400, T.size)
    lo_q = np.maximum(q - 300, 0)
    hi_q = np.minimum(q + 19 + 500, R.size)
    seeds = np.stack([t, q, np.full_like(t, 19), lo_t, hi_t, lo_q, hi_q], axis=1).astype(np.int64)
    return W.to_ascii(T), W.to_ascii(W.revcomp_codes(R)), seeds


@pytest.mark.parametrize("seed", [0, 1])
def test_strand_symmetry(seed):
    """Extending T against revcomp(Q) is extending revcomp(T) against Q with
    the seed mirrored: complementing both sequences keeps every
    substitution's class (transitions stay transitions), so each side's
    matrix is the same, the left and right sides trade places and the CIGAR
    runs come out in reverse order."""
    T, Q, s1 = _strand_case(seed)
    nT, nQ = T.size, Q.size
    h1, w1, o1 = oracle.run(T, oracle.revcomp(Q), s1, SC, 9400, threads=4)
    s2 = s1.copy()
    s2[:, 0] = nT - s1[:, 0] - s1[:, 2]
    s2[:, 1] = nQ - s1[:, 1] - s1[:, 2]
    s2[:, 3], s2[:, 4] = nT - s1[:, 4], nT - s1[:, 3]
    s2[:, 5], s2[:, 6] = nQ - s1[:, 6], nQ - s1[:, 5]
    h2, w2, o2 = oracle.run(oracle.revcomp(T), Q, s2, SC, 9400, threads=4)
    assert (h1["status"] == 0).all() and (h2["status"] == 0).all()
    assert (h1["score"] > 19 * 91).any()            # some seeds do extend
    for k in range(len(s1)):
        a, b = h1[k], h2[k]
        assert a["score"] == b["score"]
        assert (a["score_l"], a["score_r"]) == (b["score_r"], b["score_l"])
        assert (a["cells_l"], a["cells_r"]) == (b["cells_r"], b["cells_l"])
        assert (b["t_begin"], b["t_end"]) == (nT - a["t_end"], nT - a["t_begin"])
        assert (b["q_begin"], b["q_end"]) == (nQ - a["q_end"], nQ - a["q_begin"])
        c1 = w1[o1[k]:o1[k] + a["n_runs"]]
        c2 = w2[o2[k]:o2[k] + b["n_runs"]]
        assert np.array_equal(c1[::-1], c2)


# ---------------------------------------------------------- seed stage --

def test_find_seeds_hand_example():
    """T = ACGTACGT, Q = CGTA, k = 3: CGT at t 1 and 5 matches q 0, GTA at
    t 2 matches q 1.  Diagonal 1 holds (1, 0) and (2, 1), one run, so the
    dedup keeps (1, 0); (5, 0) is alone on diagonal 5."""
    s, n = oracle.find_seeds("ACGTACGT", "CGTA", k=3, flank=2, dedup=False)
    assert n == 3
    assert s[:, :2].tolist() == [[1, 0], [2, 1], [5, 0]]
    s, n = oracle.find_seeds("ACGTACGT", "CGTA", k=3, flank=2, dedup=True)
    assert s.tolist() == [[1, 0, 3, 0, 6, 0, 4], [5, 0, 3, 3, 8, 0, 4]]


def _seeds_by_enumeration(T, Q, k, flank, dedup):
    """Every start pair compared as strings, ordered by (t - q, t), runs cut
    by a walk: the definition written out with loops."""
    T, Q = T.upper(), Q.upper()
    hits = []
    for t in range(len(T) - k + 1):
        for q in range(len(Q) - k + 1):
            if T[t:t + k] == Q[q:q + k] and "N" not in T[t:t + k]:
                hits.append((t - q, t, q))
    hits.sort()
    out = []
    prev = None
    for dg, t, q in hits:
        if not (dedup and prev is not None and prev[0] == dg and prev[1] == t - 1):
            out.append([t, q, k, max(t - flank, 0), min(t + k + flank, len(T)), max(q - flank, 0),
                        min(q + k + flank, len(Q))])
        prev = (dg, t)
    return out, len(hits)


@pytest.mark.parametrize("seed,k,alphabet", [(0, 3, "ACGT"), (1, 5, "ACGT"), (2, 8, "ACGT"), (3, 4, "ACGT"),
                                             (4, 3, "ACGTN"), (5, 6, "AAACGTN")])
def test_find_seeds_enumeration(seed, k, alphabet):
    """Random pairs with planted repeats and mutated copies, against the
    enumeration of all start pairs (N matches nothing)."""
    rng = random.Random(seed)
    T = "".join(rng.choice(alphabet) for _ in range(150))
    rep = "".join(rng.choice("ACGT") for _ in range(12))
    T = T[:30] + rep + T[42:90] + rep + T[102:]
    Q = list(T[20:140])
    for _ in range(10):
        Q[rng.randrange(len(Q))] = rng.choice(alphabet)
    Q = "".join(Q) + rep.lower()
    for dedup in (False, True):
        got, n = oracle.find_seeds(T, Q, k=k, flank=7, dedup=dedup)
        exp, ne = _seeds_by_enumeration(T, Q, k, 7, dedup)
        assert n == ne
        assert got.tolist() == exp


def test_find_seeds_reverse_strand_and_edges():
    rng = random.Random(9)
    T = "".join(rng.choice("ACGT") for _ in range(200))
    Q = "".join(rng.choice("ACGT") for _ in range(180))
    a, na = oracle.find_seeds(T, Q, k=4, flank=5, query_rc=True)
    b, nb = oracle.find_seeds(T, oracle.revcomp(Q).tobytes(), k=4, flank=5)
    assert na == nb and np.array_equal(a, b)
    assert oracle.find_seeds("ACG", "ACGT", k=4)[0].shape == (0, 7)        # target shorter than k
    with pytest.raises(ValueError):
        oracle.find_seeds("ACGR", "ACGT", k=2)
    # N matches nothing, not even N; k-mers around it still do
    s, n = oracle.find_seeds("ACNNGT", "ACNNGT", k=2, flank=0)
    assert n == 2 and s[:, :2].tolist() == [[0, 0], [4, 4]]


# ---- 4x4 substitution matrix and N -------------------------------------

def rand_matrix_scoring(rng):
    """An asymmetric int8 matrix (rows = target base) and an N score."""
    return dict(matrix=[[rng.randint(-128, 127) for _ in range(4)] for _ in range(4)],
                n_score=rng.randint(-128, 127), gap_open=rng.randint(1, 400), gap_extend=rng.randint(1, 60))


@pytest.mark.parametrize("case", range(120))
def test_bruteforce_matrix(case):
    """Random asymmetric matrices, N in either sequence (either case), with
    and without pruning, against path enumeration."""
    rng = random.Random(7000 + case)
    alphabet = ["ACGTN", "ACGTn", "AN", "CGT"][case % 4]
    a = rand_seq(rng, rng.randint(0, 5), alphabet)
    b = rand_seq(rng, rng.randint(0, 5), alphabet)
    sc = rand_matrix_scoring(rng)
    check_against_brute(a, b, sc, None if case % 2 else rng.randint(0, 300))


@pytest.mark.parametrize("case", range(40))
def test_local_bruteforce_matrix(case):
    rng = random.Random(7500 + case)
    a = rand_seq(rng, rng.randint(0, 5), "ACGTN")
    b = rand_seq(rng, rng.randint(0, 5), "ACGTN")
    sc = rand_matrix_scoring(rng)
    hits, _, _ = oracle.run(a, b, np.array([[0, 0, 0, 0, len(a), 0, len(b)]], dtype=np.int64), sc, 0,
                            local=True, threads=1)
    br = bf.local_brute(a, b, sc)
    assert hits["status"][0] == 0
    assert hits["score"][0] == br["score"]


def matrix_of(sc):
    """The triple written as a matrix: equal bases score match, A<->G and
    C<->T score transition, every other pair transversion."""
    cls = {0: "match", 2: "transition"}
    return [[sc[cls.get(x ^ y, "transversion")] for y in range(4)] for x in range(4)]


def test_matrix_of_triple_equals_triple(tiny_small):
    """The matrix mode with the triple's matrix gives the triple's results,
    CIGARs included, on the tiny batch."""
    w = tiny_small
    sc_m = dict(matrix=matrix_of(w["scoring"]), n_score=-100, gap_open=w["scoring"]["gap_open"],
                gap_extend=w["scoring"]["gap_extend"])
    h1, c1, o1 = oracle.run(w["target"], w["query"], w["seeds"], w["scoring"], w["ydrop"], threads=4)
    h2, c2, o2 = oracle.run(w["target"], w["query"], w["seeds"], sc_m, w["ydrop"], threads=4)
    assert np.array_equal(h1, h2) and np.array_equal(c1, c2) and np.array_equal(o1, o2)


@pytest.mark.parametrize("seed", range(4))
def test_matrix_transpose_symmetry(seed):
    """Swapping target and query with the matrix transposed keeps the score
    (an alignment read the other way has the same columns), with pruning."""
    rng = random.Random(7900 + seed)
    sc = rand_matrix_scoring(rng)
    sc["matrix"] = [[rng.randint(-60, 100) if x == y else rng.randint(-128, -20) for y in range(4)]
                    for x in range(4)]
    a = rand_seq(rng, 300, "ACGT")
    b = list(a)
    for _ in range(30):
        b[rng.randrange(len(b))] = rng.choice("ACGTN")
    b = "".join(b)
    scT = dict(sc, matrix=[list(r) for r in zip(*sc["matrix"])])
    for ydrop in (oracle.YDROP_INF, 500):
        x = oracle.side(a, b, sc, ydrop)
        y = oracle.side(b, a, scT, ydrop)
        assert x["status"] == 0 and y["status"] == 0
        assert x["score"] == y["score"]


def test_n_needs_a_matrix():
    """Without a matrix N is an invalid base; with one it scores n_score."""
    r = oracle.side("ACNT", "ACGT", SC, oracle.YDROP_INF)
    assert r["status"] != 0
    sc = dict(matrix=matrix_of(SC), n_score=-7, gap_open=SC["gap_open"], gap_extend=SC["gap_extend"])
    r = oracle.side("ACNT", "ACGT", sc, oracle.YDROP_INF)
    assert r["status"] == 0 and r["score"] == 3 * SC["match"] - 7 and (r["ie"], r["je"]) == (4, 4)


def test_matrix_orientation_closed_form():
    """sub[a][b] scores target base a against query base b.  With an
    asymmetric matrix the two orientations give different hand-derived
    results; the transpose-symmetry pin alone would pass a consistently
    transposed lookup."""
    m = [[91, 50, -31, -123],
         [-200, 91, -123, -31],
         [-31, -123, 91, -123],
         [-123, -31, -123, 91]]
    sc = dict(matrix=m, n_score=-100, gap_open=400, gap_extend=30)
    # target A against query C scores +50 per column: 4 * 50
    r = oracle.side("AAAA", "CCCC", sc, oracle.YDROP_INF)
    assert (r["score"], r["ie"], r["je"], r["ops"]) == (200, 4, 4, "MMMM")
    # target C against query A scores -200, a gap 430: the empty extension wins
    r = oracle.side("CCCC", "AAAA", sc, oracle.YDROP_INF)
    assert (r["score"], r["ie"], r["je"], r["ops"]) == (0, 0, 0, "")
    # one N in the target among matches: 3 * 91 + n_score
    r = oracle.side("ANAA", "ACAA", sc, oracle.YDROP_INF)
    assert (r["score"], r["ie"], r["je"]) == (3 * 91 - 100, 4, 4)


# ---- covered-seed suppression by rounds --------------------------------

def test_rounds_single_round_equals_run():
    """With one round nothing is suppressed: the results are run()'s."""
    w = W.homolog_rounds(length=12_000, seed=2)
    n = len(w["seeds"])
    a = oracle.run(w["target"], w["query"], w["seeds"], w["scoring"], w["ydrop"], min_tb=w["min_tb"])
    b = oracle.extend_rounds(w["target"], w["query"], w["seeds"], w["scoring"], w["ydrop"], w["min_tb"], n)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_rounds_hand_example():
    """Identical 400-base sequences: the seed at 50 aligns the whole main
    diagonal, so the seed at 200 on it is covered when it comes in a later
    round, not when both share a round.  A seed on another diagonal is
    never covered by it."""
    rng = random.Random(3)
    T = rand_seq(rng, 400)
    Q = T
    seeds = np.array([[50, 50, 19, 0, 400, 0, 400],
                      [200, 200, 19, 0, 400, 0, 400],
                      [10, 300, 5, 0, 400, 0, 400]], dtype=np.int64)
    h, w, o = oracle.extend_rounds(T, Q, seeds, SC, 9400, 0, 1)
    assert h["n_runs"][0] > 0 and oracle.cigar_string(w[o[0]:o[0] + h["n_runs"][0]]) == "400M"
    assert h["status"][1] == oracle.STATUS_COVERED and h["score"][1] == 0 and h["n_runs"][1] == 0
    assert h["status"][2] == 0
    h2, _, _ = oracle.extend_rounds(T, Q, seeds, SC, 9400, 0, 2)
    assert h2["status"][1] == 0 and h2["score"][1] == h["score"][0]
    # untraced alignments (score not above min_tb) cover nothing
    h3, _, _ = oracle.extend_rounds(T, Q, seeds, SC, 9400, 10 ** 9, 1)
    assert not (h3["status"] & oracle.STATUS_COVERED).any()


def test_rounds_seed_outside_sequences_never_covered():
    """A seed whose columns run past an end of the sequences is not covered,
    even where its columns inside overlap an earlier alignment: it is
    extended as a plain batch extends it, which reports the seed invalid.
    A seed inside the sequences on the same cells is covered."""
    rng = random.Random(5)
    T = rand_seq(rng, 400)
    Q = T
    seeds = np.array([[50, 50, 19, 0, 400, 0, 400],        # aligns 400M
                      [390, 390, 19, 0, 400, 0, 400],      # columns 390..408: past both ends
                      [-5, -5, 19, 0, 400, 0, 400],        # columns -5..13: before both starts
                      [380, 380, 19, 0, 400, 0, 400]], dtype=np.int64)   # inside, on the 400M cells
    h, w, o = oracle.extend_rounds(T, Q, seeds, SC, 9400, 0, 1)
    assert oracle.cigar_string(w[o[0]:o[0] + h["n_runs"][0]]) == "400M"
    for k in (1, 2):
        assert not h["status"][k] & oracle.STATUS_COVERED, k
        assert h["status"][k] & oracle.STATUS_ESEED, k
    assert h["status"][3] == oracle.STATUS_COVERED


def _cells_of(T, Q, hit, words):
    """Every aligned (t, q) cell of one alignment, read from its text CIGAR
    one column at a time."""
    import re
    t, q = int(hit["t_begin"]), int(hit["q_begin"])
    cells = set()
    for ln, op in re.findall(r"(\d+)([MID])", oracle.cigar_string(words)):
        for _ in range(int(ln)):
            if op == "M":
                cells.add((t, q))
                t += 1
                q += 1
            elif op == "I":
                q += 1
            else:
                t += 1
    assert (t, q) == (int(hit["t_end"]), int(hit["q_end"]))
    return cells


def test_round_bounds():
    assert oracle.round_bounds(10, 3) == [(0, 3), (3, 6), (6, 9), (9, 10)]
    assert oracle.round_bounds(10, 1, doubling=True) == [(0, 1), (1, 3), (3, 7), (7, 10)]
    assert oracle.round_bounds(0, 4) == []


@pytest.mark.parametrize("round_size,doubling", [(3, False), (10, False), (40, False), (1, True), (4, True)])
def test_rounds_coverage_by_cells(round_size, doubling):
    """Coverage recomputed from explicit cell sets: a seed is covered exactly
    when one of its columns is an aligned cell of an alignment traced in an
    earlier round; every extended seed has run()'s result."""
    w = W.homolog_rounds(length=16_000, seed=4)
    S = w["seeds"]
    h, words, offs = oracle.extend_rounds(w["target"], w["query"], S, w["scoring"], w["ydrop"], w["min_tb"],
                                          round_size, doubling=doubling)
    ref, rw, ro = oracle.run(w["target"], w["query"], S, w["scoring"], w["ydrop"], min_tb=w["min_tb"])
    earlier = set()
    n_cov = 0
    bounds = []
    r0, size = 0, round_size
    while r0 < len(S):                      # the schedule, written out again
        bounds.append((r0, min(r0 + size, len(S))))
        r0 += size
        size *= 2 if doubling else 1
    for r0, r1 in bounds:
        this_round = set()
        for k in range(r0, r1):
            t, q, L = (int(x) for x in S[k, :3])
            # a seed's columns are matrix cells only when they all lie inside
            # the two sequences; a seed without such columns is never covered
            inside = L >= 1 and t >= 0 and q >= 0 and t + L <= len(w["target"]) and q + L <= len(w["query"])
            cov = inside and any((t + i, q + i) in earlier for i in range(L))
            assert bool(h["status"][k] & oracle.STATUS_COVERED) == cov, k
            if cov:
                n_cov += 1
                assert h["score"][k] == 0 and h["n_runs"][k] == 0
                continue
            assert h[k] == ref[k]
            got = words[offs[k]:offs[k] + h["n_runs"][k]]
            assert np.array_equal(got, rw[ro[k]:ro[k] + ref["n_runs"][k]])
            if h["n_runs"][k]:
                this_round |= _cells_of(w["target"], w["query"], h[k], got)
        earlier |= this_round
    assert 0 < n_cov < len(S)


# ------------------------------------------------------ CIGAR rescoring --

def test_rescore_hand_examples():
    """oracle.rescore (the full-size invariant check) against scores written
    out by hand: M columns by match / transition / transversion, a gap run
    of g at -(open + g * extend), I on the query only, D on the target only."""
    m, ts, tv, go, ge = SC["match"], SC["transition"], SC["transversion"], SC["gap_open"], SC["gap_extend"]
    T = b"ACGTACGTAC"
    Q = b"ACGAACGTTTAC"
    # 8M: A-A C-C G-G T-A (transversion) A-A C-C G-G T-T
    W8 = np.array([8 << 4], dtype=np.uint32)
    # 3M 2I 5M from (0, 0): ACG/ACG, insert "AA" in the query, then CGTAC/CGTTT
    WI = np.array([3 << 4, (2 << 4) | 1, 5 << 4], dtype=np.uint32)
    # 2M 1D 2M from (0, 0): AC/AC, skip target G, TA/GA (transversion T-G, then A-A)
    WD = np.array([2 << 4, (1 << 4) | 2, 2 << 4], dtype=np.uint32)
    words = np.concatenate([W8, WI, WD])
    s, te, qe, bad = oracle.rescore(T, Q, [0, 0, 0], [0, 0, 0], [0, 1, 4], [1, 3, 3], words, SC)
    assert bad == 0
    assert s[0] == 7 * m + tv and (te[0], qe[0]) == (8, 8)
    assert (te[1], qe[1]) == (8, 10)
    # WI's 5M aligns T[3:8] = "TACGT" with Q[5:10] = "CGTTT": T-C ts, A-G ts, C-T ts, G-T tv, T-T m
    assert s[1] == 3 * m - (go + 2 * ge) + (ts + ts + ts + tv + m)
    assert s[2] == 2 * m - (go + ge) + (tv + m) and (te[2], qe[2]) == (5, 4)


def test_rescore_flags_bad_rows():
    T, Q = b"ACGT", b"ACGT"
    words = np.array([5 << 4, 2 << 4, (1 << 4) | 7], dtype=np.uint32)
    s, te, qe, bad = oracle.rescore(T, Q, [0, 3, 0], [0, 0, 0], [0, 1, 2], [1, 1, 1], words, SC)
    assert bad == 3 and (s == 0).all()


def test_rescore_matches_oracle_alignments(tiny_small):
    """Every alignment the oracle traces rescores to its own score and end."""
    w = tiny_small
    oh, ow, oo = oracle.run(w["target"], w["query"], w["seeds"], w["scoring"], w["ydrop"])
    ok = (oh["status"] == 0) & (oh["n_runs"] > 0)
    s, te, qe, bad = oracle.rescore(w["target"], w["query"], oh["t_begin"][ok], oh["q_begin"][ok], oo[ok],
                                    oh["n_runs"][ok], ow, w["scoring"])
    assert bad == 0 and ok.sum() > 50
    assert (s == oh["score"][ok]).all() and (te == oh["t_end"][ok]).all() and (qe == oh["q_end"][ok]).all()

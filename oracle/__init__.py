"""CPU oracle for batched gapped seed extension -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product library never does, and this package never
imports the product.  The arithmetic lives in ``fz_oracle.c`` (plain C,
int64, anti-diagonal order, value-based traceback); this module only builds
that file with gcc and marshals numpy arrays through ctypes.

See the header of ``fz_oracle.c`` for the passages of the FastZ paper (SC'21)
each part follows.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fz_oracle.c")
_LIB = os.path.join(_HERE, "libfz_oracle.so")

YDROP_INF = 2147483647

STATUS_ESEED, STATUS_EBASE, STATUS_ERANGE, STATUS_ENOMEM = 1, 2, 4, 8
STATUS_COVERED = 128          # extend_rounds: the seed lies on an earlier round's alignment

HIT_FIELDS = ["score", "t_begin", "t_end", "q_begin", "q_end",
              "score_l", "i_l", "j_l", "score_r", "i_r", "j_r",
              "cells_l", "cells_r", "dend_l", "dend_r", "n_runs", "status"]
HIT_DTYPE = np.dtype([(f, np.int64) for f in HIT_FIELDS])
SEED_FIELDS = ["t_pos", "q_pos", "seed_len", "t_lo", "t_hi", "q_lo", "q_hi"]


def build(force=True):
    """Compile the oracle with gcc (plain -O2, pthreads)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
                           "-pthread", _SRC, "-o", tmp])
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.fzo_run.restype = P
        lib.fzo_run.argtypes = [P, i64, P, i64, P, i64, P, i64, i64, ctypes.c_int, ctypes.c_int,
                                ctypes.c_int, P]
        lib.fzo_copy_cigars.restype = None
        lib.fzo_copy_cigars.argtypes = [P, P, P]
        lib.fzo_free.restype = None
        lib.fzo_free.argtypes = [P]
        lib.fzo_side_matrix.restype = i64
        lib.fzo_side_matrix.argtypes = [P, i64, P, i64, P, i64, P, P, P, P, P, P]
        lib.fzo_rescore.restype = i64
        lib.fzo_rescore.argtypes = [P, i64, P, i64, P, P, P, P, P, P, i64, P]
        _lib = lib
    return _lib


def _scoring_arr(scoring):
    """The C struct's fields in order.  A scoring dict with a "matrix" (4x4,
    rows = target base, columns = query base, order A, C, G, T) and an
    "n_score" (a pair with N) uses them instead of match / transition /
    transversion, and then accepts N in the sequences."""
    mat = scoring.get("matrix")
    use = mat is not None
    sub = np.asarray(mat, dtype=np.int64).reshape(16) if use else np.zeros(16, dtype=np.int64)
    head = [scoring.get("match", 0), scoring.get("transition", 0), scoring.get("transversion", 0),
            scoring["gap_open"], scoring["gap_extend"], int(use)]
    return np.concatenate([np.array(head, dtype=np.int64), sub,
                           np.array([scoring.get("n_score", 0) if use else 0], dtype=np.int64)])


def _as_bytes(seq):
    if isinstance(seq, (bytes, bytearray)):
        return np.frombuffer(bytes(seq), dtype=np.uint8).copy()
    if isinstance(seq, str):
        return np.frombuffer(seq.encode(), dtype=np.uint8).copy()
    return np.ascontiguousarray(seq, dtype=np.uint8)


# Complement of each ASCII base: A<->T, C<->G in either case; any other byte
# maps to itself, so the batch still rejects it as a non-ACGT input.
_COMPLEMENT = np.arange(256, dtype=np.uint8)
for _a, _b in ("AT", "TA", "CG", "GC", "at", "ta", "cg", "gc"):
    _COMPLEMENT[ord(_a)] = ord(_b)


def revcomp(seq):
    """Reverse complement of an ASCII sequence: the other strand read in its
    own direction, base j being the complement of base len-1-j.

    FastZ (SC'21), section 2, places the extension inside whole-genome
    alignment, which searches both strands of the query; the pages do not
    spell out the reverse strand, so this is the textbook definition, and an
    extension on the reverse strand is the forward extension against this
    sequence (seeds and windows in its coordinates).
    """
    return _COMPLEMENT[_as_bytes(seq)[::-1]]


_CODE = np.full(256, -1, dtype=np.int64)
for _k, _c in enumerate("ACGT"):
    _CODE[ord(_c)] = _k
    _CODE[ord(_c.lower())] = _k


def find_seeds(target, query, k=19, flank=32768, dedup=True, query_rc=False):
    """The seed stage: every (t, q) with target[t:t+k] == query[q:q+k] (with
    query_rc, q indexes the query's reverse complement), N (the unknown base,
    either case) matching nothing, not even N.

    FastZ (SC'21), section 2: whole-genome alignment first finds short exact
    matches (19 bases) between the two sequences as seed sites and then
    filters them before the gapped extension.  The filter here is the
    plainest one: with dedup, of each run of hits on consecutive positions of
    one diagonal t - q only the first is kept.  Seeds are ordered by diagonal
    t - q, then t; windows are [x - flank, x + k + flank) clipped to each
    sequence.  Returns (seeds, n_hits): an (n, 7) int64 array in
    SEED_FIELDS order and the number of hits before the dedup.
    """
    T = _as_bytes(target)
    Q = revcomp(query) if query_rc else _as_bytes(query)
    tc, qc = _CODE[T], _CODE[Q]
    tn, qn = (T | 0x20) == ord("n"), (Q | 0x20) == ord("n")
    if ((tc < 0) & ~tn).any() or ((qc < 0) & ~qn).any():
        raise ValueError("sequence holds a byte other than A, C, G, T, N")
    if not 1 <= k <= 32:
        raise ValueError("k must be 1..32")
    nt, nq = T.size - k + 1, Q.size - k + 1
    if nt <= 0 or nq <= 0:
        return np.zeros((0, 7), dtype=np.int64), 0

    def kmers(c, isn, n):
        # the k codes from each start as a base-4 number, first base most
        # significant; and whether the k bases hold no N (N is no base: a
        # k-mer with N matches nothing)
        v = np.zeros(n, dtype=np.uint64)
        bad = np.zeros(n, dtype=bool)
        for i in range(k):
            v = v * np.uint64(4) + np.maximum(c[i:i + n], 0).astype(np.uint64)
            bad |= isn[i:i + n]
        return v, ~bad

    tk, tv = kmers(tc, tn, nt)
    qk, qv = kmers(qc, qn, nq)
    tpos = np.nonzero(tv)[0]
    tk = tk[tv]
    order = np.argsort(tk, kind="stable")
    st = tk[order]
    lo = np.searchsorted(st, qk, "left")
    hi = np.searchsorted(st, qk, "right")
    cnt = np.where(qv, hi - lo, 0)
    n_hits = int(cnt.sum())
    q = np.repeat(np.arange(nq, dtype=np.int64), cnt)
    first = np.repeat(lo, cnt)
    nth = np.arange(n_hits, dtype=np.int64) - np.repeat(np.cumsum(cnt) - cnt, cnt)
    t = tpos[order[first + nth]].astype(np.int64)
    diag = t - q
    o = np.lexsort((t, diag))
    t, q, diag = t[o], q[o], diag[o]
    if dedup and n_hits:
        keep = np.ones(n_hits, dtype=bool)
        keep[1:] = ~((diag[1:] == diag[:-1]) & (t[1:] == t[:-1] + 1))
        t, q = t[keep], q[keep]
    out = np.empty((t.size, 7), dtype=np.int64)
    out[:, 0], out[:, 1], out[:, 2] = t, q, k
    out[:, 3] = np.maximum(t - flank, 0)
    out[:, 4] = np.minimum(t + k + flank, T.size)
    out[:, 5] = np.maximum(q - flank, 0)
    out[:, 6] = np.minimum(q + k + flank, Q.size)
    return out, n_hits


def seeds_array(seeds):
    """Seeds as an (n, 7) int64 array in SEED_FIELDS order."""
    if isinstance(seeds, np.ndarray) and seeds.dtype.names:
        return np.stack([seeds[f].astype(np.int64) for f in SEED_FIELDS], axis=1).copy()
    a = np.ascontiguousarray(seeds, dtype=np.int64)
    return a.reshape(-1, 7)


def default_threads():
    """Worker threads of a batch run: the CPUs this process may use, at most
    16 (a GPU host's share per GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def run(target, query, seeds, scoring, ydrop, min_tb=None, traceback=True, local=False,
        threads=None):
    """Run the oracle on a batch.

    Returns (hits, cigar_words, cigar_offsets): hits is a structured array with
    HIT_FIELDS, cigar_words the concatenated BAM-style run words (len << 4 | op,
    op 0=M 1=I 2=D) of every seed that was traced, cigar_offsets[k] the start of
    seed k's runs (n_runs of them).
    """
    lib = _load()
    T = _as_bytes(target)
    Q = _as_bytes(query)
    S = seeds_array(seeds)
    n = S.shape[0]
    sc = _scoring_arr(scoring)
    hits = np.zeros(n, dtype=HIT_DTYPE)
    if threads is None:
        threads = default_threads()
    if min_tb is None:
        min_tb = -(1 << 62)
    h = lib.fzo_run(T.ctypes.data, T.size, Q.ctypes.data, Q.size, S.ctypes.data, n, sc.ctypes.data,
                    int(ydrop), int(min_tb), int(bool(traceback)), int(bool(local)), int(threads),
                    hits.ctypes.data)
    if not h:
        raise MemoryError("oracle batch allocation failed")
    try:
        total = int(hits["n_runs"].sum())
        words = np.zeros(max(total, 1), dtype=np.uint32)
        lib.fzo_copy_cigars(h, hits.ctypes.data, words.ctypes.data)
    finally:
        lib.fzo_free(h)
    offs = np.zeros(n, dtype=np.int64)
    if n:
        offs[1:] = np.cumsum(hits["n_runs"])[:-1]
    return hits, words[:total], offs


def side(a, b, scoring, ydrop, matrices=False, traceback=True):
    """One side on explicit sequences a (rows, length m) and b (columns, n).

    Returns dict(score, ie, je, cells, dend, ops[, S, I, D]); ops end-first
    ('M', 'I', 'D'); matrices hold None for cells never evaluated or dead.
    """
    lib = _load()
    A = _as_bytes(a)
    B = _as_bytes(b)
    m, n = A.size, B.size
    sc = _scoring_arr(scoring)
    out5 = np.zeros(5, dtype=np.int64)
    Sm = Im = Dm = None
    if matrices:
        Sm = np.zeros((m + 1, n + 1), dtype=np.int64)
        Im = np.zeros_like(Sm)
        Dm = np.zeros_like(Sm)
    ops = ctypes.create_string_buffer(m + n + 2) if traceback else None
    nops = ctypes.c_int64(0)
    Ap = A.ctypes.data if m else ctypes.c_void_p(ctypes.addressof(ctypes.c_char()))
    Bp = B.ctypes.data if n else ctypes.c_void_p(ctypes.addressof(ctypes.c_char()))
    st = lib.fzo_side_matrix(Ap, m, Bp, n, sc.ctypes.data, int(ydrop), out5.ctypes.data,
                             Sm.ctypes.data if matrices else None,
                             Im.ctypes.data if matrices else None,
                             Dm.ctypes.data if matrices else None,
                             ops, ctypes.byref(nops) if traceback else None)
    res = dict(score=int(out5[0]), ie=int(out5[1]), je=int(out5[2]), cells=int(out5[3]),
               dend=int(out5[4]), status=int(st))
    if traceback:
        res["ops"] = ops.raw[:nops.value].decode()
    if matrices:
        NEG = np.iinfo(np.int64).min
        res["S"], res["I"], res["D"] = [np.where(x == NEG, None, x).astype(object) for x in (Sm, Im, Dm)]
    return res


def aligned_segments(hits, words, offs):
    """The aligned (M) columns of every traced alignment, as segments on
    diagonals: (t - q, t_first, t_last + 1) for each M run, walking each
    CIGAR from (t_begin, q_begin) (I consumes query, D consumes target)."""
    segs = []
    for k in range(len(hits)):
        n = int(hits["n_runs"][k])
        if n == 0:
            continue
        t, q = int(hits["t_begin"][k]), int(hits["q_begin"][k])
        for w in words[offs[k]:offs[k] + n].tolist():
            ln, op = w >> 4, w & 15
            if op == 0:
                segs.append((t - q, t, t + ln))
                t += ln
                q += ln
            elif op == 1:
                q += ln
            else:
                t += ln
    return segs


def round_bounds(n, round_size, doubling=False):
    """[start, end) of each round: round_size seeds each, or, with doubling,
    round_size for the first round and twice the previous size after it."""
    out, r0, size = [], 0, int(round_size)
    while r0 < n:
        out.append((r0, min(r0 + size, n)))
        r0 += size
        if doubling:
            size *= 2
    return out


def extend_rounds(target, query, seeds, scoring, ydrop, min_tb, round_size, threads=None, doubling=False):
    """Covered-seed suppression by rounds.

    FastZ (SC'21) section 2.1 describes LASTZ ending a seed extension that
    runs into an alignment it found before (joining the two would not pay),
    and section 3.4 why FastZ drops that rule: it depends on the order of
    the extensions.  Reading taken here, the data-parallel form of the rule:
    seeds are taken in the given order in rounds of `round_size` (with
    doubling, each round after the first twice the size of the one before;
    see round_bounds); a seed of
    round r whose exact-match columns (t_pos + k, q_pos + k), k < seed_len,
    share a cell with the aligned (M) columns of an alignment traced (given
    a CIGAR) in rounds before r (a seed without columns, or with columns
    outside the sequences, shares none) is not extended and gets status
    STATUS_COVERED with every other field zero; every other seed of round r
    is extended on its own, as run() extends it.  Seeds of one round never
    suppress each other.

    Returns (hits, words, offsets) as run(); a seed's CIGAR words are those
    run() gives it, concatenated in seed order.
    """
    S = seeds_array(seeds)
    n = S.shape[0]
    T_len, Q_len = _as_bytes(target).size, _as_bytes(query).size
    if round_size < 1:
        raise ValueError("round_size must be >= 1")
    hits = np.zeros(n, dtype=HIT_DTYPE)
    cig = [np.zeros(0, dtype=np.uint32) for _ in range(n)]
    by_diag = {}                       # diagonal -> list of (t_first, t_end) of earlier rounds
    for r0, r1 in round_bounds(n, round_size, doubling):
        idx = np.arange(r0, r1)
        keep = []
        for k in idx:
            t, q, L = int(S[k, 0]), int(S[k, 1]), int(S[k, 2])
            inside = L >= 1 and t >= 0 and q >= 0 and t + L <= T_len and q + L <= Q_len
            covered = inside and any(a < t + L and b > t for a, b in by_diag.get(t - q, ()))
            if covered:
                hits["status"][k] = STATUS_COVERED
            else:
                keep.append(k)
        if not keep:
            continue
        keep = np.array(keep)
        h, w, o = run(target, query, S[keep], scoring, ydrop, min_tb=min_tb, threads=threads)
        hits[keep] = h
        for j, k in enumerate(keep):
            cig[k] = w[o[j]:o[j] + h["n_runs"][j]]
        for dg, a, b in aligned_segments(h, w, o):
            by_diag.setdefault(dg, []).append((a, b))
    words = np.concatenate(cig) if n else np.zeros(0, dtype=np.uint32)
    offs = np.zeros(n, dtype=np.int64)
    if n:
        offs[1:] = np.cumsum(hits["n_runs"])[:-1]
    return hits, words.astype(np.uint32), offs


def cigar_string(words):
    """BAM-style run words -> text CIGAR."""
    return "".join("%d%s" % (w >> 4, "MID"[w & 15]) for w in np.asarray(words, dtype=np.uint32).tolist())


def rescore(target, query, t_begin, q_begin, cigar_off, cigar_len, words, scoring):
    """Score CIGARs laid on the sequences (a check of alignments at any batch
    size): row k's runs words[cigar_off[k] : cigar_off[k] + cigar_len[k]]
    from (t_begin[k], q_begin[k]), M columns by their substitution scores,
    each gap run of length g at -(gap_open + g * gap_extend).  Returns
    (score, t_end, q_end, n_bad) with int64 arrays; rows that leave the
    sequences or hold an unknown code or base count in n_bad and read 0."""
    lib = _load()
    T = _as_bytes(target)
    Q = _as_bytes(query)
    sc = _scoring_arr(scoring)
    tb = np.ascontiguousarray(t_begin, dtype=np.int64)
    qb = np.ascontiguousarray(q_begin, dtype=np.int64)
    off = np.ascontiguousarray(cigar_off, dtype=np.int64)
    ln = np.ascontiguousarray(cigar_len, dtype=np.int64)
    W = np.ascontiguousarray(words, dtype=np.uint32)
    if W.size == 0:
        W = np.zeros(1, dtype=np.uint32)
    n = tb.size
    out = np.zeros((max(n, 1), 3), dtype=np.int64)
    bad = lib.fzo_rescore(T.ctypes.data, T.size, Q.ctypes.data, Q.size, sc.ctypes.data, tb.ctypes.data,
                          qb.ctypes.data, off.ctypes.data, ln.ctypes.data, W.ctypes.data, n, out.ctypes.data)
    return out[:n, 0].copy(), out[:n, 1].copy(), out[:n, 2].copy(), int(bad)

"""Seeded synthetic inputs for batched gapped seed extension.

This module only draws sequences and seed lists; it holds none of the
alignment arithmetic, so both the GPU path and the CPU oracle can be fed from
it.  Every generator is deterministic in its `seed` argument
(numpy.random.default_rng).

The FastZ paper measures on real chromosome pairs (its Table 1 and Fig. 6:
nematode, fly and mosquito chromosomes of 12-31 Mbp, one million seed sites
near one random site, section 4).  Those genomes are not available here, so
these generators produce inputs with the same shapes: chromosome-scale
sequences, 19-bp exact seeds, and the skewed alignment-length mix of the
paper's section 1 (most seed sites give alignments of at most 128 bp, a few
run to tens of kb) and Table 2.

Bases are ASCII bytes 'A', 'C', 'G', 'T' (and 'N', the unknown base, in the
matrix workloads).  A seed record is seven int64s:
(t_pos, q_pos, seed_len, t_lo, t_hi, q_lo, q_hi); the windows are half-open.
"""
import numpy as np

ACGT = np.frombuffer(b"ACGT", dtype=np.uint8)
SEED_LEN = 19
WINDOW_FLANK = 32768          # largest length bin of FastZ section 3.3

DEFAULT_SCORING = dict(match=91, transition=-31, transversion=-123, gap_open=400, gap_extend=30)
DEFAULT_YDROP = 9400

# A synthetic asymmetric 4x4 substitution matrix (rows = target base,
# columns = query base, order A, C, G, T) of the same magnitudes as the
# default triple: matches 92..100, transitions about -30, transversions
# about -120; and a score for any pair with the unknown base N.
DEFAULT_MATRIX = [[95, -120, -30, -125],
                  [-115, 100, -120, -35],
                  [-32, -118, 98, -110],
                  [-122, -28, -116, 92]]
DEFAULT_N_SCORE = -100


def matrix_scoring(matrix=None, n_score=DEFAULT_N_SCORE, gap_open=400, gap_extend=30):
    return dict(matrix=[list(r) for r in (DEFAULT_MATRIX if matrix is None else matrix)], n_score=n_score,
                gap_open=gap_open, gap_extend=gap_extend)


def plant_n_runs(rng, ascii_seq, n_runs, len_min, len_max, keep=None):
    """A copy of an ASCII sequence with `n_runs` runs of 'N' (lengths
    U{len_min..len_max}, uniform start positions); positions where `keep`
    is true keep their bases."""
    out = np.array(ascii_seq, dtype=np.uint8, copy=True)
    if out.size == 0 or n_runs <= 0:
        return out
    starts = rng.integers(0, out.size, size=n_runs)
    lens = rng.integers(len_min, len_max + 1, size=n_runs)
    cover = np.zeros(out.size + 1, dtype=np.int64)
    np.add.at(cover, starts, 1)
    np.add.at(cover, np.minimum(starts + lens, out.size), -1)
    mask = np.cumsum(cover[:-1]) > 0
    if keep is not None:
        mask &= ~keep
    out[mask] = ord("N")
    return out


def seed_span_mask(seeds, length, col_pos, col_len=2):
    """True on every base covered by a seed's exact-match columns."""
    cover = np.zeros(length + 1, dtype=np.int64)
    if len(seeds):
        s = seeds[:, col_pos]
        np.add.at(cover, s, 1)
        np.add.at(cover, np.minimum(s + seeds[:, col_len], length), -1)
    return np.cumsum(cover[:-1]) > 0


def with_matrix_and_n(w, n_runs, len_min, len_max, seed):
    """The workload scored with DEFAULT_MATRIX, with runs of N planted in
    both sequences outside every seed's exact columns."""
    rng = np.random.default_rng(seed)
    out = dict(w)
    out["name"] = w["name"] + "_matrix"
    out["scoring"] = matrix_scoring(gap_open=w["scoring"]["gap_open"], gap_extend=w["scoring"]["gap_extend"])
    S = w["seeds"]
    out["target"] = plant_n_runs(rng, w["target"], n_runs, len_min, len_max,
                                 keep=seed_span_mask(S, w["target"].size, 0))
    if w.get("query_rc"):
        # seed columns are on the reverse complement: mirror them
        L = w["query"].size
        m = seed_span_mask(S, L, 1)[::-1]
    else:
        m = seed_span_mask(S, w["query"].size, 1)
    out["query"] = plant_n_runs(rng, w["query"], n_runs, len_min, len_max, keep=m)
    out["info"] = dict(w.get("info", {}), n_runs=n_runs)
    return out


def to_ascii(codes):
    return ACGT[np.asarray(codes, dtype=np.int64)]


def random_codes(rng, n):
    return rng.integers(0, 4, size=int(n), dtype=np.int8)


def revcomp_codes(codes):
    """Reverse complement in base codes (A=0, C=1, G=2, T=3, so the
    complement of c is 3 - c)."""
    return (3 - np.asarray(codes, dtype=np.int8))[::-1].copy()


def mutate(rng, src, sub_rate, indel_rate, p_geom, ts_frac=2.0 / 3.0):
    """Mutated copy of a code array (0..3 = A, C, G, T).

    Walking the source, each position starts an indel with probability
    `indel_rate` (half insertions of Geom(p) random bases placed before the
    position, half deletions of Geom(p) source bases starting there); every
    other position is substituted with probability `sub_rate`, by a
    transition (A<->G, C<->T) with probability `ts_frac`, else by one of the
    two transversions.  Rates may be scalars or per-position arrays.
    """
    src = np.asarray(src, dtype=np.int8)
    n = src.size
    if n == 0:
        return src.copy()
    indel = rng.random(n) < indel_rate
    is_ins = indel & (rng.random(n) < 0.5)
    is_del = indel & ~is_ins
    lens = rng.geometric(p_geom, size=n).astype(np.int64)
    diff = np.zeros(n + 1, dtype=np.int64)
    dpos = np.nonzero(is_del)[0]
    np.add.at(diff, dpos, 1)
    np.add.at(diff, np.minimum(dpos + lens[dpos], n), -1)
    deleted = np.cumsum(diff[:n]) > 0
    subst = (~indel) & (rng.random(n) < sub_rate)
    ts = rng.random(n) < ts_frac
    tv_pick = np.where(rng.random(n) < 0.5, 1, 3).astype(np.int8)
    xor = np.where(ts, np.int8(2), tv_pick).astype(np.int8)
    base = np.where(subst, src ^ xor, src).astype(np.int8)
    ins_n = np.where(is_ins, lens, 0)
    keep = ~deleted
    cnt = ins_n + keep
    total = int(cnt.sum())
    starts = np.cumsum(cnt) - cnt
    out = random_codes(rng, total)
    kp = np.nonzero(keep)[0]
    out[starts[kp] + ins_n[kp]] = base[kp]
    return out


def kmer_keys(codes, k=SEED_LEN):
    """2-bit packed k-mer key at every start position (uint64)."""
    c = np.asarray(codes, dtype=np.uint64)
    n = c.size - k + 1
    if n <= 0:
        return np.zeros(0, dtype=np.uint64)
    key = np.zeros(n, dtype=np.uint64)
    for t in range(k):
        key = (key << np.uint64(2)) | c[t:t + n]
    return key


def shared_kmers(t_codes, q_codes, k=SEED_LEN, t_mask=None, q_mask=None):
    """Every (t, q) with equal k-mers (sort-merge join on packed keys).

    Optional boolean masks drop k-mer start positions before the join.
    Returns (t_pos, q_pos) int64 arrays, sorted by q then t.
    """
    kt = kmer_keys(t_codes, k)
    kq = kmer_keys(q_codes, k)
    tpos = np.arange(kt.size, dtype=np.int64)
    qpos = np.arange(kq.size, dtype=np.int64)
    if t_mask is not None:
        tpos = tpos[t_mask[:kt.size]]
        kt = kt[tpos]
    if q_mask is not None:
        qpos = qpos[q_mask[:kq.size]]
        kq = kq[qpos]
    order = np.argsort(kt, kind="stable")
    st = kt[order]
    # sorted queries make the merge walk memory in order
    qorder = np.argsort(kq, kind="stable")
    kq = kq[qorder]
    qpos = qpos[qorder]
    lo = np.searchsorted(st, kq, "left")
    hi = np.searchsorted(st, kq, "right")
    cnt = hi - lo
    tot = int(cnt.sum())
    qi = np.repeat(qpos, cnt)
    within = np.arange(tot, dtype=np.int64) - np.repeat(np.cumsum(cnt) - cnt, cnt)
    ti = tpos[order[np.repeat(lo, cnt) + within]]
    o = np.lexsort((ti, qi))
    return ti[o], qi[o]


def _windows(t_pos, q_pos, tlen, qlen, flank=WINDOW_FLANK, L=SEED_LEN):
    t_lo = np.maximum(t_pos - flank, 0)
    q_lo = np.maximum(q_pos - flank, 0)
    t_hi = np.minimum(t_pos + L + flank, tlen)
    q_hi = np.minimum(q_pos + L + flank, qlen)
    return t_lo, t_hi, q_lo, q_hi


def _pack(t_pos, q_pos, L, t_lo, t_hi, q_lo, q_hi):
    n = len(t_pos)
    s = np.empty((n, 7), dtype=np.int64)
    s[:, 0] = t_pos
    s[:, 1] = q_pos
    s[:, 2] = L
    s[:, 3] = t_lo
    s[:, 4] = t_hi
    s[:, 5] = q_lo
    s[:, 6] = q_hi
    return s


def _workload(name, t_codes, q_codes, seeds, local=False, min_tb=None, query_rc=False, **info):
    """query_rc: the seeds lie on the reverse complement of `query` (the
    library is called with FZ_QUERY_RC; `query` is the forward strand)."""
    return dict(name=name, target=to_ascii(t_codes), query=to_ascii(q_codes), seeds=seeds,
                scoring=dict(DEFAULT_SCORING), ydrop=DEFAULT_YDROP, local=local,
                traceback=not local, min_tb=min_tb, query_rc=query_rc, info=info)


def tiny(n_seeds=1000, flank=256, seed=0):
    """Tiny batch: each record is a target piece of flank + 19 + flank random
    bases and a query piece mut(left flank) + the same 19-bp seed +
    mut(right flank) (8% substitutions at 2:1 transition:transversion, 1%
    indels of Geom(0.5) length); mutated flanks are cut to at most `flank`
    bases next to the seed.  Windows are the pieces; every seed is traced."""
    rng = np.random.default_rng(seed)
    tparts, qparts, rows = [], [], []
    toff = qoff = 0
    for _ in range(n_seeds):
        left = random_codes(rng, flank)
        core = random_codes(rng, SEED_LEN)
        right = random_codes(rng, flank)
        ml = mutate(rng, left, 0.08, 0.01, 0.5)[-flank:]
        mr = mutate(rng, right, 0.08, 0.01, 0.5)[:flank]
        tp = np.concatenate([left, core, right])
        qp = np.concatenate([ml, core, mr])
        rows.append((toff + flank, qoff + ml.size, SEED_LEN, toff, toff + tp.size, qoff, qoff + qp.size))
        tparts.append(tp)
        qparts.append(qp)
        toff += tp.size
        qoff += qp.size
    seeds = np.array(rows, dtype=np.int64).reshape(-1, 7)
    return _workload("tiny", np.concatenate(tparts), np.concatenate(qparts), seeds,
                     n_seeds=n_seeds, flank=flank)


def local_pairs(n_pairs=4096, length=2048, seed=0):
    """Local-mode batch: independent uniform pairs of `length` bases; each
    record's windows are one pair (seed_len 0)."""
    rng = np.random.default_rng(seed)
    t = random_codes(rng, n_pairs * length)
    q = random_codes(rng, n_pairs * length)
    lo = np.arange(n_pairs, dtype=np.int64) * length
    seeds = _pack(lo, lo, 0, lo, lo + length, lo, lo + length)
    return _workload("local", t, q, seeds, local=True, n_pairs=n_pairs, length=length)


def _homology_with_blocks(rng, src_len, unrelated_frac, run_min, run_max):
    """Run lengths (log-uniform) of homologous stretches and the size of the
    unrelated blocks placed between them, covering src_len bases."""
    runs = []
    hom_target = (1.0 - unrelated_frac) * src_len
    total = 0.0
    while total < hom_target:
        r = int(np.exp(rng.uniform(np.log(run_min), np.log(run_max))))
        runs.append(r)
        total += r
    block = int(round(unrelated_frac * src_len / max(len(runs), 1)))
    return runs, block


def skewed(target_len=10_000_000, n_seeds=1_000_000, short_frac=0.78, long_frac=0.19,
           n_short=150, n_long=50, copies=32, sub_rate=0.15, indel_rate=0.015, p_geom=0.4,
           unrelated_frac=0.10, flank=WINDOW_FLANK, min_tb=3000, seed=0):
    """Skewed seed batch (one million seeds by default).

    Target: uniform random.  Query: a mutated copy of the target (15%
    substitutions 2:1, 1.5% indels of Geom(0.4) length) in which about 10% is
    replaced by unrelated blocks placed between homologous runs of
    log-uniform length 128 bp .. 64 kb.  Repeat families: random strings
    planted as `copies` exact copies at random non-overlapping places in
    target and in query (after the mutation); `n_short` families of
    U{19..34} bases and `n_long` of U{35..100}.  Seeds are shared 19-mers
    drawn uniformly from the hits of each group: `short_frac` from short
    families (both extensions end within 16 bases, the eager-traceback
    class of FastZ Table 2), `long_frac` from long families (alignments of
    at most about 128 bp), the rest from the other shared 19-mers
    (homologous hits that run to tens of kb).  Windows reach `flank` bases
    past each side of the seed."""
    rng = np.random.default_rng(seed)
    T = random_codes(rng, target_len)
    # query: homologous runs separated by unrelated blocks
    runs, block = _homology_with_blocks(rng, target_len, unrelated_frac, 128, 65536)
    parts = []
    pos = 0
    for r in runs:
        if pos >= target_len:
            break
        seg = T[pos:pos + r]
        parts.append(mutate(rng, seg, sub_rate, indel_rate, p_geom))
        pos += r + block
        parts.append(random_codes(rng, block))
    Q = np.concatenate(parts)
    # repeat families, planted in non-overlapping slots
    n_families = n_short + n_long
    fam_len = np.concatenate([rng.integers(SEED_LEN, 35, size=n_short),
                              rng.integers(35, 101, size=n_long)])
    fams = [random_codes(rng, L) for L in fam_len]
    slot = 128

    def plant(seq):
        nslots = seq.size // slot
        picks = rng.choice(nslots, size=n_families * copies, replace=False)
        starts = picks.reshape(n_families, copies) * slot + rng.integers(0, slot - 100, size=(n_families, copies))
        for f in range(n_families):
            for c in range(copies):
                s = starts[f, c]
                seq[s:s + fam_len[f]] = fams[f]
        return starts

    t_starts = plant(T)
    q_starts = plant(Q)

    # family hits: family f, offset o, target copy a, query copy b
    def family_hits(fam_ids, count):
        w = (fam_len[fam_ids] - SEED_LEN + 1).astype(np.float64)
        f = fam_ids[rng.choice(fam_ids.size, size=count, p=w / w.sum())]
        o = (rng.random(count) * (fam_len[f] - SEED_LEN + 1)).astype(np.int64)
        a = rng.integers(0, copies, size=count)
        b = rng.integers(0, copies, size=count)
        return t_starts[f, a] + o, q_starts[f, b] + o

    n_sh = int(round(n_seeds * short_frac))
    n_lg = int(round(n_seeds * long_frac))
    st_, sq_ = family_hits(np.arange(n_short), n_sh)
    lt_, lq_ = family_hits(np.arange(n_short, n_families), n_lg)

    # other hits: shared 19-mers whose positions touch no family copy
    def fam_mask(seq_len, starts):
        cover = np.zeros(seq_len + 1, dtype=np.int64)
        for fi in range(n_families):
            s = starts[fi]
            np.add.at(cover, np.maximum(s - SEED_LEN + 1, 0), 1)
            np.add.at(cover, np.minimum(s + fam_len[fi], seq_len), -1)
        return np.cumsum(cover[:seq_len]) == 0

    ht, hq = shared_kmers(T, Q, t_mask=fam_mask(T.size, t_starts), q_mask=fam_mask(Q.size, q_starts))
    n_hom = n_seeds - n_sh - n_lg
    pick = rng.choice(ht.size, size=min(n_hom, ht.size), replace=False)
    t_pos = np.concatenate([st_, lt_, ht[pick]])
    q_pos = np.concatenate([sq_, lq_, hq[pick]])
    perm = rng.permutation(t_pos.size)
    t_pos, q_pos = t_pos[perm], q_pos[perm]
    t_lo, t_hi, q_lo, q_hi = _windows(t_pos, q_pos, T.size, Q.size, flank)
    seeds = _pack(t_pos, q_pos, SEED_LEN, t_lo, t_hi, q_lo, q_hi)
    return _workload("skewed", T, Q, seeds, min_tb=min_tb, n_short_family_seeds=n_sh,
                     n_long_family_seeds=n_lg, n_other_seeds=int(pick.size),
                     n_other_hits=int(ht.size), query_len=int(Q.size))


def executor_heavy(n_pairs=100_000, len_min=1000, len_max=20000, unrelated=2048, seed=0):
    """Executor-heavy batch: per pair, identity U(0.70, 0.90) (substitutions
    1 - identity at 2:1), 2% indels of Geom(0.5) length, homologous length
    log-uniform in [len_min, len_max].  Target pair = 19-bp seed + L bases +
    `unrelated` random bases; query pair = the same seed + mut(L bases) +
    `unrelated` independent random bases.  The seed sits at the pair start
    (empty left side); every seed is traced."""
    rng = np.random.default_rng(seed)
    ident = rng.uniform(0.70, 0.90, size=n_pairs)
    L = np.exp(rng.uniform(np.log(len_min), np.log(len_max), size=n_pairs)).astype(np.int64)
    tparts, qparts, rows = [], [], []
    toff = qoff = 0
    for k in range(n_pairs):
        core = random_codes(rng, SEED_LEN)
        hom = random_codes(rng, L[k])
        mh = mutate(rng, hom, 1.0 - ident[k], 0.02, 0.5)
        tp = np.concatenate([core, hom, random_codes(rng, unrelated)])
        qp = np.concatenate([core, mh, random_codes(rng, unrelated)])
        rows.append((toff, qoff, SEED_LEN, toff, toff + tp.size, qoff, qoff + qp.size))
        tparts.append(tp)
        qparts.append(qp)
        toff += tp.size
        qoff += qp.size
    seeds = np.array(rows, dtype=np.int64).reshape(-1, 7)
    return _workload("executor_heavy", np.concatenate(tparts), np.concatenate(qparts), seeds,
                     n_pairs=n_pairs, mean_len=float(L.mean()))


def _chromosome_pair(length, sub_rate, indel_rate, p_geom, n_inversions, inv_min, inv_max, unrelated_frac, seed):
    rng = np.random.default_rng(seed)
    C1 = random_codes(rng, length)
    C2 = mutate(rng, C1, sub_rate, indel_rate, p_geom)
    n2 = C2.size
    # non-overlapping inversions
    span = n2 // n_inversions
    for k in range(n_inversions):
        L = int(rng.integers(inv_min, inv_max + 1))
        s = k * span + int(rng.integers(0, max(span - L, 1)))
        C2[s:s + L] = revcomp_codes(C2[s:s + L])
    ub = int(unrelated_frac * n2)
    us = int(rng.integers(0, n2 - ub))
    C2[us:us + ub] = random_codes(rng, ub)
    return C1, C2


def _diagonal_dedup_seeds(t, q, tlen, qlen, flank):
    """Each run of hits on consecutive positions of one diagonal (t - q)
    becomes one seed at the run start; windows +-flank."""
    diag = t - q
    order = np.lexsort((t, diag))
    t, q, diag = t[order], q[order], diag[order]
    start = np.ones(t.size, dtype=bool)
    start[1:] = ~((diag[1:] == diag[:-1]) & (t[1:] == t[:-1] + 1))
    t, q = t[start], q[start]
    t_lo, t_hi, q_lo, q_hi = _windows(t, q, tlen, qlen, flank)
    return _pack(t, q, SEED_LEN, t_lo, t_hi, q_lo, q_hi)


def chromosome(length=20_000_000, sub_rate=0.12, indel_rate=0.01, p_geom=0.3, n_inversions=5,
               inv_min=50_000, inv_max=500_000, unrelated_frac=0.20, flank=WINDOW_FLANK, seed=0):
    """Chromosome-scale pair: C2 = mut(C1) (12% substitutions 2:1, 1% indels of
    Geom(0.3)), then `n_inversions` non-overlapping reverse-complement
    inversions of U(50 kb, 500 kb), then one contiguous unrelated block of
    20% of the length.  Seeds are all forward-strand shared 19-mers after
    diagonal dedup: each run of hits on consecutive positions of one
    diagonal (t - q) becomes one seed at the run start."""
    C1, C2 = _chromosome_pair(length, sub_rate, indel_rate, p_geom, n_inversions, inv_min, inv_max,
                              unrelated_frac, seed)
    t, q = shared_kmers(C1, C2)
    seeds = _diagonal_dedup_seeds(t, q, C1.size, C2.size, flank)
    return _workload("chromosome", C1, C2, seeds, n_seeds=len(seeds))


def chromosome_rc(length=20_000_000, sub_rate=0.12, indel_rate=0.01, p_geom=0.3, n_inversions=5,
                  inv_min=50_000, inv_max=500_000, unrelated_frac=0.20, flank=WINDOW_FLANK, seed=0):
    """The pair of `chromosome` (same parameters, same draw) searched on the
    other strand: seeds are the shared 19-mers of C1 and the reverse
    complement of C2 (mostly inside the inversions), diagonal-deduplicated,
    in the coordinates of that reverse complement.  The query passed is C2
    itself, with query_rc set."""
    C1, C2 = _chromosome_pair(length, sub_rate, indel_rate, p_geom, n_inversions, inv_min, inv_max,
                              unrelated_frac, seed)
    R2 = revcomp_codes(C2)
    t, q = shared_kmers(C1, R2)
    seeds = _diagonal_dedup_seeds(t, q, C1.size, R2.size, flank)
    return _workload("chromosome_rc", C1, C2, seeds, query_rc=True, n_seeds=len(seeds))


def chromosome_seed_stage(length=20_000_000, sub_rate=0.12, indel_rate=0.01, p_geom=0.3, n_inversions=5,
                          inv_min=50_000, inv_max=500_000, unrelated_frac=0.20, flank=WINDOW_FLANK, seed=0):
    """Input of the seed stage itself: the pair of `chromosome` (same
    parameters, same draw) as ASCII, with the seed length and window flank.
    The stage runs on both strands of the query."""
    C1, C2 = _chromosome_pair(length, sub_rate, indel_rate, p_geom, n_inversions, inv_min, inv_max,
                              unrelated_frac, seed)
    return {"name": "chromosome_seed_stage", "target": to_ascii(C1), "query": to_ascii(C2), "k": SEED_LEN,
            "flank": flank}


def homolog_rounds(length=40_000, sub_rate=0.12, indel_rate=0.01, p_geom=0.3, block=6000, gap=2000, flank=3000,
                   min_tb=3000, seed=0):
    """Input for covered-seed suppression: a homologous pair (C2 = mut(C1),
    12% substitutions 2:1, 1% indels of Geom(0.3)) in which every `block`
    bases of C2 end with `gap` unrelated ones, so that it holds several
    alignments; seeds = the shared 19-mers after diagonal dedup (many seeds
    per alignment: every indel starts a new diagonal), windows +-flank, in
    a seeded random order."""
    rng = np.random.default_rng(seed)
    C1 = random_codes(rng, length)
    C2 = mutate(rng, C1, sub_rate, indel_rate, p_geom)
    for s0 in range(block - gap, C2.size, block):
        C2[s0:s0 + gap] = random_codes(rng, min(gap, C2.size - s0))
    t, q = shared_kmers(C1, C2)
    seeds = _diagonal_dedup_seeds(t, q, C1.size, C2.size, flank)
    seeds = seeds[rng.permutation(len(seeds))]
    return _workload("homolog_rounds", C1, C2, seeds, min_tb=min_tb, n_seeds=len(seeds))


def chromosome_rounds(length=20_000_000, seed=0, **kw):
    """The chromosome pair's forward seeds (144,179 at full size) in a seeded
    random order, for covered-seed suppression."""
    w = chromosome(length=length, seed=seed, **kw)
    rng = np.random.default_rng(1000 + seed)
    w = dict(w, seeds=w["seeds"][rng.permutation(len(w["seeds"]))], min_tb=3000)
    w["name"] = "chromosome_rounds"
    return w


def skewed_matrix(seed=0, **kw):
    """The skewed batch scored with the 4x4 matrix, with 400 runs of N of
    10..1000 bases planted in each sequence (about 2% of it) outside the
    seeds' exact columns."""
    return with_matrix_and_n(skewed(seed=seed, **kw), 400, 10, 1000, seed=100 + seed)


WORKLOADS = {
    "tiny": tiny,
    "local": local_pairs,
    "skewed": skewed,
    "executor_heavy": executor_heavy,
    "chromosome": chromosome,
    "chromosome_rc": chromosome_rc,
    "skewed_matrix": skewed_matrix,
    "chromosome_rounds": chromosome_rounds,
}

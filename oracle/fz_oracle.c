/*
 * fz_oracle.c -- plain, slow CPU reference for batched gapped seed extension.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or constant with
 * the GPU path.
 *
 * What it computes follows "FastZ: Accelerating Gapped Whole Genome Alignment
 * on GPUs" (Gundabolu, Vijaykumar, Thottethodi, SC'21):
 *   - the affine-gap Smith-Waterman cell with a total score S, a gap state I
 *     and a gap state D (section 1, Fig. 1).  The figure's recurrence did not
 *     survive extraction; the form below is the one fixed by the operation
 *     counts of section 2.2 observation (1) (five reads, five additions, four
 *     comparisons) and by section 3.1.3 (I and D each choose between two
 *     candidates, S between three), so extension mode has no zero term;
 *   - y-drop pruning (section 2.1, Fig. 3a) in the form of section 3.4
 *     "work reduction": the threshold only uses scores of cells that are
 *     already complete, i.e. of earlier anti-diagonals;
 *   - traceback from the highest-scoring cell (section 2.1, Fig. 3b);
 *   - left and right extensions of a seed done separately, then joined
 *     (section 3.1.2).
 * Local mode (full-window local alignment, zero floor, no y-drop) follows the
 * textbook local recurrence with a zero clamp applied last, as the DPX article
 * ("DPX" page, section 1.1 and section 3.2) describes it, extended to affine
 * gaps.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   gap of length g costs open + g*extend; substitution is match /
 *   transition (A<->G, C<->T) / transversion, or, when a 4x4 matrix is
 *   given, its entry for (target base, query base), with N (either case)
 *   against anything, N included, scoring a separate n_score (N is an
 *   invalid base without a matrix); a cell is dead when S < T_d
 *   (strict), T_d = best score over live cells of diagonals < d minus ydrop,
 *   and a dead cell has S = I = D = -inf; the end cell is the highest S, ties
 *   to the smallest anti-diagonal then the smallest i; traceback prefers the
 *   diagonal move, then I, then D, and inside a gap prefers "opened here" over
 *   "extended"; I consumes query only, D consumes target only; the seed's own
 *   columns are scored with the substitution score.
 *
 * Arithmetic is int64; every live value is checked to fit in int32.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <pthread.h>

#define NEG INT64_MIN          /* minus infinity; any candidate built from NEG stays NEG */
#define NEG32 INT32_MIN        /* the same marker in int32 storage */
#define YDROP_INF 2147483647LL /* ydrop >= this value means "no pruning" */

enum { FZO_OK = 0, FZO_ESEED = 1, FZO_EBASE = 2, FZO_ERANGE = 4, FZO_ENOMEM = 8 };

typedef struct {
    int64_t match, transition, transversion, gap_open, gap_extend;
    int64_t use_matrix;                  /* nonzero: sub[][] and n_score replace the three scores */
    int64_t sub[4][4];                   /* [target base][query base], order A, C, G, T */
    int64_t n_score;                     /* a pair with N on either side */
} fzo_scoring;

typedef struct {
    int64_t t_pos, q_pos, seed_len, t_lo, t_hi, q_lo, q_hi;
} fzo_seed;

typedef struct {
    int64_t score;                       /* seed total, or local maximum */
    int64_t t_begin, t_end, q_begin, q_end;
    int64_t score_l, i_l, j_l;           /* left side: best score and end cell */
    int64_t score_r, i_r, j_r;           /* right side */
    int64_t cells_l, cells_r;            /* canonical cell counts per side */
    int64_t dend_l, dend_r;              /* last anti-diagonal evaluated per side */
    int64_t n_runs;                      /* CIGAR runs (0 when no traceback) */
    int64_t status;
} fzo_hit;

/* ---------------------------------------------------------------- bases -- */

/* 0..3 for A, C, G, T (either case); 4 for N (either case) when a matrix
 * is in use; -1 otherwise.  (The table holds the code plus one; 0 = none.) */
static const signed char CODE1[256] = {
    ['A'] = 1, ['a'] = 1, ['C'] = 2, ['c'] = 2, ['G'] = 3, ['g'] = 3, ['T'] = 4, ['t'] = 4, ['N'] = 5, ['n'] = 5,
};

static int base_code(uint8_t c, const fzo_scoring *sc)
{
    int code = CODE1[c] - 1;
    if (code == 4 && !sc->use_matrix) code = -1;
    return code;
}

/* Substitution score.  With a matrix: its entry, or n_score for a pair with
 * N.  Otherwise transitions are purine<->purine (A,G) and
 * pyrimidine<->pyrimidine (C,T); every other mismatch is a transversion. */
static int64_t sub_score(int a, int b, const fzo_scoring *sc)
{
    if (sc->use_matrix) return (a == 4 || b == 4) ? sc->n_score : sc->sub[a][b];
    if (a == b) return sc->match;
    int a_purine = (a == 0 || a == 2), b_purine = (b == 0 || b == 2);
    if (a_purine == b_purine) return sc->transition;
    return sc->transversion;
}

/* sub_score for every pair of codes 0..4, looked up in the per-cell loops
 * (the same values, evaluated once per extension). */
static void sub_table(const fzo_scoring *sc, int64_t tab[5][5])
{
    for (int a = 0; a < 5; a++)
        for (int b = 0; b < 5; b++)
            tab[a][b] = (a < 4 && b < 4) || sc->use_matrix ? sub_score(a, b, sc) : 0;
}

static int64_t add(int64_t x, int64_t y) { return (x == NEG) ? NEG : x + y; }
static int64_t max2(int64_t x, int64_t y) { return x > y ? x : y; }

/* ------------------------------------------------ one-sided extension ---- */

/* The matrix of one side is stored one anti-diagonal at a time: diagonal d
 * holds the evaluated cells i in [lo[d], hi[d]] (j = d - i) at values
 * S/I/D[off[d] + (i - lo[d])].  Cells never evaluated read as -inf. */
typedef struct {
    int64_t nd, capd;
    int64_t *lo, *hi, *off;
    int64_t *live_lo, *live_hi;          /* hull of live cells, live_lo > live_hi if none */
    int64_t ncell, capc;
    int32_t *S, *I, *D;
    int err;
} band;

static int band_reserve(band *b, int64_t nd, int64_t nc)
{
    if (nd > b->capd) {
        int64_t cap = b->capd ? b->capd : 64;
        while (cap < nd) cap *= 2;
        int64_t **arrs[5] = {&b->lo, &b->hi, &b->off, &b->live_lo, &b->live_hi};
        for (int k = 0; k < 5; k++) {
            int64_t *p = realloc(*arrs[k], (size_t)cap * sizeof(int64_t));
            if (!p) return -1;
            *arrs[k] = p;
        }
        b->capd = cap;
    }
    if (nc > b->capc) {
        int64_t cap = b->capc ? b->capc : 1024;
        while (cap < nc) cap *= 2;
        int32_t **arrs[3] = {&b->S, &b->I, &b->D};
        for (int k = 0; k < 3; k++) {
            int32_t *p = realloc(*arrs[k], (size_t)cap * sizeof(int32_t));
            if (!p) return -1;
            *arrs[k] = p;
        }
        b->capc = cap;
    }
    return 0;
}

static void band_free(band *b)
{
    free(b->lo); free(b->hi); free(b->off); free(b->live_lo); free(b->live_hi);
    free(b->S); free(b->I); free(b->D);
    memset(b, 0, sizeof *b);
}

static int64_t load(const band *b, const int32_t *arr, int64_t i, int64_t j)
{
    int64_t d = i + j;
    if (i < 0 || j < 0 || d >= b->nd) return NEG;
    if (i < b->lo[d] || i > b->hi[d]) return NEG;
    int32_t v = arr[b->off[d] + (i - b->lo[d])];
    return v == NEG32 ? NEG : (int64_t)v;
}

static int32_t store_val(band *b, int64_t v)
{
    if (v == NEG) return NEG32;
    if (v <= (int64_t)INT32_MIN || v > (int64_t)INT32_MAX) { b->err |= FZO_ERANGE; return NEG32; }
    return (int32_t)v;
}

typedef struct {
    const uint8_t *t; int64_t tdir;      /* a_i = t[tdir * i], i = 1..m */
    const uint8_t *q; int64_t qdir;      /* b_j = q[qdir * j], j = 1..n */
    int64_t m, n;
} side_seq;

static int side_base(const uint8_t *p, int64_t dir, int64_t idx, const fzo_scoring *sc, int *err)
{
    int c = base_code(p[dir * idx], sc);
    if (c < 0) { *err |= FZO_EBASE; c = 0; }
    return c;
}

typedef struct {
    int64_t score, ie, je, cells, dend;
} side_result;

/*
 * Anti-diagonal-synchronous y-drop extension of one side (FastZ section 2.1
 * and section 3.4).  Diagonal d is evaluated on the range R_d: the hull of
 * the cells that can have a live predecessor -- (i, j-1) and (i-1, j) on d-1,
 * (i-1, j-1) on d-2 -- clipped to the matrix.  The run stops when R_d is
 * empty.  Every cell of R_d is counted in `cells`.
 */
static void extend_side(const side_seq *s, const fzo_scoring *sc, int64_t ydrop,
                        band *b, side_result *r)
{
    const int64_t OE = sc->gap_open + sc->gap_extend, E = sc->gap_extend;
    int64_t tab[5][5];
    sub_table(sc, tab);
    b->nd = 0; b->ncell = 0; b->err = 0;
    r->score = 0; r->ie = 0; r->je = 0; r->cells = 0; r->dend = 0;

    int64_t best = 0, best_i = 0, best_j = 0;
    for (int64_t d = 0;; d++) {
        int64_t lo, hi;
        if (d == 0) {
            lo = 0; hi = 0;
        } else {
            lo = INT64_MAX; hi = INT64_MIN;
            for (int64_t back = 1; back <= 2 && d - back >= 0; back++) {
                int64_t pl = b->live_lo[d - back], ph = b->live_hi[d - back];
                if (pl > ph) continue;
                /* from d-1: (i, j-1) -> i, (i-1, j) -> i+1;  from d-2: (i-1, j-1) -> i+1 */
                int64_t cl = (back == 1) ? pl : pl + 1, ch = ph + 1;
                if (cl < lo) lo = cl;
                if (ch > hi) hi = ch;
            }
            if (lo < d - s->n) lo = d - s->n;
            if (lo < 0) lo = 0;
            if (hi > s->m) hi = s->m;
            if (hi > d) hi = d;
            if (lo > hi) break;                       /* R_d empty: extension over */
        }
        if (band_reserve(b, d + 1, b->ncell + (hi - lo + 1)) != 0) { b->err |= FZO_ENOMEM; break; }
        b->lo[d] = lo; b->hi[d] = hi; b->off[d] = b->ncell;
        b->ncell += hi - lo + 1;
        b->nd = d + 1;
        r->cells += hi - lo + 1;
        r->dend = d;

        int64_t thr = (ydrop >= YDROP_INF) ? NEG : best - ydrop;   /* T_d from diagonals < d */
        int64_t llo = INT64_MAX, lhi = INT64_MIN;
        int64_t dbest = NEG, dbest_i = 0;
        for (int64_t i = lo; i <= hi; i++) {
            int64_t j = d - i, S, I, D;
            if (d == 0) {
                S = 0; I = NEG; D = NEG;
            } else {
                /* I: gap consuming query only, entered from the left. */
                I = max2(add(load(b, b->I, i, j - 1), -E), add(load(b, b->S, i, j - 1), -OE));
                /* D: gap consuming target only, entered from above. */
                D = max2(add(load(b, b->D, i - 1, j), -E), add(load(b, b->S, i - 1, j), -OE));
                int64_t H = NEG;
                if (i >= 1 && j >= 1) {
                    int e = 0;
                    int ca = side_base(s->t, s->tdir, i, sc, &e), cb = side_base(s->q, s->qdir, j, sc, &e);
                    b->err |= e;
                    H = add(load(b, b->S, i - 1, j - 1), tab[ca][cb]);
                }
                S = max2(H, max2(I, D));
                if (S == NEG || (thr != NEG && S < thr)) { S = NEG; I = NEG; D = NEG; }
            }
            int64_t k = b->off[d] + (i - lo);
            b->S[k] = store_val(b, S); b->I[k] = store_val(b, I); b->D[k] = store_val(b, D);
            if (S != NEG) {
                if (i < llo) llo = i;
                if (i > lhi) lhi = i;
                if (S > dbest) { dbest = S; dbest_i = i; }
            }
        }
        b->live_lo[d] = (llo <= lhi) ? llo : 1;
        b->live_hi[d] = (llo <= lhi) ? lhi : 0;
        if (dbest != NEG && (d == 0 || dbest > best)) { best = dbest; best_i = dbest_i; best_j = d - dbest_i; }
    }
    r->score = best; r->ie = best_i; r->je = best_j;
}

/* Traceback from (ie, je) in state S back to (0,0), re-deriving every choice
 * from the stored values (no pointers).  Ops are emitted end-first:
 * 'M' consumes a_i and b_j, 'I' consumes b_j only, 'D' consumes a_i only. */
static int64_t traceback(const side_seq *s, const fzo_scoring *sc, const band *b,
                         int64_t ie, int64_t je, char *ops, int *err)
{
    const int64_t OE = sc->gap_open + sc->gap_extend, E = sc->gap_extend;
    int64_t i = ie, j = je, n = 0;
    enum { ST_S, ST_I, ST_D } st = ST_S;
    while (!(st == ST_S && i == 0 && j == 0)) {
        if (st == ST_S) {
            int64_t Sv = load(b, b->S, i, j);
            int64_t H = NEG;
            if (i >= 1 && j >= 1) {
                int e = 0;
                H = add(load(b, b->S, i - 1, j - 1),
                        sub_score(side_base(s->t, s->tdir, i, sc, &e), side_base(s->q, s->qdir, j, sc, &e), sc));
            }
            if (Sv != NEG && Sv == H) { ops[n++] = 'M'; i--; j--; }
            else if (Sv != NEG && Sv == load(b, b->I, i, j)) st = ST_I;
            else if (Sv != NEG && Sv == load(b, b->D, i, j)) st = ST_D;
            else { *err |= FZO_ERANGE; return n; }
        } else if (st == ST_I) {
            int64_t Iv = load(b, b->I, i, j);
            ops[n++] = 'I';
            if (Iv != NEG && Iv == add(load(b, b->S, i, j - 1), -OE)) st = ST_S;     /* opened here */
            else if (Iv == NEG || Iv != add(load(b, b->I, i, j - 1), -E)) { *err |= FZO_ERANGE; return n; }
            j--;
        } else {
            int64_t Dv = load(b, b->D, i, j);
            ops[n++] = 'D';
            if (Dv != NEG && Dv == add(load(b, b->S, i - 1, j), -OE)) st = ST_S;
            else if (Dv == NEG || Dv != add(load(b, b->D, i - 1, j), -E)) { *err |= FZO_ERANGE; return n; }
            i--;
        }
        if (i < 0 || j < 0) { *err |= FZO_ERANGE; return n; }
    }
    return n;
}

/* ----------------------------------------------------------- one seed --- */

typedef struct {
    band bl, br;
    char *ops; int64_t capops;
} worker_mem;

/* Run-length encode an op string into BAM-style words: len << 4 | code,
 * code 0 = M, 1 = I, 2 = D. */
static int64_t rle_append(uint32_t *out, int64_t nruns, char op, int64_t count)
{
    if (count <= 0) return nruns;
    uint32_t code = (op == 'M') ? 0u : (op == 'I') ? 1u : 2u;
    if (nruns > 0 && (out[nruns - 1] & 15u) == code) {
        out[nruns - 1] += (uint32_t)count << 4;
        return nruns;
    }
    out[nruns] = ((uint32_t)count << 4) | code;
    return nruns + 1;
}

/* Two-sided extension of one seed: left side reads T and Q backwards from
 * the seed start, right side forwards from the seed end (FastZ 3.1.2).
 * If traceback is wanted and the total exceeds min_tb, the CIGAR words are
 * written to *cigar (malloc'd).  Returns status. */
static int64_t extend_seed(const uint8_t *T, int64_t tlen, const uint8_t *Q, int64_t qlen,
                           const fzo_seed *sd, const fzo_scoring *sc, int64_t ydrop,
                           int64_t min_tb, int want_tb, worker_mem *w,
                           fzo_hit *h, uint32_t **cigar)
{
    memset(h, 0, sizeof *h);
    *cigar = NULL;
    int64_t L = sd->seed_len;
    if (L < 0 || sd->t_lo < 0 || sd->q_lo < 0 || sd->t_hi > tlen || sd->q_hi > qlen ||
        sd->t_pos < sd->t_lo || sd->q_pos < sd->q_lo ||
        sd->t_pos + L > sd->t_hi || sd->q_pos + L > sd->q_hi) {
        h->status = FZO_ESEED;
        return h->status;
    }
    side_seq left = { T + sd->t_pos, -1, Q + sd->q_pos, -1, sd->t_pos - sd->t_lo, sd->q_pos - sd->q_lo };
    side_seq right = { T + sd->t_pos + L - 1, 1, Q + sd->q_pos + L - 1, 1,
                       sd->t_hi - sd->t_pos - L, sd->q_hi - sd->q_pos - L };
    side_result rl, rr;
    extend_side(&left, sc, ydrop, &w->bl, &rl);
    extend_side(&right, sc, ydrop, &w->br, &rr);
    int err = w->bl.err | w->br.err;

    int64_t seed_score = 0;
    for (int64_t k = 0; k < L; k++) {
        int ca = base_code(T[sd->t_pos + k], sc), cb = base_code(Q[sd->q_pos + k], sc);
        if (ca < 0 || cb < 0) { err |= FZO_EBASE; continue; }
        seed_score += sub_score(ca, cb, sc);
    }
    h->score = rl.score + seed_score + rr.score;
    h->score_l = rl.score; h->i_l = rl.ie; h->j_l = rl.je;
    h->score_r = rr.score; h->i_r = rr.ie; h->j_r = rr.je;
    h->cells_l = rl.cells; h->cells_r = rr.cells;
    h->dend_l = rl.dend; h->dend_r = rr.dend;
    h->t_begin = sd->t_pos - rl.ie; h->q_begin = sd->q_pos - rl.je;
    h->t_end = sd->t_pos + L + rr.ie; h->q_end = sd->q_pos + L + rr.je;
    if (h->score > INT32_MAX || h->score < INT32_MIN) err |= FZO_ERANGE;

    if (want_tb && h->score > min_tb && err == 0) {
        int64_t need = rl.ie + rl.je + rr.ie + rr.je + 2;
        if (need > w->capops) {
            char *p = realloc(w->ops, (size_t)need);
            if (!p) { h->status = FZO_ENOMEM; return h->status; }
            w->ops = p; w->capops = need;
        }
        int64_t nl = traceback(&left, sc, &w->bl, rl.ie, rl.je, w->ops, &err);
        int64_t nr = traceback(&right, sc, &w->br, rr.ie, rr.je, w->ops + nl, &err);
        uint32_t *out = malloc((size_t)(nl + nr + 1) * sizeof(uint32_t));
        if (!out) { h->status = FZO_ENOMEM; return h->status; }
        int64_t nruns = 0;
        /* left ops come out in forward genome order already */
        for (int64_t k = 0; k < nl; k++) nruns = rle_append(out, nruns, w->ops[k], 1);
        nruns = rle_append(out, nruns, 'M', L);
        /* right ops come out end-first: reverse them */
        for (int64_t k = nl + nr - 1; k >= nl; k--) nruns = rle_append(out, nruns, w->ops[k], 1);
        *cigar = out;
        h->n_runs = nruns;
    }
    h->status = err;
    return err;
}

/* --------------------------------------------------------- local mode --- */

/* Full-window local alignment with affine gaps: S = max(0, H, I, D) over the
 * whole window, boundary row and column S = 0, I = D = -inf; no y-drop.
 * Score = max S; end = smallest anti-diagonal, then smallest i. */
static int64_t local_pair(const uint8_t *a, int64_t m, const uint8_t *bq, int64_t n,
                          const fzo_scoring *sc, fzo_hit *h)
{
    const int64_t OE = sc->gap_open + sc->gap_extend, E = sc->gap_extend;
    int64_t tab[5][5];
    sub_table(sc, tab);
    memset(h, 0, sizeof *h);
    int64_t *Sp = malloc((size_t)(n + 1) * sizeof(int64_t));   /* row i-1 */
    int64_t *Sc = malloc((size_t)(n + 1) * sizeof(int64_t));   /* row i */
    int64_t *Dp = malloc((size_t)(n + 1) * sizeof(int64_t));   /* D of row i-1 */
    int64_t *Dc = malloc((size_t)(n + 1) * sizeof(int64_t));
    int *cb = malloc((size_t)(n + 1) * sizeof(int));
    if (!Sp || !Sc || !Dp || !Dc || !cb) {
        free(Sp); free(Sc); free(Dp); free(Dc); free(cb);
        h->status = FZO_ENOMEM; return h->status;
    }
    int err = 0;
    for (int64_t j = 1; j <= n; j++) {
        cb[j] = base_code(bq[j - 1], sc);
        if (cb[j] < 0) { err |= FZO_EBASE; cb[j] = 0; }
    }
    for (int64_t j = 0; j <= n; j++) { Sp[j] = 0; Dp[j] = NEG; }
    int64_t best = 0, bi = 0, bj = 0;
    for (int64_t i = 1; i <= m; i++) {
        int ca = base_code(a[i - 1], sc);
        if (ca < 0) { err |= FZO_EBASE; ca = 0; }
        Sc[0] = 0; Dc[0] = NEG;
        int64_t I = NEG;                 /* I(i, j-1) */
        for (int64_t j = 1; j <= n; j++) {
            I = max2(add(I, -E), Sc[j - 1] - OE);
            int64_t D = max2(add(Dp[j], -E), Sp[j] - OE);
            int64_t H = Sp[j - 1] + tab[ca][cb[j]];
            int64_t S = max2(0, max2(H, max2(I, D)));
            Sc[j] = S; Dc[j] = D;
            if (S > INT32_MAX) err |= FZO_ERANGE;
            if (S > best || (S == best && (i + j < bi + bj || (i + j == bi + bj && i < bi)))) {
                best = S; bi = i; bj = j;
            }
        }
        int64_t *t = Sp; Sp = Sc; Sc = t;
        t = Dp; Dp = Dc; Dc = t;
    }
    if (best == 0) { bi = 0; bj = 0; }
    h->score = best;
    h->t_begin = 0; h->q_begin = 0; h->t_end = bi; h->q_end = bj;   /* window-relative end cell */
    h->i_r = bi; h->j_r = bj;
    h->cells_r = m * n;
    h->status = err;
    free(Sp); free(Sc); free(Dp); free(Dc); free(cb);
    return err;
}

/* ------------------------------------------------------------- batches --- */

typedef struct {
    const uint8_t *T, *Q; int64_t tlen, qlen;
    const fzo_seed *seeds; int64_t n;
    fzo_scoring sc; int64_t ydrop, min_tb; int want_tb, local;
    fzo_hit *hits; uint32_t **cigars;
    int64_t next;
    pthread_mutex_t mu;
} batch_job;

static void *batch_worker(void *arg)
{
    batch_job *job = arg;
    worker_mem w;
    memset(&w, 0, sizeof w);
    for (;;) {
        pthread_mutex_lock(&job->mu);
        int64_t k = job->next++;
        pthread_mutex_unlock(&job->mu);
        if (k >= job->n) break;
        const fzo_seed *sd = &job->seeds[k];
        if (job->local) {
            if (sd->t_lo < 0 || sd->q_lo < 0 || sd->t_hi > job->tlen || sd->q_hi > job->qlen ||
                sd->t_lo > sd->t_hi || sd->q_lo > sd->q_hi) {
                memset(&job->hits[k], 0, sizeof(fzo_hit));
                job->hits[k].status = FZO_ESEED;
                continue;
            }
            local_pair(job->T + sd->t_lo, sd->t_hi - sd->t_lo, job->Q + sd->q_lo, sd->q_hi - sd->q_lo,
                       &job->sc, &job->hits[k]);
            job->hits[k].t_begin += sd->t_lo; job->hits[k].t_end += sd->t_lo;
            job->hits[k].q_begin += sd->q_lo; job->hits[k].q_end += sd->q_lo;
            job->cigars[k] = NULL;
        } else {
            extend_seed(job->T, job->tlen, job->Q, job->qlen, sd, &job->sc, job->ydrop,
                        job->min_tb, job->want_tb, &w, &job->hits[k], &job->cigars[k]);
        }
    }
    band_free(&w.bl); band_free(&w.br); free(w.ops);
    return NULL;
}

typedef struct {
    int64_t n;
    uint32_t **cigars;
} fzo_batch;

/* Run a whole batch on `nthreads` threads.  Results go to hits[n]; CIGARs
 * stay in the returned handle until fzo_take_cigars / fzo_free. */
fzo_batch *fzo_run(const uint8_t *T, int64_t tlen, const uint8_t *Q, int64_t qlen,
                   const fzo_seed *seeds, int64_t n, const fzo_scoring *sc,
                   int64_t ydrop, int64_t min_tb, int want_tb, int local,
                   int nthreads, fzo_hit *hits)
{
    fzo_batch *bt = calloc(1, sizeof *bt);
    if (!bt) return NULL;
    bt->n = n;
    bt->cigars = calloc((size_t)(n > 0 ? n : 1), sizeof(uint32_t *));
    if (!bt->cigars) { free(bt); return NULL; }
    batch_job job;
    memset(&job, 0, sizeof job);
    job.T = T; job.Q = Q; job.tlen = tlen; job.qlen = qlen;
    job.seeds = seeds; job.n = n; job.sc = *sc; job.ydrop = ydrop; job.min_tb = min_tb;
    job.want_tb = want_tb; job.local = local; job.hits = hits; job.cigars = bt->cigars;
    pthread_mutex_init(&job.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    pthread_t *th = malloc((size_t)nthreads * sizeof(pthread_t));
    int started = 0;
    for (int t = 0; th && t < nthreads; t++)
        if (pthread_create(&th[t], NULL, batch_worker, &job) == 0) started++;
    if (started == 0) batch_worker(&job);
    for (int t = 0; t < started; t++) pthread_join(th[t], NULL);
    free(th);
    pthread_mutex_destroy(&job.mu);
    return bt;
}

/* Copy CIGAR words of every seed into out (concatenated in seed order). */
void fzo_copy_cigars(const fzo_batch *bt, const fzo_hit *hits, uint32_t *out)
{
    int64_t o = 0;
    for (int64_t k = 0; k < bt->n; k++) {
        if (!bt->cigars[k]) continue;
        memcpy(out + o, bt->cigars[k], (size_t)hits[k].n_runs * sizeof(uint32_t));
        o += hits[k].n_runs;
    }
}

void fzo_free(fzo_batch *bt)
{
    if (!bt) return;
    for (int64_t k = 0; k < bt->n; k++) free(bt->cigars[k]);
    free(bt->cigars);
    free(bt);
}

/* One side on explicit sequences, with per-cell access for tests: fills
 * S/I/D (m+1)x(n+1) row-major with INT64_MIN for cells never evaluated or
 * dead, and ops (end-first) when ops != NULL.  Returns status. */
int64_t fzo_side_matrix(const uint8_t *a, int64_t m, const uint8_t *bq, int64_t n,
                        const fzo_scoring *sc, int64_t ydrop,
                        int64_t *out5 /* score, ie, je, cells, dend */,
                        int64_t *S, int64_t *I, int64_t *D,
                        char *ops, int64_t *nops)
{
    side_seq s = { a - 1, 1, bq - 1, 1, m, n };
    band b;
    memset(&b, 0, sizeof b);
    side_result r;
    extend_side(&s, sc, ydrop, &b, &r);
    int err = b.err;
    out5[0] = r.score; out5[1] = r.ie; out5[2] = r.je; out5[3] = r.cells; out5[4] = r.dend;
    if (S) {
        for (int64_t i = 0; i <= m; i++)
            for (int64_t j = 0; j <= n; j++) {
                S[i * (n + 1) + j] = load(&b, b.S, i, j);
                I[i * (n + 1) + j] = load(&b, b.I, i, j);
                D[i * (n + 1) + j] = load(&b, b.D, i, j);
            }
    }
    if (ops) *nops = (err == 0) ? traceback(&s, sc, &b, r.ie, r.je, ops, &err) : 0;
    band_free(&b);
    return err;
}

/* ------------------------------------------------------ CIGAR rescoring -- */

/* The score of an alignment given as a CIGAR, for checks at any batch size.
 * Row k lays words[off[k] .. off[k] + len[k]) (BAM-style runs, len << 4 |
 * code, code 0 = M: target and query advance; 1 = I: query only; 2 = D:
 * target only) on the sequences from (t_begin[k], q_begin[k]): the sum of
 * the substitution scores of its M columns (the seed's own included) minus
 * gap_open + g * gap_extend for every gap run of length g.  out[3k] gets the
 * score, out[3k + 1] and out[3k + 2] the end coordinates (one past the last
 * column).  Returns the number of rows that leave the sequences, hold an
 * unknown code or an invalid base (their out entries are left at 0). */
int64_t fzo_rescore(const uint8_t *T, int64_t tlen, const uint8_t *Q, int64_t qlen, const fzo_scoring *sc,
                    const int64_t *t_begin, const int64_t *q_begin, const int64_t *off, const int64_t *len,
                    const uint32_t *words, int64_t n, int64_t *out)
{
    int64_t tab[5][5];
    sub_table(sc, tab);
    int64_t bad = 0;
    for (int64_t k = 0; k < n; k++) {
        int64_t t = t_begin[k], q = q_begin[k], score = 0;
        int ok = t >= 0 && q >= 0;
        for (int64_t r = 0; ok && r < len[k]; r++) {
            const uint32_t w = words[off[k] + r];
            const int64_t g = (int64_t)(w >> 4);
            const uint32_t code = w & 15u;
            if (code == 0) {
                if (t + g > tlen || q + g > qlen) { ok = 0; break; }
                for (int64_t c = 0; c < g; c++) {
                    const int a = base_code(T[t + c], sc), b = base_code(Q[q + c], sc);
                    if (a < 0 || b < 0) { ok = 0; break; }
                    score += tab[a][b];
                }
                t += g;
                q += g;
            } else if (code == 1 || code == 2) {
                score -= sc->gap_open + g * sc->gap_extend;
                if (code == 1) q += g; else t += g;
                if (t > tlen || q > qlen) ok = 0;
            } else {
                ok = 0;
            }
        }
        if (ok) {
            out[3 * k] = score;
            out[3 * k + 1] = t;
            out[3 * k + 2] = q;
        } else {
            out[3 * k] = out[3 * k + 1] = out[3 * k + 2] = 0;
            bad++;
        }
    }
    return bad;
}

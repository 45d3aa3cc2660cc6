/*
 * fz.h -- C ABI of libfz: batched gapped seed extension on one MI355X (gfx950).
 *
 * The operation follows "FastZ: Accelerating Gapped Whole Genome Alignment on
 * GPUs" (Gundabolu, Vijaykumar, Thottethodi, SC'21).  FastZ is a drop-in
 * replacement for the gapped-extension stage of LASTZ: the host picks 19-bp
 * seeds, sequences and seeds go in, alignments come out (section 1 and
 * section 3.4 "implementation").  Each seed is extended on both sides
 * separately (section 3.1.2) with affine-gap Smith-Waterman (section 1,
 * Fig. 1) pruned by y-drop (section 2.1, Fig. 3a, in the "previously
 * completed scores" form of section 3.4), then traced back from the best cell
 * (section 2.1, Fig. 3b).
 *
 * Exact definition computed for one side (a_1..a_m from the target, b_1..b_n
 * from the query, both read outward from the seed):
 *   I(i,j) = max(I(i,j-1) - E, S(i,j-1) - O - E)   gap in the target (CIGAR 'I')
 *   D(i,j) = max(D(i-1,j) - E, S(i-1,j) - O - E)   gap in the query  (CIGAR 'D')
 *   S(i,j) = max(S(i-1,j-1) + sub(a_i, b_j), I(i,j), D(i,j)),  S(0,0) = 0
 *   anti-diagonals d = i + j are settled in order; T_d = (best S over live
 *   cells of diagonals < d) - ydrop; a cell with S < T_d is dead (S=I=D=-inf);
 *   the run ends when no cell of the next diagonal can have a live predecessor.
 *   The side's result is the best live S, ties to the smallest d then the
 *   smallest i.  Traceback prefers the diagonal move, then I, then D; inside
 *   a gap it prefers "opened here" over "extended".
 * A gap of g bases costs O + g*E.  sub() is `match` for equal bases,
 * `transition` for A<->G and C<->T, `transversion` otherwise, or, when an
 * fz_matrix is passed, its entry for (target base, query base), with N
 * against anything scoring its n_score.  The seed's own columns are scored
 * with sub() and added to the two sides' scores.
 *
 * Around that path: FZ_QUERY_RC aligns against the query's reverse
 * complement; fz_find_seeds is the seed stage that produces the seeds
 * (section 2); fz_extend_rounds runs batches in rounds and skips seeds that
 * lie on alignments of earlier rounds (LASTZ's rule of section 2.1, made
 * data-parallel per round).
 *
 * Local mode (FZ_LOCAL): each record's windows are one pair; the whole
 * window is scored with S = max(0, H, I, D), no y-drop, and the result is
 * the best S and its cell (same tie rule).  No traceback in local mode.
 *
 * Memory: every pointer marked "device" must be device memory of the
 * context's GPU (e.g. a torch tensor's data_ptr()); the library never frees
 * caller memory.  All work is enqueued on `stream` (a hipStream_t, NULL = the
 * null stream); fz_extend_batch synchronises that stream before it returns
 * because it reads sizes back between its phases, so outputs are complete on
 * return.
 *
 * Errors: call-level problems return a negative FZ_E* code and set a message
 * readable with fz_last_error(); per-seed problems set bits in
 * fz_hit.status and leave the rest of the batch valid.
 */
#ifndef FZ_H
#define FZ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct fz_ctx fz_ctx;

/* Scores (signed) and gap costs (>= 0).  A gap of g bases costs
 * gap_open + g * gap_extend. */
typedef struct {
    int32_t match, transition, transversion;
    int32_t gap_open, gap_extend;
} fz_scoring;

/* A full substitution matrix, used instead of the three scores of
 * fz_scoring when passed to fz_extend_batch.  sub[a][b] scores target base
 * a against query base b, bases in the order A, C, G, T (the matrix need
 * not be symmetric).  With a matrix the sequences may also hold N (either
 * case), the unknown base: a pair with N on either side, N against N
 * included, scores n_score.  Every entry and n_score must lie in
 * -128..127.  (FastZ fixes no scoring; LASTZ, whose extension it
 * accelerates, scores with such a matrix.) */
typedef struct {
    int32_t sub[4][4];
    int32_t n_score;
} fz_matrix;

/* One seed: an exact match of seed_len bases at target[t_pos..] and
 * query[q_pos..], plus half-open windows that bound the extension (the
 * extension treats a window edge as a sequence end).  Requires
 * t_lo <= t_pos, t_pos + seed_len <= t_hi <= target_len (same for q).
 * In FZ_LOCAL mode only the windows are read.  56 bytes, int64 fields, so a
 * (n, 7) int64 array in this field order is an array of fz_seed. */
typedef struct {
    int64_t t_pos, q_pos, seed_len;
    int64_t t_lo, t_hi, q_lo, q_hi;
} fz_seed;

/* Result per seed.  Coordinates are 0-based half-open on the forward
 * strand.  cigar_off / cigar_len index the CIGAR word array returned by the
 * call (cigar_len 0 when the seed was not traced).  96 bytes, int64 fields. */
typedef struct {
    int64_t score;                 /* left + seed columns + right (local: best S) */
    int64_t status;                /* FZ_HIT_* bits */
    int64_t t_begin, t_end, q_begin, q_end;
    int64_t cigar_off, cigar_len;
    int64_t cells;                 /* canonical cells evaluated, both sides */
    int64_t score_left, score_right;
    int64_t bin;                   /* executor length bin of the longer side, -1 if none */
} fz_hit;

/* Statistics of one call (host struct, optional). */
typedef struct {
    uint64_t cells;                /* canonical cells, all seeds, both sides */
    uint64_t executor_cells;       /* cells recomputed by the executor */
    uint64_t pointer_bytes;        /* traceback pointer bytes written */
    uint64_t n_sides, n_eager, n_executor, n_overflow;
    uint64_t bin_hist[8];
    uint64_t n_batches;
    uint64_t max_band;             /* widest range R_d (cells of one anti-diagonal) of any side */
    uint64_t n_packed;             /* sides swept in the packed 16-bit layouts after their first 34
                                    * anti-diagonals (0 with FZ_EXACT32, FZ_LOCAL, or a scoring
                                    * outside the packed range) */
    uint64_t n_onepass;            /* sides the one-pass executor extended and traced (see
                                    * FZ_TWO_PASS); executor_cells and pointer_bytes do not
                                    * count them */
    uint64_t onepass_cells;        /* their canonical cells (all of them, best to band's end too) */
    uint64_t onepass_bytes;        /* pool bytes their row blocks, block tables and arenas took */
    uint64_t n_tail_walked;        /* one-pass sides walked while the one-pass executor still ran
                                    * (FZ_DEBUG_TAIL_WALK) */
    float ms_pack, ms_inspect, ms_bin, ms_exec, ms_walk, ms_gather;
                                   /* phase spans between HIP events on the call's stream;
                                    * ms_inspect includes the one-pass executor; ms_walk is the
                                    * summed duration of the traceback walker launches, which run
                                    * inside the executor phase (ms_exec) on its streams, beside
                                    * other batches */
    float ms_main;                 /* the dominant kernel alone (inspector, or the local kernel) */
    float ms_onepass;              /* the one-pass executor launch (0 when none ran) */
} fz_stats;

/* Phase times of one fz_find_seeds call, milliseconds between HIP events on
 * the call's stream.  A phase that did not run (no hits) reads 0. */
typedef struct {
    float ms_pack;                 /* ASCII -> codes, both sequences, validation */
    float ms_keys;                 /* k-mer key of every target start position */
    float ms_sort_keys;            /* radix sort of the target's (key, position) pairs */
    float ms_index;                /* bucket table over the sorted keys' top bits */
    float ms_join;                 /* per query position, its key and range of equal target keys */
    float ms_scan;                 /* exclusive scan of the per-position hit counts */
    float ms_emit;                 /* every hit written as one 64-bit word */
    float ms_sort_hits;            /* radix sort of the hit words (diagonal, then t) */
    float ms_runs;                 /* run starts on each diagonal and their ranks */
    float ms_write;                /* the seed records */
    float ms_total;                /* first to last event, the count read-back included */
} fz_seed_stats;

enum {
    FZ_TRACEBACK = 1u << 0,        /* CIGAR for every seed whose score > min_traceback_score */
    FZ_LOCAL = 1u << 1,            /* full-window local alignment, score and end cell only */
    FZ_STATS = 1u << 2,            /* fill *stats (adds stream syncs for phase timings) */
    FZ_QUERY_RC = 1u << 3,         /* seeds lie on the query's reverse complement (see below) */
    FZ_SEEDS_ALL = 1u << 4,        /* fz_find_seeds: every shared k-mer, no diagonal dedup */
    FZ_SEEDS_REUSE_INDEX = 1u << 5,/* fz_find_seeds: reuse the target index of an earlier call */
    FZ_ROUNDS_DOUBLING = 1u << 6,  /* fz_extend_rounds: each round twice the size of the one before */
    FZ_EXACT32 = 1u << 7,          /* fz_extend_batch: keep every cell in a 32-bit lane (see below) */
    FZ_TWO_PASS = 1u << 8          /* fz_extend_batch / _rounds: no one-pass executor (see below) */
};

/* FZ_EXACT32: by default, scorings with int8 match / transition /
 * transversion, ydrop <= 16000 and gap_open + 2 * gap_extend <= 4000 are
 * computed with two cells per 32-bit lane register (16-bit values relative
 * to the y-drop threshold, which hold every value that can decide a result
 * exactly); the results are identical either way.  This flag keeps the
 * 32-bit layouts, e.g. to check that. */

/* FZ_TWO_PASS: by default (packed layouts, with FZ_TRACEBACK), a side whose
 * best score at anti-diagonal 256 already makes its seed traced, whatever
 * the other side scores (best >= min_traceback_score - seed score + 1), and
 * whose best was found within the last 64 anti-diagonals, leaves the
 * inspector there: a one-pass executor extends it again from the start to
 * its end, finding its best cell and writing its pointer rows in the same
 * pass, so that the inspector does not sweep it to its end before the
 * executor sweeps it again to its best cell.  Its rows go to blocks of 64
 * anti-diagonals carved from a device pool that the context keeps; sides
 * that do not fit go back to the inspector and the two-pass executor.
 * The results are identical either way; this flag keeps every side in the
 * inspector / executor scheme of FastZ section 3. */

/* FZ_QUERY_RC: the call aligns the target against the reverse complement
 * of `query` (base j of it is the complement of query[query_len - 1 - j];
 * A<->T, C<->G).  Seed positions, windows and the q_begin / q_end of the
 * results are coordinates on that reverse complement; the forward-strand
 * span of a hit is [query_len - q_end, query_len - q_begin).  The query
 * buffer itself is read, never written.  Works with and without FZ_LOCAL.
 * (FastZ and LASTZ search both strands; the reverse strand is this
 * transform of the input, the kernels are the same.) */

enum {
    FZ_OK = 0,
    FZ_EINVAL = -1,                /* bad argument, or a byte the call does not accept */
    FZ_ENOMEM = -2,                /* device allocation failed */
    FZ_EDEVICE = -3                /* HIP runtime error, or an internal check that failed */
};
/* A band too wide for the widest window is a per-seed condition
 * (FZ_HIT_EBAND below), never a call-level error. */

enum {
    FZ_HIT_TRACED = 1,             /* CIGAR present */
    FZ_HIT_EAGER_LEFT = 2,         /* left side traced inside the inspector (<= 16x16) */
    FZ_HIT_EAGER_RIGHT = 4,
    FZ_HIT_BELOW_MIN = 8,          /* score <= min_traceback_score: no CIGAR by request */
    FZ_HIT_EBAND = 16,             /* a side's band outgrew the widest kernel: result invalid */
    FZ_HIT_ESEED = 32,             /* seed outside its window or window outside the sequences */
    FZ_HIT_ERANGE = 64,            /* window too long for int32 scores with these parameters, or a
                                    * side window longer than 2^28 bases */
    FZ_HIT_COVERED = 128,          /* fz_extend_rounds: seed on an earlier round's alignment, not extended */
    FZ_HIT_EEXEC = 256,            /* the executor's recompute of a side disagreed with the inspector
                                    * (best score, best cell or pointer-row size): score and
                                    * coordinates stand, no CIGAR is given (FZ_HIT_TRACED is clear) */
    FZ_HIT_WIDE = 512              /* information only: a side's band passed 384 positions and the
                                    * side was redone in the 1024-position window */
};

#define FZ_YDROP_INF 2147483647    /* ydrop >= this: no pruning */

/* Create a context on HIP device `device`.  The context owns its device
 * workspace (grown on demand, reused across calls) and the CIGAR buffer.
 * workspace_bytes caps the traceback-pointer workspace, the one large
 * buffer (as fz_set_pointer_workspace; 0 = the default there).  Returns
 * FZ_OK or a negative code; *out is NULL on failure. */
int fz_create(fz_ctx **out, int device, uint64_t workspace_bytes);

/* Free the context and every device buffer it owns.  NULL is ignored. */
void fz_destroy(fz_ctx *ctx);

/* Message of the last failed call on ctx ("" if none).  Valid until the
 * next call on ctx.  Not thread-safe per context. */
const char *fz_last_error(const fz_ctx *ctx);

/* Cap (bytes) of the traceback-pointer workspace, shared by the executor's
 * streams (three workspaces of a third each, each at least twice the
 * largest side's pointer rows); the executor works in batches that fit.
 * The one-pass executor's pool (FZ_TWO_PASS) is held to the same cap
 * (sides it cannot hold go to the two-pass executor).
 * 0 restores the default: 70% of the device memory free at the call, at
 * most 200 GiB (allocated on first need and kept by the context); the
 * pool's default is sized from the deferred sides' windows, at most 70% of
 * the free memory and 60% of the device, and the executor's workspaces are
 * released when the pool must grow.  Several contexts that work at once on
 * one GPU should each be given a cap, since each default is taken from the
 * memory free when that context asks. */
int fz_set_pointer_workspace(fz_ctx *ctx, uint64_t bytes);

/*
 * Extend a batch of seeds (or, with FZ_LOCAL, align a batch of windows).
 *   target, query   device, ASCII bases (A/C/G/T in either case, and N
 *                   when a matrix is given; any other byte makes the call
 *                   fail with FZ_EINVAL), lengths in bytes
 *   seeds           device, n_seeds records
 *   scoring         host; costs must be >= 0
 *   matrix          host or NULL: a substitution matrix replacing
 *                   scoring's match / transition / transversion (its gap
 *                   costs still apply); FZ_EINVAL for an entry outside
 *                   -128..127
 *   ydrop           >= 0; FZ_YDROP_INF disables pruning (ignored in local mode)
 *   min_traceback_score   with FZ_TRACEBACK, seeds whose score is strictly
 *                   greater get a CIGAR; others get FZ_HIT_BELOW_MIN
 *   flags           FZ_TRACEBACK | FZ_LOCAL | FZ_STATS | FZ_QUERY_RC
 *   hits            device, n_seeds records, written by the call
 *   cigar           out (may be NULL): device pointer to the CIGAR words,
 *                   BAM-style (length << 4 | op, op 0 = M, 1 = I, 2 = D),
 *                   owned by ctx, valid until the next call or fz_destroy
 *   cigar_words     out (may be NULL): number of words at *cigar
 *   stats           host, optional
 *   stream          hipStream_t or NULL
 * Returns FZ_OK or a negative FZ_E* code.
 */
int fz_extend_batch(fz_ctx *ctx,
                    const uint8_t *target, uint64_t target_len,
                    const uint8_t *query, uint64_t query_len,
                    const fz_seed *seeds, uint64_t n_seeds,
                    const fz_scoring *scoring, const fz_matrix *matrix, int32_t ydrop,
                    int64_t min_traceback_score, uint32_t flags,
                    fz_hit *hits, const uint32_t **cigar, uint64_t *cigar_words,
                    fz_stats *stats, void *stream);

/*
 * For callers that cannot allocate device memory (code under graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * score-only form of fz_extend_batch (no FZ_TRACEBACK, no FZ_LOCAL) that
 * allocates nothing.  Every buffer its kernels use beyond the caller's
 * inputs and outputs lives in a static device array of
 * FZ_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until
 * the process ends; the call takes at most FZ_NOALLOC_MAX_SEEDS seeds and
 * sequences of at most FZ_NOALLOC_MAX_BASES bases each, and rejects larger
 * inputs with FZ_EINVAL.  Arguments, results (hits, and stats' cells,
 * n_sides, n_overflow and ms_main) and errors are those of fz_extend_batch
 * without traceback; flags may hold FZ_STATS and FZ_QUERY_RC.  All calls
 * on one GPU share that GPU's array: calls that overlap in time on one GPU
 * (other streams, other contexts, other threads) race and must not be
 * made.  The call returns after its stream has run it.
 */
#define FZ_NOALLOC_MAX_SEEDS 65536
#define FZ_NOALLOC_MAX_BASES 4194304
#define FZ_NOALLOC_SCRATCH_BYTES 83886080
int fz_extend_batch_noalloc(fz_ctx *ctx,
                            const uint8_t *target, uint64_t target_len,
                            const uint8_t *query, uint64_t query_len,
                            const fz_seed *seeds, uint64_t n_seeds,
                            const fz_scoring *scoring, const fz_matrix *matrix, int32_t ydrop,
                            uint32_t flags, fz_hit *hits, fz_stats *stats, void *stream);

/*
 * Covered-seed suppression by rounds.  FastZ (SC'21) section 2.1 describes
 * LASTZ ending a seed extension that reaches an alignment found earlier;
 * section 3.4 explains why FastZ drops that rule (it orders the
 * extensions).  This call applies it between rounds and keeps each round a
 * data-parallel batch: seeds are taken in the given order in rounds of
 * round_size; a seed of round r whose exact-match columns (t_pos + k,
 * q_pos + k), k < seed_len, share a cell with an aligned (M) column of an
 * alignment traced in an earlier round is not extended (its record is all
 * zero but status = FZ_HIT_COVERED and bin = -1); every other seed of the
 * round is extended exactly as fz_extend_batch extends it.  Seeds of one
 * round never suppress each other, and alignments without a CIGAR (score
 * not above min_traceback_score) suppress nothing.  A seed without columns,
 * or with columns outside the sequences, is never covered; coverage looks at
 * the columns only, so a seed outside its window may still be covered
 * (else it reports FZ_HIT_ESEED as in fz_extend_batch).
 *   arguments       as fz_extend_batch; flags must hold FZ_TRACEBACK and
 *                   not FZ_LOCAL, and may add FZ_ROUNDS_DOUBLING; sequences
 *                   shorter than 2^31 bases
 *   round_size      >= 1 seeds per round (>= n_seeds: one round, the same
 *                   results as fz_extend_batch); with FZ_ROUNDS_DOUBLING in
 *                   flags, the size of the first round, each later round
 *                   holding twice as many seeds as the one before (few
 *                   early extensions cover most seeds, in few rounds)
 *   cigar, cigar_words   the words of all rounds, in seed order within a
 *                   round and round after round; hits' cigar_off index them
 *   stats           sums over the rounds
 * The context keeps the aligned segments of the call (16 bytes per M run)
 * until the next call.  Returns FZ_OK or a negative FZ_E* code.
 */
int fz_extend_rounds(fz_ctx *ctx,
                     const uint8_t *target, uint64_t target_len,
                     const uint8_t *query, uint64_t query_len,
                     const fz_seed *seeds, uint64_t n_seeds,
                     const fz_scoring *scoring, const fz_matrix *matrix, int32_t ydrop,
                     int64_t min_traceback_score, uint32_t flags, uint64_t round_size,
                     fz_hit *hits, const uint32_t **cigar, uint64_t *cigar_words,
                     fz_stats *stats, void *stream);

/*
 * Seed stage (FastZ, SC'21, section 2: whole-genome alignment first finds
 * short exact matches between the two sequences as seed sites, then filters
 * them, then runs the gapped extension).  Finds every pair (t, q) with
 * target[t .. t+k) == query[q .. q+k) (with FZ_QUERY_RC: equal to the
 * query's reverse complement, q counted on it) and, unless FZ_SEEDS_ALL,
 * keeps one seed per run of hits on consecutive positions of one diagonal
 * t - q (the run's first hit).  Seeds come out ordered by diagonal t - q,
 * then by t, with seed_len = k and windows [t - flank, t + k + flank) and
 * [q - flank, q + k + flank) clipped to the sequences: an fz_seed array
 * fz_extend_batch takes as it is (with the same FZ_QUERY_RC).
 *   target, query   device, ASCII bases as for fz_extend_batch; each
 *                   shorter than 2^31 bases
 *   k               1..32
 *   flank           >= 0
 *   flags           FZ_QUERY_RC | FZ_SEEDS_ALL | FZ_SEEDS_REUSE_INDEX
 *   seeds           out (may be NULL): device pointer to *n_seeds records,
 *                   owned by ctx, valid until the next fz_find_seeds or
 *                   fz_destroy (fz_copy_seeds copies them out)
 *   n_seeds         out: number of seeds
 *   n_hits          out (may be NULL): shared k-mer hits before the dedup
 *   stats           out (may be NULL): phase times from HIP events on
 *                   `stream` (recording them costs a little)
 *   stream          hipStream_t or NULL
 * Every hit is materialized (16 bytes each in device memory, plus sort
 * scratch); more than 2^31 hits fail with FZ_ENOMEM.  The call reads counts
 * back, so it returns after the stream has finished it.  Returns FZ_OK or a
 * negative FZ_E* code (FZ_EINVAL for bad arguments or a non-ACGT byte).
 */
int fz_find_seeds(fz_ctx *ctx,
                  const uint8_t *target, uint64_t target_len,
                  const uint8_t *query, uint64_t query_len,
                  uint32_t k, int64_t flank, uint32_t flags,
                  const fz_seed **seeds, uint64_t *n_seeds, uint64_t *n_hits,
                  fz_seed_stats *stats, void *stream);

/* FZ_SEEDS_REUSE_INDEX: every call without this flag builds an index of the
 * target (its k-mers sorted, and a bucket table over them) and keeps it on
 * ctx once the call has succeeded.  A call with the flag skips that build
 * and uses the kept index; the target pointer, target_len and k must equal
 * those of the call that built it (else FZ_EINVAL), and the caller
 * guarantees the target bytes have not changed since.  Searching both
 * strands of one query, or many queries against one target, builds the
 * index once.  fz_extend_batch does not touch the index. */

/* Failure injection for tests of the library's own checks.
 * FZ_DEBUG_SHRINK_ROWS: every executor side is given `value` fewer
 * pointer-row words than the inspector sized for it, so that the executor's
 * row-capacity check trips on each side that needs rows (its results then
 * carry FZ_HIT_EEXEC); 0 restores normal sizing (while it is set, no side
 * goes to the one-pass executor).
 * FZ_DEBUG_ONEPASS_POOL: the one-pass executor's pool is `value` bytes, so
 * that sides run out of it and go back to the inspector; 0 turns the
 * one-pass executor off, -1 restores the library's sizing.
 * FZ_DEBUG_ONEPASS_ORDER: 1 (the default) launches the one-pass executor's
 * sides longest first by a predicted length, 0 in the order the inspector
 * handed them over (results are the same either way).
 * FZ_DEBUG_TAIL_WALK: 1 (the default) walks the one-pass sides that have
 * finished while the one-pass executor's last waves still run (the tail
 * walk), 0 walks every one-pass side after it, 2 runs the tail walk after
 * the executor (so that it takes every side whose runs fit), a larger value
 * runs it after the executor with at most `value` run words for all sides
 * (the rest fall back to the later walk); results are the same in every
 * case.  Returns FZ_OK, or FZ_EINVAL for an unknown `what` or a value out
 * of range. */
enum { FZ_DEBUG_SHRINK_ROWS = 1, FZ_DEBUG_ONEPASS_POOL = 2, FZ_DEBUG_ONEPASS_ORDER = 3, FZ_DEBUG_TAIL_WALK = 4 };
int fz_debug_set(fz_ctx *ctx, int what, int64_t value);

/* Copy the first n seeds of the last successful fz_find_seeds to dst
 * (device, n records). */
int fz_copy_seeds(fz_ctx *ctx, fz_seed *dst, uint64_t n, void *stream);

/* Copy the first `words` CIGAR words of the last successful fz_extend_batch
 * on ctx into caller device memory `dst` (enqueued on `stream`, which is
 * synchronised before return).  words must not exceed the count that call
 * returned.  Returns FZ_OK or a negative code. */
int fz_copy_cigar(fz_ctx *ctx, uint32_t *dst, uint64_t words, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FZ_H */

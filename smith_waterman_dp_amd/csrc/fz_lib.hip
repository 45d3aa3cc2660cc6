// fz_lib.hip -- C ABI of libfz: batched gapped seed extension on gfx950.
//
// Phases of one fz_extend_batch call (FastZ, SC'21, section 3 and Fig. 8):
//   pack      ASCII -> codes, forward and reversed copies, with validation
//   setup     seeds -> two side tasks each, seed-column scores
//   inspect   score-only y-drop extension of every side, one wave per side;
//             the hardware dispatcher starts a new wave wherever one retires,
//             which takes the place of the paper's 32 CUDA streams against
//             load imbalance (section 3.4); sides whose best cell is in the
//             16 x 16 corner are traced here
//   widen     sides whose band outgrew the window are redone with a wider one
//   bin       per seed totals; executor sides counted and scattered by length
//             bin, longest bins first (section 3.3)
//   execute   in batches that fit the pointer workspace: pruned recompute
//             with 4-bit pointers, then one lane per side walks them back
//   gather    left ops + seed + reversed right ops, merged into CIGAR words
// Local mode runs pack and one full-window kernel.  fz_find_seeds is the seed
// stage before all this (fz_seeds.hpp).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <thread>
#include <chrono>
#include <string>
#include <vector>

#include "../../include/fz.h"
#include "fz_aux.hpp"
#include "fz_device.hpp"
#include "fz_extend.hpp"
#include "fz_packed.hpp"
#include "fz_local.hpp"
#include "fz_seeds.hpp"
#include "fz_rounds.hpp"
#include "fz_sort.hpp"

using namespace fz;

namespace {

struct DevBuf {
    void *p = nullptr;
    size_t cap = 0;
};

// Scalars the kernels update, one allocation.
struct Counters {
    uint32_t err;               // bit 0: non-ACGT byte; bit 1: broken traceback
    uint32_t overflow_count[2];
    uint32_t bin_count[EXEC_CLASSES * NBINS];
    uint32_t bin_base[EXEC_CLASSES * NBINS];
    uint32_t bin_fill[EXEC_CLASSES * NBINS];
    int64_t max_ptr;
    int64_t exec_cells;
    int64_t totals[4];
    int64_t max_band;
    uint32_t defer_count;                   // one-pass executor: sides handed over
    uint64_t defer_diags;                   // the deferred sides' anti-diagonals (m + n + 1 each)
    int64_t op_cells;
    int64_t op_runs_total;                  // run capacity of a round's walked sides
    // per one-pass round (cleared before each): sides given back, sides
    // finished, pool bytes taken
    struct {
        uint32_t fail, done;
        uint64_t pool_used;
    } op_round;
    uint32_t op_key_hist[OP_KEYS];          // one-pass launch order: keys' counts, then cursors
    uint32_t op_key_cur[OP_KEYS];
    struct {
        uint32_t count, pad;                // the wide retry's sides traced beside the one-pass executor
        uint64_t bytes;                     // their rows' workspace
    } early;
    struct {
        uint64_t used;                      // tail walk: run words taken of the tail buffer (per round)
        uint32_t sides;                     // one-pass sides it walked (per call)
        uint32_t flushed;                   // the round's tail flush began (tail_flush_kernel)
    } tail;
};

// One wave per workgroup for the wave-per-side kernels: sides differ in
// length by orders of magnitude, and a workgroup's slot on the CU is held
// until its longest wave ends, so larger groups strand short waves' slots
// (measured: about half the occupancy with four waves per group).
constexpr int EXT_WAVES = 1;
constexpr int LOCAL_WAVES = 4;          // local mode: every wave does the same work
// Executor batches go round-robin to this many streams, each with its own
// pointer workspace, so that a batch's last long sides overlap the next
// batches instead of leaving the machine idle (a batch holds only a few
// thousand sides, about one round of resident waves).
constexpr int EXEC_STREAMS = 3;
constexpr int C_STD = 6;                // window 384 positions
constexpr int C_WIDE = 16;              // window 1024 positions
constexpr int LOCAL_RL = 32;            // rows per lane in local mode

}  // namespace

// ---- static scratch of fz_extend_batch_noalloc --------------------------
// For callers that cannot allocate device memory (code under graph capture,
// tight serving loops): every buffer that call's kernels use beyond the
// caller's inputs and outputs lives in one file-scope device array, sized
// for at most FZ_NOALLOC_MAX_SEEDS seeds and sequences of at most
// FZ_NOALLOC_MAX_BASES bases each.  Each GPU the library runs on holds its
// own copy until the process ends.  In host code `scratch` only names the
// symbol: its device address comes from hipGetSymbolAddress, taken once per
// device (fz_create, with that device current) and kept in noalloc_base[].
namespace {

constexpr int64_t NA_SEQ = FZ_NOALLOC_MAX_BASES + 2 * PAD + 64;      // one packed copy
constexpr int64_t NA_SIDES = 2 * (int64_t)FZ_NOALLOC_MAX_SEEDS;
constexpr int64_t na_up(int64_t x) { return (x + 255) & ~(int64_t)255; }
// byte offsets of the regions, each 256-aligned
constexpr int64_t NA_TF = 0;
constexpr int64_t NA_TR = NA_TF + na_up(NA_SEQ);
constexpr int64_t NA_QF = NA_TR + na_up(NA_SEQ);
constexpr int64_t NA_QR = NA_QF + na_up(NA_SEQ);
constexpr int64_t NA_TF16 = NA_QR + na_up(NA_SEQ);
constexpr int64_t NA_TR16 = NA_TF16 + na_up(2 * NA_SEQ);
constexpr int64_t NA_QF16 = NA_TR16 + na_up(2 * NA_SEQ);
constexpr int64_t NA_QR16 = NA_QF16 + na_up(2 * NA_SEQ);
constexpr int64_t NA_TASKS = NA_QR16 + na_up(2 * NA_SEQ);
constexpr int64_t NA_INFO = NA_TASKS + na_up(NA_SIDES * (int64_t)sizeof(SideTask));
constexpr int64_t NA_OUT = NA_INFO + na_up(FZ_NOALLOC_MAX_SEEDS * (int64_t)sizeof(SeedInfo));
constexpr int64_t NA_EAGER = NA_OUT + na_up(NA_SIDES * (int64_t)sizeof(SideOut));
constexpr int64_t NA_OVL0 = NA_EAGER + na_up(NA_SIDES * EAGER_OPS);
constexpr int64_t NA_OVL1 = NA_OVL0 + na_up(NA_SIDES * 4);
constexpr int64_t NA_TRACE = NA_OVL1 + na_up(NA_SIDES * 4);
constexpr int64_t NA_RUNCAP = NA_TRACE + na_up(NA_SIDES * 4);
constexpr int64_t NA_COUNTERS = NA_RUNCAP + na_up(NA_SIDES * 8);
constexpr int64_t NA_END = NA_COUNTERS + na_up((int64_t)sizeof(Counters));
static_assert(NA_END <= FZ_NOALLOC_SCRATCH_BYTES, "noalloc scratch layout exceeds its array");

constexpr int NA_MAX_DEVICES = 64;
std::mutex noalloc_mu;
uint8_t *noalloc_base[NA_MAX_DEVICES] = {};

}  // namespace

static __device__ __align__(256) uint8_t scratch[FZ_NOALLOC_SCRATCH_BYTES];

struct fz_ctx {
    int device = 0;
    int n_cu = 256;
    std::string err;
    uint64_t ptr_cap = 0;               // 0 = default
    int64_t dbg_shrink_rows = 0;        // fz_debug_set(FZ_DEBUG_SHRINK_ROWS)
    int64_t dbg_op_pool = -1;           // fz_debug_set(FZ_DEBUG_ONEPASS_POOL): pool bytes (-1: sized by the library)
    int64_t dbg_tail = 1;               // fz_debug_set(FZ_DEBUG_TAIL_WALK): 0 off, 1 beside the executor,
                                        // 2 after it, more: after it within that many run words
    int64_t dbg_op_order = 1;           // fz_debug_set(FZ_DEBUG_ONEPASS_ORDER): predicted longest first (0: as deferred)
    std::vector<hipEvent_t> walk_ev;    // brackets of the walker launches (FZ_STATS)
    uint64_t last_words = 0;            // CIGAR words of the last successful call
    DevBuf Tf, Tr, Qf, Qr;
    DevBuf Tf16, Tr16, Qf16, Qr16;      // 16-bit code copies of the packed layouts
    DevBuf tasks, info, out, eager, side_trace, run_cap, run_off, run_len, runs;
    DevBuf items, batch_first, scan_tmp, cig, cigar, counters, ovl0, ovl1, bnd;
    DevBuf rs_cnt, ps_tmp;              // radix-sort digit counts, tile totals of the generic scans
    DevBuf ptr_ws[EXEC_STREAMS];        // one pointer workspace per executor stream
    // one-pass executor: deferred sides, sides given back, block tables (by
    // side), the pool of row blocks
    DevBuf defer_list, op_fail, op_btab, op_pool, op_key, op_order, early_items, early_ws;
    // one-pass rounds: the other round's list of sides given back, the
    // finished sides, their walk items, the walks' scratch (a run per move
    // at most), and the runs of sides walked before the pool was used again,
    // packed (by side: where they start)
    DevBuf op_fail2, op_done, op_items, op_runs_tmp, op_runs, op_run_off;
    // tail walk: finished flags by list index, the runs of the sides it walked
    DevBuf op_fin, tail_runs;
    // seed stage: target keys and positions (two of each for the sort), query
    // keys, join ranges and counts, hits (two for the sort), run flags and
    // ranks, and the seeds of the last fz_find_seeds
    DevBuf sk_tk, sk_tk2, sk_tp, sk_tp2, sk_valid, sk_vpos, sk_bend, sk_boff, sk_lo, sk_cnt, sk_off, sk_hit, sk_hit2, sk_flag, sk_rank, sk_out;
    uint64_t last_seeds = 0;
    // covered-seed rounds: round flags, scan, packed seeds and results, CIGAR
    // words of all rounds, aligned segments (keys and ends, two of each for
    // the sort), running maxima
    DevBuf rd_keep, rd_pos, rd_seeds, rd_hits, rd_cnt, rd_off, rd_cig, sg_key, sg_key2, sg_end, sg_end2, sg_v, sg_max;
    // the target index held in sk_tk2 / sk_tp2 / sk_boff (FZ_SEEDS_REUSE_INDEX)
    bool idx_valid = false;
    const uint8_t *idx_target = nullptr;
    uint64_t idx_tlen = 0;
    uint32_t idx_k = 0;
    int64_t idx_keys = 0;               // target k-mers without N in the index
    hipStream_t xs[EXEC_STREAMS - 1] = {};   // executor streams besides the caller's
    hipEvent_t fork_ev = nullptr, join_ev[EXEC_STREAMS - 1] = {};
    hipStream_t xw = nullptr;           // the wide-window executor and walker, beside the batches
    hipEvent_t wide_ev = nullptr;
    hipEvent_t op_ev = nullptr;         // the one-pass sides' walks joined
    hipEvent_t tail_ev[2] = {};         // a one-pass round's list ready; its tail walk done
    hipEvent_t op_end_ev = nullptr;     // a one-pass round's executor done
    uint32_t *op_started = nullptr;     // (coherent pinned host memory) the round's last executor wave started
    hipEvent_t ev[12] = {};
    hipEvent_t kev[4] = {};             // brackets the dominant kernel, then the one-pass executor
};

namespace {

int fail(fz_ctx *ctx, int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    ctx->err = buf;
    return code;
}

#define HIP_OK(call)                                                                                   \
    do {                                                                                               \
        hipError_t e_ = (call);                                                                        \
        if (e_ != hipSuccess) return fail(ctx, FZ_EDEVICE, "%s: %s", #call, hipGetErrorString(e_));    \
    } while (0)

int ensure(fz_ctx *ctx, DevBuf &b, size_t bytes)
{
    if (bytes == 0) bytes = 256;
    if (b.cap >= bytes) return FZ_OK;
    if (b.p) {
        (void)hipFree(b.p);
        b.p = nullptr;
        b.cap = 0;
    }
    size_t want = bytes + std::min<size_t>(bytes / 8, (size_t)1 << 30);   // room to grow, at most 1 GiB
    if (hipMalloc(&b.p, want) != hipSuccess) {
        (void)hipGetLastError();
        if (hipMalloc(&b.p, bytes) != hipSuccess) {
            (void)hipGetLastError();
            b.p = nullptr;
            return fail(ctx, FZ_ENOMEM, "device allocation of %zu bytes failed", bytes);
        }
        want = bytes;
    }
    b.cap = want;
    return FZ_OK;
}

#define ENSURE(buf, bytes)                                   \
    do {                                                     \
        int r_ = ensure(ctx, (buf), (size_t)(bytes));        \
        if (r_ != FZ_OK) return r_;                          \
    } while (0)

template <class T>
T *as(DevBuf &b) { return reinterpret_cast<T *>(b.p); }

inline unsigned blocks_for(int64_t n, int threads) { return (unsigned)((n + threads - 1) / threads); }

__global__ void zero_kernel(uint32_t *p, int64_t nwords)
{
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < nwords; k += (int64_t)gridDim.x * blockDim.x)
        p[k] = 0u;
}

int zero(fz_ctx *ctx, void *p, size_t bytes, hipStream_t st)
{
    const int64_t w = (int64_t)((bytes + 3) / 4);
    zero_kernel<<<std::min<int64_t>(blocks_for(w, 256), 4096), 256, 0, st>>>((uint32_t *)p, w);
    HIP_OK(hipGetLastError());
    return FZ_OK;
}

// Exclusive scan of n int64 values read at vals[k * stride] into
// out[k * ostride]; the total lands in *d_total (device).
int scan(fz_ctx *ctx, const int64_t *vals, int64_t stride, int64_t n, int64_t *outv, int64_t ostride,
         int64_t *d_total, hipStream_t st)
{
    const int64_t nb = std::max<int64_t>(1, (n + SCAN_TILE - 1) / SCAN_TILE);
    ENSURE(ctx->scan_tmp, (size_t)nb * sizeof(int64_t));
    int64_t *bs = as<int64_t>(ctx->scan_tmp);
    if (n > 0) {
        scan_reduce_kernel<<<(unsigned)nb, SCAN_BLOCK, 0, st>>>(vals, stride, n, bs);
        HIP_OK(hipGetLastError());
    }
    scan_top_kernel<<<1, SCAN_BLOCK, 0, st>>>(bs, n > 0 ? nb : 0, d_total);
    HIP_OK(hipGetLastError());
    if (n > 0) {
        scan_apply_kernel<<<(unsigned)nb, SCAN_BLOCK, 0, st>>>(vals, stride, n, bs, outv, ostride);
        HIP_OK(hipGetLastError());
    }
    return FZ_OK;
}

// Scan of n values with OP (fz_sort.hpp), exclusive or inclusive; out may
// be in.  Uses ctx->ps_tmp for the tile totals.
template <class T, class OP, bool INCL>
int device_scan(fz_ctx *ctx, const T *in, T *out, int64_t n, hipStream_t st)
{
    if (n <= 0) return FZ_OK;
    const int64_t nt = (n + PS_TILE - 1) / PS_TILE;
    ENSURE(ctx->ps_tmp, (size_t)nt * sizeof(T));
    T *tt = as<T>(ctx->ps_tmp);
    pscan_reduce_kernel<T, OP><<<(unsigned)nt, PS_BLOCK, 0, st>>>(in, n, tt);
    HIP_OK(hipGetLastError());
    pscan_top_kernel<T, OP><<<1, PS_BLOCK, 0, st>>>(tt, nt);
    HIP_OK(hipGetLastError());
    pscan_apply_kernel<T, OP, INCL><<<(unsigned)nt, PS_BLOCK, 0, st>>>(in, n, tt, out);
    HIP_OK(hipGetLastError());
    return FZ_OK;
}

// Stable sort of n 64-bit keys (and their 32-bit values when va is given)
// by bits [0, bits), eight per pass, ping-ponging between the a and b
// buffers (both hold n entries).  *in_b tells where the result ends up.
int radix_sort(fz_ctx *ctx, uint64_t *ka, uint64_t *kb, uint32_t *va, uint32_t *vb, int64_t n, int bits,
               hipStream_t st, bool *in_b)
{
    *in_b = false;
    if (n <= 1 || bits <= 0) return FZ_OK;
    if (n >= ((int64_t)1 << 32)) return fail(ctx, FZ_EINVAL, "radix sort of %lld keys: at most 2^32 - 1", (long long)n);
    const int64_t ntiles = (n + RS_TILE - 1) / RS_TILE;
    ENSURE(ctx->rs_cnt, (size_t)RS_BINS * ntiles * sizeof(uint32_t));
    uint32_t *cnt = as<uint32_t>(ctx->rs_cnt);
    for (int shift = 0; shift < bits; shift += 8) {
        rs_hist_kernel<<<(unsigned)ntiles, RS_BLOCK, 0, st>>>(ka, n, shift, cnt, ntiles);
        HIP_OK(hipGetLastError());
        int rc = device_scan<uint32_t, ScanSum, false>(ctx, cnt, cnt, (int64_t)RS_BINS * ntiles, st);
        if (rc) return rc;
        if (va) rs_scatter_kernel<true><<<(unsigned)ntiles, RS_BLOCK, 0, st>>>(ka, kb, va, vb, n, shift, cnt, ntiles);
        else rs_scatter_kernel<false><<<(unsigned)ntiles, RS_BLOCK, 0, st>>>(ka, kb, nullptr, nullptr, n, shift, cnt,
                                                                              ntiles);
        HIP_OK(hipGetLastError());
        std::swap(ka, kb);
        std::swap(va, vb);
        *in_b = !*in_b;
    }
    return FZ_OK;
}

const char *bad_byte_msg(const Scoring &sc)
{
    return sc.mode == SUB_MATRIX ? "sequence holds a byte other than A, C, G, T, N"
                                 : "sequence holds a byte other than A, C, G, T (N needs a substitution matrix)";
}

Scoring make_scoring(const fz_scoring *s, const fz_matrix *mx, int32_t ydrop)
{
    Scoring sc = {};
    sc.match = s->match;
    sc.ts = s->transition;
    sc.tv = s->transversion;
    sc.oe = s->gap_open + s->gap_extend;
    sc.e = s->gap_extend;
    auto fits = [](int v) { return v >= -128 && v <= 127; };
    auto mag = [](int v) { return v < 0 ? -v : v; };
    sc.small = fits(sc.match) && fits(sc.ts) && fits(sc.tv);
    // xor code of two base codes: 0 equal, 2 transition, 1 or 3 transversion
    sc.lut = ((uint32_t)(sc.match & 0xFF)) | ((uint32_t)(sc.tv & 0xFF) << 8) | ((uint32_t)(sc.ts & 0xFF) << 16) |
             ((uint32_t)(sc.tv & 0xFF) << 24);
    sc.ydrop = (int64_t)ydrop >= SCORE_LIMIT ? (int32_t)SCORE_LIMIT : ydrop;
    if (mx) {
        sc.mode = SUB_MATRIX;
        sc.small = 1;
        sc.nsc = mx->n_score;
        sc.nrep = 0x01010101u * ((uint32_t)mx->n_score & 0xFFu);
        sc.msub = mag(mx->n_score);
        for (int a = 0; a < 4; ++a) {
            sc.mrow[a] = 0;
            for (int b = 0; b < 4; ++b) {
                sc.mrow[a] |= ((uint32_t)mx->sub[a][b] & 0xFFu) << (8 * b);
                sc.msub = std::max(sc.msub, mag(mx->sub[a][b]));
            }
        }
    } else {
        sc.mode = sc.small ? SUB_LUT : SUB_WIDE;
        sc.msub = std::max(mag(sc.match), std::max(mag(sc.ts), mag(sc.tv)));
    }
    return sc;
}

// The packed 16-bit layouts give the same results as the 32-bit ones for
// scorings within their exact range (fz_packed.hpp).
bool packed_ok(const Scoring &sc, uint32_t flags)
{
    return !(flags & FZ_EXACT32) && sc.mode == SUB_LUT && sc.ydrop <= PK_MAX_YDROP && sc.oe + sc.e <= PK_MAX_OE;
}

template <int C, bool EXEC>
int launch_extend(fz_ctx *ctx, const ExtendArgs &a, int64_t nwork, hipStream_t st, bool pk = false)
{
    if (nwork <= 0) return FZ_OK;
    const unsigned blocks = (unsigned)((nwork + EXT_WAVES - 1) / EXT_WAVES);
    if constexpr (C == C_STD) {
        if (pk) {
            extend_kernel<C, EXEC, SUB_LUT, EXT_WAVES, true><<<blocks, 64 * EXT_WAVES, 0, st>>>(a);
            HIP_OK(hipGetLastError());
            return FZ_OK;
        }
    }
    if (a.sc.mode == SUB_MATRIX) extend_kernel<C, EXEC, SUB_MATRIX, EXT_WAVES><<<blocks, 64 * EXT_WAVES, 0, st>>>(a);
    else if (a.sc.mode == SUB_LUT) extend_kernel<C, EXEC, SUB_LUT, EXT_WAVES><<<blocks, 64 * EXT_WAVES, 0, st>>>(a);
    else extend_kernel<C, EXEC, SUB_WIDE, EXT_WAVES><<<blocks, 64 * EXT_WAVES, 0, st>>>(a);
    HIP_OK(hipGetLastError());
    return FZ_OK;
}

// The packed two-pass executor over sides of the shortest length bin: four
// waves (sides) per workgroup.  These sides are short and alike, so a group
// is not held long by one of them, and a quarter of the workgroups keeps
// the dispatcher, which short one-wave groups outrun, from bounding the
// launch.
int launch_exec_short(fz_ctx *ctx, const ExtendArgs &a, int64_t nwork, hipStream_t st)
{
    if (nwork <= 0) return FZ_OK;
    constexpr int G = 4;
    extend_kernel<C_STD, true, SUB_LUT, G, true><<<(unsigned)((nwork + G - 1) / G), 64 * G, 0, st>>>(a);
    HIP_OK(hipGetLastError());
    return FZ_OK;
}

// The one-pass executor over a.list (one wave per side, like the others).
int launch_onepass(fz_ctx *ctx, const ExtendArgs &a, int64_t nwork, hipStream_t st)
{
    if (nwork <= 0) return FZ_OK;
    extend_kernel<C_STD, true, SUB_LUT, 1, true, true><<<(unsigned)nwork, 64, 0, st>>>(a);
    HIP_OK(hipGetLastError());
    return FZ_OK;
}

int check_args(fz_ctx *ctx, const uint8_t *target, uint64_t tlen, const uint8_t *query, uint64_t qlen,
               const fz_seed *seeds, uint64_t n, const fz_scoring *sc, const fz_matrix *mx, int32_t ydrop,
               uint32_t flags, fz_hit *hits)
{
    if (!sc) return fail(ctx, FZ_EINVAL, "scoring is NULL");
    if (mx) {
        bool ok = mx->n_score >= -128 && mx->n_score <= 127;
        for (int a = 0; a < 4; ++a)
            for (int b = 0; b < 4; ++b) ok = ok && mx->sub[a][b] >= -128 && mx->sub[a][b] <= 127;
        if (!ok) return fail(ctx, FZ_EINVAL, "matrix entries and n_score must lie in -128..127");
    }
    if (n > 0 && (!seeds || !hits)) return fail(ctx, FZ_EINVAL, "seeds or hits is NULL");
    if ((tlen > 0 && !target) || (qlen > 0 && !query)) return fail(ctx, FZ_EINVAL, "sequence pointer is NULL");
    if (tlen >= ((uint64_t)1 << 40) || qlen >= ((uint64_t)1 << 40)) return fail(ctx, FZ_EINVAL, "sequence too long");
    if (n >= ((uint64_t)1 << 30)) return fail(ctx, FZ_EINVAL, "too many seeds (max 2^30 - 1 per call)");
    if (sc->gap_open < 0 || sc->gap_extend < 0) return fail(ctx, FZ_EINVAL, "gap costs must be >= 0");
    const int64_t lim = (int64_t)1 << 24;
    if (sc->gap_open > lim || sc->gap_extend > lim || sc->match > lim || sc->match < -lim || sc->transition > lim ||
        sc->transition < -lim || sc->transversion > lim || sc->transversion < -lim)
        return fail(ctx, FZ_EINVAL, "scoring values must lie in [-2^24, 2^24]");
    if (!(flags & FZ_LOCAL) && ydrop < 0) return fail(ctx, FZ_EINVAL, "ydrop must be >= 0");
    if (flags & ~(uint32_t)(FZ_TRACEBACK | FZ_LOCAL | FZ_STATS | FZ_QUERY_RC | FZ_EXACT32 | FZ_TWO_PASS))
        return fail(ctx, FZ_EINVAL, "unknown flag bits");
    if ((flags & FZ_LOCAL) && (flags & FZ_TRACEBACK)) return fail(ctx, FZ_EINVAL, "local mode has no traceback");
    return FZ_OK;
}

struct Timer {
    fz_ctx *ctx;
    hipStream_t st;
    bool on;
    int k = 0;
    void mark()
    {
        if (on && k < 12) (void)hipEventRecord(ctx->ev[k++], st);
    }
    float ms(int a, int b)
    {
        if (!on || b >= k) return 0.f;
        float v = 0.f;
        (void)hipEventElapsedTime(&v, ctx->ev[a], ctx->ev[b]);
        return v;
    }
};

int run_local(fz_ctx *ctx, const fz_seed *seeds, uint64_t n, uint64_t tlen, uint64_t qlen, const Scoring &sc,
              fz_hit *hits, int64_t *d_max2, hipStream_t st)
{
    // windows taller than one strip spill their strip's last row; size that
    // buffer by the largest windows (read back once)
    window_max_kernel<<<blocks_for((int64_t)n, 256), 256, 0, st>>>(seeds, (int64_t)n, d_max2);
    HIP_OK(hipGetLastError());
    int64_t mx[2] = {0, 0};
    HIP_OK(hipMemcpyAsync(mx, d_max2, sizeof mx, hipMemcpyDeviceToHost, st));
    HIP_OK(hipStreamSynchronize(st));
    int64_t stride = 0;
    if (mx[0] > 64 * LOCAL_RL) stride = 2 * (std::max<int64_t>(mx[1], 0) + 1);
    ENSURE(ctx->bnd, (size_t)std::max<int64_t>(stride, 1) * sizeof(int32_t) * (stride ? (size_t)n : 1));
    LocalArgs a;
    a.seeds = seeds;
    a.n = (int64_t)n;
    a.tlen = (int64_t)tlen;
    a.qlen = (int64_t)qlen;
    a.Tf = as<uint8_t>(ctx->Tf);
    a.Qf = as<uint8_t>(ctx->Qf);
    a.sc = sc;
    a.hits = hits;
    a.bnd = as<int32_t>(ctx->bnd);
    a.bnd_stride = stride;
    const unsigned blocks = blocks_for((int64_t)n, LOCAL_WAVES);
    HIP_OK(hipEventRecord(ctx->kev[0], st));
    if (sc.mode == SUB_MATRIX) local_kernel<LOCAL_RL, SUB_MATRIX, LOCAL_WAVES><<<blocks, 64 * LOCAL_WAVES, 0, st>>>(a);
    else if (sc.mode == SUB_LUT) local_kernel<LOCAL_RL, SUB_LUT, LOCAL_WAVES><<<blocks, 64 * LOCAL_WAVES, 0, st>>>(a);
    else local_kernel<LOCAL_RL, SUB_WIDE, LOCAL_WAVES><<<blocks, 64 * LOCAL_WAVES, 0, st>>>(a);
    HIP_OK(hipGetLastError());
    HIP_OK(hipEventRecord(ctx->kev[1], st));
    return FZ_OK;
}

// The seed stage (fz_seeds.hpp), on `st`; synchronous at its two read-backs
// and at the end.
static int seeds_impl(fz_ctx *ctx, const uint8_t *target, uint64_t tlen, const uint8_t *query, uint64_t qlen,
                      uint32_t k, int64_t flank, uint32_t flags, const fz_seed **seeds, uint64_t *n_seeds,
                      uint64_t *n_hits, fz_seed_stats *stats, hipStream_t st)
{
    if (!n_seeds) return fail(ctx, FZ_EINVAL, "n_seeds is NULL");
    *n_seeds = 0;
    if (n_hits) *n_hits = 0;
    if (stats) *stats = fz_seed_stats{};
    Timer tm{ctx, st, stats != nullptr};
    if (seeds) *seeds = nullptr;
    ctx->last_seeds = 0;
    if (k < 1 || k > 32) return fail(ctx, FZ_EINVAL, "k must be 1..32 (got %u)", k);
    if (flank < 0) return fail(ctx, FZ_EINVAL, "flank must be >= 0");
    if (flags & ~(uint32_t)(FZ_QUERY_RC | FZ_SEEDS_ALL | FZ_SEEDS_REUSE_INDEX))
        return fail(ctx, FZ_EINVAL, "unknown flag bits");
    if ((tlen && !target) || (qlen && !query)) return fail(ctx, FZ_EINVAL, "NULL sequence");
    if (tlen >= (1ull << 31) || qlen >= (1ull << 31))
        return fail(ctx, FZ_EINVAL, "sequences must be shorter than 2^31 bases for the seed stage");
    const bool reuse = (flags & FZ_SEEDS_REUSE_INDEX) != 0;
    if (reuse && !(ctx->idx_valid && ctx->idx_target == target && ctx->idx_tlen == tlen && ctx->idx_k == k))
        return fail(ctx, FZ_EINVAL, "FZ_SEEDS_REUSE_INDEX: no index of this target (pointer, length, k) on ctx");
    if (!reuse) ctx->idx_valid = false;
    if (tlen < k || qlen < k) return FZ_OK;
    const int64_t nt = (int64_t)(tlen - k + 1), nq = (int64_t)(qlen - k + 1);
    const int64_t NT = (int64_t)tlen + 2 * PAD, NQ = (int64_t)qlen + 2 * PAD;

    // codes, validated (the extension's own staging)
    ENSURE(ctx->counters, sizeof(Counters));
    Counters *dc = as<Counters>(ctx->counters);
    int rc = zero(ctx, dc, sizeof(Counters), st);
    if (rc) return rc;
    ENSURE(ctx->Tf, NT + 64);
    ENSURE(ctx->Tr, NT + 64);
    ENSURE(ctx->Qf, NQ + 64);
    ENSURE(ctx->Qr, NQ + 64);
    tm.mark();
    if (!reuse)
        pack_kernel<<<std::min<int64_t>(blocks_for(NT, 256), 8192), 256, 0, st>>>(
            target, (int64_t)tlen, as<uint8_t>(ctx->Tf), as<uint8_t>(ctx->Tr), NT, &dc->err, 0, 3);
    pack_kernel<<<std::min<int64_t>(blocks_for(NQ, 256), 8192), 256, 0, st>>>(
        query, (int64_t)qlen, as<uint8_t>(ctx->Qf), as<uint8_t>(ctx->Qr), NQ, &dc->err, (flags & FZ_QUERY_RC) ? 1 : 0,
        3);
    HIP_OK(hipGetLastError());
    tm.mark();

    // target keys without N, sorted with their positions, and a bucket
    // table over the top bits of the key: about as many buckets as keys (at
    // most 2^30), all 2k bits when that is fewer
    const unsigned gb = 4 * (unsigned)ctx->n_cu * 4;
    int64_t ntv = reuse ? ctx->idx_keys : 0;
    auto table_bits = [&](int64_t nkeys) {
        int bits = 1;
        while (bits < 30 && (1ll << bits) < nkeys) ++bits;
        return std::min(bits, (int)(2 * k));
    };
    if (!reuse) {
        ENSURE(ctx->sk_tk, nt * sizeof(uint64_t));
        ENSURE(ctx->sk_tk2, nt * sizeof(uint64_t));
        ENSURE(ctx->sk_tp, nt * sizeof(uint32_t));
        ENSURE(ctx->sk_tp2, nt * sizeof(uint32_t));
        ENSURE(ctx->sk_valid, nt * sizeof(uint32_t));
        ENSURE(ctx->sk_vpos, nt * sizeof(uint32_t));
        kmer_keys_kernel<<<gb, 256, 0, st>>>(as<uint8_t>(ctx->Tf) + PAD, nt, (int)k, as<uint64_t>(ctx->sk_tk),
                                             as<uint32_t>(ctx->sk_tp), as<uint32_t>(ctx->sk_valid));
        HIP_OK(hipGetLastError());
        rc = device_scan<uint32_t, ScanSum, false>(ctx, as<uint32_t>(ctx->sk_valid), as<uint32_t>(ctx->sk_vpos),
                                                   nt, st);
        if (rc) return rc;
        uint32_t lv[2] = {0, 0};
        HIP_OK(hipMemcpyAsync(&lv[0], as<uint32_t>(ctx->sk_vpos) + (nt - 1), sizeof(uint32_t), hipMemcpyDeviceToHost,
                              st));
        HIP_OK(hipMemcpyAsync(&lv[1], as<uint32_t>(ctx->sk_valid) + (nt - 1), sizeof(uint32_t),
                              hipMemcpyDeviceToHost, st));
        HIP_OK(hipStreamSynchronize(st));
        ntv = (int64_t)lv[0] + lv[1];
        if (ntv < nt) {         // k-mers with N: keep the others, in order
            compact_keys_kernel<<<gb, 256, 0, st>>>(as<uint64_t>(ctx->sk_tk), as<uint32_t>(ctx->sk_tp),
                                                    as<uint32_t>(ctx->sk_valid), as<uint32_t>(ctx->sk_vpos), nt,
                                                    as<uint64_t>(ctx->sk_tk2), as<uint32_t>(ctx->sk_tp2));
            HIP_OK(hipGetLastError());
            std::swap(ctx->sk_tk, ctx->sk_tk2);
            std::swap(ctx->sk_tp, ctx->sk_tp2);
        }
    }
    const int nb_bits = table_bits(ntv);
    const int shift = (int)(2 * k) - nb_bits;
    const int64_t NB = 1ll << nb_bits;
    if (reuse || ntv == 0) {
        tm.mark();              // keys (done above unless reused), sort, table
        tm.mark();
        tm.mark();
    } else {
        tm.mark();
        // the sorted index ends in sk_tk2 / sk_tp2
        bool in_b = false;
        rc = radix_sort(ctx, as<uint64_t>(ctx->sk_tk), as<uint64_t>(ctx->sk_tk2), as<uint32_t>(ctx->sk_tp),
                        as<uint32_t>(ctx->sk_tp2), ntv, (int)(2 * k), st, &in_b);
        if (rc) return rc;
        if (!in_b) {
            std::swap(ctx->sk_tk, ctx->sk_tk2);
            std::swap(ctx->sk_tp, ctx->sk_tp2);
        }
        tm.mark();
        ENSURE(ctx->sk_bend, NB * sizeof(uint32_t));
        ENSURE(ctx->sk_boff, (NB + 1) * sizeof(uint32_t));
        rc = zero(ctx, ctx->sk_bend.p, NB * sizeof(uint32_t), st);
        if (rc) return rc;
        rc = zero(ctx, ctx->sk_boff.p, sizeof(uint32_t), st);
        if (rc) return rc;
        bucket_end_kernel<<<gb, 256, 0, st>>>(as<uint64_t>(ctx->sk_tk2), ntv, shift, as<uint32_t>(ctx->sk_bend));
        HIP_OK(hipGetLastError());
        rc = device_scan<uint32_t, ScanMax, true>(ctx, as<uint32_t>(ctx->sk_bend), as<uint32_t>(ctx->sk_boff) + 1, NB,
                                                  st);
        if (rc) return rc;
        tm.mark();
    }

    // join: per query position, the range of equal target keys
    ENSURE(ctx->sk_lo, nq * sizeof(uint32_t));
    ENSURE(ctx->sk_cnt, nq * sizeof(uint64_t));
    ENSURE(ctx->sk_off, nq * sizeof(uint64_t));
    join_count_kernel<<<gb, 256, 0, st>>>(as<uint64_t>(ctx->sk_tk2), ntv, as<uint32_t>(ctx->sk_boff), shift,
                                          as<uint8_t>(ctx->Qf) + PAD, nq, (int)k, as<uint32_t>(ctx->sk_lo),
                                          as<uint64_t>(ctx->sk_cnt));
    HIP_OK(hipGetLastError());
    tm.mark();
    rc = device_scan<uint64_t, ScanSum, false>(ctx, as<uint64_t>(ctx->sk_cnt), as<uint64_t>(ctx->sk_off), nq, st);
    if (rc) return rc;
    tm.mark();
    uint64_t last[2] = {0, 0};
    HIP_OK(hipMemcpyAsync(&last[0], as<uint64_t>(ctx->sk_off) + (nq - 1), sizeof(uint64_t), hipMemcpyDeviceToHost, st));
    HIP_OK(hipMemcpyAsync(&last[1], as<uint64_t>(ctx->sk_cnt) + (nq - 1), sizeof(uint64_t), hipMemcpyDeviceToHost, st));
    Counters hc;
    HIP_OK(hipMemcpyAsync(&hc, dc, sizeof(Counters), hipMemcpyDeviceToHost, st));
    HIP_OK(hipStreamSynchronize(st));
    if (hc.err & 1u) return fail(ctx, FZ_EINVAL, "sequence holds a byte other than A, C, G, T, N");
    if (!reuse) {
        ctx->idx_valid = true;
        ctx->idx_target = target;
        ctx->idx_tlen = tlen;
        ctx->idx_k = k;
        ctx->idx_keys = ntv;
    }
    const uint64_t H = last[0] + last[1];
    if (n_hits) *n_hits = H;
    auto finish = [&]() -> int {
        if (!stats) return FZ_OK;
        HIP_OK(hipStreamSynchronize(st));
        stats->ms_pack = tm.ms(0, 1);
        stats->ms_keys = tm.ms(1, 2);
        stats->ms_sort_keys = tm.ms(2, 3);
        stats->ms_index = tm.ms(3, 4);
        stats->ms_join = tm.ms(4, 5);
        stats->ms_scan = tm.ms(5, 6);
        stats->ms_emit = tm.ms(6, 7);
        stats->ms_sort_hits = tm.ms(7, 8);
        stats->ms_runs = tm.ms(8, 9);
        stats->ms_write = tm.ms(9, 10);
        stats->ms_total = tm.ms(0, tm.k - 1);
        return FZ_OK;
    };
    if (H == 0) return finish();
    if (H >= (1ull << 31)) return fail(ctx, FZ_ENOMEM, "%llu shared k-mer hits: more than the stage handles (2^31)",
                                       (unsigned long long)H);

    // hits, sorted by diagonal then t; run starts; their ranks
    ENSURE(ctx->sk_hit, H * sizeof(uint64_t));
    ENSURE(ctx->sk_hit2, H * sizeof(uint64_t));
    ENSURE(ctx->sk_flag, H * sizeof(uint64_t));
    ENSURE(ctx->sk_rank, H * sizeof(uint64_t));
    emit_hits_kernel<<<gb, 256, 0, st>>>(as<uint32_t>(ctx->sk_tp2), as<uint32_t>(ctx->sk_lo),
                                         as<uint64_t>(ctx->sk_cnt), as<uint64_t>(ctx->sk_off), nq, (int64_t)qlen,
                                         as<uint64_t>(ctx->sk_hit));
    HIP_OK(hipGetLastError());
    tm.mark();
    {
        // the word's diagonal field holds t - q + query_len < target_len + query_len;
        // the sorted words end in sk_hit2
        int bits = 32;
        while (bits < 64 && (tlen + qlen) >> (bits - 32)) ++bits;
        bool in_b = false;
        rc = radix_sort(ctx, as<uint64_t>(ctx->sk_hit), as<uint64_t>(ctx->sk_hit2), nullptr, nullptr, (int64_t)H, bits,
                        st, &in_b);
        if (rc) return rc;
        if (!in_b) std::swap(ctx->sk_hit, ctx->sk_hit2);
    }
    tm.mark();
    run_start_kernel<<<gb, 256, 0, st>>>(as<uint64_t>(ctx->sk_hit2), (int64_t)H, (flags & FZ_SEEDS_ALL) ? 0 : 1,
                                         as<uint64_t>(ctx->sk_flag));
    HIP_OK(hipGetLastError());
    rc = device_scan<uint64_t, ScanSum, false>(ctx, as<uint64_t>(ctx->sk_flag), as<uint64_t>(ctx->sk_rank), (int64_t)H,
                                               st);
    if (rc) return rc;
    tm.mark();
    HIP_OK(hipMemcpyAsync(&last[0], as<uint64_t>(ctx->sk_rank) + (H - 1), sizeof(uint64_t), hipMemcpyDeviceToHost, st));
    HIP_OK(hipMemcpyAsync(&last[1], as<uint64_t>(ctx->sk_flag) + (H - 1), sizeof(uint64_t), hipMemcpyDeviceToHost, st));
    HIP_OK(hipStreamSynchronize(st));
    const uint64_t n = last[0] + last[1];

    // the seed records
    ENSURE(ctx->sk_out, n * sizeof(fz_seed));
    write_seeds_kernel<<<gb, 256, 0, st>>>(as<uint64_t>(ctx->sk_hit2), as<uint64_t>(ctx->sk_flag),
                                           as<uint64_t>(ctx->sk_rank), (int64_t)H, (int)k, flank, (int64_t)tlen,
                                           (int64_t)qlen, as<fz_seed>(ctx->sk_out));
    HIP_OK(hipGetLastError());
    tm.mark();
    HIP_OK(hipStreamSynchronize(st));
    ctx->last_seeds = n;
    *n_seeds = n;
    if (seeds) *seeds = as<fz_seed>(ctx->sk_out);
    return finish();
}

}  // namespace

extern "C" {

int fz_create(fz_ctx **out, int device, uint64_t workspace_bytes)
{
    if (!out) return FZ_EINVAL;
    *out = nullptr;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev) {
        (void)hipGetLastError();
        return FZ_EDEVICE;
    }
    fz_ctx *ctx = new fz_ctx;
    ctx->device = device;
    ctx->ptr_cap = workspace_bytes;
    int prev = 0;
    (void)hipGetDevice(&prev);
    if (hipSetDevice(device) != hipSuccess) {
        delete ctx;
        return FZ_EDEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) == hipSuccess && prop.multiProcessorCount > 0)
        ctx->n_cu = prop.multiProcessorCount;
    {
        // this device's copy of the no-allocation scratch array, once per
        // device, with the device current
        std::lock_guard<std::mutex> lk(noalloc_mu);
        if (device < NA_MAX_DEVICES && !noalloc_base[device]) {
            void *p = nullptr;
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
                (void)hipGetLastError();
                (void)hipSetDevice(prev);
                fz_destroy(ctx);
                return FZ_EDEVICE;
            }
            noalloc_base[device] = reinterpret_cast<uint8_t *>(p);
        }
    }
    for (auto &e : ctx->kev) {
        if (hipEventCreate(&e) != hipSuccess) {
            (void)hipSetDevice(prev);
            fz_destroy(ctx);
            return FZ_EDEVICE;
        }
    }
    for (auto &e : ctx->ev) {
        if (hipEventCreate(&e) != hipSuccess) {
            (void)hipSetDevice(prev);
            fz_destroy(ctx);
            return FZ_EDEVICE;
        }
    }
    bool ok = hipEventCreateWithFlags(&ctx->fork_ev, hipEventDisableTiming) == hipSuccess;
    for (auto &e : ctx->join_ev) ok = ok && hipEventCreateWithFlags(&e, hipEventDisableTiming) == hipSuccess;
    ok = ok && hipEventCreateWithFlags(&ctx->wide_ev, hipEventDisableTiming) == hipSuccess;
    ok = ok && hipEventCreateWithFlags(&ctx->op_ev, hipEventDisableTiming) == hipSuccess;
    for (auto &e : ctx->tail_ev) ok = ok && hipEventCreateWithFlags(&e, hipEventDisableTiming) == hipSuccess;
    ok = ok && hipEventCreateWithFlags(&ctx->op_end_ev, hipEventDisableTiming) == hipSuccess;
    ok = ok && hipHostMalloc((void **)&ctx->op_started, 256, hipHostMallocCoherent) == hipSuccess;
    // default priority, no implicit ordering with the null stream
    for (auto &x : ctx->xs) ok = ok && hipStreamCreateWithFlags(&x, hipStreamNonBlocking) == hipSuccess;
    ok = ok && hipStreamCreateWithFlags(&ctx->xw, hipStreamNonBlocking) == hipSuccess;
    if (!ok) {
        (void)hipSetDevice(prev);
        fz_destroy(ctx);
        return FZ_EDEVICE;
    }
    (void)hipSetDevice(prev);
    *out = ctx;
    return FZ_OK;
}

void fz_destroy(fz_ctx *ctx)
{
    if (!ctx) return;
    int prev = 0;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(ctx->device);
    DevBuf *bufs[] = {&ctx->Tf, &ctx->Tr, &ctx->Qf, &ctx->Qr, &ctx->Tf16, &ctx->Tr16, &ctx->Qf16, &ctx->Qr16,
                      &ctx->tasks, &ctx->info, &ctx->out,
                      &ctx->eager, &ctx->side_trace, &ctx->run_cap, &ctx->run_off, &ctx->run_len, &ctx->runs,
                      &ctx->items, &ctx->batch_first, &ctx->scan_tmp, &ctx->cig, &ctx->cigar,
                      &ctx->counters, &ctx->ovl0, &ctx->ovl1, &ctx->bnd,
                      &ctx->sk_tk, &ctx->sk_tk2, &ctx->sk_tp, &ctx->sk_tp2, &ctx->sk_valid, &ctx->sk_vpos,
                      &ctx->sk_bend, &ctx->sk_boff, &ctx->sk_lo, &ctx->sk_cnt,
                      &ctx->sk_off, &ctx->sk_hit, &ctx->sk_hit2, &ctx->sk_flag, &ctx->sk_rank,
                      &ctx->sk_out, &ctx->rd_keep, &ctx->rd_pos, &ctx->rd_seeds, &ctx->rd_hits, &ctx->rd_cnt,
                      &ctx->rd_off, &ctx->rd_cig, &ctx->sg_key, &ctx->sg_key2, &ctx->sg_end, &ctx->sg_end2,
                      &ctx->sg_v, &ctx->sg_max, &ctx->rs_cnt, &ctx->ps_tmp, &ctx->defer_list, &ctx->op_fail,
                      &ctx->op_btab, &ctx->op_pool, &ctx->op_fail2, &ctx->op_done, &ctx->op_items,
                      &ctx->op_runs_tmp, &ctx->op_runs, &ctx->op_run_off, &ctx->op_key, &ctx->op_order,
                      &ctx->early_items, &ctx->early_ws, &ctx->op_fin, &ctx->tail_runs};
    for (auto &x : ctx->xs)
        if (x) (void)hipStreamSynchronize(x);
    if (ctx->xw) (void)hipStreamSynchronize(ctx->xw);
    for (DevBuf *b : bufs)
        if (b->p) (void)hipFree(b->p);
    for (auto &b : ctx->ptr_ws)
        if (b.p) (void)hipFree(b.p);
    for (auto &x : ctx->xs)
        if (x) (void)hipStreamDestroy(x);
    if (ctx->xw) (void)hipStreamDestroy(ctx->xw);
    if (ctx->wide_ev) (void)hipEventDestroy(ctx->wide_ev);
    if (ctx->op_ev) (void)hipEventDestroy(ctx->op_ev);
    for (auto &e : ctx->tail_ev)
        if (e) (void)hipEventDestroy(e);
    if (ctx->op_end_ev) (void)hipEventDestroy(ctx->op_end_ev);
    if (ctx->op_started) (void)hipHostFree(ctx->op_started);
    if (ctx->fork_ev) (void)hipEventDestroy(ctx->fork_ev);
    for (auto &e : ctx->join_ev)
        if (e) (void)hipEventDestroy(e);
    for (auto &e : ctx->ev)
        if (e) (void)hipEventDestroy(e);
    for (auto &e : ctx->kev)
        if (e) (void)hipEventDestroy(e);
    for (auto &e : ctx->walk_ev)
        if (e) (void)hipEventDestroy(e);
    (void)hipSetDevice(prev);
    delete ctx;
}

const char *fz_last_error(const fz_ctx *ctx) { return ctx ? ctx->err.c_str() : "null context"; }

int fz_set_pointer_workspace(fz_ctx *ctx, uint64_t bytes)
{
    if (!ctx) return FZ_EINVAL;
    ctx->ptr_cap = bytes;
    return FZ_OK;
}

int fz_debug_set(fz_ctx *ctx, int what, int64_t value)
{
    if (!ctx) return FZ_EINVAL;
    if (what == FZ_DEBUG_SHRINK_ROWS && value >= 0) {
        ctx->dbg_shrink_rows = value;
        return FZ_OK;
    }
    if (what == FZ_DEBUG_ONEPASS_POOL && value >= -1) {
        ctx->dbg_op_pool = value;
        return FZ_OK;
    }
    if (what == FZ_DEBUG_ONEPASS_ORDER && (value == 0 || value == 1)) {
        ctx->dbg_op_order = value;
        return FZ_OK;
    }
    if (what == FZ_DEBUG_TAIL_WALK && value >= 0 && value <= ((int64_t)1 << 40)) {
        ctx->dbg_tail = value;
        return FZ_OK;
    }
    return fail(ctx, FZ_EINVAL, "unknown debug setting or value out of range");
}

static int grow_keep(fz_ctx *ctx, DevBuf &b, size_t bytes, size_t keep, hipStream_t st);

// The one-pass executor's pool, sized for n deferred sides whose windows
// hold `diags` anti-diagonals in all (each side m + n + 1): a 256-position
// row with its header per anti-diagonal, plus an arena and a block table
// per side; at most 3/4 of the free device memory (this context's pointer
// workspaces counted as free, and released when the pool must grow), 3/4
// of the device, and the context's pointer-memory cap.  *bytes is the
// pool's usable size, 0 when there is none (too little memory: the deferred
// sides then go back to the inspector).
static int prepare_onepass_pool(fz_ctx *ctx, int64_t n, uint64_t diags, int64_t nsides, hipStream_t st,
                                uint64_t *bytes)
{
    *bytes = 0;
    ENSURE(ctx->op_btab, nsides * sizeof(uint64_t));
    uint64_t want = 0;
    if (ctx->dbg_op_pool > 0) {
        want = (uint64_t)ctx->dbg_op_pool;
    } else {
        size_t fr = 0, tot = 0;
        HIP_OK(hipMemGetInfo(&fr, &tot));
        uint64_t avail = (uint64_t)fr + ctx->op_pool.cap;
        for (const auto &b : ctx->ptr_ws) avail += b.cap;
        // three quarters of what is available: a pool that runs short
        // costs a round (a walk and the kernel's tail) per refill
        const uint64_t cap = std::min<uint64_t>(avail / 4 * 3, (uint64_t)tot / 4 * 3);
        const uint64_t need = diags * (8 + 4 * 32) + (uint64_t)n * (uint64_t)(OP_ARENA + 8192) + ((uint64_t)64 << 20);
        want = std::min(need, cap);
        // a pointer-memory cap set on the context bounds the pool too
        if (ctx->ptr_cap) want = std::min<uint64_t>(want, ctx->ptr_cap);
    }
    if (ctx->op_pool.cap < want) {
        size_t fr = 0, tot = 0;
        HIP_OK(hipMemGetInfo(&fr, &tot));
        if ((uint64_t)fr < want - ctx->op_pool.cap + ((uint64_t)1 << 30)) {
            // the executor's workspaces come back later at their own size
            HIP_OK(hipStreamSynchronize(st));
            for (auto &b : ctx->ptr_ws)
                if (b.p) {
                    (void)hipFree(b.p);
                    b.p = nullptr;
                    b.cap = 0;
                }
        }
        if (ctx->op_pool.p) {
            HIP_OK(hipStreamSynchronize(st));
            (void)hipFree(ctx->op_pool.p);
            ctx->op_pool.p = nullptr;
            ctx->op_pool.cap = 0;
        }
        // what the device gives, down to a quarter of the request
        for (uint64_t b = want; b >= want / 4 && b >= (uint64_t)OP_ARENA; b /= 2) {
            if (hipMalloc(&ctx->op_pool.p, b) == hipSuccess) {
                ctx->op_pool.cap = b;
                break;
            }
            (void)hipGetLastError();
            ctx->op_pool.p = nullptr;
        }
    }
    const uint64_t pool_bytes = ctx->op_pool.p ? std::min<uint64_t>(want, ctx->op_pool.cap - WALK_PAD) : 0;
    // (the pool's sink and one arena at least)
    *bytes = pool_bytes >= (uint64_t)(OP_BLOCK_BYTES + OP_ARENA) ? pool_bytes : 0;
    return FZ_OK;
}

// One round of the one-pass executor over list[0, n): sides it finishes go
// to `done`, sides the pool could not hold to `fail` (counts in
// Counters::op_round, cleared by the caller).
static int launch_onepass_round(fz_ctx *ctx, const ExtendArgs &ea, const int32_t *list, int64_t n,
                                uint64_t pool_bytes, int32_t *fail, int32_t *done, uint32_t *fin,
                                uint32_t *last_started, void *counters, hipStream_t st)
{
    Counters *dc = static_cast<Counters *>(counters);
    ExtendArgs oa = ea;
    oa.list = list;
    oa.nlist = (int32_t)n;
    oa.exec_cells = &dc->op_cells;
    oa.op_pool = as<uint8_t>(ctx->op_pool);
    oa.op_pool_bytes = pool_bytes;
    oa.op_pool_used = reinterpret_cast<unsigned long long *>(&dc->op_round.pool_used);
    oa.op_btab = as<uint64_t>(ctx->op_btab);
    oa.op_fail_list = fail;
    oa.op_fail_count = &dc->op_round.fail;
    oa.op_done_list = done;
    oa.op_done_count = &dc->op_round.done;
    oa.op_fin = fin;
    oa.op_last_started = last_started;
    oa.op_flushed = &dc->tail.flushed;
    return launch_onepass(ctx, oa, n, st);
}

static int extend_impl(fz_ctx *ctx, const uint8_t *target, uint64_t tlen, const uint8_t *query, uint64_t qlen,
                       const fz_seed *seeds, uint64_t n_seeds, const fz_scoring *scoring, const fz_matrix *matrix,
                       int32_t ydrop, int64_t min_tb, uint32_t flags, fz_hit *hits, const uint32_t **cigar,
                       uint64_t *cigar_words, fz_stats *stats, hipStream_t st)
{
    int rc = check_args(ctx, target, tlen, query, qlen, seeds, n_seeds, scoring, matrix, ydrop, flags, hits);
    if (rc != FZ_OK) return rc;
    if (cigar) *cigar = nullptr;
    if (cigar_words) *cigar_words = 0;
    fz_stats S;
    memset(&S, 0, sizeof S);
    Timer tm{ctx, st, (flags & FZ_STATS) != 0};
    const int64_t n = (int64_t)n_seeds;
    if (n == 0) {
        if (stats) *stats = S;
        return FZ_OK;
    }
    const Scoring sc = make_scoring(scoring, matrix, ydrop);
    const int64_t NT = (int64_t)tlen + 2 * PAD, NQ = (int64_t)qlen + 2 * PAD;

    ENSURE(ctx->counters, sizeof(Counters));
    Counters *dc = as<Counters>(ctx->counters);
    rc = zero(ctx, dc, sizeof(Counters), st);
    if (rc) return rc;

    tm.mark();
    // ---- pack
    ENSURE(ctx->Tf, NT + 64);
    ENSURE(ctx->Tr, NT + 64);
    ENSURE(ctx->Qf, NQ + 64);
    ENSURE(ctx->Qr, NQ + 64);
    const bool pk = !(flags & FZ_LOCAL) && packed_ok(sc, flags);
    if (pk) {
        ENSURE(ctx->Tf16, 2 * (NT + 64));
        ENSURE(ctx->Tr16, 2 * (NT + 64));
        ENSURE(ctx->Qf16, 2 * (NQ + 64));
        ENSURE(ctx->Qr16, 2 * (NQ + 64));
    }
    {
        const unsigned bt = std::min<int64_t>(blocks_for(NT, 256), 8192);
        const int mxr = sc.mode == SUB_MATRIX ? 1 : 0;     // matrix mode: role codes, N accepted
        pack_kernel<<<bt, 256, 0, st>>>(target, (int64_t)tlen, as<uint8_t>(ctx->Tf), as<uint8_t>(ctx->Tr), NT,
                                        &dc->err, 0, mxr, pk ? as<uint16_t>(ctx->Tf16) : nullptr,
                                        pk ? as<uint16_t>(ctx->Tr16) : nullptr, 0);
        HIP_OK(hipGetLastError());
        const unsigned bq = std::min<int64_t>(blocks_for(NQ, 256), 8192);
        // with FZ_QUERY_RC every later step sees the query's reverse
        // complement: seeds, windows and results are in its coordinates
        pack_kernel<<<bq, 256, 0, st>>>(query, (int64_t)qlen, as<uint8_t>(ctx->Qf), as<uint8_t>(ctx->Qr), NQ,
                                        &dc->err, (flags & FZ_QUERY_RC) ? 1 : 0, 2 * mxr,
                                        pk ? as<uint16_t>(ctx->Qf16) : nullptr, pk ? as<uint16_t>(ctx->Qr16) : nullptr,
                                        1);
        HIP_OK(hipGetLastError());
    }
    Counters hc;
    auto read_counters = [&]() -> int {
        HIP_OK(hipMemcpyAsync(&hc, dc, sizeof(Counters), hipMemcpyDeviceToHost, st));
        HIP_OK(hipStreamSynchronize(st));
        return FZ_OK;
    };

    if (flags & FZ_LOCAL) {
        rc = run_local(ctx, seeds, n_seeds, tlen, qlen, sc, hits, &dc->totals[0], st);
        if (rc) return rc;
        tm.mark();
        if ((rc = read_counters())) return rc;
        if (hc.err & 1u) return fail(ctx, FZ_EINVAL, "%s", bad_byte_msg(sc));
        if (stats) {
            S.ms_inspect = tm.ms(0, 1);
            (void)hipEventElapsedTime(&S.ms_main, ctx->kev[0], ctx->kev[1]);
            *stats = S;
        }
        return FZ_OK;
    }

    // ---- setup
    const int64_t nsides = 2 * n;
    ENSURE(ctx->tasks, nsides * sizeof(SideTask));
    ENSURE(ctx->info, n * sizeof(SeedInfo));
    ENSURE(ctx->out, nsides * sizeof(SideOut));
    ENSURE(ctx->eager, nsides * EAGER_OPS);
    // sides certain to be traced go to the one-pass executor (packed
    // layouts, with traceback; not under the test-only row shrink, which
    // exercises the two-pass executor's disagreement check)
    const bool defer_on = pk && (flags & FZ_TRACEBACK) && !(flags & FZ_TWO_PASS) && ctx->dbg_shrink_rows == 0 &&
                          ctx->dbg_op_pool != 0;
    setup_kernel<<<blocks_for(n, 256), 256, 0, st>>>(seeds, n, (int64_t)tlen, (int64_t)qlen, as<uint8_t>(ctx->Tf),
                                                      as<uint8_t>(ctx->Tr), as<uint8_t>(ctx->Qf),
                                                      as<uint8_t>(ctx->Qr), NT, NQ, sc, as<SideTask>(ctx->tasks),
                                                      as<SeedInfo>(ctx->info), pk ? as<uint8_t>(ctx->Tf16) : nullptr,
                                                      pk ? as<uint8_t>(ctx->Tr16) : nullptr,
                                                      pk ? as<uint8_t>(ctx->Qf16) : nullptr,
                                                      pk ? as<uint8_t>(ctx->Qr16) : nullptr, defer_on, min_tb);
    HIP_OK(hipGetLastError());
    tm.mark();

    // ---- inspect
    ENSURE(ctx->ovl0, nsides * sizeof(int32_t));
    ENSURE(ctx->ovl1, nsides * sizeof(int32_t));
    ExtendArgs ea = {};
    ea.tasks = as<SideTask>(ctx->tasks);
    ea.list = nullptr;
    ea.nlist = (int32_t)nsides;
    ea.out = as<SideOut>(ctx->out);
    ea.eager_ops = as<uint8_t>(ctx->eager);
    ea.overflow_list = as<int32_t>(ctx->ovl0);
    ea.overflow_count = &dc->overflow_count[0];
    ea.exec_cells = &dc->exec_cells;
    ea.result_flags = 0;
    ea.sc = sc;
    if (defer_on) {
        ENSURE(ctx->defer_list, nsides * sizeof(int32_t));
        ea.defer_list = as<int32_t>(ctx->defer_list);
        ea.defer_count = &dc->defer_count;
        ea.defer_diags = reinterpret_cast<unsigned long long *>(&dc->defer_diags);
    }
    HIP_OK(hipEventRecord(ctx->kev[0], st));
    rc = launch_extend<C_STD, false>(ctx, ea, nsides, st, pk);
    if (rc) return rc;
    HIP_OK(hipEventRecord(ctx->kev[1], st));
    if (defer_on) {
        onepass_pick_kernel<<<blocks_for(n, 256), 256, 0, st>>>(
            n, as<SeedInfo>(ctx->info), as<SideOut>(ctx->out), as<SideTask>(ctx->tasks), min_tb, SHORT_BIN_LEN,
            as<int32_t>(ctx->defer_list), &dc->defer_count, reinterpret_cast<unsigned long long *>(&dc->defer_diags));
        HIP_OK(hipGetLastError());
    }
    if ((rc = read_counters())) return rc;
    if (hc.err & 1u) return fail(ctx, FZ_EINVAL, "%s", bad_byte_msg(sc));
    // wide retry (the 1024-position window, a few long latency-bound waves)
    // of the overflow list [first, first + count)
    auto wide_retry = [&](uint32_t first, uint32_t count, hipStream_t ws, bool early) -> int {
        ExtendArgs wa = ea;
        wa.list = as<int32_t>(ctx->ovl0) + first;
        wa.nlist = (int32_t)count;
        wa.overflow_list = as<int32_t>(ctx->ovl1);
        wa.overflow_count = &dc->overflow_count[1];
        wa.result_flags = SO_WIDE_FLAG;
        if (early && (flags & FZ_TRACEBACK)) {
            // beside the one-pass executor: sides certain to be traced are
            // traced in the retry's own wave (a handful of long waves that
            // would otherwise end the executor phase alone)
            size_t fr = 0, tot = 0;
            HIP_OK(hipMemGetInfo(&fr, &tot));
            uint64_t cap = std::min<uint64_t>((uint64_t)2 << 30, (uint64_t)fr / 16);
            if (ctx->ptr_cap) cap = std::min<uint64_t>(cap, ctx->ptr_cap);     // (a pointer-memory cap bounds it too)
            ENSURE(ctx->early_items, (int64_t)count * sizeof(ExecItem));
            ENSURE(ctx->early_ws, (int64_t)cap + WALK_PAD);
            wa.early_ws = as<uint8_t>(ctx->early_ws);
            wa.early_cap = std::min<uint64_t>(cap, ctx->early_ws.cap - WALK_PAD);
            wa.early_bytes = reinterpret_cast<unsigned long long *>(&dc->early.bytes);
            wa.early_items = as<ExecItem>(ctx->early_items);
            wa.early_count = &dc->early.count;
            wa.info = as<SeedInfo>(ctx->info);
            wa.min_tb = min_tb;
        }
        return launch_extend<C_WIDE, false>(ctx, wa, wa.nlist, ws);
    };
    // the inspector's overflow sides go to the wide retry beside the
    // one-pass executor; those of the one-pass executor (and of sides it
    // gives back) after it
    const uint32_t n_ovl_first = hc.defer_count > 0 ? hc.overflow_count[0] : 0;
    if (n_ovl_first > 0) {
        HIP_OK(hipEventRecord(ctx->fork_ev, st));
        HIP_OK(hipStreamWaitEvent(ctx->xw, ctx->fork_ev, 0));
        if ((rc = wide_retry(0, n_ovl_first, ctx->xw, true))) return rc;
    }
    bool onepass_ran = false;
    bool tail_ran = false;              // a tail walk beside the one-pass executor (tail_ev[1] its end)
    int64_t n_early = 0;                // the wide retry's sides traced beside the one-pass executor
    if (hc.defer_count > 0) {
        // ---- one-pass executor over the deferred sides, in rounds: when the
        // pool cannot hold all their rows at once, the sides a round
        // finished are walked at once and the pool serves the next round
        // (the sides that did not fit); the last round's sides are walked
        // beside the two-pass executor.  A round that finishes no side
        // gives the rest back to the inspector.
        // Tail walk: the one-pass executor's last waves run for tens of
        // milliseconds after its last dispatch, with most of the machine
        // idle.  A walk launched beside it (on an executor stream no one
        // uses yet) takes the sides that have finished by the time its wave
        // runs, into a run buffer of its own (1/64 of the free memory, at
        // most 1 GiB, taken once per context, before the pool).
        const bool tail_on = ctx->dbg_tail != 0;
        if (tail_on) {
            if (!ctx->tail_runs.p) {
                size_t fr = 0, tot = 0;
                HIP_OK(hipMemGetInfo(&fr, &tot));
                ENSURE(ctx->tail_runs, std::max<uint64_t>(std::min<uint64_t>((uint64_t)fr / 64, (uint64_t)1 << 30), 4096));
            }
            ENSURE(ctx->op_fin, nsides * sizeof(uint32_t));
            ENSURE(ctx->op_run_off, nsides * sizeof(int64_t));
            rc = zero(ctx, &dc->tail, sizeof dc->tail, st);
            if (rc) return rc;
        }
        // (test settings: after the executor on the caller's stream, where
        // every finished side is taken, within a given number of run words)
        const uint64_t tail_cap = ctx->dbg_tail > 2 ? std::min<uint64_t>(ctx->tail_runs.cap / sizeof(uint32_t),
                                                                          (uint64_t)ctx->dbg_tail)
                                                    : ctx->tail_runs.cap / sizeof(uint32_t);
        const hipStream_t ts = ctx->dbg_tail >= 2 ? st : ctx->xs[0];
        uint64_t pool_bytes = 0;
        rc = prepare_onepass_pool(ctx, (int64_t)hc.defer_count, hc.defer_diags, nsides, st, &pool_bytes);
        if (rc) return rc;
        ENSURE(ctx->op_fail, nsides * sizeof(int32_t));
        ENSURE(ctx->op_fail2, nsides * sizeof(int32_t));
        ENSURE(ctx->op_done, nsides * sizeof(int32_t));
        ENSURE(ctx->run_len, nsides * sizeof(int64_t));
        const int32_t *L = as<int32_t>(ctx->defer_list);
        uint32_t nL = hc.defer_count;
        if (nL > 1 && ctx->dbg_op_order) {
            // longest sides first (predicted)
            ENSURE(ctx->op_key, (int64_t)nL);
            ENSURE(ctx->op_order, (int64_t)nL * sizeof(int32_t));
            rc = zero(ctx, dc->op_key_hist, 2 * OP_KEYS * sizeof(uint32_t), st);
            if (rc) return rc;
            op_key_kernel<<<blocks_for(nL, OP_KEY_WAVES), 64 * OP_KEY_WAVES, 0, st>>>(
                L, (int64_t)nL, as<SideTask>(ctx->tasks), as<uint8_t>(ctx->op_key), dc->op_key_hist);
            HIP_OK(hipGetLastError());
            op_order_kernel<<<blocks_for(nL, 256), 256, 0, st>>>(L, (int64_t)nL, as<uint8_t>(ctx->op_key),
                                                                 dc->op_key_hist, dc->op_key_cur,
                                                                 as<int32_t>(ctx->op_order));
            HIP_OK(hipGetLastError());
            L = as<int32_t>(ctx->op_order);
        }
        const int32_t *back = nullptr;
        uint32_t n_back = 0;
        if (pool_bytes == 0) {
            back = L;
            n_back = nL;
            nL = 0;
        }
        int64_t runs_base = 0;
        for (int fb = 0; nL > 0; fb ^= 1) {
            rc = zero(ctx, &dc->op_round, sizeof dc->op_round, st);
            if (rc) return rc;
            int32_t *fl = fb ? as<int32_t>(ctx->op_fail2) : as<int32_t>(ctx->op_fail);
            if (tail_on) {
                rc = zero(ctx, ctx->op_fin.p, (size_t)nL * sizeof(uint32_t), st);
                if (rc) return rc;
                rc = zero(ctx, &dc->tail.flushed, sizeof dc->tail.flushed, st);
                if (rc) return rc;
                HIP_OK(hipEventRecord(ctx->tail_ev[0], st));
            }
            if (!onepass_ran) HIP_OK(hipEventRecord(ctx->kev[2], st));
            const bool tail_beside = tail_on && ts != st;
            uint32_t *started_dev = nullptr;
            if (tail_beside) {
                __atomic_store_n(ctx->op_started, 0u, __ATOMIC_RELEASE);
                HIP_OK(hipHostGetDevicePointer((void **)&started_dev, ctx->op_started, 0));
            }
            rc = launch_onepass_round(ctx, ea, L, nL, pool_bytes, fl, as<int32_t>(ctx->op_done),
                                      tail_on ? as<uint32_t>(ctx->op_fin) : nullptr, started_dev, dc, st);
            if (rc) return rc;
            onepass_ran = true;
            if (tail_beside) {
                // hold the tail walk back until the executor's last wave has
                // started (or the executor has ended): launched earlier, its
                // waves would take slots from executor waves not yet started
                HIP_OK(hipEventRecord(ctx->op_end_ev, st));
                while (__atomic_load_n(ctx->op_started, __ATOMIC_ACQUIRE) == 0) {
                    const hipError_t q = hipEventQuery(ctx->op_end_ev);
                    if (q != hipErrorNotReady) {
                        HIP_OK(q);
                        break;
                    }
                    std::this_thread::sleep_for(std::chrono::microseconds(200));
                }
            }
            if (tail_on) {
                // (after the executor in host order: the device dispatches it
                // once the executor's grid is dispatched, or its waves find
                // few sides finished)
                HIP_OK(hipStreamWaitEvent(ts, ctx->tail_ev[0], 0));
                tail_flush_kernel<<<TAIL_FLUSH_GROUPS, 64, 0, ts>>>(&dc->tail.flushed);
                HIP_OK(hipGetLastError());
                WalkArgs wk = {};
                wk.begin = 0;
                wk.end = nL;
                wk.op_btab = as<uint64_t>(ctx->op_btab);
                wk.out = as<SideOut>(ctx->out);
                wk.runs = as<uint32_t>(ctx->tail_runs);
                wk.run_len = as<int64_t>(ctx->run_len);
                wk.tail_list = L;
                wk.tail_fin = as<uint32_t>(ctx->op_fin);
                wk.tail_used = reinterpret_cast<unsigned long long *>(&dc->tail.used);
                wk.tail_cap = tail_cap;
                wk.op_run_off = as<int64_t>(ctx->op_run_off);
                wk.tail_sides = &dc->tail.sides;
                walk_wave_kernel<true><<<nL, 64, 0, ts>>>(wk);
                HIP_OK(hipGetLastError());
                HIP_OK(hipEventRecord(ctx->tail_ev[1], ts));
                tail_ran = true;
            }
            if ((rc = read_counters())) return rc;
            const uint32_t nd = hc.op_round.done, nf = hc.op_round.fail;
            S.n_onepass += nd;
            S.onepass_bytes += std::min<uint64_t>(hc.op_round.pool_used, pool_bytes);
            if (nd == 0) {
                back = fl;
                n_back = nf;
                break;
            }
            if (nf == 0) break;
            // the pool serves the next round: walk this round's sides now
            // (those the tail walk took have their runs already)
            if (tail_on) HIP_OK(hipStreamWaitEvent(st, ctx->tail_ev[1], 0));
            ENSURE(ctx->op_items, (int64_t)nd * sizeof(ExecItem));
            ExecItem *items = as<ExecItem>(ctx->op_items);
            op_items_kernel<<<blocks_for(nd, 256), 256, 0, st>>>(as<int32_t>(ctx->op_done), (int64_t)nd,
                                                                 as<SideOut>(ctx->out), items);
            HIP_OK(hipGetLastError());
            const int64_t stride = sizeof(ExecItem) / sizeof(int64_t);
            rc = scan(ctx, reinterpret_cast<const int64_t *>(&items->ptr_bytes), stride, nd,
                      reinterpret_cast<int64_t *>(&items->ptr_off), stride, &dc->op_runs_total, st);
            if (rc) return rc;
            if ((rc = read_counters())) return rc;
            ENSURE(ctx->op_runs_tmp, std::max<int64_t>(hc.op_runs_total, 1) * sizeof(uint32_t));
            WalkArgs wk = {};
            wk.items = items;
            wk.begin = 0;
            wk.end = nd;
            wk.op_btab = as<uint64_t>(ctx->op_btab);
            wk.runs_by_item = 1;
            wk.out = as<SideOut>(ctx->out);
            wk.runs = as<uint32_t>(ctx->op_runs_tmp);
            wk.run_len = as<int64_t>(ctx->run_len);
            walk_wave_kernel<true><<<nd, 64, 0, st>>>(wk);
            HIP_OK(hipGetLastError());
            // pack the runs (a walk writes far fewer than its capacity)
            op_run_count_kernel<<<blocks_for(nd, 256), 256, 0, st>>>(items, (int64_t)nd, as<int64_t>(ctx->run_len));
            HIP_OK(hipGetLastError());
            rc = scan(ctx, reinterpret_cast<const int64_t *>(&items->batch), stride, nd,
                      reinterpret_cast<int64_t *>(&items->ptr_bytes), stride, &dc->op_runs_total, st);
            if (rc) return rc;
            if ((rc = read_counters())) return rc;
            const int64_t packed = hc.op_runs_total;
            rc = grow_keep(ctx, ctx->op_runs, (size_t)std::max<int64_t>(runs_base + packed, 1) * sizeof(uint32_t),
                           (size_t)runs_base * sizeof(uint32_t), st);
            if (rc) return rc;
            ENSURE(ctx->op_run_off, nsides * sizeof(int64_t));
            op_run_pack_kernel<<<blocks_for(nd, 256), 256, 0, st>>>(
                items, (int64_t)nd, as<uint32_t>(ctx->op_runs_tmp), as<uint32_t>(ctx->tail_runs),
                as<SideOut>(ctx->out), as<uint32_t>(ctx->op_runs), runs_base, as<int64_t>(ctx->op_run_off));
            HIP_OK(hipGetLastError());
            runs_base += packed;
            // (the tail buffer's runs are packed: the next round's tail walk
            // starts it over)
            if (tail_on && (rc = zero(ctx, &dc->tail.used, sizeof dc->tail.used, st))) return rc;
            L = fl;
            nL = nf;
        }
        if (onepass_ran) HIP_OK(hipEventRecord(ctx->kev[3], st));
        S.onepass_cells = (uint64_t)hc.op_cells;
        if (n_back > 0) {
            // the pool held none of them: the inspector takes those sides
            // back and keeps them (the two-pass executor traces them)
            undefer_kernel<<<blocks_for(n_back, 256), 256, 0, st>>>(back, (int64_t)n_back, as<SideTask>(ctx->tasks));
            HIP_OK(hipGetLastError());
            ExtendArgs ra = ea;
            ra.list = back;
            ra.nlist = (int32_t)n_back;
            rc = launch_extend<C_STD, false>(ctx, ra, ra.nlist, st, pk);
            if (rc) return rc;
            if ((rc = read_counters())) return rc;
        }
    }
    S.n_overflow = hc.overflow_count[0];
    if (hc.overflow_count[0] > n_ovl_first &&
        (rc = wide_retry(n_ovl_first, hc.overflow_count[0] - n_ovl_first, st, false)))
        return rc;
    if (n_ovl_first > 0) {
        HIP_OK(hipEventRecord(ctx->wide_ev, ctx->xw));
        HIP_OK(hipStreamWaitEvent(st, ctx->wide_ev, 0));
    }
    tm.mark();

    // ---- combine + bin
    ENSURE(ctx->side_trace, nsides * sizeof(int32_t));
    ENSURE(ctx->run_cap, nsides * sizeof(int64_t));
    ENSURE(ctx->run_off, nsides * sizeof(int64_t));
    ENSURE(ctx->run_len, nsides * sizeof(int64_t));
    CombineArgs ca;
    ca.seeds = seeds;
    ca.n = n;
    ca.out = as<SideOut>(ctx->out);
    ca.info = as<SeedInfo>(ctx->info);
    ca.min_tb = min_tb;
    ca.traceback = (flags & FZ_TRACEBACK) ? 1 : 0;
    ca.hits = hits;
    ca.side_trace = as<int32_t>(ctx->side_trace);
    ca.run_cap = as<int64_t>(ctx->run_cap);
    ca.bin_count = dc->bin_count;
    ca.max_ptr = &dc->max_ptr;
    ca.cells_total = &dc->totals[3];
    ca.max_band = &dc->max_band;
    combine_kernel<<<blocks_for(n, 256), 256, 0, st>>>(ca);
    HIP_OK(hipGetLastError());
    // run slots of traced sides
    rc = scan(ctx, as<int64_t>(ctx->run_cap), 1, nsides, as<int64_t>(ctx->run_off), 1, &dc->totals[0], st);
    if (rc) return rc;
    if ((rc = read_counters())) return rc;
    const int64_t total_runs = hc.totals[0];
    uint32_t base[EXEC_CLASSES * NBINS];
    // item order: one-pass sides (walked only), then wide-window sides (few
    // and slow, so they overlap everything after them), then the standard
    // ones, each class longest bins first; items [0, n_op) are one-pass,
    // [n_op, n_wide) wide
    int64_t n_exec = 0, n_op = 0, n_wide = 0, n_short = 0;
    for (int cls = EXEC_CLASSES - 1; cls >= 0; --cls)
        for (int b = NBINS - 1; b >= 0; --b) {
            base[cls * NBINS + b] = (uint32_t)n_exec;
            if (cls == EXEC_CLASS_STD && b == 0) n_short = n_exec;   // the shortest standard bin from here
            n_exec += hc.bin_count[cls * NBINS + b];
            if (cls == EXEC_CLASS_ONEPASS) n_op = n_exec;
            if (cls == EXEC_CLASS_WIDE) n_wide = n_exec;
            S.bin_hist[b] += hc.bin_count[cls * NBINS + b];
        }
    S.n_executor = (uint64_t)(n_exec - n_op);
    ENSURE(ctx->runs, std::max<int64_t>(total_runs, 1) * sizeof(uint32_t));
    if (n_exec > 0) {
        HIP_OK(hipMemcpyAsync(dc->bin_base, base, sizeof base, hipMemcpyHostToDevice, st));
        ENSURE(ctx->items, n_exec * sizeof(ExecItem));
        bin_scatter_kernel<<<blocks_for(nsides, 256), 256, 0, st>>>(nsides, as<int32_t>(ctx->side_trace),
                                                                    as<SideOut>(ctx->out), dc->bin_base,
                                                                    dc->bin_fill, as<ExecItem>(ctx->items),
                                                                    ctx->dbg_shrink_rows);
        HIP_OK(hipGetLastError());
        const int64_t stride = sizeof(ExecItem) / sizeof(int64_t);
        ExecItem *it = as<ExecItem>(ctx->items);
        rc = scan(ctx, reinterpret_cast<const int64_t *>(&it->ptr_bytes), stride, n_exec,
                  reinterpret_cast<int64_t *>(&it->ptr_off), stride, &dc->totals[1], st);
        if (rc) return rc;
    }
    eager_runs_kernel<<<blocks_for(nsides, 256), 256, 0, st>>>(nsides, as<int32_t>(ctx->side_trace),
                                                               as<SideOut>(ctx->out), as<uint8_t>(ctx->eager),
                                                               as<int64_t>(ctx->run_off), as<uint32_t>(ctx->runs),
                                                               as<int64_t>(ctx->run_len));
    HIP_OK(hipGetLastError());
    tm.mark();

    // the early list's traced sides (their rows written by the wide retry
    // beside the one-pass executor; the stream joined the retry's after it)
    n_early = (int64_t)hc.early.count;
    if (n_early > 0) {
        WalkArgs wk = {};
        wk.items = as<ExecItem>(ctx->early_items);
        wk.begin = 0;
        wk.end = n_early;
        wk.ptr_ws = as<uint8_t>(ctx->early_ws);
        wk.ptr_base_off = 0;
        wk.out = as<SideOut>(ctx->out);
        wk.run_off = as<int64_t>(ctx->run_off);
        wk.runs = as<uint32_t>(ctx->runs);
        wk.run_len = as<int64_t>(ctx->run_len);
        wk.side_trace = as<int32_t>(ctx->side_trace);
        walk_wave_kernel<false><<<(unsigned)n_early, 64, 0, st>>>(wk);
        HIP_OK(hipGetLastError());
        S.n_executor += (uint64_t)n_early;
    }

    // ---- execute + walk, in batches
    size_t n_walks = 0;
    if (n_exec > 0) {
        if ((rc = read_counters())) return rc;
        const int64_t total_ptr = hc.totals[1], max_item = hc.max_ptr;
        S.pointer_bytes = (uint64_t)total_ptr;
        uint64_t cap = ctx->ptr_cap;
        if (cap == 0) {
            size_t fr = 0, tot = 0;
            HIP_OK(hipMemGetInfo(&fr, &tot));
            // the context's own workspaces count as available
            uint64_t avail = (uint64_t)fr;
            for (const auto &b : ctx->ptr_ws) avail += b.cap;
            // most of what is available: a batch lasts at least as long as
            // its longest side, so fewer, larger batches finish sooner
            cap = std::min<uint64_t>(avail / 10 * 7, (uint64_t)200 << 30);
        }
        // the cap covers all workspaces; each holds at least two of the
        // largest sides
        uint64_t cap1 = std::max<uint64_t>(cap / EXEC_STREAMS, (uint64_t)2 * (uint64_t)max_item + 4096);
        // room for every side at once when the cap allows (one batch): a
        // batch b holds the items whose offsets fall in [b*step, (b+1)*step),
        // the last of which may reach max_item past the step
        const int64_t ws = std::min<int64_t>((int64_t)cap1, total_ptr + max_item + 256);
        const int64_t step = std::max<int64_t>(1, ws - max_item);
        const int64_t nb = (total_ptr + step - 1) / step;
        const int nbuf = (int)std::min<int64_t>(nb, EXEC_STREAMS);
        for (int k = 0; k < nbuf; ++k) ENSURE(ctx->ptr_ws[k], ws + WALK_PAD);
        ENSURE(ctx->batch_first, (nb + 1) * sizeof(int64_t));
        fill_i64_kernel<<<blocks_for(nb + 1, 256), 256, 0, st>>>(as<int64_t>(ctx->batch_first), nb + 1, n_exec);
        HIP_OK(hipGetLastError());
        batch_assign_kernel<<<blocks_for(n_exec, 256), 256, 0, st>>>(as<ExecItem>(ctx->items), n_exec, step,
                                                                     as<int64_t>(ctx->batch_first));
        HIP_OK(hipGetLastError());
        std::vector<int64_t> first((size_t)nb + 1);
        HIP_OK(hipMemcpyAsync(first.data(), ctx->batch_first.p, nb * sizeof(int64_t), hipMemcpyDeviceToHost, st));
        HIP_OK(hipStreamSynchronize(st));
        first[(size_t)nb] = n_exec;
        // batches that own no item start where the next one does
        for (int64_t b = nb - 1; b >= 0; --b)
            if (first[(size_t)b] > first[(size_t)b + 1]) first[(size_t)b] = first[(size_t)b + 1];
        S.n_batches = (uint64_t)nb;
        // batch b runs on stream b % nbuf with workspace b % nbuf; a
        // workspace is reused only by later batches of its own stream.  When
        // no workspace is reused (one batch per stream), the wide-window
        // items (a few hundred long, low-occupancy waves) run on a stream of
        // their own beside the batches, in their batch's workspace region.
        const bool wide_apart = nb <= nbuf && n_wide > n_op;
        // the one-pass sides' walks: on an executor stream that no batch
        // uses, else beside the wide-window items (streams share the
        // device's few hardware queues, so no stream is added for them)
        const bool op_own = nbuf < EXEC_STREAMS;         // an executor stream without a batch
        const hipStream_t xop = op_own ? ctx->xs[std::max(nbuf, 1) - 1] : ctx->xw;
        const bool use_xw = wide_apart || (n_op > 0 && !op_own);
        if (nbuf > 1 || use_xw || n_op > 0) {
            HIP_OK(hipEventRecord(ctx->fork_ev, st));
            for (int k = 1; k < nbuf; ++k) HIP_OK(hipStreamWaitEvent(ctx->xs[k - 1], ctx->fork_ev, 0));
            if (use_xw) HIP_OK(hipStreamWaitEvent(ctx->xw, ctx->fork_ev, 0));
            if (n_op > 0 && op_own) HIP_OK(hipStreamWaitEvent(xop, ctx->fork_ev, 0));
        }
        auto walk = [&](int64_t s0, int64_t s1, hipStream_t xst, uint8_t *wsp, int64_t base_off, bool op) -> int {
            WalkArgs wk = {};
            wk.items = as<ExecItem>(ctx->items);
            wk.begin = s0;
            wk.end = s1;
            wk.ptr_ws = wsp;
            wk.ptr_base_off = base_off;
            wk.op_btab = as<uint64_t>(ctx->op_btab);
            wk.out = as<SideOut>(ctx->out);
            wk.run_off = as<int64_t>(ctx->run_off);
            wk.runs = as<uint32_t>(ctx->runs);
            wk.run_len = as<int64_t>(ctx->run_len);
            if (tm.on) {
                // a pair of events around each walker launch (ms_walk)
                while (ctx->walk_ev.size() < 2 * (n_walks + 1)) {
                    hipEvent_t e = nullptr;
                    HIP_OK(hipEventCreate(&e));
                    ctx->walk_ev.push_back(e);
                }
                HIP_OK(hipEventRecord(ctx->walk_ev[2 * n_walks], xst));
            }
            if (op) walk_wave_kernel<true><<<(unsigned)(s1 - s0), 64, 0, xst>>>(wk);
            else walk_wave_kernel<false><<<(unsigned)(s1 - s0), 64, 0, xst>>>(wk);
            HIP_OK(hipGetLastError());
            if (tm.on) HIP_OK(hipEventRecord(ctx->walk_ev[2 * n_walks++ + 1], xst));
            return FZ_OK;
        };
        if (n_op > 0 && tail_ran) HIP_OK(hipStreamWaitEvent(xop, ctx->tail_ev[1], 0));
        if (n_op > 0 && (rc = walk(0, n_op, xop, nullptr, 0, true))) return rc;
        for (int64_t b = 0; b < nb; ++b) {
            const int64_t lo = first[(size_t)b], hi = first[(size_t)b + 1];
            if (hi <= lo) continue;
            const int kb = (int)(b % nbuf);
            const hipStream_t bst = kb == 0 ? st : ctx->xs[kb - 1];
            uint8_t *wsp = as<uint8_t>(ctx->ptr_ws[kb]);
            // wide-window items come before the standard ones in the list
            // (and one-pass ones, not executed, before both)
            const int64_t segs[2][2] = {{std::max(lo, n_wide), hi}, {std::max(lo, n_op), std::min(hi, n_wide)}};
            for (int cls = 1; cls >= 0; --cls) {
                const int64_t s0 = segs[cls][0], s1 = segs[cls][1];
                if (s1 <= s0) continue;
                const hipStream_t xst = (cls == 1 && wide_apart) ? ctx->xw : bst;
                ExtendArgs xa = ea;
                xa.exec = as<ExecItem>(ctx->items);
                xa.exec_begin = s0;
                xa.nlist = (int32_t)(s1 - s0);
                xa.ptr_ws = wsp;
                xa.ptr_base_off = b * step;
                if (cls == 0 && pk && s1 > n_short) {
                    // the shortest bin's sides in groups of four
                    const int64_t m = std::max(s0, n_short);
                    xa.nlist = (int32_t)(m - s0);
                    if ((rc = launch_extend<C_STD, true>(ctx, xa, m - s0, xst, pk))) return rc;
                    ExtendArgs sa = xa;
                    sa.exec_begin = m;
                    sa.nlist = (int32_t)(s1 - m);
                    rc = launch_exec_short(ctx, sa, s1 - m, xst);
                } else {
                    rc = cls == 0 ? launch_extend<C_STD, true>(ctx, xa, s1 - s0, xst, pk)
                                  : launch_extend<C_WIDE, true>(ctx, xa, s1 - s0, xst);
                }
                if (rc) return rc;
                if ((rc = walk(s0, s1, xst, wsp, b * step, false))) return rc;
            }
        }
        for (int k = 1; k < nbuf; ++k) {
            HIP_OK(hipEventRecord(ctx->join_ev[k - 1], ctx->xs[k - 1]));
            HIP_OK(hipStreamWaitEvent(st, ctx->join_ev[k - 1], 0));
        }
        if (use_xw) {
            HIP_OK(hipEventRecord(ctx->wide_ev, ctx->xw));
            HIP_OK(hipStreamWaitEvent(st, ctx->wide_ev, 0));
        }
        if (n_op > 0 && op_own) {
            HIP_OK(hipEventRecord(ctx->op_ev, xop));
            HIP_OK(hipStreamWaitEvent(st, ctx->op_ev, 0));
        }
    }
    tm.mark();

    // ---- gather CIGARs
    if (tail_ran) HIP_OK(hipStreamWaitEvent(st, ctx->tail_ev[1], 0));
    ENSURE(ctx->cig, n * sizeof(int64_t));
    AssembleArgs aa = {};
    aa.op_run_off = as<int64_t>(ctx->op_run_off);
    aa.op_runs = as<uint32_t>(ctx->op_runs);
    aa.tail_runs = as<uint32_t>(ctx->tail_runs);
    aa.seeds = seeds;
    aa.out = as<SideOut>(ctx->out);
    aa.n = n;
    aa.run_off = as<int64_t>(ctx->run_off);
    aa.run_len = as<int64_t>(ctx->run_len);
    aa.runs = as<uint32_t>(ctx->runs);
    aa.hits = hits;
    aa.cig_len = as<int64_t>(ctx->cig);
    aa.cigar = nullptr;
    aa.err = &dc->err;
    assemble_kernel<false><<<blocks_for(n, 256), 256, 0, st>>>(aa);
    HIP_OK(hipGetLastError());
    rc = scan(ctx, as<int64_t>(ctx->cig), 1, n, as<int64_t>(ctx->cig), 1, &dc->totals[2], st);
    if (rc) return rc;
    if ((rc = read_counters())) return rc;
    const int64_t total_words = hc.totals[2];
    S.n_tail_walked = tail_ran ? hc.tail.sides : 0;
    ENSURE(ctx->cigar, std::max<int64_t>(total_words, 1) * sizeof(uint32_t));
    aa.cigar = as<uint32_t>(ctx->cigar);
    assemble_kernel<true><<<blocks_for(n, 256), 256, 0, st>>>(aa);
    HIP_OK(hipGetLastError());
    tm.mark();
    if ((rc = read_counters())) return rc;
    if (hc.err & 2u) return fail(ctx, FZ_EDEVICE, "internal error: a traceback walk did not reach the origin");
    if (cigar) *cigar = as<uint32_t>(ctx->cigar);
    if (cigar_words) *cigar_words = (uint64_t)total_words;
    ctx->last_words = (uint64_t)total_words;
    if (stats) {
        S.n_sides = (uint64_t)nsides;
        S.cells = (uint64_t)hc.totals[3];
        S.executor_cells = (uint64_t)hc.exec_cells;
        S.max_band = (uint64_t)hc.max_band;
        S.n_packed = pk ? (uint64_t)nsides : 0;
        if (onepass_ran) (void)hipEventElapsedTime(&S.ms_onepass, ctx->kev[2], ctx->kev[3]);
        for (size_t w = 0; w < n_walks; ++w) {
            float v = 0.f;
            (void)hipEventElapsedTime(&v, ctx->walk_ev[2 * w], ctx->walk_ev[2 * w + 1]);
            S.ms_walk += v;
        }
        S.ms_pack = tm.ms(0, 1);
        S.ms_inspect = tm.ms(1, 2);
        S.ms_bin = tm.ms(2, 3);
        S.ms_exec = tm.ms(3, 4);
        S.ms_gather = tm.ms(4, 5);
        (void)hipEventElapsedTime(&S.ms_main, ctx->kev[0], ctx->kev[1]);
        *stats = S;
    }
    return FZ_OK;
}

// fz_extend_batch_noalloc: the score-only extension path (pack, setup,
// inspector, wide retry, combine) with every buffer carved from this
// device's static scratch array.  No device allocation and no allocating
// library call; the one read-back (the overflow count) goes to host stack
// memory.
static int noalloc_impl(fz_ctx *ctx, const uint8_t *target, uint64_t tlen, const uint8_t *query, uint64_t qlen,
                        const fz_seed *seeds, uint64_t n_seeds, const fz_scoring *scoring, const fz_matrix *matrix,
                        int32_t ydrop, uint32_t flags, fz_hit *hits, fz_stats *stats, hipStream_t st)
{
    int rc = check_args(ctx, target, tlen, query, qlen, seeds, n_seeds, scoring, matrix, ydrop, flags, hits);
    if (rc != FZ_OK) return rc;
    if (flags & (FZ_TRACEBACK | FZ_LOCAL))
        return fail(ctx, FZ_EINVAL, "fz_extend_batch_noalloc is score-only: FZ_TRACEBACK and FZ_LOCAL are not accepted");
    if (n_seeds > (uint64_t)FZ_NOALLOC_MAX_SEEDS)
        return fail(ctx, FZ_EINVAL, "fz_extend_batch_noalloc takes at most %d seeds (got %llu)", FZ_NOALLOC_MAX_SEEDS,
                    (unsigned long long)n_seeds);
    if (tlen > (uint64_t)FZ_NOALLOC_MAX_BASES || qlen > (uint64_t)FZ_NOALLOC_MAX_BASES)
        return fail(ctx, FZ_EINVAL, "fz_extend_batch_noalloc takes sequences of at most %d bases (got %llu and %llu)",
                    FZ_NOALLOC_MAX_BASES, (unsigned long long)tlen, (unsigned long long)qlen);
    uint8_t *base = ctx->device < NA_MAX_DEVICES ? noalloc_base[ctx->device] : nullptr;
    if (!base) return fail(ctx, FZ_EDEVICE, "no scratch address for device %d", ctx->device);
    fz_stats S;
    memset(&S, 0, sizeof S);
    const int64_t n = (int64_t)n_seeds;
    if (n == 0) {
        if (stats) *stats = S;
        return FZ_OK;
    }
    const Scoring sc = make_scoring(scoring, matrix, ydrop);
    const int64_t NT = (int64_t)tlen + 2 * PAD, NQ = (int64_t)qlen + 2 * PAD;
    uint8_t *Tf = base + NA_TF, *Tr = base + NA_TR, *Qf = base + NA_QF, *Qr = base + NA_QR;
    const bool pk = packed_ok(sc, flags);
    uint16_t *Tf16 = pk ? reinterpret_cast<uint16_t *>(base + NA_TF16) : nullptr;
    uint16_t *Tr16 = pk ? reinterpret_cast<uint16_t *>(base + NA_TR16) : nullptr;
    uint16_t *Qf16 = pk ? reinterpret_cast<uint16_t *>(base + NA_QF16) : nullptr;
    uint16_t *Qr16 = pk ? reinterpret_cast<uint16_t *>(base + NA_QR16) : nullptr;
    SideTask *tasks = reinterpret_cast<SideTask *>(base + NA_TASKS);
    SeedInfo *info = reinterpret_cast<SeedInfo *>(base + NA_INFO);
    SideOut *out = reinterpret_cast<SideOut *>(base + NA_OUT);
    Counters *dc = reinterpret_cast<Counters *>(base + NA_COUNTERS);
    // the counters keep the last call's values: clear them (a kernel, not a memset)
    rc = zero(ctx, dc, sizeof(Counters), st);
    if (rc) return rc;
    const int mxr = sc.mode == SUB_MATRIX ? 1 : 0;
    pack_kernel<<<std::min<int64_t>(blocks_for(NT, 256), 8192), 256, 0, st>>>(target, (int64_t)tlen, Tf, Tr, NT,
                                                                                &dc->err, 0, mxr, Tf16, Tr16, 0);
    HIP_OK(hipGetLastError());
    pack_kernel<<<std::min<int64_t>(blocks_for(NQ, 256), 8192), 256, 0, st>>>(
        query, (int64_t)qlen, Qf, Qr, NQ, &dc->err, (flags & FZ_QUERY_RC) ? 1 : 0, 2 * mxr, Qf16, Qr16, 1);
    HIP_OK(hipGetLastError());
    setup_kernel<<<blocks_for(n, 256), 256, 0, st>>>(seeds, n, (int64_t)tlen, (int64_t)qlen, Tf, Tr, Qf, Qr, NT, NQ,
                                                      sc, tasks, info, reinterpret_cast<uint8_t *>(Tf16),
                                                      reinterpret_cast<uint8_t *>(Tr16),
                                                      reinterpret_cast<uint8_t *>(Qf16),
                                                      reinterpret_cast<uint8_t *>(Qr16));
    HIP_OK(hipGetLastError());
    const int64_t nsides = 2 * n;
    ExtendArgs ea = {};
    ea.tasks = tasks;
    ea.list = nullptr;
    ea.nlist = (int32_t)nsides;
    ea.out = out;
    ea.eager_ops = base + NA_EAGER;
    ea.overflow_list = reinterpret_cast<int32_t *>(base + NA_OVL0);
    ea.overflow_count = &dc->overflow_count[0];
    ea.exec_cells = &dc->exec_cells;
    ea.result_flags = 0;
    ea.sc = sc;
    HIP_OK(hipEventRecord(ctx->kev[0], st));
    rc = launch_extend<C_STD, false>(ctx, ea, nsides, st, pk);
    if (rc) return rc;
    HIP_OK(hipEventRecord(ctx->kev[1], st));
    Counters hc;
    HIP_OK(hipMemcpyAsync(&hc, dc, sizeof(Counters), hipMemcpyDeviceToHost, st));
    HIP_OK(hipStreamSynchronize(st));
    if (hc.err & 1u) return fail(ctx, FZ_EINVAL, "%s", bad_byte_msg(sc));
    if (hc.overflow_count[0] > 0) {
        ExtendArgs wa = ea;
        wa.list = reinterpret_cast<int32_t *>(base + NA_OVL0);
        wa.nlist = (int32_t)hc.overflow_count[0];
        wa.overflow_list = reinterpret_cast<int32_t *>(base + NA_OVL1);
        wa.overflow_count = &dc->overflow_count[1];
        wa.result_flags = SO_WIDE_FLAG;
        rc = launch_extend<C_WIDE, false>(ctx, wa, wa.nlist, st);
        if (rc) return rc;
    }
    CombineArgs ca;
    ca.seeds = seeds;
    ca.n = n;
    ca.out = out;
    ca.info = info;
    ca.min_tb = 0;
    ca.traceback = 0;
    ca.hits = hits;
    ca.side_trace = reinterpret_cast<int32_t *>(base + NA_TRACE);
    ca.run_cap = reinterpret_cast<int64_t *>(base + NA_RUNCAP);
    ca.bin_count = dc->bin_count;
    ca.max_ptr = &dc->max_ptr;
    ca.cells_total = &dc->totals[3];
    ca.max_band = &dc->max_band;
    combine_kernel<<<blocks_for(n, 256), 256, 0, st>>>(ca);
    HIP_OK(hipGetLastError());
    if (stats) {
        HIP_OK(hipMemcpyAsync(&hc, dc, sizeof(Counters), hipMemcpyDeviceToHost, st));
        HIP_OK(hipStreamSynchronize(st));
        S.n_sides = (uint64_t)nsides;
        S.cells = (uint64_t)hc.totals[3];
        S.max_band = (uint64_t)hc.max_band;
        S.n_packed = pk ? (uint64_t)nsides : 0;
        S.n_overflow = hc.overflow_count[0];
        (void)hipEventElapsedTime(&S.ms_main, ctx->kev[0], ctx->kev[1]);
        *stats = S;
    }
    return FZ_OK;
}

// Grow b to at least `bytes`, keeping its first `keep` bytes.
static int grow_keep(fz_ctx *ctx, DevBuf &b, size_t bytes, size_t keep, hipStream_t st)
{
    if (b.cap >= bytes) return FZ_OK;
    DevBuf nb;
    int rc = ensure(ctx, nb, bytes);
    if (rc) return rc;
    if (keep && b.p) {
        HIP_OK(hipMemcpyAsync(nb.p, b.p, keep, hipMemcpyDeviceToDevice, st));
        HIP_OK(hipStreamSynchronize(st));
    }
    if (b.p) (void)hipFree(b.p);
    b = nb;
    return FZ_OK;
}

static int rounds_impl(fz_ctx *ctx, const uint8_t *target, uint64_t tlen, const uint8_t *query, uint64_t qlen,
                       const fz_seed *seeds, uint64_t n_seeds, const fz_scoring *scoring, const fz_matrix *matrix,
                       int32_t ydrop, int64_t min_tb, uint32_t flags, uint64_t round_size, fz_hit *hits,
                       const uint32_t **cigar, uint64_t *cigar_words, fz_stats *stats, hipStream_t st)
{
    if (cigar) *cigar = nullptr;
    if (cigar_words) *cigar_words = 0;
    const bool doubling = (flags & FZ_ROUNDS_DOUBLING) != 0;
    flags &= ~(uint32_t)FZ_ROUNDS_DOUBLING;
    int rc = check_args(ctx, target, tlen, query, qlen, seeds, n_seeds, scoring, matrix, ydrop, flags, hits);
    if (rc != FZ_OK) return rc;
    if (!(flags & FZ_TRACEBACK) || (flags & FZ_LOCAL))
        return fail(ctx, FZ_EINVAL, "fz_extend_rounds needs FZ_TRACEBACK and no FZ_LOCAL");
    if (round_size < 1) return fail(ctx, FZ_EINVAL, "round_size must be >= 1");
    if (tlen >= (1ull << 31) || qlen >= (1ull << 31))
        return fail(ctx, FZ_EINVAL, "sequences must be shorter than 2^31 bases for fz_extend_rounds");
    fz_stats tot;
    memset(&tot, 0, sizeof tot);
    const int64_t n = (int64_t)n_seeds;
    int64_t B = (int64_t)std::min<uint64_t>(round_size, std::max<uint64_t>(n_seeds, 1));
    int64_t acc_words = 0, nseg = 0;
    for (int64_t r0 = 0; r0 < n; r0 += B, B = doubling ? std::min<int64_t>(2 * B, n) : B) {
        const int64_t nb = std::min<int64_t>(B, n - r0);
        // the per-round buffers may grow (doubling rounds): let the last
        // round's kernels finish before any is reallocated
        if (r0 > 0) HIP_OK(hipStreamSynchronize(st));
        ENSURE(ctx->rd_keep, nb * sizeof(uint32_t));
        ENSURE(ctx->rd_pos, nb * sizeof(uint32_t));
        ENSURE(ctx->rd_seeds, nb * sizeof(fz_seed));
        ENSURE(ctx->rd_hits, nb * sizeof(fz_hit));
        ENSURE(ctx->rd_cnt, nb * sizeof(uint64_t));
        ENSURE(ctx->rd_off, nb * sizeof(uint64_t));
        const fz_seed *rs = seeds + r0;
        uint32_t *keep = as<uint32_t>(ctx->rd_keep), *pos = as<uint32_t>(ctx->rd_pos);
        // which seeds of the round an earlier round covers
        cover_kernel<<<blocks_for(nb, 256), 256, 0, st>>>(rs, nb, (int64_t)tlen, (int64_t)qlen,
                                                          as<uint64_t>(ctx->sg_key), as<uint64_t>(ctx->sg_max),
                                                          nseg, keep);
        HIP_OK(hipGetLastError());
        rc = device_scan<uint32_t, ScanSum, false>(ctx, keep, pos, nb, st);
        if (rc) return rc;
        uint32_t lastv[2] = {0, 0};
        HIP_OK(hipMemcpyAsync(&lastv[0], pos + (nb - 1), sizeof(uint32_t), hipMemcpyDeviceToHost, st));
        HIP_OK(hipMemcpyAsync(&lastv[1], keep + (nb - 1), sizeof(uint32_t), hipMemcpyDeviceToHost, st));
        HIP_OK(hipStreamSynchronize(st));
        const int64_t nkeep = (int64_t)lastv[0] + lastv[1];
        compact_seeds_kernel<<<blocks_for(nb, 256), 256, 0, st>>>(rs, nb, keep, pos, as<fz_seed>(ctx->rd_seeds));
        HIP_OK(hipGetLastError());
        // the round: one ordinary batch
        uint64_t words = 0;
        if (nkeep > 0) {
            fz_stats rsst;
            rc = extend_impl(ctx, target, tlen, query, qlen, as<fz_seed>(ctx->rd_seeds), (uint64_t)nkeep, scoring,
                             matrix, ydrop, min_tb, flags, as<fz_hit>(ctx->rd_hits), nullptr, &words,
                             stats ? &rsst : nullptr, st);
            if (rc) return rc;
            if (stats) {
                tot.cells += rsst.cells;
                tot.executor_cells += rsst.executor_cells;
                tot.pointer_bytes += rsst.pointer_bytes;
                tot.n_sides += rsst.n_sides;
                tot.n_eager += rsst.n_eager;
                tot.n_executor += rsst.n_executor;
                tot.n_overflow += rsst.n_overflow;
                for (int b = 0; b < NBINS; ++b) tot.bin_hist[b] += rsst.bin_hist[b];
                tot.n_batches += rsst.n_batches;
                tot.ms_pack += rsst.ms_pack;
                tot.ms_inspect += rsst.ms_inspect;
                tot.ms_bin += rsst.ms_bin;
                tot.ms_exec += rsst.ms_exec;
                tot.ms_walk += rsst.ms_walk;
                tot.ms_gather += rsst.ms_gather;
                tot.ms_main += rsst.ms_main;
                tot.max_band = std::max(tot.max_band, rsst.max_band);
                tot.n_packed += rsst.n_packed;
                tot.n_onepass += rsst.n_onepass;
                tot.onepass_cells += rsst.onepass_cells;
                tot.onepass_bytes = std::max(tot.onepass_bytes, rsst.onepass_bytes);
                tot.ms_onepass += rsst.ms_onepass;
            }
            rc = grow_keep(ctx, ctx->rd_cig, (size_t)(acc_words + (int64_t)words + 1) * sizeof(uint32_t),
                           (size_t)acc_words * sizeof(uint32_t), st);
            if (rc) return rc;
            if (words)
                HIP_OK(hipMemcpyAsync(as<uint32_t>(ctx->rd_cig) + acc_words, ctx->cigar.p, words * sizeof(uint32_t),
                                      hipMemcpyDeviceToDevice, st));
        }
        scatter_hits_kernel<<<blocks_for(nb, 256), 256, 0, st>>>(as<fz_hit>(ctx->rd_hits), nb, keep, pos, acc_words,
                                                                 hits + r0);
        HIP_OK(hipGetLastError());
        acc_words += (int64_t)words;
        if (nkeep == 0 || r0 + nb >= n) continue;     // nothing new, or no later round to cover
        // this round's aligned segments, added to the sorted set
        seg_count_kernel<<<blocks_for(nkeep, 256), 256, 0, st>>>(as<fz_hit>(ctx->rd_hits), nkeep,
                                                                 as<uint32_t>(ctx->cigar), as<uint64_t>(ctx->rd_cnt));
        HIP_OK(hipGetLastError());
        rc = device_scan<uint64_t, ScanSum, false>(ctx, as<uint64_t>(ctx->rd_cnt), as<uint64_t>(ctx->rd_off), nkeep,
                                                   st);
        if (rc) return rc;
        uint64_t lastm[2] = {0, 0};
        HIP_OK(hipMemcpyAsync(&lastm[0], as<uint64_t>(ctx->rd_off) + (nkeep - 1), sizeof(uint64_t),
                              hipMemcpyDeviceToHost, st));
        HIP_OK(hipMemcpyAsync(&lastm[1], as<uint64_t>(ctx->rd_cnt) + (nkeep - 1), sizeof(uint64_t),
                              hipMemcpyDeviceToHost, st));
        HIP_OK(hipStreamSynchronize(st));
        const int64_t m = (int64_t)(lastm[0] + lastm[1]);
        if (m == 0) continue;
        if (nseg + m >= (1ll << 31)) return fail(ctx, FZ_ENOMEM, "more than 2^31 aligned segments");
        const int64_t ns = nseg + m;
        rc = grow_keep(ctx, ctx->sg_key, ns * sizeof(uint64_t), nseg * sizeof(uint64_t), st);
        if (rc) return rc;
        rc = grow_keep(ctx, ctx->sg_end, ns * sizeof(uint32_t), nseg * sizeof(uint32_t), st);
        if (rc) return rc;
        ENSURE(ctx->sg_key2, ns * sizeof(uint64_t));
        ENSURE(ctx->sg_end2, ns * sizeof(uint32_t));
        ENSURE(ctx->sg_v, ns * sizeof(uint64_t));
        ENSURE(ctx->sg_max, ns * sizeof(uint64_t));
        seg_emit_kernel<<<blocks_for(nkeep, 256), 256, 0, st>>>(as<fz_hit>(ctx->rd_hits), nkeep,
                                                                as<uint32_t>(ctx->cigar), as<uint64_t>(ctx->rd_off),
                                                                (int64_t)qlen, as<uint64_t>(ctx->sg_key) + nseg,
                                                                as<uint32_t>(ctx->sg_end) + nseg);
        HIP_OK(hipGetLastError());
        {
            // keys are (t - q + query_len) << 32 | t; the sorted set ends in sg_key / sg_end
            int bits = 32;
            while (bits < 64 && (tlen + qlen) >> (bits - 32)) ++bits;
            bool in_b = false;
            rc = radix_sort(ctx, as<uint64_t>(ctx->sg_key), as<uint64_t>(ctx->sg_key2), as<uint32_t>(ctx->sg_end),
                            as<uint32_t>(ctx->sg_end2), ns, bits, st, &in_b);
            if (rc) return rc;
            if (in_b) {
                std::swap(ctx->sg_key, ctx->sg_key2);
                std::swap(ctx->sg_end, ctx->sg_end2);
            }
        }
        seg_diag_end_kernel<<<blocks_for(ns, 256), 256, 0, st>>>(as<uint64_t>(ctx->sg_key), as<uint32_t>(ctx->sg_end),
                                                                 ns, as<uint64_t>(ctx->sg_v));
        HIP_OK(hipGetLastError());
        rc = device_scan<uint64_t, ScanMax, true>(ctx, as<uint64_t>(ctx->sg_v), as<uint64_t>(ctx->sg_max), ns, st);
        if (rc) return rc;
        nseg = ns;
    }
    HIP_OK(hipStreamSynchronize(st));
    // the words of every round become the context's CIGAR buffer
    std::swap(ctx->cigar, ctx->rd_cig);
    ctx->last_words = (uint64_t)acc_words;
    if (cigar) *cigar = as<uint32_t>(ctx->cigar);
    if (cigar_words) *cigar_words = (uint64_t)acc_words;
    if (stats) *stats = tot;
    return FZ_OK;
}

int fz_extend_rounds(fz_ctx *ctx, const uint8_t *target, uint64_t target_len, const uint8_t *query,
                     uint64_t query_len, const fz_seed *seeds, uint64_t n_seeds, const fz_scoring *scoring,
                     const fz_matrix *matrix, int32_t ydrop, int64_t min_traceback_score, uint32_t flags,
                     uint64_t round_size, fz_hit *hits, const uint32_t **cigar, uint64_t *cigar_words,
                     fz_stats *stats, void *stream)
{
    if (!ctx) return FZ_EINVAL;
    ctx->err.clear();
    ctx->last_words = 0;
    int prev = 0;
    if (hipGetDevice(&prev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(ctx, FZ_EDEVICE, "hipGetDevice failed");
    }
    if (prev != ctx->device && hipSetDevice(ctx->device) != hipSuccess) {
        (void)hipGetLastError();
        return fail(ctx, FZ_EDEVICE, "hipSetDevice(%d) failed", ctx->device);
    }
    const int rc = rounds_impl(ctx, target, target_len, query, query_len, seeds, n_seeds, scoring, matrix, ydrop,
                               min_traceback_score, flags, round_size, hits, cigar, cigar_words, stats,
                               (hipStream_t)stream);
    if (prev != ctx->device) (void)hipSetDevice(prev);
    return rc;
}

int fz_extend_batch(fz_ctx *ctx, const uint8_t *target, uint64_t target_len, const uint8_t *query, uint64_t query_len,
                    const fz_seed *seeds, uint64_t n_seeds, const fz_scoring *scoring, const fz_matrix *matrix,
                    int32_t ydrop,
                    int64_t min_traceback_score, uint32_t flags, fz_hit *hits, const uint32_t **cigar,
                    uint64_t *cigar_words, fz_stats *stats, void *stream)
{
    if (!ctx) return FZ_EINVAL;
    ctx->err.clear();
    ctx->last_words = 0;
    int prev = 0;
    if (hipGetDevice(&prev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(ctx, FZ_EDEVICE, "hipGetDevice failed");
    }
    if (prev != ctx->device && hipSetDevice(ctx->device) != hipSuccess) {
        (void)hipGetLastError();
        return fail(ctx, FZ_EDEVICE, "hipSetDevice(%d) failed", ctx->device);
    }
    const int rc = extend_impl(ctx, target, target_len, query, query_len, seeds, n_seeds, scoring, matrix, ydrop,
                               min_traceback_score, flags, hits, cigar, cigar_words, stats, (hipStream_t)stream);
    if (prev != ctx->device) (void)hipSetDevice(prev);
    return rc;
}

int fz_extend_batch_noalloc(fz_ctx *ctx, const uint8_t *target, uint64_t target_len, const uint8_t *query,
                            uint64_t query_len, const fz_seed *seeds, uint64_t n_seeds, const fz_scoring *scoring,
                            const fz_matrix *matrix, int32_t ydrop, uint32_t flags, fz_hit *hits, fz_stats *stats,
                            void *stream)
{
    if (!ctx) return FZ_EINVAL;
    ctx->err.clear();
    int prev = 0;
    if (hipGetDevice(&prev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(ctx, FZ_EDEVICE, "hipGetDevice failed");
    }
    if (prev != ctx->device && hipSetDevice(ctx->device) != hipSuccess) {
        (void)hipGetLastError();
        return fail(ctx, FZ_EDEVICE, "hipSetDevice(%d) failed", ctx->device);
    }
    const int rc = noalloc_impl(ctx, target, target_len, query, query_len, seeds, n_seeds, scoring, matrix, ydrop,
                                flags, hits, stats, (hipStream_t)stream);
    if (prev != ctx->device) (void)hipSetDevice(prev);
    return rc;
}

int fz_find_seeds(fz_ctx *ctx, const uint8_t *target, uint64_t target_len, const uint8_t *query, uint64_t query_len,
                  uint32_t k, int64_t flank, uint32_t flags, const fz_seed **seeds, uint64_t *n_seeds,
                  uint64_t *n_hits, fz_seed_stats *stats, void *stream)
{
    if (!ctx) return FZ_EINVAL;
    ctx->err.clear();
    int prev = 0;
    if (hipGetDevice(&prev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(ctx, FZ_EDEVICE, "hipGetDevice failed");
    }
    if (prev != ctx->device && hipSetDevice(ctx->device) != hipSuccess) {
        (void)hipGetLastError();
        return fail(ctx, FZ_EDEVICE, "hipSetDevice(%d) failed", ctx->device);
    }
    const int rc = seeds_impl(ctx, target, target_len, query, query_len, k, flank, flags, seeds, n_seeds, n_hits,
                              stats, (hipStream_t)stream);
    if (prev != ctx->device) (void)hipSetDevice(prev);
    return rc;
}

int fz_copy_seeds(fz_ctx *ctx, fz_seed *dst, uint64_t n, void *stream)
{
    if (!ctx) return FZ_EINVAL;
    if (n > ctx->last_seeds) return fail(ctx, FZ_EINVAL, "asked for %llu seeds, the last seed stage found %llu",
                                         (unsigned long long)n, (unsigned long long)ctx->last_seeds);
    if (n == 0) return FZ_OK;
    if (!dst) return fail(ctx, FZ_EINVAL, "dst is NULL");
    hipStream_t st = (hipStream_t)stream;
    HIP_OK(hipMemcpyAsync(dst, ctx->sk_out.p, n * sizeof(fz_seed), hipMemcpyDeviceToDevice, st));
    HIP_OK(hipStreamSynchronize(st));
    return FZ_OK;
}

int fz_copy_cigar(fz_ctx *ctx, uint32_t *dst, uint64_t words, void *stream)
{
    if (!ctx) return FZ_EINVAL;
    if (words > ctx->last_words) return fail(ctx, FZ_EINVAL, "asked for %llu CIGAR words, last call made %llu",
                                             (unsigned long long)words, (unsigned long long)ctx->last_words);
    if (words == 0) return FZ_OK;
    if (!dst) return fail(ctx, FZ_EINVAL, "dst is NULL");
    hipStream_t st = (hipStream_t)stream;
    HIP_OK(hipMemcpyAsync(dst, ctx->cigar.p, words * sizeof(uint32_t), hipMemcpyDeviceToDevice, st));
    HIP_OK(hipStreamSynchronize(st));
    return FZ_OK;
}

}  // extern "C"

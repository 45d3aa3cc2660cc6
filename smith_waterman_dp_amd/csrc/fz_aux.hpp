// fz_aux.hpp -- staging, binning, scans, traceback walker and CIGAR assembly.
#pragma once

#include "../../include/fz.h"
#include "fz_device.hpp"

namespace fz {

// ------------------------------------------------------------------ pack --
// ASCII -> 2-bit codes (A0 C1 G2 T3) one per byte, forward and reversed,
// with PAD code-0 bases on both ends.  Any other byte raises *err.
__global__ void pack_kernel(const uint8_t *__restrict__ ascii, int64_t len, uint8_t *__restrict__ fwd,
                            uint8_t *__restrict__ rev, int64_t padded, uint32_t *err)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    bool bad = false;
    for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < padded; x += stride) {
        const int64_t s = x - PAD;
        uint8_t code = 0;
        if (s >= 0 && s < len) {
            const uint8_t c = ascii[s] & 0xDF;   // upper-case
            code = c == 'A' ? 0 : c == 'C' ? 1 : c == 'G' ? 2 : c == 'T' ? 3 : 255;
            if (code == 255) {
                bad = true;
                code = 0;
            }
        }
        fwd[x] = code;
        rev[padded - 1 - x] = code;
    }
    if (__ballot(bad) && lane_id() == 0) atomicOr(err, 1u);
}

__device__ __forceinline__ int sub_codes(int a, int b, const Scoring &sc)
{
    const int x = a ^ b;
    return x == 0 ? sc.match : (x == 2 ? sc.ts : sc.tv);
}

// ----------------------------------------------------------------- setup --
struct SeedInfo {
    int64_t seed_score;
    int64_t status;
};

__global__ void setup_kernel(const fz_seed *__restrict__ seeds, int64_t n, int64_t tlen, int64_t qlen,
                             const uint8_t *Tf, const uint8_t *Tr, const uint8_t *Qf, const uint8_t *Qr,
                             int64_t NT, int64_t NQ, Scoring sc, SideTask *__restrict__ tasks,
                             SeedInfo *__restrict__ info)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n) return;
    const fz_seed s = seeds[k];
    SideTask L = {}, R = {};
    L.seed = R.seed = (int32_t)k;
    L.side = 0;
    R.side = 1;
    L.m = L.n = R.m = R.n = -1;
    SeedInfo in = {0, 0};
    const int64_t Ls = s.seed_len;
    const bool ok = Ls >= 0 && s.t_lo >= 0 && s.q_lo >= 0 && s.t_hi <= tlen && s.q_hi <= qlen &&
                    s.t_pos >= s.t_lo && s.q_pos >= s.q_lo && s.t_pos + Ls <= s.t_hi && s.q_pos + Ls <= s.q_hi;
    if (!ok) {
        in.status = FZ_HIT_ESEED;
    } else {
        const int64_t ml = s.t_pos - s.t_lo, nl = s.q_pos - s.q_lo;
        const int64_t mr = s.t_hi - s.t_pos - Ls, nr = s.q_hi - s.q_pos - Ls;
        // worst case of any score reachable inside the windows must stay
        // far from the int32 sentinels
        int64_t msub = sc.match;
        msub = max(msub, (int64_t)(sc.ts < 0 ? -sc.ts : sc.ts));
        msub = max(msub, (int64_t)(sc.tv < 0 ? -sc.tv : sc.tv));
        const int64_t span = (s.t_hi - s.t_lo) + (s.q_hi - s.q_lo) + 2;
        if ((msub + sc.e) * span + sc.oe >= SCORE_LIMIT / 2) {
            in.status = FZ_HIT_ERANGE;
        } else {
            int64_t ss = 0;
            for (int64_t c = 0; c < Ls; ++c) ss += sub_codes(Tf[PAD + s.t_pos + c], Qf[PAD + s.q_pos + c], sc);
            in.seed_score = ss;
            L.A = Tr;
            L.abase = NT - 1 - PAD - s.t_pos;
            L.B = Qf;
            L.bbase = PAD + s.q_pos;
            L.m = (int32_t)ml;
            L.n = (int32_t)nl;
            R.A = Tf;
            R.abase = PAD + s.t_pos + Ls - 1;
            R.B = Qr;
            R.bbase = NQ - PAD - s.q_pos - Ls;
            R.m = (int32_t)mr;
            R.n = (int32_t)nr;
        }
    }
    tasks[2 * k] = L;
    tasks[2 * k + 1] = R;
    info[k] = in;
}

__device__ __forceinline__ int bin_of(int64_t len)
{
    int b = 0;
    int64_t edge = 512;
    while (len > edge && b < NBINS - 1) {
        edge *= 4;
        ++b;
    }
    return b;
}

// --------------------------------------------------------------- combine --
// Per seed: total score, coordinates, which sides need the executor, and a
// histogram of executor sides by (class, bin).  class 0 = sides done by the
// standard window, 1 = sides redone by the wide window.
struct CombineArgs {
    const fz_seed *seeds;
    int64_t n;
    const SideOut *out;
    const SeedInfo *info;
    int64_t min_tb;
    int32_t traceback;
    fz_hit *hits;
    int32_t *side_trace;        // per side: 0 none, 1 eager, 2 executor
    int64_t *run_cap;           // per side: run-word capacity (0 when not traced)
    uint32_t *bin_count;        // [2][NBINS]
    int64_t *max_ptr;           // max executor pointer bytes of one side
    int64_t *cells_total;       // canonical cells over the batch
};

__global__ void combine_kernel(CombineArgs a)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= a.n) return;
    const fz_seed s = a.seeds[k];
    const SeedInfo in = a.info[k];
    const SideOut L = a.out[2 * k], R = a.out[2 * k + 1];
    fz_hit h = {};
    h.bin = -1;
    int tr[2] = {0, 0};
    if (in.status) {
        h.status = in.status;
    } else if ((L.flags | R.flags) & SO_OVERFLOW) {
        h.status = FZ_HIT_EBAND;
    } else {
        h.score = (int64_t)L.score + in.seed_score + R.score;
        h.score_left = L.score;
        h.score_right = R.score;
        h.t_begin = s.t_pos - L.ie;
        h.q_begin = s.q_pos - L.je;
        h.t_end = s.t_pos + s.seed_len + R.ie;
        h.q_end = s.q_pos + s.seed_len + R.je;
        h.cells = L.cells + R.cells;
        atomicAdd((unsigned long long *)a.cells_total, (unsigned long long)h.cells);
        if (a.traceback) {
            if (h.score > a.min_tb) {
                h.status |= FZ_HIT_TRACED;
                const SideOut *sd[2] = {&L, &R};
                int64_t longest = -1;
                for (int q = 0; q < 2; ++q) {
                    if (sd[q]->flags & SO_EAGER) {
                        tr[q] = 1;
                        h.status |= q == 0 ? FZ_HIT_EAGER_LEFT : FZ_HIT_EAGER_RIGHT;
                    } else {
                        tr[q] = 2;
                        const int64_t len = max(sd[q]->ie, sd[q]->je);
                        const int cls = (sd[q]->flags & SO_WIDE_FLAG) ? 1 : 0;
                        atomicAdd(&a.bin_count[cls * NBINS + bin_of(len)], 1u);
                        atomicMax((unsigned long long *)a.max_ptr, (unsigned long long)sd[q]->ptr_bytes);
                        longest = max(longest, len);
                    }
                }
                if (longest >= 0) h.bin = bin_of(longest);
            } else {
                h.status |= FZ_HIT_BELOW_MIN;
            }
        }
    }
    for (int q = 0; q < 2; ++q) {
        const SideOut &o = q == 0 ? L : R;
        a.side_trace[2 * k + q] = tr[q];
        a.run_cap[2 * k + q] = tr[q] ? (int64_t)o.ie + o.je + 1 : 0;
    }
    a.hits[k] = h;
}

// Scatter executor sides by (class, bin): class 0 first, larger bins first.
__global__ void bin_scatter_kernel(int64_t nsides, const int32_t *side_trace, const SideOut *out,
                                   const uint32_t *bin_base, uint32_t *bin_fill, ExecItem *items)
{
    const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= nsides || side_trace[s] != 2) return;
    const SideOut o = out[s];
    const int cls = (o.flags & SO_WIDE_FLAG) ? 1 : 0;
    const int b = cls * NBINS + bin_of(max(o.ie, o.je));
    const uint32_t slot = bin_base[b] + atomicAdd(&bin_fill[b], 1u);
    ExecItem it;
    it.side = (int32_t)s;
    it.dstar = o.ie + o.je;
    it.ptr_off = 0;
    it.ptr_bytes = o.ptr_bytes;
    it.batch = 0;
    items[slot] = it;
}

// ------------------------------------------------------------------ scan --
// Exclusive scan of int64 values in three launches (block sums, scan of the
// block sums in one block, local scans).  Values are read through a strided
// view so that struct fields can be scanned in place.
constexpr int SCAN_BLOCK = 256;
constexpr int SCAN_ITEMS = 8;
constexpr int SCAN_TILE = SCAN_BLOCK * SCAN_ITEMS;

__device__ __forceinline__ int64_t block_exclusive_scan(int64_t v, int64_t *sh, int64_t &total)
{
    const int t = threadIdx.x;
    sh[t] = v;
    __syncthreads();
    for (int off = 1; off < SCAN_BLOCK; off <<= 1) {
        int64_t add = t >= off ? sh[t - off] : 0;
        __syncthreads();
        sh[t] += add;
        __syncthreads();
    }
    total = sh[SCAN_BLOCK - 1];
    const int64_t incl = sh[t];
    __syncthreads();
    return incl - v;
}

__global__ __launch_bounds__(SCAN_BLOCK) void scan_reduce_kernel(const int64_t *vals, int64_t stride, int64_t n,
                                                                  int64_t *block_sums)
{
    __shared__ int64_t sh[SCAN_BLOCK];
    const int64_t base = (int64_t)blockIdx.x * SCAN_TILE + (int64_t)threadIdx.x * SCAN_ITEMS;
    int64_t s = 0;
    for (int k = 0; k < SCAN_ITEMS; ++k)
        if (base + k < n) s += vals[(base + k) * stride];
    int64_t tot;
    block_exclusive_scan(s, sh, tot);
    if (threadIdx.x == 0) block_sums[blockIdx.x] = tot;
}

__global__ __launch_bounds__(SCAN_BLOCK) void scan_top_kernel(int64_t *block_sums, int64_t nblocks, int64_t *total)
{
    __shared__ int64_t sh[SCAN_BLOCK];
    int64_t carry = 0;
    for (int64_t base = 0; base < nblocks; base += SCAN_BLOCK) {
        const int64_t i = base + threadIdx.x;
        const int64_t v = i < nblocks ? block_sums[i] : 0;
        int64_t tot;
        const int64_t ex = block_exclusive_scan(v, sh, tot);
        if (i < nblocks) block_sums[i] = carry + ex;
        carry += tot;
    }
    if (threadIdx.x == 0) *total = carry;
}

__global__ __launch_bounds__(SCAN_BLOCK) void scan_apply_kernel(const int64_t *vals, int64_t stride, int64_t n,
                                                                 const int64_t *block_sums, int64_t *outv,
                                                                 int64_t ostride)
{
    __shared__ int64_t sh[SCAN_BLOCK];
    const int64_t base = (int64_t)blockIdx.x * SCAN_TILE + (int64_t)threadIdx.x * SCAN_ITEMS;
    int64_t v[SCAN_ITEMS];
    int64_t s = 0;
    for (int k = 0; k < SCAN_ITEMS; ++k) {
        v[k] = base + k < n ? vals[(base + k) * stride] : 0;
        s += v[k];
    }
    int64_t tot;
    int64_t run = block_sums[blockIdx.x] + block_exclusive_scan(s, sh, tot);
    for (int k = 0; k < SCAN_ITEMS; ++k) {
        if (base + k < n) outv[(base + k) * ostride] = run;
        run += v[k];
    }
}

// Batch of each executor item: pointer bytes are packed back to back; a
// batch holds the items whose start offset falls in [b * step, (b+1) * step),
// so it spans at most step + (largest item) bytes.
__global__ void batch_assign_kernel(ExecItem *items, int64_t n, int64_t step, int64_t *batch_first)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n) return;
    const int64_t b = items[k].ptr_off / step;
    const int64_t bp = k > 0 ? items[k - 1].ptr_off / step : -1;
    items[k].batch = b;
    for (int64_t q = bp + 1; q <= b; ++q) batch_first[q] = k;
}

__global__ void fill_i64_kernel(int64_t *p, int64_t n, int64_t v)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k < n) p[k] = v;
}

// Largest target and query window over the records (local mode sizing).
__global__ void window_max_kernel(const fz_seed *seeds, int64_t n, int64_t *out2)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n) return;
    const fz_seed s = seeds[k];
    atomicMax((long long *)&out2[0], (long long)(s.t_hi - s.t_lo));
    atomicMax((long long *)&out2[1], (long long)(s.q_hi - s.q_lo));
}

// ---------------------------------------------------------------- walker --
// Follow the executor's 4-bit pointers from the best cell back to (0,0),
// emitting run-length words end-first.  Pointer nibble: bits 0-1 source of
// S (0 diagonal, 1 I, 2 D), bit 2 "the I entering the right neighbour
// extends", bit 3 "the D entering the lower neighbour extends".
struct WalkArgs {
    const ExecItem *items;
    int64_t begin, end;
    const uint8_t *ptr_ws;
    int64_t ptr_base_off;
    int32_t C;
    const SideOut *out;
    const int64_t *run_off;
    uint32_t *runs;
    int64_t *run_len;
};

__device__ __forceinline__ void rle_push(uint32_t *runs, int64_t &n, uint32_t &cur_op, uint32_t &cur_len, uint32_t op)
{
    if (cur_len && op == cur_op) {
        ++cur_len;
        return;
    }
    if (cur_len) runs[n++] = (cur_len << 4) | cur_op;
    cur_op = op;
    cur_len = 1;
}

// Traceback walk (FastZ section 2.1, Fig. 3b; section 3.1.3) over the
// executor's pointer rows, one wave per side, 64 anti-diagonals at a time.
// The walk has no parallelism inside one extension (FastZ runs it one thread
// per extension), and a lane per side would pay two dependent memory round
// trips (row header, then pointer word) per step.  Here, for each
// chunk of anti-diagonals d - 63 .. d below the walk's current cell (i, j),
// lane r loads row d - 63 + r's header and the pointer words the walk can
// reach on it (i never grows, and falls by at most one per anti-diagonal)
// into LDS; the wave then walks the chunk from LDS in uniform control flow.
constexpr int WALK_CHUNK = 64;

template <int C>
__global__ __launch_bounds__(64) void walk_wave_kernel(WalkArgs a)
{
    constexpr int NW = (C + 7) / 8;                      // pointer words per lane per row
    constexpr int WPR = (WALK_CHUNK / C + 2) * NW;       // words staged per row
    __shared__ uint32_t wl[WALK_CHUNK][WPR];
    __shared__ int32_t w0l[WALK_CHUNK];                  // first staged word (relative to the row)
    __shared__ int32_t ibl[WALK_CHUNK];                  // i of the row's first stored position
    __shared__ int32_t nwl[WALK_CHUNK];                  // words stored in the row
    const int lane = lane_id();
    const int64_t k = a.begin + (int64_t)blockIdx.x;
    if (k >= a.end) return;
    const ExecItem it = a.items[k];
    const SideOut o = a.out[it.side];
    const uint8_t *base = a.ptr_ws + (it.ptr_off - a.ptr_base_off);
    const RowHdr *hdr = reinterpret_cast<const RowHdr *>(base);
    const uint32_t *rows = reinterpret_cast<const uint32_t *>(base + 8 * ((int64_t)it.dstar + 1));
    uint32_t *runs = a.runs + a.run_off[it.side];
    const uint32_t total_rows = (uint32_t)((it.ptr_bytes - 8 * ((int64_t)it.dstar + 1)) / 4);

    // states: 0 = S; 1 = arrived in I (continue if the cell's bit 2 says
    // the gap extends); 2 = arrived in D (bit 3)
    int i = o.ie, j = o.je, st = 0;
    bool bad = i < 0 || j < 0 || i + j > it.dstar;
    int64_t n = 0, moves = 0;
    uint32_t cop = 0, clen = 0;
    const int64_t limit = (int64_t)o.ie + o.je;
    auto emit = [&](uint32_t op) {
        if (clen && op == cop) {
            ++clen;
            return;
        }
        if (clen && lane == 0) runs[n] = (clen << 4) | cop;
        if (clen) ++n;
        cop = op;
        clen = 1;
    };
    while (!bad && !(st == 0 && i == 0 && j == 0)) {
        const int d = i + j;
        const int dlo = max(0, d - (WALK_CHUNK - 1));
        {
            const int dr = dlo + lane;
            if (dr <= d) {
                const RowHdr h = hdr[dr];
                // (clamped to the side's rows, so that no header value can
                // send a read outside them)
                const uint32_t row_end = min(dr < it.dstar ? hdr[dr + 1].off : total_rows, total_rows);
                const int plo = max(0, i - (d - dr)) - h.ibase;
                const int w0 = plo <= 0 ? 0 : (plo / C) * NW;
                const int nw = row_end > h.off ? (int)(row_end - h.off) : 0;
#pragma unroll
                for (int q = 0; q < WPR; ++q) {
                    const int w = w0 + q;
                    wl[lane][q] = w < nw ? rows[h.off + (uint32_t)w] : 0u;
                }
                w0l[lane] = w0;
                ibl[lane] = h.ibase;
                nwl[lane] = nw;
            }
        }
        __syncthreads();
        // walk down to anti-diagonal dlo
        while (!(st == 0 && i == 0 && j == 0)) {
            const int dd = i + j;
            if (dd < dlo) break;
            const int r = dd - dlo;
            const int p = i - ibl[r];
            const int w = p < 0 ? -1 : (p / C) * NW + (p % C) / 8;
            const int q = w - w0l[r];
            if (p < 0 || w >= nwl[r] || q < 0 || q >= WPR || moves > limit) {
                bad = true;
                break;
            }
            const uint32_t x = (wl[r][q] >> (4 * ((p % C) % 8))) & 0xFu;
            if (st == 1 && (x & 4u)) {
                emit(1);
                --j;
            } else if (st == 2 && (x & 8u)) {
                emit(2);
                --i;
            } else {
                // the gap (if any) ends here: this cell is taken in S
                st = 0;
                if (i == 0 && j == 0) break;
                const uint32_t src = x & 3u;
                if (src == 0) {
                    emit(0);
                    --i;
                    --j;
                } else if (src == 1) {
                    emit(1);
                    --j;
                    st = 1;
                } else {
                    emit(2);
                    --i;
                    st = 2;
                }
            }
            ++moves;
            if (i < 0 || j < 0) {
                bad = true;
                break;
            }
        }
        __syncthreads();
    }
    if (clen && lane == 0) runs[n] = (clen << 4) | cop;
    if (clen) ++n;
    if (lane == 0) a.run_len[it.side] = (!bad && i == 0 && j == 0 && st == 0) ? n : -1;
}

// Eager sides: op bytes (end-first) -> run words (end-first).
__global__ void eager_runs_kernel(int64_t nsides, const int32_t *side_trace, const SideOut *out,
                                  const uint8_t *eager_ops, const int64_t *run_off, uint32_t *runs_all,
                                  int64_t *run_len)
{
    const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= nsides || side_trace[s] != 1) return;
    const int len = out[s].eager_len;
    if (len < 0) {
        run_len[s] = -1;
        return;
    }
    const uint8_t *ops = eager_ops + s * EAGER_OPS;
    uint32_t *runs = runs_all + run_off[s];
    int64_t n = 0;
    uint32_t cop = 0, clen = 0;
    for (int q = 0; q < len; ++q) rle_push(runs, n, cop, clen, ops[q]);
    if (clen) runs[n++] = (clen << 4) | cop;
    run_len[s] = n;
}

// -------------------------------------------------------------- assemble --
// CIGAR of a traced seed = left ops (already in forward order, since the
// left side runs backwards along the genome) + seed_len x M + right ops
// reversed; adjacent equal ops merge.
template <bool WRITE>
__device__ __forceinline__ int64_t assemble_one(const uint32_t *lr, int64_t nl, int64_t seed_len, const uint32_t *rr,
                                                int64_t nr, uint32_t *dst)
{
    int64_t n = 0;
    uint32_t cop = 0xFFFFFFFFu;
    uint64_t clen = 0;
    auto emit = [&](uint32_t op, uint64_t len) {
        if (len == 0) return;
        if (op == cop) {
            clen += len;
            return;
        }
        if (clen) {
            if (WRITE) dst[n] = (uint32_t)(clen << 4) | cop;
            ++n;
        }
        cop = op;
        clen = len;
    };
    for (int64_t q = 0; q < nl; ++q) emit(lr[q] & 15u, lr[q] >> 4);
    emit(0u, (uint64_t)seed_len);
    for (int64_t q = nr - 1; q >= 0; --q) emit(rr[q] & 15u, rr[q] >> 4);
    if (clen) {
        if (WRITE) dst[n] = (uint32_t)(clen << 4) | cop;
        ++n;
    }
    return n;
}

struct AssembleArgs {
    const fz_seed *seeds;
    int64_t n;
    const int64_t *run_off;
    const int64_t *run_len;
    const uint32_t *runs;
    fz_hit *hits;
    int64_t *cig_len;           // count pass output / write pass input (offsets after scan)
    uint32_t *cigar;
    uint32_t *err;
};

template <bool WRITE>
__global__ void assemble_kernel(AssembleArgs a)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= a.n) return;
    fz_hit *h = &a.hits[k];
    if (!(h->status & FZ_HIT_TRACED)) {
        if (!WRITE) a.cig_len[k] = 0;
        else {
            h->cigar_off = 0;
            h->cigar_len = 0;
        }
        return;
    }
    const int64_t nl = a.run_len[2 * k], nr = a.run_len[2 * k + 1];
    if (nl < 0 || nr < 0) {
        if (!WRITE) {
            a.cig_len[k] = 0;
            atomicOr(a.err, 2u);
        } else {
            h->cigar_off = 0;
            h->cigar_len = 0;
        }
        return;
    }
    const uint32_t *lr = a.runs + a.run_off[2 * k];
    const uint32_t *rr = a.runs + a.run_off[2 * k + 1];
    if (!WRITE) {
        a.cig_len[k] = assemble_one<false>(lr, nl, a.seeds[k].seed_len, rr, nr, nullptr);
    } else {
        const int64_t off = a.cig_len[k];
        const int64_t cnt = assemble_one<true>(lr, nl, a.seeds[k].seed_len, rr, nr, a.cigar + off);
        h->cigar_off = off;
        h->cigar_len = cnt;
    }
}

}  // namespace fz

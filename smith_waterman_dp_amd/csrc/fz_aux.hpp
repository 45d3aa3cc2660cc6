// fz_aux.hpp -- staging, binning, scans, traceback walker and CIGAR assembly.
#pragma once

#include "../../include/fz.h"
#include "fz_device.hpp"

namespace fz {

// ------------------------------------------------------------------ pack --
// ASCII -> 2-bit codes (A0 C1 G2 T3) one per byte, forward and reversed,
// with PAD code-0 bases on both ends.  Any other byte raises *err.
// ASCII -> byte codes, forward and reversed, with PAD zero bytes on each
// side.  role 0: codes 0..3 for A, C, G, T (N is an error); role 1 / 2: the
// matrix mode's target / query codes (mx_target_code, the base itself),
// with N (either case) accepted as MX_N; role 3: codes 0..3 with N as MX_N
// (the seed stage).  revcomp: the reverse complement
// is coded instead (complement = base ^ 3 with A=0, C=1, G=2, T=3; N stays
// N).  Any other byte sets bit 0 of *err and is coded as A.
// With fwd16 (role 0 only), the same codes are also written as the 16-bit
// pairs of the packed layouts: target (2c, 2c + 1) when pk_query is 0,
// query (2c, 2c) when it is 1 (see pk_target_code, pk_query_code).
__global__ void pack_kernel(const uint8_t *__restrict__ ascii, int64_t len, uint8_t *__restrict__ fwd,
                            uint8_t *__restrict__ rev, int64_t padded, uint32_t *err, int revcomp, int role,
                            uint16_t *__restrict__ fwd16 = nullptr, uint16_t *__restrict__ rev16 = nullptr,
                            int pk_query = 0)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    bool bad = false;
    for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < padded; x += stride) {
        const int64_t s = x - PAD;
        uint32_t code = 0;
        if (s >= 0 && s < len) {
            const uint8_t c = ascii[revcomp ? len - 1 - s : s] & 0xDF;   // upper-case
            code = c == 'A' ? 0 : c == 'C' ? 1 : c == 'G' ? 2 : c == 'T' ? 3 : (c == 'N' && role) ? MX_N : 255;
            if (code == 255) {
                bad = true;
                code = 0;
            } else if (code != MX_N) {
                if (revcomp) code ^= 3;
                if (role == 1) code = mx_target_code(code);     // roles 2, 3: the base itself
            }
        }
        fwd[x] = (uint8_t)code;
        rev[padded - 1 - x] = (uint8_t)code;
        if (fwd16) {
            const uint16_t c2 = (uint16_t)((2u * code) | ((2u * code + (pk_query ? 0u : 1u)) << 8));
            fwd16[x] = c2;
            rev16[padded - 1 - x] = c2;
        }
    }
    if (__ballot(bad) && lane_id() == 0) atomicOr(err, 1u);
}


// ----------------------------------------------------------------- setup --
struct SeedInfo {
    int64_t seed_score;
    int64_t status;
};
// (the wide retry reads seed_score through ExtendArgs::info as int64 pairs)
static_assert(sizeof(SeedInfo) == 16 && offsetof(SeedInfo, seed_score) == 0, "SeedInfo layout");

// T16f .. Q16r: the 16-bit copies of the packed layouts (may be null when
// they are not used).
__global__ void setup_kernel(const fz_seed *__restrict__ seeds, int64_t n, int64_t tlen, int64_t qlen,
                             const uint8_t *Tf, const uint8_t *Tr, const uint8_t *Qf, const uint8_t *Qr,
                             int64_t NT, int64_t NQ, Scoring sc, SideTask *__restrict__ tasks,
                             SeedInfo *__restrict__ info, const uint8_t *T16f = nullptr,
                             const uint8_t *T16r = nullptr, const uint8_t *Q16f = nullptr,
                             const uint8_t *Q16r = nullptr, bool defer_on = false, int64_t min_tb = 0)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n) return;
    const fz_seed s = seeds[k];
    SideTask L = {}, R = {};
    L.seed = R.seed = (int32_t)k;
    L.side = 0;
    R.side = 1;
    L.m = L.n = R.m = R.n = -1;
    L.defer_need = R.defer_need = INT32_MAX;
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
        const int64_t msub = sc.msub;
        const int64_t span = (s.t_hi - s.t_lo) + (s.q_hi - s.q_lo) + 2;
        if ((msub + sc.e) * span + sc.oe >= SCORE_LIMIT / 2 || s.t_hi - s.t_lo > MAX_SIDE_LEN ||
            s.q_hi - s.q_lo > MAX_SIDE_LEN) {
            in.status = FZ_HIT_ERANGE;
        } else {
            int64_t ss = 0;
            for (int64_t c = 0; c < Ls; ++c) ss += sub_pair(Tf[PAD + s.t_pos + c], Qf[PAD + s.q_pos + c], sc);
            in.seed_score = ss;
            L.A = Tr;
            L.A16 = T16r;
            L.B16 = Q16f;
            L.abase = NT - 1 - PAD - s.t_pos;
            L.B = Qf;
            L.bbase = PAD + s.q_pos;
            L.m = (int32_t)ml;
            L.n = (int32_t)nl;
            R.A = Tf;
            R.A16 = T16f;
            R.B16 = Q16r;
            R.abase = PAD + s.t_pos + Ls - 1;
            R.B = Qr;
            R.bbase = NQ - PAD - s.q_pos - Ls;
            R.m = (int32_t)mr;
            R.n = (int32_t)nr;
            if (defer_on) {
                // a seed is traced when left + seed + right > min_tb, and
                // neither side scores below 0
                const int64_t need = min_tb - ss + 1;
                L.defer_need = R.defer_need = (int32_t)max<int64_t>(min<int64_t>(need, SCORE_LIMIT), -SCORE_LIMIT);
            }
        }
    }
    tasks[2 * k] = L;
    tasks[2 * k + 1] = R;
    info[k] = in;
}

// Classes of traced sides past the eager block, in the order of the
// executor's item list: one-pass sides (walked only), wide-window sides,
// standard ones.
enum : int { EXEC_CLASS_STD = 0, EXEC_CLASS_WIDE = 1, EXEC_CLASS_ONEPASS = 2, EXEC_CLASSES = 3 };
__device__ __forceinline__ int exec_class(int32_t flags)
{
    return (flags & SO_ONEPASS) ? EXEC_CLASS_ONEPASS : (flags & SO_WIDE_FLAG) ? EXEC_CLASS_WIDE : EXEC_CLASS_STD;
}

constexpr int SHORT_BIN_LEN = 512;          // the shortest executor bin: sides of at most this length
__device__ __forceinline__ int bin_of(int64_t len)
{
    int b = 0;
    int64_t edge = SHORT_BIN_LEN;
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
    uint32_t *bin_count;        // [EXEC_CLASSES][NBINS]
    int64_t *max_ptr;           // max executor pointer bytes of one side
    int64_t *cells_total;       // canonical cells over the batch
    int64_t *max_band;          // widest range R_d over the batch
};

// Wave-wide sum and maximum (every lane of the wave takes part).
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v)
{
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
    for (int off = 32; off > 0; off >>= 1) v = max(v, (uint64_t)__shfl_xor(v, off, 64));
    return v;
}

// counts[key] += 1 for every active lane, with one atomic per distinct key
// in the wave; returns the counter's old value plus this lane's rank among
// the wave's lanes with the same key (every lane of the wave takes part).
__device__ __forceinline__ uint32_t wave_grouped_inc(uint32_t *counts, int key, bool active)
{
    const int lane = lane_id();
    uint32_t r = 0;
    uint64_t todo = ballot(active);
    while (todo) {
        const int leader = ctz64(todo);
        const int kk = __shfl(key, leader, 64);
        const bool mine = active && key == kk;
        const uint64_t grp = ballot(mine);
        uint32_t old = 0;
        if (lane == leader) old = atomicAdd(&counts[kk], (uint32_t)__popcll(grp));
        old = (uint32_t)__shfl((int)old, leader, 64);
        if (mine) r = old + (uint32_t)__popcll(grp & ((1ull << lane) - 1ull));
        todo &= ~grp;
    }
    return r;
}

__global__ void combine_kernel(CombineArgs a)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool valid = k < a.n;
    fz_hit h = {};
    h.bin = -1;
    int tr[2] = {0, 0};
    int bkey[2] = {0, 0};
    bool binned[2] = {false, false};
    uint64_t pmax = 0, bmax = 0;
    fz_seed s = {};
    SeedInfo in = {0, 0};
    SideOut L = {}, R = {};
    if (valid) {
        s = a.seeds[k];
        in = a.info[k];
        L = a.out[2 * k];
        R = a.out[2 * k + 1];
    }
    if (!valid) {
    } else if (in.status) {
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
        bmax = (uint64_t)max(L.max_band, R.max_band);
        if ((L.flags | R.flags) & SO_WIDE_FLAG) h.status |= FZ_HIT_WIDE;
        if (a.traceback) {
            if (h.score > a.min_tb) {
                h.status |= FZ_HIT_TRACED;
                const SideOut *sd[2] = {&L, &R};
                int64_t longest = -1;
                for (int q = 0; q < 2; ++q) {
                    if (sd[q]->flags & SO_EAGER) {
                        tr[q] = 1;
                        h.status |= q == 0 ? FZ_HIT_EAGER_LEFT : FZ_HIT_EAGER_RIGHT;
                    } else if (sd[q]->flags & SO_WALKED) {
                        tr[q] = 3;      // walked already, runs in the one-pass buffer
                        longest = max(longest, (int64_t)max(sd[q]->ie, sd[q]->je));
                    } else {
                        tr[q] = 2;
                        const int64_t len = max(sd[q]->ie, sd[q]->je);
                        const int cls = exec_class(sd[q]->flags);
                        bkey[q] = cls * NBINS + bin_of(len);
                        binned[q] = !(sd[q]->flags & SO_EARLY);     // (early sides: walked from their own list)
                        // (one-pass and early sides have their rows already)
                        if (cls != EXEC_CLASS_ONEPASS && binned[q]) pmax = max(pmax, (uint64_t)sd[q]->ptr_bytes);
                        longest = max(longest, len);
                    }
                }
                if (longest >= 0) h.bin = bin_of(longest);
            } else {
                h.status |= FZ_HIT_BELOW_MIN;
            }
        }
    }
    // totals with one atomic per wave (per bin: per distinct bin)
    const uint64_t csum = wave_sum_u64((uint64_t)h.cells);
    const uint64_t cmax = wave_max_u64(pmax);
    const uint64_t wmax = wave_max_u64(bmax);
    if (lane_id() == 0) {
        if (csum) atomicAdd((unsigned long long *)a.cells_total, (unsigned long long)csum);
        if (cmax) atomicMax((unsigned long long *)a.max_ptr, (unsigned long long)cmax);
        if (wmax) atomicMax((unsigned long long *)a.max_band, (unsigned long long)wmax);
    }
    for (int q = 0; q < 2; ++q) (void)wave_grouped_inc(a.bin_count, bkey[q], tr[q] == 2 && binned[q]);
    if (!valid) return;
    for (int q = 0; q < 2; ++q) {
        const SideOut &o = q == 0 ? L : R;
        a.side_trace[2 * k + q] = tr[q];
        a.run_cap[2 * k + q] = (tr[q] == 1 || tr[q] == 2) ? (int64_t)o.ie + o.je + 1 : 0;
    }
    a.hits[k] = h;
}

// Scatter executor sides by (class, bin): class 0 first, larger bins first.
// shrink_words > 0 (failure injection only) gives every side that many
// fewer pointer-row words than the inspector sized, at least one.
__global__ void bin_scatter_kernel(int64_t nsides, const int32_t *side_trace, const SideOut *out,
                                   const uint32_t *bin_base, uint32_t *bin_fill, ExecItem *items,
                                   int64_t shrink_words)
{
    const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    bool active = s < nsides && side_trace[s] == 2;
    SideOut o = {};
    int b = 0;
    if (active) {
        o = out[s];
        active = !(o.flags & SO_EARLY);         // (as the combine counted)
        b = exec_class(o.flags) * NBINS + bin_of(max(o.ie, o.je));
    }
    const uint32_t r = wave_grouped_inc(bin_fill, b, active);     // every lane of the wave
    if (!active) return;
    const uint32_t slot = bin_base[b] + r;
    ExecItem it;
    it.side = (int32_t)s;
    it.dstar = o.ie + o.je;
    it.ptr_off = 0;
    it.ptr_bytes = (o.flags & SO_ONEPASS) ? 0 : o.ptr_bytes;    // (one-pass rows are in the pool)
    if (shrink_words > 0 && !(o.flags & SO_ONEPASS)) {
        const int64_t hdr_bytes = 8 * ((int64_t)it.dstar + 1);
        it.ptr_bytes = max(hdr_bytes + 4, it.ptr_bytes - 4 * shrink_words);
    }
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

// Walk items of the one-pass sides in done[0, n) (walked before the pool is
// used again): the best cell's anti-diagonal, the side's run capacity
// (ie + je + 1, into ptr_bytes, scanned into ptr_off), SO_WALKED set.
__global__ void op_items_kernel(const int32_t *done, int64_t n, SideOut *out, ExecItem *items)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n) return;
    const int32_t s = done[k];
    SideOut o = out[s];
    ExecItem it;
    it.side = s;
    it.dstar = o.ie + o.je;
    it.ptr_off = 0;
    // (a tail-walked side has its runs already: no scratch)
    it.ptr_bytes = (o.flags & SO_TAIL) ? 0 : (int64_t)o.ie + o.je + 1;
    it.batch = 0;
    items[k] = it;
    out[s].flags = o.flags | SO_WALKED;
}

// The walked sides' run counts (a walk that failed counts 0) into the
// items' batch field, to be scanned into compact offsets.
__global__ void op_run_count_kernel(ExecItem *items, int64_t n, const int64_t *run_len)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k < n) items[k].batch = max(run_len[items[k].side], (int64_t)0);
}

// Copy each walked side's runs from the round's scratch (at its item's
// ptr_off, capacity ie + je + 1), or from the tail buffer for a side the tail
// walk took (at op_run_off), to the one-pass runs buffer, packed (at base +
// the scanned count, kept in the item's ptr_bytes field).
__global__ void op_run_pack_kernel(const ExecItem *items, int64_t n, const uint32_t *scratch,
                                   const uint32_t *tail_runs, SideOut *out, uint32_t *runs, int64_t base,
                                   int64_t *op_run_off)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n) return;
    const ExecItem it = items[k];
    const int64_t dst = base + it.ptr_bytes;
    const int32_t fl = out[it.side].flags;
    const uint32_t *src = (fl & SO_TAIL) ? tail_runs + op_run_off[it.side] : scratch + it.ptr_off;
    for (int64_t q = 0; q < it.batch; ++q) runs[dst + q] = src[q];
    op_run_off[it.side] = dst;
    if (fl & SO_TAIL) out[it.side].flags = fl & ~SO_TAIL;
}

// Traced sides the inspector finished that are longer than the shortest
// executor bin join the one-pass executor's list: there they are swept once
// more with their rows among the other one-pass sides, longest first,
// instead of as two-pass executor waves that end a batch alone, and walked
// with them.  A seed with a deferred side is certain to be traced; one whose
// sides both finished is traced when its score passes min_tb (as the
// combine decides).  Seeds with an overflowed side (its wide retry still to
// come) are left to the two-pass path.
__global__ void onepass_pick_kernel(int64_t n, const SeedInfo *__restrict__ info, SideOut *__restrict__ out,
                                    const SideTask *__restrict__ tasks, int64_t min_tb, int32_t min_len,
                                    int32_t *__restrict__ defer_list, uint32_t *__restrict__ defer_count,
                                    unsigned long long *__restrict__ defer_diags)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n || info[k].status) return;
    const SideOut L = out[2 * k], R = out[2 * k + 1];
    if ((L.flags | R.flags) & (SO_OVERFLOW | SO_SKIPPED)) return;
    const bool traced = ((L.flags | R.flags) & SO_DEFERRED) ||
                        (int64_t)L.score + info[k].seed_score + R.score > min_tb;
    if (!traced) return;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const SideOut &o = q ? R : L;
        if ((o.flags & (SO_DEFERRED | SO_EAGER)) || max(o.ie, o.je) <= min_len) continue;
        const int64_t sid = 2 * k + q;
        out[sid].flags = SO_DEFERRED;
        defer_list[atomicAdd(defer_count, 1u)] = (int32_t)sid;
        atomicAdd(defer_diags, (unsigned long long)((int64_t)tasks[sid].m + tasks[sid].n + 1));
    }
}

// Sides the one-pass executor gave back (pool exhausted): the inspector
// takes them again and keeps them.
__global__ void undefer_kernel(const int32_t *list, int64_t n, SideTask *tasks)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k < n) tasks[list[k]].defer_need = INT32_MAX;
}

// ------------------------------------------- one-pass launch order --
// The one-pass executor's waves are latency-bound: a side of tens of
// thousands of anti-diagonals takes about as long alone on the machine as
// among others, so one started late ends the kernel long after the rest.
// Its sides go longest first, by a predicted length: how far homology runs
// along the side's diagonal.  The prediction follows the diagonal in steps
// of OP_TRACK_STEP bases, comparing windows of OP_TRACK_LEN bases of A with
// B: four windows a quarter step apart at offsets within 8 of the diagonal
// found so far, else two at offsets within OP_TRACK_WIDE (clusters of indels
// move the diagonal by tens of bases now and then); a window with
// OP_TRACK_HIT (OP_TRACK_HIT_WIDE) or more equal bases at some offset is
// homology there (the offset becomes the diagonal).  OP_TRACK_MISS steps in a row without homology end it (an
// alignment under a y-drop of thousands bridges shorter unrelated
// stretches; a long side predicted short costs more than the reverse), and
// so does the window's end.  The key is the predicted length in units of
// 4 steps.  Only the order of the sides depends on it, not any result.
constexpr int OP_TRACK_STEP = 256;
constexpr int OP_TRACK_LEN = 32;
constexpr int OP_TRACK_HIT = 17;            // 53% (random sequence: 25%), kept low: diverged stretches
                                            // still extend an alignment
constexpr int OP_TRACK_HIT_WIDE = 19;       // (8 times the offsets: fewer chance hits)
constexpr int OP_TRACK_MISS = 3;
constexpr int OP_TRACK_WIDE = 128;
constexpr int OP_TRACK_WIDE0 = 320;
constexpr int OP_TRACK_MAX = 64;            // steps (16 kb: longer sides all go first, early enough
                                            // that even the longest windows end with the rest)
constexpr int OP_KEYS = 64;

// Equal bases of a[0 .. OP_TRACK_LEN - 1] (A, ascending) and b[0], b[-1],
// .., b[-(OP_TRACK_LEN - 1)] (B, descending addresses), with 16-byte loads.
__device__ __forceinline__ int window_matches(const GlobalU8 *a, const GlobalU8 *b)
{
    constexpr int NW = OP_TRACK_LEN / 4;
    uint32_t va[NW], vb[NW];
#pragma unroll
    for (int h = 0; h < NW / 4; ++h) {
        load_unaligned<4>(a + 16 * h, *reinterpret_cast<uint32_t(*)[4]>(&va[4 * h]));
        load_unaligned<4>(b - (OP_TRACK_LEN - 1) + 16 * h, *reinterpret_cast<uint32_t(*)[4]>(&vb[4 * h]));
    }
    int cnt = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        // B's dword NW - 1 - w holds positions 4w + 3 .. 4w in memory order
        const uint32_t x = va[w] ^ __builtin_amdgcn_perm(0u, vb[NW - 1 - w], 0x00010203u);
        const uint32_t z = ~(((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x) & 0x80808080u;     // a byte's top bit: it is 0
        cnt += __builtin_popcount(z);
    }
    return cnt;
}

// One wave per side, OP_KEY_WAVES sides per workgroup (tiny workgroups
// would cap the resident waves below what hides the loads' latency).
constexpr int OP_KEY_WAVES = 4;
__global__ __launch_bounds__(64 * OP_KEY_WAVES) void op_key_kernel(const int32_t *__restrict__ list, int64_t n,
                                                                   const SideTask *__restrict__ tasks,
                                                                   uint8_t *__restrict__ key,
                                                                   uint32_t *__restrict__ hist)
{
    const int64_t k = (int64_t)blockIdx.x * OP_KEY_WAVES + uniform((int)(threadIdx.x / 64));
    if (k >= n) return;
    const int lane = lane_id();
    const SideTask t = tasks[list[k]];
    // base i of the side's A at A[i], base j of its B at B[-j] (1-based)
    const GlobalU8 *A = reinterpret_cast<const GlobalU8 *>(reinterpret_cast<uintptr_t>(t.A + t.abase));
    const GlobalU8 *B = reinterpret_cast<const GlobalU8 *>(reinterpret_cast<uintptr_t>(t.B + t.bbase));
    const int lim = min(t.m, t.n);
    const int g = lane >> 4, o = (lane & 15) - 8;
    // windows at i = x .. x + LEN - 1 and j = x + delta .. x + delta + LEN
    // - 1: in [1, lim] when x + LEN - 1 + |delta| <= lim and x + delta >= 1
    auto count = [&](int x, int delta) -> int {
        return x + delta >= 1 ? window_matches(A + x, B - (x + delta)) : 0;
    };
    int center = 0, steps = 0, miss = 0;
    for (int s = 1; s <= OP_TRACK_MAX; ++s) {
        const int xs = OP_TRACK_STEP * s;
        constexpr int Q = OP_TRACK_STEP / 4;
        // (the first step searches wider: the alignment may have opened a gap
        // of a few hundred bases near the seed)
        const int wide = s == 1 ? OP_TRACK_WIDE0 : OP_TRACK_WIDE;
        if (xs + 3 * Q + OP_TRACK_LEN + abs(center) + wide > lim) {
            steps = s;                  // the window's end
            break;
        }
        int delta = center + o;
        int c = count(xs + Q * g, delta);
        int best = c >= OP_TRACK_HIT ? c : 0, bdelta = delta;
        if (ballot(best > 0) == 0) {
            for (int d0 = -wide; d0 < wide; d0 += 64) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    delta = center + d0 + lane;
                    c = count(xs + 2 * Q * h, delta);
                    if (c >= OP_TRACK_HIT_WIDE && c > best) {
                        best = c;
                        bdelta = delta;
                    }
                }
            }
        }
        if (ballot(best > 0)) {
            // the offset of the most equal bases
            const int top = wave_max(best);
            center = __builtin_amdgcn_readlane(bdelta, ctz64(ballot(best == top)));
            steps = s;
            miss = 0;
        } else if (++miss == OP_TRACK_MISS) {
            break;
        }
    }
    if (lane == 0) {
        const int kk = min(OP_KEYS - 1, steps >> 2);
        key[k] = (uint8_t)kk;
        atomicAdd(&hist[kk], 1u);
    }
}

// list[k] to out in descending key order (hist: the keys' counts; cur:
// zeroed cursors; the order within a key is arbitrary).  Blocks of 256
// count their keys in LDS and take one range per key.
__global__ __launch_bounds__(256) void op_order_kernel(const int32_t *__restrict__ list, int64_t n,
                                                       const uint8_t *__restrict__ key,
                                                       const uint32_t *__restrict__ hist, uint32_t *__restrict__ cur,
                                                       int32_t *__restrict__ out)
{
    __shared__ uint32_t lcnt[OP_KEYS], lbase[OP_KEYS];
    const int tid = (int)threadIdx.x;
    if (tid < OP_KEYS) lcnt[tid] = 0;
    __syncthreads();
    const int64_t k = (int64_t)blockIdx.x * 256 + tid;
    int kk = -1;
    uint32_t lpos = 0;
    if (k < n) {
        kk = key[k];
        lpos = atomicAdd(&lcnt[kk], 1u);
    }
    __syncthreads();
    if (tid < OP_KEYS) {
        uint32_t base = 0;
        for (int b = OP_KEYS - 1; b > tid; --b) base += hist[b];
        lbase[tid] = lcnt[tid] ? base + atomicAdd(&cur[tid], lcnt[tid]) : 0u;
    }
    __syncthreads();
    if (kk >= 0) out[lbase[kk] + lpos] = list[k];
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
// Follow the executor's 4-bit pointers (PTR_* in fz_device.hpp) from the
// best cell back to (0,0), emitting run-length words end-first.
struct WalkArgs {
    const ExecItem *items;
    int64_t begin, end;
    const uint8_t *ptr_ws;
    int64_t ptr_base_off;
    const uint64_t *op_btab;    // one-pass sides (OP): each side's block table
    int32_t runs_by_item;       // a side's runs at runs + its item's ptr_off (else runs + run_off[side])
    SideOut *out;
    const int64_t *run_off;
    uint32_t *runs;
    int64_t *run_len;
    const int32_t *side_trace;  // (early list) items whose side is not traced through the executor are skipped
    // Tail walk (OP, tail_list set): wave k takes one-pass list entry
    // tail_list[k] if tail_fin[k] already says its side finished, takes
    // TAIL_RUNS(ie + je) run words of the tail buffer (runs, tail_cap words,
    // tail_used taken), and on success records run_len, op_run_off and
    // SO_TAIL.  A side it skips, cannot fit or cannot finish is walked later
    // as before.  The other OP walks skip SO_TAIL sides.
    const int32_t *tail_list;
    const uint32_t *tail_fin;
    unsigned long long *tail_used;
    uint64_t tail_cap;
    int64_t *op_run_off;
    uint32_t *tail_sides;       // sides the tail walk finished (stats)
};

// Before the tail walk: sets the flag that one-pass waves ending from now on
// read (they then write back their own L2), waits until it is acknowledged,
// then writes back the L2 of the XCD it runs on; launched with
// TAIL_FLUSH_GROUPS single-wave groups, which the dispatcher spreads over
// every XCD.  Sides that ended before the flag was set are then readable by
// the walk, which starts after this kernel has ended.
constexpr int TAIL_FLUSH_GROUPS = 64;
__global__ void tail_flush_kernel(uint32_t *flushed)
{
    if (threadIdx.x == 0) __hip_atomic_store(flushed, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Run words a tail walk may write for a side whose best cell is on
// anti-diagonal dstar: a CIGAR with more runs (a gap every 32 moves or so)
// is left to the walk after the executor, which has room for one run per move.
__device__ __forceinline__ int64_t TAIL_RUNS(int64_t dstar) { return min(dstar + 1, dstar / 32 + 256); }

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
// executor's pointer rows, one wave per side, 128 anti-diagonals at a time.
// The walk has no parallelism inside one extension (FastZ runs it one thread
// per extension), and a lane per side would pay two dependent memory round
// trips (row header, then pointer word) per step.  Here, for each chunk of
// anti-diagonals d - 127 .. d below the walk's current cell (i, j), lane l
// loads rows d - 127 + l and d - 63 + l: header, and the pointer words the
// walk can reach on the row (i never grows, and falls by at most one per
// anti-diagonal: on row d - k, positions i - k .. i), all loads in flight at
// once, into LDS.  The wave then
// walks the chunk from LDS in uniform control flow; a run of diagonal moves
// is taken in one round, lane l testing the l-th cell down the diagonal.
constexpr int WALK_LANES = 64;
constexpr int WALK_CHUNK = 2 * WALK_LANES;

// Rows hold 6 or 8 positions per word (RowHdr); position p of a row is in
// word p / cpw at nibble shift 4 * (cpw - 1 - p % cpw).
__device__ __forceinline__ int row_word(int p, bool cpw8) { return cpw8 ? (p >> 3) : p / 6; }
// bit offset of cell p's nibble in its word (formats at RowHdr)
__device__ __forceinline__ int row_shift(int p, bool cpw8, bool pk)
{
    if (!pk) return cpw8 ? 4 * (7 - (p & 7)) : 4 * (5 - p % 6);
    const int k = cpw8 ? (p & 7) : p % 6;
    return 16 * (k >> 2) + 8 * (k & 1) + 4 * ((k >> 1) & 1);
}

// OP: the side's rows are the one-pass executor's blocks (fz_device.hpp,
// OP_BLOCK), found through its block table; else one executor area.
template <bool OP>
__global__ __launch_bounds__(64) void walk_wave_kernel(WalkArgs a)
{
    constexpr int WPR = WALK_CHUNK / 6 + 2;              // words staged per row (at most)
    constexpr int WPR4 = (WPR + 3) / 4;                  // 16-byte loads per row
    static_assert(16 * WPR4 <= WALK_PAD + 4, "the row loads must stay within a pointer area's pad");
    __shared__ uint32_t wl[WALK_CHUNK][WPR];
    const int lane = lane_id();
    const int64_t k = a.begin + (int64_t)blockIdx.x;
    if (k >= a.end) return;
    const bool tail = OP && a.tail_list != nullptr;
    ExecItem it = {};
    SideOut o;
    int64_t cap = INT64_MAX;        // run words this walk may write
    uint64_t slot = 0;
    if (tail) {
        // (acquire: the executor wave's rows and result, written back past
        // its XCD's L2 before the flag, are read past this one's)
        const uint32_t fin = __hip_atomic_load(a.tail_fin + k, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
        if (uniform((int)fin) != 1) return;
        it.side = a.tail_list[k];
        o = a.out[it.side];
        if (o.flags & (SO_EXEC_MISMATCH | SO_TAIL)) return;
        it.dstar = o.ie + o.je;
        cap = TAIL_RUNS(it.dstar);
        if (lane == 0) slot = atomicAdd(a.tail_used, (unsigned long long)cap);
        slot = uniform64(slot);
        if (slot > a.tail_cap || (uint64_t)cap > a.tail_cap - slot) return;
    } else {
        it = a.items[k];
        if (a.side_trace && a.side_trace[it.side] != 2) return;
        o = a.out[it.side];
        if (OP && (o.flags & SO_TAIL)) return;      // (walked by the tail walk)
    }
    const uint8_t *base = OP ? nullptr : a.ptr_ws + (it.ptr_off - a.ptr_base_off);
    const RowHdr *hdr = reinterpret_cast<const RowHdr *>(base);
    const uint32_t *rows = OP ? nullptr : reinterpret_cast<const uint32_t *>(base + 8 * ((int64_t)it.dstar + 1));
    typedef __attribute__((address_space(1))) const uint64_t GlobalU64;
    GlobalU64 *btab = OP ? reinterpret_cast<GlobalU64 *>(a.op_btab[it.side]) : nullptr;
    uint32_t *runs = a.runs + (tail ? (int64_t)slot : a.runs_by_item ? it.ptr_off : a.run_off[it.side]);
    const uint32_t total_rows = OP ? OP_BLOCK_WORDS : (uint32_t)((it.ptr_bytes - 8 * ((int64_t)it.dstar + 1)) / 4);

    // states: 0 = S; 1 = arrived in I (continue if the cell's PTR_EXT_I
    // says the gap extends); 2 = arrived in D (PTR_EXT_D)
    if (o.flags & SO_EXEC_MISMATCH) {
        // the recompute disagreed with the inspector: its rows are not
        // trusted; the seed is reported without a CIGAR (FZ_HIT_EEXEC)
        if (lane == 0) a.run_len[it.side] = 0;
        return;
    }
    int i = o.ie, j = o.je, st = 0;
    bool bad = i < 0 || j < 0 || i + j > it.dstar || total_rows == 0 || (OP && !btab);
    int64_t n = 0, moves = 0;
    uint32_t cop = 0, clen = 0;
    const int64_t limit = (int64_t)o.ie + o.je;
    auto emit = [&](uint32_t op, uint32_t cnt) {
        if (clen && op == cop) {
            clen += cnt;
            return;
        }
        if (clen && lane == 0 && n < cap) runs[n] = (clen << 4) | cop;
        if (clen) ++n;
        cop = op;
        clen = cnt;
    };
    // the staged pointer nibble of cell (ii, dd - ii) on chunk row r, or 16
    // when the row does not hold it (fields of row r live in lane r % 64;
    // the row's format flags are the top two bits of ib8 (ROW_CPW8, ROW_PK),
    // ib8 & ROW_OFF_MASK its ibase biased by 2^29)
    auto nib_at = [&](int r, int ii, int ib8, int w0, int nw) -> uint32_t {
        const bool cpw8 = ((uint32_t)ib8 & ROW_CPW8) != 0, pk = ((uint32_t)ib8 & ROW_PK) != 0;
        const int p = ii - ((int)((uint32_t)ib8 & ROW_OFF_MASK) - (1 << 29));
        if (p < 0) return 16u;
        const int w = row_word(p, cpw8);
        const int q = w - w0;
        if (w >= nw || q < 0 || q >= WPR) return 16u;
        // (packed rows hold PTR_DIAG and PTR_FROM_I inverted)
        return ((wl[r][q] >> row_shift(p, cpw8, pk)) & 0xFu) ^ (pk ? (PTR_DIAG | PTR_FROM_I) : 0u);
    };
    // one-pass blocks: lane k < 8 holds the address of block pf_b0 + k,
    // loaded one chunk ahead (a chunk's rows lie in at most three blocks)
    uint64_t pf = 0;
    int pf_b0 = -(1 << 30);
    while (!bad && !(st == 0 && i == 0 && j == 0)) {
        const int d = i + j;
        const int dlo = max(0, d - (WALK_CHUNK - 1));
        int rib[2] = {0, 0}, rw0[2] = {0, 0}, rnw[2] = {0, 0};
        uint64_t cur = 0;
        int cur_b0 = 0;
        if constexpr (OP) {
            const int b0 = dlo / OP_BLOCK, bmax = it.dstar / OP_BLOCK;
            if (b0 < pf_b0 || d / OP_BLOCK > pf_b0 + 7) {
                // (the first chunk, or a walk that left the prefetched range)
                pf = (lane < 8 && b0 + lane <= bmax) ? btab[b0 + lane] : 0;
                pf_b0 = b0;
            }
            cur = pf;
            cur_b0 = pf_b0;
            // the next chunk ends below dlo and starts at or above dlo - 128
            const int nb0 = max(0, dlo - WALK_CHUNK) / OP_BLOCK;
            pf = (lane < 8 && nb0 + lane <= bmax) ? btab[nb0 + lane] : 0;
            pf_b0 = nb0;
        }
        {
            // both rows' headers, then every word load of both rows, then
            // the LDS stores: two memory round trips per chunk (one-pass
            // blocks: the block addresses come from the chunk before)
            RowHdr h[2];
            uint32_t rend[2];
            const uint32_t *rb[2] = {rows, rows};
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                // rows past d are not needed: they read row d's header,
                // unconditionally (no divergent branch between the loads)
                const int dr = min(dlo + h2 * WALK_LANES + lane, d);
                if constexpr (OP) {
                    // the block's headers hold one more slot, the block's
                    // word count, so the next header is the row's end also
                    // for the block's last row (and the side's)
                    const int src = dr / OP_BLOCK - cur_b0;      // 0..2
                    const uint32_t alo = (uint32_t)__shfl((int)(uint32_t)cur, src);
                    const uint32_t ahi = (uint32_t)__shfl((int)(uint32_t)(cur >> 32), src);
                    const uint64_t blk = ((uint64_t)ahi << 32) | alo;
                    GlobalU64 *bh = reinterpret_cast<GlobalU64 *>(blk);
                    const int q = dr & (OP_BLOCK - 1);
                    const uint64_t h0 = bh[q], h1 = bh[q + 1];
                    h[h2].off = (uint32_t)h0;
                    h[h2].ibase = (int32_t)(h0 >> 32);
                    rend[h2] = min((uint32_t)h1 & ROW_OFF_MASK, total_rows);
                    rb[h2] = reinterpret_cast<const uint32_t *>(blk + 8 * OP_HDRS);
                } else {
                    h[h2] = hdr[dr];
                    // (clamped to the side's rows, so that no header value
                    // can send a read outside them)
                    const uint32_t next_off = hdr[min(dr + 1, it.dstar)].off & ROW_OFF_MASK;
                    rend[h2] = min(dr < it.dstar ? next_off : total_rows, total_rows);
                }
            }
            uint32_t v[2][WPR4 * 4];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int dr = dlo + h2 * WALK_LANES + lane;
                const bool cpw8 = (h[h2].off & ROW_CPW8) != 0;
                const uint32_t off = h[h2].off & ROW_OFF_MASK;
                const int plo = max(0, i - (d - dr)) - h[h2].ibase;
                rw0[h2] = plo <= 0 ? 0 : row_word(plo, cpw8);
                rnw[h2] = (dr <= d && rend[h2] > off) ? (int)(rend[h2] - off) : 0;
                // words past the highest reachable position (i never grows)
                // are never read: the row ends there for this chunk, and the
                // clamped loads below repeat its last word (cache hits)
                const int phi = i - h[h2].ibase;
                rnw[h2] = min(rnw[h2], phi < 0 ? 0 : row_word(phi, cpw8) + 1);
                // ibase biased by 2^29 (rows' ibase lies within +-2^29: sides
                // are at most MAX_SIDE_LEN long), the format flags above it
                rib[h2] = (int)((uint32_t)(h[h2].ibase + (1 << 29)) | (h[h2].off & (ROW_CPW8 | ROW_PK)));
                // 16-byte loads from the window's first word (the rows'
                // first word when the row has none in the window), all
                // issued before any is used: they reach at most 4 WPR4 - 1
                // words past a row's last word, which every pointer area
                // has after it (WALK_PAD)
                const uint32_t w0 = rw0[h2] < rnw[h2] ? off + (uint32_t)rw0[h2] : 0u;
                const GlobalU8 *src = reinterpret_cast<const GlobalU8 *>(reinterpret_cast<uintptr_t>(rb[h2] + w0));
#pragma unroll
                for (int g = 0; g < WPR4; ++g) {
                    uint32_t t[4];
                    load_unaligned<4>(src + 16 * g, t);
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[h2][4 * g + e] = t[e];
                }
            }
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int q = 0; q < WPR; ++q)
                    wl[h2 * WALK_LANES + lane][q] = rw0[h2] + q < rnw[h2] ? v[h2][q] : 0u;
        }
        __syncthreads();
        // Length of a run of one kind of move from the current cell (i, j)
        // on chunk row r: lane l tests cell (i - l di, j - l dj), on row
        // r - l (di + dj), for the pointer bit; the run ends at the first
        // cell without it, outside the chunk or the matrix, or (with
        // stop_at_origin) at (0,0).  Row r' has its fields in lane r' % 64.
        auto run_of = [&](int r, int di, int dj, uint32_t bit, bool stop_at_origin) -> int {
            const int rl = r - (di + dj) * lane;
            const int sl = rl < 0 ? 0 : rl;
            const int src_lane = sl % WALK_LANES;
            const int ib0 = __shfl(rib[0], src_lane), ib1 = __shfl(rib[1], src_lane);
            const int w00 = __shfl(rw0[0], src_lane), w01 = __shfl(rw0[1], src_lane);
            const int nw0 = __shfl(rnw[0], src_lane), nw1 = __shfl(rnw[1], src_lane);
            const bool lo_half = sl < WALK_LANES;
            const int lib = lo_half ? ib0 : ib1, lw0 = lo_half ? w00 : w01, lnw = lo_half ? nw0 : nw1;
            const int il = i - di * lane, jl = j - dj * lane;
            bool m = rl >= 0 && il >= 0 && jl >= 0 && !(stop_at_origin && il == 0 && jl == 0);
            if (m) {
                const uint32_t xl = nib_at(rl, il, lib, lw0, lnw);
                m = xl <= 15u && (xl & bit);
            }
            const uint64_t stop = ~ballot(m);
            return stop ? ctz64(stop) : WALK_LANES;
        };
        while (!(st == 0 && i == 0 && j == 0)) {
            const int dd = i + j;
            if (dd < dlo) break;
            const int r = dd - dlo;
            const int hr = r / WALK_LANES, lr = r % WALK_LANES;
            const int ib = __builtin_amdgcn_readlane(hr ? rib[1] : rib[0], lr);
            const int w0 = __builtin_amdgcn_readlane(hr ? rw0[1] : rw0[0], lr);
            const int nw = __builtin_amdgcn_readlane(hr ? rnw[1] : rnw[0], lr);
            const uint32_t x = (uint32_t)uniform((int)nib_at(r, i, ib, w0, nw));
            if (x > 15u || moves > limit) {
                bad = true;
                break;
            }
            // in a gap, the run of cells whose pointer extends it (lane 0
            // is this cell, so the run is empty exactly when the gap ends)
            const int g = st == 0 ? 0 : run_of(r, st == 2 ? 1 : 0, st == 1 ? 1 : 0, st == 1 ? PTR_EXT_I : PTR_EXT_D,
                                               false);
            if (g > 0) {
                emit((uint32_t)st, (uint32_t)g);
                if (st == 1) j -= g;
                else i -= g;
                moves += g;
            } else {
                // the gap (if any) ends here: this cell is taken in S
                st = 0;
                if (i == 0 && j == 0) break;
                const uint32_t src = ptr_src(x);
                if (src == 0) {
                    // diagonal moves from here, up to the first cell that is
                    // not a diagonal move, the origin, or the chunk's end
                    const int f = run_of(r, 1, 1, PTR_DIAG, true);
                    if (f == 0) {
                        bad = true;     // cannot happen; never loop without progress
                        break;
                    }
                    emit(0, (uint32_t)f);
                    i -= f;
                    j -= f;
                    moves += f;
                } else if (src == 1) {
                    emit(1, 1);
                    --j;
                    st = 1;
                    ++moves;
                } else {
                    emit(2, 1);
                    --i;
                    st = 2;
                    ++moves;
                }
            }
            if (i < 0 || j < 0) {
                bad = true;
                break;
            }
        }
        __syncthreads();
    }
    if (clen && lane == 0 && n < cap) runs[n] = (clen << 4) | cop;
    if (clen) ++n;
    const bool ok = !bad && i == 0 && j == 0 && st == 0;
    if (tail) {
        // (a side that did not fit its run words or did not reach the
        // origin is walked again after the executor, which reports it)
        if (ok && n <= cap && lane == 0) {
            a.run_len[it.side] = n;
            a.op_run_off[it.side] = (int64_t)slot;
            atomicOr(&a.out[it.side].flags, SO_TAIL);
            atomicAdd(a.tail_sides, 1u);
        }
        return;
    }
    if (lane == 0) a.run_len[it.side] = ok ? n : -1;
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
    const SideOut *out;
    int64_t n;
    const int64_t *run_off;
    const int64_t *run_len;
    const uint32_t *runs;
    const int64_t *op_run_off;  // SO_WALKED sides: their runs at op_runs + op_run_off[side]
    const uint32_t *op_runs;
    const uint32_t *tail_runs;  // SO_TAIL sides: at tail_runs + op_run_off[side]
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
    if (!WRITE && (h->status & FZ_HIT_TRACED) &&
        ((a.out[2 * k].flags | a.out[2 * k + 1].flags) & SO_EXEC_MISMATCH)) {
        // the executor disagreed with the inspector on a side: no CIGAR
        h->status = (h->status & ~(int64_t)FZ_HIT_TRACED) | FZ_HIT_EEXEC;
    }
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
    auto runs_of = [&](int64_t sd) -> const uint32_t * {
        const int32_t fl = a.out[sd].flags;
        return (fl & SO_TAIL) ? a.tail_runs + a.op_run_off[sd]
               : (fl & SO_WALKED) ? a.op_runs + a.op_run_off[sd] : a.runs + a.run_off[sd];
    };
    const uint32_t *lr = runs_of(2 * k);
    const uint32_t *rr = runs_of(2 * k + 1);
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

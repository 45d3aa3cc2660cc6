// fz_extend.hpp -- one-sided y-drop extension, one wave64 per side (gfx950).
//
// Used twice, as in the inspector-executor scheme of FastZ (SC'21, section 3):
//   inspector (EXEC = false): score only; finds the best cell, the canonical
//     cell count, the executor's pointer-memory size, and traces sides whose
//     best cell lies in the 16 x 16 corner at once (section 3.1.2);
//   executor  (EXEC = true):  recomputes the same band up to the best cell's
//     anti-diagonal and stores a 4-bit pointer per cell (section 3.1.3).
//
// Layout.  The wave works one anti-diagonal d = i + j at a time (FastZ
// section 2.2, observations (2) and (3)).  Cells of the current band sit at
// "positions" p = i - o_d, o_d = (d + K) >> 1, of a window of W = 64 * C
// positions: lane l holds positions l*C .. l*C + C - 1 in registers.  A
// position keeps its k = i - j from one diagonal to the next-but-one, so the
// diagonal predecessor (i-1, j-1) is the same register; the up and left
// predecessors are the same or the adjacent position, and only one value per
// diagonal crosses a lane boundary (one DPP move).  Three diagonals live in
// registers (S of d-1 and d-2, plus the gap states handed on from d-1): the
// circular use-and-discard buffer of section 3.2.  K is even, so
// o_d - o_(d-1) is 1 on even d and 0 on odd d; the loop is unrolled by two
// to make that a compile-time fact.  When the band nears a window edge the
// window slides by whole lanes; a band wider than the window sets
// SO_OVERFLOW and the side is redone by a wider instantiation.
//
// Per cell (positions are lane-private): H = S(d-2) + sub; S = max3(H, I, D);
// live iff S >= T_d; U = S - (O + E); the I handed right is max(I - E, U),
// the D handed down is max(D - E, U).  A dead cell only keeps S = -inf: its
// handed-on gap values are below T_d <= T_(d+1) and cannot revive a cell or
// tie a live one, so live values and traceback choices equal the definition
// where dead cells hold -inf in all three states.
#pragma once

#include "fz_device.hpp"

namespace fz {

struct ExtendArgs {
    const SideTask *tasks;
    const int32_t *list;        // inspector: side ids (NULL = identity); executor: unused
    int32_t nlist;
    const ExecItem *exec;       // executor items (EXEC only)
    int64_t exec_begin;         // executor batch [begin, begin + nlist) into exec
    uint8_t *ptr_ws;            // executor pointer workspace
    int64_t ptr_base_off;       // list offset that maps to ptr_ws[0] for this batch
    SideOut *out;
    uint8_t *eager_ops;         // EAGER_OPS bytes per side (op codes 0 M, 1 I, 2 D; end-first)
    int32_t *overflow_list;     // sides that outgrew the window
    uint32_t *overflow_count;
    int64_t *exec_cells;        // executor: cells recomputed (stats)
    int32_t result_flags;       // OR'ed into every inspector result (SO_WIDE_FLAG for the wide pass)
    // inspector: sides stopped for the one-pass executor (SO_DEFERRED)
    int32_t *defer_list;
    uint32_t *defer_count;
    unsigned long long *defer_diags;    // sum of their m + n + 1 (one-pass pool sizing)
    // one-pass executor: the pool its arenas come from, each side's block
    // table address (by side), and the sides it could not finish for lack of
    // pool (they go back to the inspector)
    uint8_t *op_pool;
    uint64_t op_pool_bytes;
    unsigned long long *op_pool_used;
    uint64_t *op_btab;
    int32_t *op_fail_list;
    uint32_t *op_fail_count;
    int32_t *op_done_list;      // ... and the sides it finished
    uint32_t *op_done_count;
    uint32_t *op_fin;           // (nullable) by list index: 1 once the side finished, its rows
                                // and result visible on every XCD (agent-scope release)
    uint32_t *op_last_started;  // (nullable, host memory) 1 once the list's last wave started
    const uint32_t *op_flushed; // 1 once the tail walk's flush began (tail_flush_kernel)
    // the wide retry beside the one-pass executor: a side whose seed is then
    // certain to be traced gets its rows in the same wave (SO_EARLY), in the
    // early workspace (early_bytes taken of early_cap), listed in early_items
    uint8_t *early_ws;
    uint64_t early_cap;
    unsigned long long *early_bytes;
    ExecItem *early_items;
    uint32_t *early_count;
    const void *info;           // the seeds' SeedInfo (seed scores)
    int64_t min_tb;
    Scoring sc;
};

template <int C, bool EXEC, int SUB>
struct SideDP {
    static constexpr bool SMALL = SUB != SUB_WIDE;       // one byte per substitution score
    static constexpr int W = 64 * C;
    static constexpr int NDW = (C + 3) / 4;             // dwords of bases per lane
    static constexpr int P0 = 32 * C;                   // position of (0,0): lane 32, slot 0
    static constexpr int EL0 = 32 - (8 + C - 1) / C;    // lanes holding the eager block
    static constexpr int EL1 = 32 + 8 / C;
    static constexpr int NEL = EL1 - EL0 + 1;
    static constexpr int NWORD = (C + 7) / 8;           // pointer words per lane per row (8 nibbles each)
    static constexpr bool PAIRED = C == 3;              // narrow layout: two lanes per pointer dword
    // an empty live hull: far outside every window, so that the range of the
    // next diagonal comes out empty or from the other hull alone
    static constexpr int NONE_LO = 1 << 29, NONE_HI = -(1 << 29);

    // registers
    int SA[C], SB[C], R[C], Dn[C];
    uint32_t TA[NDW], QB[NDW];          // bases under this lane's slots on the current diagonal
    uint32_t TAn[NDW], QBn[NDW];        // fetched ahead for the next update of each sequence
    const GlobalU8 *ba, *bb;            // wave-uniform bases, below every byte a window can touch
    uint32_t ua, ub;                    // offset of slot 0 of lane 0 from ba at o_d = 0 / from bb at o_d - d = 0
    // wave-uniform state
    int K, dmask;               // dmask: first d whose window reaches i > m or j > n
    int lo1, hi1, lo2, hi2;     // live hulls (positions) of d-1 and d-2
    int best, bi, bj, dend;
    int T;                      // y-drop threshold of the next diagonal
    int64_t cells, cum_bytes, ptr_at_best;  // totals up to diagonal dflush
    int dflush;
    int32_t acc_cells, acc_words;   // since dflush: sum of (|R_d| - 1), of (row words - NWORD)
    int32_t bmax;               // widest range so far, minus one
    bool overflow;
    // executor
    uint32_t rowoff, rowcap;    // rows written / rows the inspector sized
    RowHdr *hdr;
    uint32_t *rows;

    const SideTask &t;
    const Scoring &sc;
    int lane;

    __device__ SideDP(const SideTask &task, const Scoring &s) : t(task), sc(s), lane(fresh_lane_id()) {}

    __device__ __forceinline__ int sub_of(uint32_t X, uint32_t P, int c) const
    {
        if (SMALL) {
            return (int)(int8_t)((P >> (8 * (c & 3))) & 0xFF);
        } else {
            const uint32_t x = (X >> (8 * (c & 3))) & 3u;
            return x == 0 ? sc.match : (x == 2 ? sc.ts : sc.tv);
        }
    }

    // Sequence bytes.  Along the diagonals the target bytes under a lane move
    // by one every even d and the query bytes by one every odd d, so each
    // diagonal updates one sequence from dwords fetched two diagonals ahead.
    // NDW dwords from base + off + this lane's first slot (any byte offset:
    // one unaligned global load, which also completes in order); base and
    // off are wave-uniform.
    __device__ __forceinline__ void fetch(const GlobalU8 *base, uint32_t off, uint32_t (&out)[NDW]) const
    {
        load_unaligned<NDW>(base + (off + (uint32_t)(lane * C)), out);
    }

    // After a slide: this diagonal's bases at the new offset, and the
    // fetches for the next update of each sequence.
    __device__ __forceinline__ void reload(int d, int od)
    {
        fetch(ba, ua + od, TA);
        fetch(bb, ub + (od - d), QB);
        fetch(ba, ua + (od + 1), TAn);          // next even diagonal
        fetch(bb, ub + (od - d - 1), QBn);      // next odd diagonal
    }

    __device__ __forceinline__ void set_dmask()
    {
        // o_d = (d + K) >> 1 reaches m - W + 2 at d = 2(m - W + 2) - K;
        // d - o_d reaches n + 1 at d = 2n + 1 + K
        dmask = min(2 * (t.m - W + 2) - K, 2 * t.n + 1 + K);
    }

    // Evaluate diagonal d.  DELTA = o_d - o_(d-1); S of d-2 is in SN (and
    // is replaced by S of d).  Returns this lane's live slots as a bit mask.
    // With PTR, word[] receives this lane's C pointer nibbles, eight per word.
    template <int DELTA, bool PTR, bool MASKED>
    __device__ __forceinline__ int cells_of(int (&SN)[C], int T, int rlo, int rhi, int &dmax,
                                            uint32_t (&word)[NWORD])
    {
        uint32_t X[NDW], P[NDW];
#pragma unroll
        for (int k = 0; k < NDW; ++k) {
            if (SUB == SUB_MATRIX) {
                X[k] = 0u;
                P[k] = matrix_scores(TA[k] | QB[k], sc);
            } else {
                X[k] = TA[k] ^ QB[k];
                P[k] = SMALL ? __builtin_amdgcn_perm(0u, sc.lut, X[k]) : 0u;
            }
        }
        // the one value that crosses a lane boundary
        int cross;
        if (DELTA == 1) cross = from_next_lane(R[0], NEG);       // left of slot C-1 is next lane's slot 0
        else cross = from_prev_lane(Dn[C - 1], NEG);            // up of slot 0 is previous lane's slot C-1

#pragma unroll
        for (int k = 0; k < NWORD; ++k) word[k] = 0;
        dmax = NEG;
        int lm = 0;
        const int mbase = MASKED ? lane * C - rlo : 0;
        int Rn[C], Dnn[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int Iv = DELTA == 1 ? (c < C - 1 ? R[c + 1] : cross) : R[c];
            const int Dv = DELTA == 1 ? Dn[c] : (c > 0 ? Dn[c - 1] : cross);
            const int H = SN[c] + sub_of(X[c / 4], P[c / 4], c);
            int S = max(max(H, Iv), Dv);
            bool ok = S >= T;
            if (MASKED) {
                // rlo <= lane*C + c <= rhi, from a per-diagonal base (no
                // per-slot constants held across the loop)
                ok = ok && (uint32_t)(mbase + c) <= (uint32_t)(rhi - rlo);
            }
            lm |= ok ? (1 << c) : 0;
            const int Sk = ok ? S : NEG;
            const int U = Sk - sc.oe;
            const int Ie = Iv - sc.e, De = Dv - sc.e;
            Rn[c] = max(Ie, U);
            Dnn[c] = max(De, U);
            if (PTR) {
                uint32_t &wd = word[c / 8];
                wd = shift_in(wd, S == H);      // PTR_DIAG
                wd = shift_in(wd, S == Iv);     // PTR_FROM_I
                wd = shift_in(wd, Ie > U);      // PTR_EXT_I
                wd = shift_in(wd, De > U);      // PTR_EXT_D
            }
            SN[c] = Sk;
            dmax = max(dmax, Sk);
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
            R[c] = Rn[c];
            Dn[c] = Dnn[c];
        }
        return lm;
    }

    __device__ __forceinline__ void slide(int s)
    {
        // s > 0: lane l takes lane l+s's registers (window moves to larger i - j)
        while (s > 0) {
#pragma unroll
            for (int c = 0; c < C; ++c) {
                SA[c] = from_next_lane(SA[c], NEG);
                SB[c] = from_next_lane(SB[c], NEG);
                R[c] = from_next_lane(R[c], NEG);
                Dn[c] = from_next_lane(Dn[c], NEG);
            }
            --s;
        }
        while (s < 0) {
#pragma unroll
            for (int c = 0; c < C; ++c) {
                SA[c] = from_prev_lane(SA[c], NEG);
                SB[c] = from_prev_lane(SB[c], NEG);
                R[c] = from_prev_lane(R[c], NEG);
                Dn[c] = from_prev_lane(Dn[c], NEG);
            }
            ++s;
        }
    }

    // One anti-diagonal.  Returns false when the extension is over.
    template <int DELTA, bool PTR>
    __device__ __forceinline__ bool step(int d, int dstop, uint32_t *eager_lds)
    {
        if (EXEC && d > dstop) return false;
        int od = (d + K) >> 1;
        // This diagonal's bases, fetched two diagonals ago, and at once the
        // fetch for the next update of the same sequence; a full step of
        // work separates each fetch from its first use.  (A slide below
        // refetches everything.)
        if (DELTA == 1) {
#pragma unroll
            for (int k = 0; k < NDW; ++k) TA[k] = TAn[k];
            fetch(ba, ua + (od + 1), TAn);
        } else {
#pragma unroll
            for (int k = 0; k < NDW; ++k) QB[k] = QBn[k];
            fetch(bb, ub + (od - d - 1), QBn);
        }
        // R_d: cells with a possibly live predecessor (hulls of d-1 and d-2)
        int rlo = min(lo1 - DELTA, lo2);
        int rhi = max(hi1 - DELTA + 1, hi2);
        bool masked = false;
        // fast path: d < dmask and 0 <= rlo <= rhi <= W - 1, i.e. four
        // terms that are all non-negative (one sign test)
        if (((dmask - 1 - d) | rlo | (W - 1 - rhi) | (rhi - rlo)) < 0) {
            // Near a matrix edge, an empty range, or the band at a window
            // edge.  (Elsewhere R_d needs no clipping: its cells have
            // 0 <= i <= d by construction and the window lies inside
            // d - n <= i <= m.)
            const int vlo = max(0, d - t.n) - od, vhi = min(t.m, d) - od;
            rlo = max(rlo, vlo);
            rhi = min(rhi, vhi);
            if (rlo > rhi) return false;
            if (rlo < 0 || rhi > W - 1) {
                // slide by s lanes so that [rlo, rhi] fits, near the centre
                const int smin = floordiv(rhi - (W - 1) + C - 1, C), smax = floordiv(rlo, C);
                if (smin > smax) {
                    overflow = true;
                    return false;
                }
                int s = floordiv((rlo + rhi + 1) / 2 - W / 2, C);
                s = s < smin ? smin : (s > smax ? smax : s);
                slide(s);
                const int sh = s * C;
                K += 2 * sh;
                od += sh;
                lo1 -= sh; hi1 -= sh; lo2 -= sh; hi2 -= sh;
                rlo -= sh; rhi -= sh;
                set_dmask();
                reload(d, od);
            }
            // positions with i > m or j > n are the only ones that can pick
            // up a live value without being in R_d; mask explicitly only when
            // the window reaches them (cells with i < 0 or j < 0 only ever
            // see -inf)
            masked = (W - 1 + od > t.m) || (d - od > t.n);
        }
        int lm, dmax;
        uint32_t word[NWORD];
        // (the uniform branch keeps the range test out of the common path)
        if (masked) {
            if (DELTA == 1) lm = cells_of<DELTA, PTR, true>(SA, T, rlo, rhi, dmax, word);   // even d
            else lm = cells_of<DELTA, PTR, true>(SB, T, rlo, rhi, dmax, word);             // odd d
        } else {
            if (DELTA == 1) lm = cells_of<DELTA, PTR, false>(SA, T, rlo, rhi, dmax, word);
            else lm = cells_of<DELTA, PTR, false>(SB, T, rlo, rhi, dmax, word);
        }

        // live hull of d: lanes from the ballot, slots from the two edge lanes
        const uint64_t anyl = ballot(lm != 0);
        int lo = NONE_LO, hi = NONE_HI, llo = 0, lhi = -1;
        if (anyl) {
            llo = ctz64(anyl);
            lhi = hibit64(anyl);
            const uint32_t mlo = (uint32_t)__builtin_amdgcn_readlane(lm, llo);
            const uint32_t mhi = (uint32_t)__builtin_amdgcn_readlane(lm, lhi);
            lo = llo * C + __builtin_ctz(mlo);
            hi = lhi * C + (31 - __builtin_clz(mhi));
        }
        // Σ|R_d| and the pointer-row sizes, as 32-bit sums that flush()
        // folds into the totals (the per-diagonal constants are added there)
        acc_cells += rhi - rlo;
        bmax = max(bmax, rhi - rlo);
        // pointer row: the lanes of the live hull; with C = 3, lane pairs
        // share a dword so that rows keep the six-cells-per-dword format
        const int rlane0 = PAIRED ? (llo & ~1) : llo;
        const int nl1 = PAIRED ? (lhi >> 1) - (llo >> 1) : lhi - llo;     // row words / NWORD - 1
        const int nl = (nl1 + 1) * NWORD;
        if (!EXEC) acc_words += nl1;

        if (ballot(dmax > best)) {
            const int nb = uniform(wave_max(dmax));
            // first position holding it: each lane finds its first slot (this
            // diagonal's S is in the register it was written to), the ballot
            // the first lane
            int slot = C;
#pragma unroll
            for (int c = C - 1; c >= 0; --c) {
                const int Sv = DELTA == 1 ? SA[c] : SB[c];
                slot = Sv == nb ? c : slot;
            }
            const int fl = ctz64(ballot(slot < C));
            const int pbest = fl * C + __builtin_amdgcn_readlane(slot, fl);
            best = nb;
            T = max(best - sc.ydrop, T_FLOOR);
            bi = pbest + od;
            bj = d - bi;
            const int n = d - dflush;
            ptr_at_best = cum_bytes + 8 * (int64_t)n + 4 * NWORD * ((int64_t)acc_words + n);
        }

        if (EXEC) {
            if (rowoff + (uint32_t)nl > rowcap) {
                // the recompute disagrees with the inspector's sizing
                overflow = true;
                return false;
            }
            if (lane == 0) {
                RowHdr h;
                h.off = rowoff | (NWORD == 2 ? ROW_CPW8 : 0u);
                h.ibase = rlane0 * C + od;
                store_hdr(hdr + d, h.off, h.ibase);
            }
            if (PAIRED) {
                // the odd lane's three nibbles go under the even lane's
                const uint32_t odd = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)word[0], 0xB1, 0xF, 0xF, false);
                if (!(lane & 1) && lane >= rlane0 && lane <= lhi)
                    gstore(rows + rowoff + ((lane - rlane0) >> 1), (word[0] << 12) | odd);
            } else if (lane >= llo && lane <= lhi) {
#pragma unroll
                for (int k = 0; k < NWORD; ++k) gstore(rows + rowoff + (lane - llo) * NWORD + k, word[k]);
            }
            rowoff += (uint32_t)nl;
        } else if (PTR) {
            if (lane >= EL0 && lane <= EL1) {
#pragma unroll
                for (int k = 0; k < NWORD; ++k) eager_lds[(d * NEL + (lane - EL0)) * NWORD + k] = word[k];
            }
        }

        lo2 = lo1; hi2 = hi1;
        lo1 = lo; hi1 = hi;
        dend = d;
        return true;
    }

    // Fold the 32-bit sums of the diagonals after dflush, up to dend, into
    // the totals.
    __device__ __forceinline__ void flush()
    {
        const int n = dend - dflush;
        cells += (int64_t)acc_cells + n;
        cum_bytes += 8 * (int64_t)n + 4 * NWORD * ((int64_t)acc_words + n);
        acc_cells = 0;
        acc_words = 0;
        dflush = dend;
    }

    // Bases of the sequence arrays for this layout.  Window positions reach
    // i = o_d + p with o_d >= -W and p < W, and j <= n + W, so every byte
    // read lies at or above abase - W - 4 in A and bbase - n - W - 4 in B;
    // the bases sit 4-aligned below that (inside the padding of the
    // sequence arrays), and the per-lane offsets stay positive.
    __device__ __forceinline__ void init_bases()
    {
        const int64_t aoff = (t.abase - W - 8) & ~(int64_t)3;
        const int64_t boff = (t.bbase - (int64_t)t.n - W - 8) & ~(int64_t)3;
        ba = reinterpret_cast<const GlobalU8 *>(reinterpret_cast<uintptr_t>(t.A + aoff));
        bb = reinterpret_cast<const GlobalU8 *>(reinterpret_cast<uintptr_t>(t.B + boff));
        ua = (uint32_t)(t.abase - aoff);
        ub = (uint32_t)(t.bbase - boff);
    }

    // d = 0 and diagonal 1 (the executor), or diagonals 0..33 with the eager
    // pointers of 1..32 (the inspector).  Returns the next diagonal, which is
    // even, or -1 when the extension is over.  The executor's area holds
    // nhdr row headers (dstop + 1 when nhdr < 0), then the rows.
    __device__ int start(int dstop, uint32_t *eager_lds, uint8_t *ptr_base, int64_t ptr_bytes, int64_t nhdr = -1)
    {
        if (nhdr < 0) nhdr = (int64_t)dstop + 1;
#pragma unroll
        for (int c = 0; c < C; ++c) { SA[c] = NEG; SB[c] = NEG; R[c] = NEG; Dn[c] = NEG; }
        K = -W;
        set_dmask();
        init_bases();
        // d = 0: the single cell (0,0), S = 0, I = D = -inf
        if (lane == P0 / C) {
            SA[0] = 0;
            R[0] = -sc.oe;
            Dn[0] = -sc.oe;
        }
        lo1 = P0; hi1 = P0; lo2 = NONE_LO; hi2 = NONE_HI;
        best = 0; bi = 0; bj = 0; dend = 0;
        T = max(-sc.ydrop, T_FLOOR);
        cells = 1;
        cum_bytes = 8 + 4 * NWORD;
        ptr_at_best = cum_bytes;
        dflush = 0; acc_cells = 0; acc_words = 0;
        bmax = 0;
        overflow = false;
        rowoff = 0;
        {
            // diagonal 1 is odd: it takes its query bytes from QBn and keeps
            // the target bytes set here; diagonal 2 takes TAn
            const int od1 = (1 + K) >> 1;
            fetch(ba, ua + od1, TA);
            fetch(bb, ub + (od1 - 1), QBn);
            fetch(ba, ua + (od1 + 1), TAn);
        }
        if (EXEC) {
            hdr = reinterpret_cast<RowHdr *>(ptr_base);
            rows = reinterpret_cast<uint32_t *>(ptr_base + 8 * nhdr);
            if (lane == 0) {
                RowHdr h;
                h.off = 0;
                h.ibase = 0;         // lane 32 slot 0 is i = 0
                store_hdr(hdr, h.off, h.ibase);
            }
            if (lane == P0 / C) {
#pragma unroll
                for (int k = 0; k < NWORD; ++k) gstore(rows + k, 0u);   // (0,0): no gap extends through it
            }
            rowoff = NWORD;
            // (row offsets share their word with the format flags: a side
            // with more rows than they can address ends in a mismatch)
            rowcap = (uint32_t)min<int64_t>((ptr_bytes - 8 * nhdr) / 4, (int64_t)ROW_OFF_MASK);
            return step<0, EXEC>(1, dstop, eager_lds) ? 2 : -1;
        }
        if (lane >= EL0 && lane <= EL1) {
#pragma unroll
            for (int k = 0; k < NWORD; ++k) eager_lds[(lane - EL0) * NWORD + k] = 0u;
        }
        // diagonals 1..32 keep pointers for the eager block
        int d = 1;
        for (; d <= EAGER_ROWS - 1; d += 2) {
            if (!step<0, true>(d, dstop, eager_lds)) return -1;
            if (!step<1, true>(d + 1, dstop, eager_lds)) return -1;
        }
        return step<0, false>(d, dstop, eager_lds) ? d + 1 : -1;
    }

    // Width of the union of the live hulls of the last two diagonals (the
    // next range is at most 3 wider), or -1 when both are empty.
    __device__ __forceinline__ int hull_width() const
    {
        const int ul = min(lo1, lo2), uh = max(hi1, hi2);
        return ul <= uh ? uh - ul : -1;
    }

    // Layout switches (standard kernel only): a side in the 192-position
    // layout moves to the 384-position one when its band widens, and back
    // when it narrows again.
    // The test runs every 8 diagonals.  Each diagonal widens the union by at
    // most 2, so a band that passed the test at width <= 172 keeps every
    // range within 172 + 2*8 = 188 <= W - C positions until the next test,
    // which always fits the 192-position window (slides go by whole lanes).
    static constexpr int SWITCH_EVERY = 8;
    static constexpr int NARROW_FROM_D = 256;
    static constexpr int NARROW_ENTER = 157;     // union hull width to enter the narrow layout
    static constexpr int NARROW_LEAVE = 172;     // ... and to leave it

    template <bool SWITCHABLE>
    __device__ __forceinline__ bool want_switch(int d) const
    {
        if (!SWITCHABLE) return false;
        const int w = hull_width();
        if (C == 6) return d >= NARROW_FROM_D && w >= 0 && w <= NARROW_ENTER;
        return w > NARROW_LEAVE;
    }

    // Diagonals from d (even) on until the extension ends (returns -1) or,
    // with SWITCHABLE, the band calls for the other layout (returns the next
    // d, again even).
    template <bool SWITCHABLE>
    __device__ int advance(int d, int dstop, uint32_t *eager_lds)
    {
        if (SWITCHABLE) {
            // lane-derived constants of this layout are formed here, inside
            // the layout's own run, not once for the whole side (where both
            // layouts' sets would occupy registers at the same time)
            lane = fresh_lane_id();
        }
        for (;; d += 2) {
            if (!step<1, EXEC>(d, dstop, eager_lds)) return -1;
            if (!step<0, EXEC>(d + 1, dstop, eager_lds)) return -1;
            if (((d + 1) & (SWITCH_EVERY - 1)) == SWITCH_EVERY - 1) {
                flush();
                if (want_switch<SWITCHABLE>(d + 1)) return d + 2;
            }
        }
    }

    // Lane registers by position, for a change of layout.  Only the union
    // [ul, uh] of the last two live hulls is handed over: elsewhere S is
    // -inf, and the handed-on gap values come from dead cells, which lie
    // below the threshold and act as -inf (see the top of this file).  x
    // holds four arrays of XFER_W entries, indexed by position - ul.
    static constexpr int XFER_W = XFER_STRIDE;
    __device__ __forceinline__ void export_regs(uint32_t *x, int ul, int uh) const
    {
        // (an opaque base keeps per-slot position constants from being
        // computed once and held in registers through the whole side)
        const int q0 = fresh_lane_id() * C - ul;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int q = q0 + c;
            if ((uint32_t)q <= (uint32_t)(uh - ul)) {
                x[q] = (uint32_t)SA[c];
                x[XFER_W + q] = (uint32_t)SB[c];
                x[2 * XFER_W + q] = (uint32_t)R[c];
                x[3 * XFER_W + q] = (uint32_t)Dn[c];
            }
        }
    }

    // Take over from a side run in another layout after its diagonal dlast:
    // position q here is position q + s there (o_d grows by s for every d,
    // which keeps K even).
    template <class O>
    __device__ __forceinline__ void adopt(const O &o, int s, const uint32_t *x, int ul, int uh, int dlast)
    {
        const int q0 = fresh_lane_id() * C + s - ul;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const bool in = (uint32_t)(q0 + c) <= (uint32_t)(uh - ul);
            const int q = in ? q0 + c : 0;
            SA[c] = in ? (int)x[q] : NEG;
            SB[c] = in ? (int)x[XFER_W + q] : NEG;
            R[c] = in ? (int)x[2 * XFER_W + q] : NEG;
            Dn[c] = in ? (int)x[3 * XFER_W + q] : NEG;
        }
        auto mlo = [&](int v) { return v == NONE_LO ? v : v - s; };
        auto mhi = [&](int v) { return v == NONE_HI ? v : v - s; };
        K = o.K + 2 * s;
        lo1 = mlo(o.lo1); hi1 = mhi(o.hi1);
        lo2 = mlo(o.lo2); hi2 = mhi(o.hi2);
        best = o.best; bi = o.bi; bj = o.bj; dend = o.dend; T = o.T;
        cells = o.cells; cum_bytes = o.cum_bytes; ptr_at_best = o.ptr_at_best;
        dflush = o.dflush; acc_cells = 0; acc_words = 0;        // (the other side flushed)
        bmax = o.bmax;
        overflow = o.overflow;
        rowoff = o.rowoff; rowcap = o.rowcap; hdr = o.hdr; rows = o.rows;
        lane = fresh_lane_id();
        set_dmask();
        init_bases();
        reload(dlast, (dlast + K) >> 1);
    }

    // Walk the eager block from (bi, bj).  The whole wave walks in step (the
    // nibble read from LDS is broadcast to a scalar), so the walk is plain
    // uniform control flow; lane 0 stores the ops, end-first.
    __device__ int eager_walk(const uint32_t *eager_lds, uint8_t *ops) const
    {
        int i = bi, j = bj, st = 0, n = 0;
        auto nib = [&](int ii, int jj) -> uint32_t {
            const int dd = ii + jj;
            const int od0 = (dd - W) >> 1;     // no slide happens before diagonal 33
            const int p = ii - od0;
            const int l = p / C, c = p % C;
            const uint32_t wd = (uint32_t)uniform((int)eager_lds[(dd * NEL + (l - EL0)) * NWORD + c / 8]);
            return (wd >> ptr_shift<C>(c)) & 0xFu;
        };
        for (int guard = 0; guard < 2 * EAGER_OPS + 2; ++guard) {
            if ((st == 0 && i == 0 && j == 0) || n >= EAGER_OPS || i < 0 || j < 0) break;
            if (st == 0) {
                const uint32_t src = ptr_src(nib(i, j));
                if (src == 0) {
                    if (lane == 0) ops[n] = 0;
                    ++n;
                    --i;
                    --j;
                } else {
                    st = (int)src;
                }
            } else if (st == 1) {
                if (lane == 0) ops[n] = 1;
                ++n;
                if (--j < 0) break;
                st = (nib(i, j) & PTR_EXT_I) ? 1 : 0;
            } else {
                if (lane == 0) ops[n] = 2;
                ++n;
                if (--i < 0) break;
                st = (nib(i, j) & PTR_EXT_D) ? 2 : 0;
            }
        }
        return (st == 0 && i == 0 && j == 0) ? n : -1;
    }
};

// What a side's extension reports, from whichever layout finished it.
struct SideResult {
    int best, bi, bj, dend, band;
    int64_t cells, ptr_at_best;
    bool overflow;
    int state = 0;              // packed layouts: SidePk's END_* reason (deferred, pool exhausted)
    template <class DP>
    __device__ __forceinline__ void take(DP &dp)
    {
        dp.flush();
        best = dp.best; bi = dp.bi; bj = dp.bj; dend = dp.dend; band = dp.bmax + 1;
        cells = dp.cells; ptr_at_best = dp.ptr_at_best;
        overflow = dp.overflow;
    }
};

// Move a side between layouts after diagonal d - 1: the union of its last
// two hulls is centred in the new window.
template <class TO, class FROM>
__device__ __forceinline__ void switch_layout(TO &to, FROM &from, uint32_t *x, int d)
{
    from.flush();
    const int ul = min(from.lo1, from.lo2), uh = max(from.hi1, from.hi2);
    const int s = ((ul + uh) >> 1) - TO::W / 2;
    from.export_regs(x, ul, uh);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    to.adopt(from, s, x, ul, uh, d - 1);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// The layout a side starts in: in the standard kernel the 192-position one
// (every band starts as the single cell (0,0), and the eager block of
// diagonals 0..32 is at most 17 positions wide); a wide retry starts and
// stays in its own.
template <int C>
struct StartLayout {
    static constexpr int value = C == 6 ? 3 : C;
};

// One side, start to end.  In the standard kernel a side runs three cells
// per lane (192 positions) while its band is narrow and six per lane (384)
// while it is wide: it moves up when the band passes 172 positions and back
// down, from diagonal 256 on, when it narrows to 157 (the narrow layout
// does about half the work per diagonal).  The executor makes the same
// moves as the inspector, since they depend only on the hulls.
template <int C, bool EXEC, int SUB>
__device__ __forceinline__ SideResult run_side(const SideTask &task, const Scoring &sc, int dstop, uint32_t *eager_lds,
                                               uint32_t *xfer, uint8_t *ptr_base, int64_t ptr_bytes)
{
    SideResult r;
    if constexpr (C != 6) {
        SideDP<C, EXEC, SUB> dp(task, sc);
        const int d = dp.start(dstop, eager_lds, ptr_base, ptr_bytes);
        if (d >= 0) dp.template advance<false>(d, dstop, eager_lds);
        r.take(dp);
        return r;
    } else {
        SideDP<3, EXEC, SUB> dn(task, sc);
        SideDP<6, EXEC, SUB> dw(task, sc);
        int d = dn.start(dstop, eager_lds, ptr_base, ptr_bytes);
        if (d < 0) {
            r.take(dn);
            return r;
        }
        for (;;) {
            d = dn.template advance<true>(d, dstop, eager_lds);
            if (d < 0) {
                r.take(dn);
                return r;
            }
            switch_layout(dw, dn, xfer, d);
            d = dw.template advance<true>(d, dstop, eager_lds);
            if (d < 0) {
                r.take(dw);
                return r;
            }
            switch_layout(dn, dw, xfer, d);
        }
    }
}

}  // namespace fz

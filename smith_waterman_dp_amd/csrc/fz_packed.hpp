// fz_packed.hpp -- the extension's cell sweep with two cells per 32-bit lane
// register (gfx950 packed 16-bit integer VALU).
//
// The layouts here hold C = 2 * C2 positions per lane (C2 registers per
// state, two positions per register: the even one in the low half, the odd
// one in the high half), so one v_pk_* instruction updates two cells.  They
// take over from the 32-bit layout of fz_extend.hpp once the eager block is
// done (diagonal 34) and run the rest of the side, for the inspector and the
// executor alike, with the same window geometry, ranges, slides, kills and
// pointer rows as the 32-bit layouts (FastZ section 2.2 and section 3.2: one
// wave per extension, three rolling anti-diagonals in registers).
//
// Scores relative to the threshold.  Each stored value is V = S - T, where
// T = best - ydrop is the y-drop threshold of the next diagonal to evaluate.
// A cell is live exactly when V >= 0, so the kill is one arithmetic shift
// (the sign of each half) and one bit select that puts DEAD (-16384) in the
// dead halves.  When the best score grows by delta, T grows by the same
// amount and every stored value is moved down by it (one packed subtraction
// per register); delta is at most the largest substitution score, since a
// cell's score exceeds its predecessors' best by no more than that.
//
// Range.  Live values: 0 <= V <= ydrop + 127.  Below: a dead cell holds
// DEAD; a gap value is at least DEAD - (gap_open + gap_extend) when formed
// (it is a maximum with the value opened from this cell) and at most
// gap_extend + 127 lower when next used; a diagonal term is at least
// DEAD - 2 * 127 - 128.  With ydrop <=
// PK_MAX_YDROP, substitution scores in [-128, 127] and gap_open +
// 2 * gap_extend <= PK_MAX_OE every value stays in [-20,800, 16,300]: no
// sum or difference wraps, and the differences the pointer bits test for
// zero are below 2^16 in magnitude.  Values below 0 never become live again
// (they only decrease), so a dead-derived value and the 32-bit layouts'
// -inf make the same decisions, and every live value, kill, best-cell
// choice and traceback bit equals the 32-bit computation's.  The host runs
// other scorings on the 32-bit layouts.
#pragma once

#include "fz_extend.hpp"

namespace fz {

constexpr int PK_MAX_YDROP = 16000;
constexpr int PK_MAX_OE = 4000;
constexpr int32_t PK_DEAD = -16384;
constexpr uint32_t PK_DEAD2 = 0xC000C000u;          // PK_DEAD in both halves
constexpr int32_t PK_DEAD_LIMIT = -8192;            // below this a value counts as dead (-inf)

// packed 16-bit helpers; the ones the compiler would scalarize are written
// as single instructions
typedef short pk_s16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ pk_s16x2 pk_v(uint32_t x) { return __builtin_bit_cast(pk_s16x2, x); }
__device__ __forceinline__ uint32_t pk_u(pk_s16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ uint32_t pk_add(uint32_t a, uint32_t b) { return pk_u(pk_v(a) + pk_v(b)); }
__device__ __forceinline__ uint32_t pk_sub(uint32_t a, uint32_t b) { return pk_u(pk_v(a) - pk_v(b)); }
__device__ __forceinline__ uint32_t pk_max(uint32_t a, uint32_t b)
{
    return pk_u(__builtin_elementwise_max(pk_v(a), pk_v(b)));
}
// 0xFFFF in each half whose value is negative, 0 elsewhere (one
// v_pk_ashrrev_i16; the compiler keeps it as a shift since only the
// inline-assembly bit select below reads it)
__device__ __forceinline__ uint32_t pk_neg_mask(uint32_t x)
{
    return pk_u(pk_v(x) >> (pk_s16x2){15, 15});
}
// (m & a) | (~m & b)
__device__ __forceinline__ uint32_t bit_select(uint32_t m, uint32_t a, uint32_t b)
{
    uint32_t r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "v"(a), "v"(b));
    return r;
}
typedef unsigned short pk_u16x2 __attribute__((ext_vector_type(2)));
// per half: 1 if the (unsigned) value is 0, else 0 (saturating 1 - x: one
// v_pk_sub_u16 with clamp)
__device__ __forceinline__ uint32_t pk_is_zero(uint32_t x)
{
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat((pk_u16x2){1, 1},
                                                                      __builtin_bit_cast(pk_u16x2, x)));
}
// per half: 1 if the (unsigned) value is not 0, else 0
__device__ __forceinline__ uint32_t pk_nonzero(uint32_t x)
{
    uint32_t r;
    asm("v_pk_min_u16 %0, %1, 1 op_sel_hi:[1,0]" : "=v"(r) : "v"(x));
    return r;
}
// per half: a - b saturated to the int16 range (keeps the sign right)
__device__ __forceinline__ uint32_t pk_sub_sat(uint32_t a, uint32_t b)
{
    return pk_u(__builtin_elementwise_sub_sat(pk_v(a), pk_v(b)));
}
// per half: a * 2 + b (a, b small unsigned)
__device__ __forceinline__ uint32_t pk_shl1_add(uint32_t a, uint32_t b)
{
    uint32_t r;
    asm("v_pk_mad_u16 %0, %1, 2, %2 op_sel_hi:[1,0,1]" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
// A VGPR copy of a wave-uniform value: the packed constants of the cell
// updates live in vector registers, which this kernel has to spare, and not
// in the scalar file, which its wave-uniform state fills.
__device__ __forceinline__ uint32_t in_vgpr(uint32_t x)
{
    uint32_t r;
    asm("v_mov_b32 %0, %1" : "=v"(r) : "s"(x));
    return r;
}
// sign-extended low / high half
__device__ __forceinline__ int pk_lo(uint32_t x) { return (int)(int16_t)(x & 0xFFFFu); }
__device__ __forceinline__ int pk_hi(uint32_t x) { return (int)(int16_t)(x >> 16); }

// Packed 16-bit codes of the two sequences: a target base a is stored as
// the byte pair (2a, 2a + 1) and a query base b as (2b, 2b), so that the
// xor of a target pair and a query pair is the byte pair (2x, 2x + 1) with
// x = a ^ b: a byte-permute selector for entry x of a table of four int16
// scores (match, transversion, transition, transversion).
__host__ __device__ constexpr uint32_t pk_target_code(uint32_t base) { return (2u * base) | ((2u * base + 1u) << 8); }
__host__ __device__ constexpr uint32_t pk_query_code(uint32_t base) { return (2u * base) | ((2u * base) << 8); }

template <int N> struct Unaligned3;
template <> struct Unaligned3<3> { typedef uint32_t T __attribute__((ext_vector_type(3), aligned(1))); };

template <int N>
__device__ __forceinline__ void load_unaligned_pk(const GlobalU8 *p, uint32_t (&out)[N])
{
    if constexpr (N == 3) {
        typedef typename Unaligned3<3>::T V;
        const V v = *reinterpret_cast<const __attribute__((address_space(1))) V *>(p);
        out[0] = v[0];
        out[1] = v[1];
        out[2] = v[2];
    } else {
        load_unaligned<N>(p, out);
    }
}

// One-pass executor state of the wave (one wave per workgroup): the pool,
// the current arena's end and the side's block table.  Touched once per
// block of OP_BLOCK anti-diagonals.
struct OpState {
    uint8_t *pool;              // the first OP_BLOCK_BYTES are a sink (see op_next_block)
    uint64_t pool_bytes;
    unsigned long long *used;   // bytes taken after the sink
    uint64_t aend;              // end of the wave's current arena (0: none)
    uint64_t *btab;             // the side's block table
    uint64_t admit;             // no side starts once `used` is past this
    int32_t out_of_pool;        // the side ran out of pool
};
__shared__ OpState op_state;

// `bytes` of pool memory at or after address cur (16-aligned), from the
// wave's arena; a new arena when it does not fit, a direct pool carve for
// requests above half an arena.  nullptr when the pool is exhausted.
// With `limit`, the carve fails also when the pool had `limit` bytes or more
// taken before it (admission of a new side, see run_side_pk).
__device__ __forceinline__ uint8_t *op_alloc(uint64_t cur, uint64_t bytes, uint64_t limit = ~(uint64_t)0)
{
    const uint64_t aend = uniform64(op_state.aend);
    if (cur != 0 && cur + bytes <= aend) return reinterpret_cast<uint8_t *>(cur);
    const uint64_t take = bytes > (uint64_t)OP_ARENA / 2 ? (bytes + 255) & ~(uint64_t)255 : (uint64_t)OP_ARENA;
    unsigned long long *used = reinterpret_cast<unsigned long long *>(uniform64((uint64_t)(uintptr_t)op_state.used));
    uint64_t off = 0;
    if (fresh_lane_id() == 0) off = atomicAdd(used, (unsigned long long)take);
    off = uniform64(off);
    const uint64_t pool_bytes = uniform64(op_state.pool_bytes) - (uint64_t)OP_BLOCK_BYTES;
    if (off > pool_bytes || take > pool_bytes - off || off >= limit) return nullptr;
    const uint64_t base = uniform64((uint64_t)(uintptr_t)op_state.pool) + (uint64_t)OP_BLOCK_BYTES + off;
    if (take == (uint64_t)OP_ARENA) op_state.aend = base + take;       // (every lane writes the same value)
    return reinterpret_cast<uint8_t *>(base);
}

template <int C2, bool EXEC, bool ONEPASS = false>
struct SidePk {
    static constexpr int C = 2 * C2;                 // positions per lane
    static constexpr int W = 64 * C;
    static constexpr bool PAIRED = C2 == 2;          // pointer rows: two lanes (16 bits each) per dword
    static constexpr int CPW = PAIRED ? 8 : C;       // cells per pointer word
    static constexpr int NWORD = 1;
    static constexpr int NONE_LO = 1 << 29, NONE_HI = -(1 << 29);
    static constexpr bool STOPS = EXEC;  // the executors test d against dstop (INT_MAX: the one-pass one)

    // registers (packed pairs)
    uint32_t SA[C2], SB[C2], R[C2], Dn[C2];
    // sequence codes in two buffers per sequence, used in turn (see step):
    // no register copies when a diagonal's prefetch becomes current
    uint32_t Ta[2][C2], Qb[2][C2];
    uint32_t crossL, crossR;    // DPP targets whose edge lane keeps PK_DEAD2
    const GlobalU8 *ba, *bb;    // 16-bit code arrays, uniform bases (bytes)
    uint32_t ua, ub;            // element offsets of slot 0 of lane 0 (as in SideDP)
    // wave-uniform state
    int K, dmask;
    int lo1, hi1, lo2, hi2;
    int best, bi, bj, dend;     // best: absolute score
    int ydrop;                  // values are stored as S - T with T = best - ydrop, the next diagonal's threshold
    int64_t cells, cum_bytes, ptr_at_best;
    int dflush;
    int32_t acc_cells, acc_words, bmax;
    bool overflow;
    int state;                  // END_* once the side stopped for another reason than its end
    uint32_t rowoff, rowcap;
    RowHdr *hdr;
    uint32_t *rows;

    const SideTask &t;
    const Scoring &sc;
    int lane;
    uint32_t oe2, e2, lut_lo, lut_hi, dead2;    // packed constants (VGPR copies)

    static constexpr int END_DEFER = 1;         // inspector: handed to the one-pass executor
    static constexpr int END_POOL = 2;          // one-pass executor: pool exhausted

    __device__ SidePk(const SideTask &task, const Scoring &s)
        : ydrop(s.ydrop), state(0), t(task), sc(s), lane(fresh_lane_id())
    {
    }

    // Flush points where advance() hands control back to the caller.
    static __device__ __forceinline__ bool at_checkpoint(int d)
    {
        if (ONEPASS) return (d & (OP_BLOCK - 1)) == 0;
        return !EXEC && (d == ONEPASS_AT || d == ONEPASS_AT2 || d == ONEPASS_AT3);
    }

    // (inspector, at a hand-over test) the side's seed is now certain to be traced
    // and its best is still growing: it goes to the one-pass executor
    // (defer_need is INT32_MAX when that is off)
    __device__ __forceinline__ bool defer_now(int d) const
    {
        return best >= t.defer_need && d - (bi + bj) <= ONEPASS_RECENT;
    }

    // One-pass executor: close the block ending before diagonal d (its last
    // header slot gets the block's word count) and open the block of d.
    // When the pool is exhausted the side's rows go to the pool's sink
    // (never read) and it is marked out of pool; the caller ends it.
    __device__ __forceinline__ void op_next_block(int d)
    {
        if (lane == 0) {
            RowHdr h;
            h.off = rowoff;
            h.ibase = 0;
            store_hdr(hdr + d, h.off, h.ibase);
        }
        const uint64_t cur = ((uint64_t)(uintptr_t)(rows + rowoff) + 15) & ~(uint64_t)15;
        // (once out of pool, the rows stay in the sink: cur lies there)
        uint8_t *blk = uniform(op_state.out_of_pool) ? nullptr : op_alloc(cur, (uint64_t)OP_BLOCK_BYTES);
        if (!blk) {
            blk = reinterpret_cast<uint8_t *>(uniform64((uint64_t)(uintptr_t)op_state.pool));
            op_state.out_of_pool = 1;
        }
        blk = reinterpret_cast<uint8_t *>(uniform64((uint64_t)(uintptr_t)blk));
        uint64_t *btab = reinterpret_cast<uint64_t *>(uniform64((uint64_t)(uintptr_t)op_state.btab));
        if (lane == 0) gstore64(btab + d / OP_BLOCK, (uint64_t)(uintptr_t)blk);
        hdr = reinterpret_cast<RowHdr *>(blk) - d;
        rows = reinterpret_cast<uint32_t *>(blk + 8 * OP_HDRS);
        rowoff = 0;
        rowcap = OP_BLOCK_WORDS;
    }

    // lane-held values of this layout's run, formed when the run starts (not
    // once per side, where both layouts' sets would hold registers)
    __device__ __forceinline__ void enter()
    {
        lane = fresh_lane_id();
        oe2 = in_vgpr(((uint32_t)sc.oe & 0xFFFFu) * 0x10001u);
        e2 = in_vgpr(((uint32_t)sc.e & 0xFFFFu) * 0x10001u);
        lut_lo = in_vgpr(((uint32_t)sc.match & 0xFFFFu) | ((uint32_t)sc.tv << 16));
        lut_hi = in_vgpr(((uint32_t)sc.ts & 0xFFFFu) | ((uint32_t)sc.tv << 16));
        dead2 = in_vgpr(PK_DEAD2);
    }

    __device__ __forceinline__ void fetch(const GlobalU8 *base, uint32_t off, uint32_t (&out)[C2]) const
    {
        load_unaligned_pk<C2>(base + 2u * (off + (uint32_t)(lane * C)), out);
    }

    // After a slide inside step<DELTA, P>(d): this diagonal's codes and the
    // prefetches, in the buffers that step uses.
    template <int DELTA, int P>
    __device__ __forceinline__ void reload(int d, int od)
    {
        fetch(ba, ua + od, Ta[P]);
        fetch(bb, ub + (od - d), Qb[DELTA == 1 ? P ^ 1 : P]);
        fetch(ba, ua + (od + 1), Ta[P ^ 1]);
        fetch(bb, ub + (od - d - 1), Qb[DELTA == 1 ? P : P ^ 1]);
    }

    // The state step<1, 0>(d + 1) starts from, after diagonal d (odd):
    // Ta[0] holds the target codes of d + 1, Qb[1] the query codes of d + 1
    // (the same as d's), Qb[0] those of d + 2.
    __device__ __forceinline__ void reload_entry(int d, int od)
    {
        fetch(ba, ua + (od + 1), Ta[0]);
        fetch(bb, ub + (od - d), Qb[1]);
        fetch(bb, ub + (od - d - 1), Qb[0]);
    }

    // Swap the buffers' roles (a single pair before the four-diagonal loop).
    __device__ __forceinline__ void swap_buffers()
    {
#pragma unroll
        for (int k = 0; k < C2; ++k) {
            const uint32_t a = Ta[0][k], b = Qb[0][k];
            Ta[0][k] = Ta[1][k];
            Qb[0][k] = Qb[1][k];
            Ta[1][k] = a;
            Qb[1][k] = b;
        }
    }

    __device__ __forceinline__ void set_dmask() { dmask = min(2 * (t.m - W + 2) - K, 2 * t.n + 1 + K); }

    __device__ __forceinline__ void init_bases()
    {
        const int64_t aoff = (t.abase - W - 8) & ~(int64_t)3;
        const int64_t boff = (t.bbase - (int64_t)t.n - W - 8) & ~(int64_t)3;
        ba = reinterpret_cast<const GlobalU8 *>(reinterpret_cast<uintptr_t>(t.A16 + 2 * aoff));
        bb = reinterpret_cast<const GlobalU8 *>(reinterpret_cast<uintptr_t>(t.B16 + 2 * boff));
        ua = (uint32_t)(t.abase - aoff);
        ub = (uint32_t)(t.bbase - boff);
    }

    // Evaluate one diagonal (DELTA = o_d - o_(d-1)); SN holds S of d-2 and
    // receives S of d.  Returns the lane's live mask (one byte per position,
    // 0xFF dead, 0x00 live; positions 0-3 in m0, 4-5 in m1) and the lane's
    // best value; with PTR, word receives the lane's pointer nibbles in the
    // row format (PAIRED: 16 bits, first position highest; else C nibbles).
    template <int DELTA, bool PTR, bool MASKED>
    __device__ __forceinline__ void cells_of(uint32_t (&SN)[C2], const uint32_t (&TA)[C2], const uint32_t (&QB)[C2],
                                             int rlo, int rhi, uint32_t &m0, uint32_t &m1, uint32_t &dmax,
                                             uint32_t &word)
    {
        uint32_t X[C2];
#pragma unroll
        for (int r = 0; r < C2; ++r) X[r] = __builtin_amdgcn_perm(lut_hi, lut_lo, TA[r] ^ QB[r]);
        uint32_t Iv[C2], Dv[C2];
        if (DELTA == 1) {
            crossL = (uint32_t)__builtin_amdgcn_update_dpp((int)crossL, (int)R[0], 0x130 /* wave_shl:1 */, 0xF, 0xF,
                                                           false);
#pragma unroll
            for (int r = 0; r < C2; ++r) {
                Iv[r] = __builtin_amdgcn_alignbyte(r + 1 < C2 ? R[r + 1 < C2 ? r + 1 : 0] : crossL, R[r], 2);
                Dv[r] = Dn[r];
            }
        } else {
            crossR = (uint32_t)__builtin_amdgcn_update_dpp((int)crossR, (int)Dn[C2 - 1], 0x138 /* wave_shr:1 */, 0xF,
                                                           0xF, false);
#pragma unroll
            for (int r = 0; r < C2; ++r) {
                Iv[r] = R[r];
                Dv[r] = __builtin_amdgcn_alignbyte(Dn[r], r > 0 ? Dn[r > 0 ? r - 1 : 0] : crossR, 2);
            }
        }
        uint32_t Kd[C2];
        const int mbase = MASKED ? lane * C - rlo : 0;
        const uint32_t span = (uint32_t)(rhi - rlo);
        uint32_t bits[C2];
#pragma unroll
        for (int r = 0; r < C2; ++r) {
            const uint32_t H = pk_add(SN[r], X[r]);
            const uint32_t S = pk_max(pk_max(H, Iv[r]), Dv[r]);
            uint32_t Kr = pk_neg_mask(S);
            if (MASKED) {
                // positions outside [rlo, rhi] are dead
                const uint32_t out_lo = (uint32_t)(mbase + 2 * r) > span ? 0x0000FFFFu : 0u;
                const uint32_t out_hi = (uint32_t)(mbase + 2 * r + 1) > span ? 0xFFFF0000u : 0u;
                Kr |= out_lo | out_hi;
            }
            Kd[r] = Kr;
            const uint32_t Sk = bit_select(Kr, dead2, S);
            const uint32_t U = pk_sub(Sk, oe2);
            const uint32_t Rn = pk_max(pk_sub(Iv[r], e2), U);
            const uint32_t Dnn = pk_max(pk_sub(Dv[r], e2), U);
            if (PTR) {
                // the four pointer bits of the register's two cells as
                // sign bits (saturating differences): H - S < 0 when S did
                // not come by the diagonal, I - S < 0 when not from I,
                // U - (I - E) < 0 when I extends, U - (D - E) < 0 when D
                // extends.  Two permutes gather the signs as 0x00 / 0xFF
                // bytes (selectors 8..11 replicate the sign bits of the
                // halves), masks place them: bytes 0, 1 hold the gap bits
                // (bits 1, 0) of the low and high cell, bytes 2, 3 the
                // "not diagonal", "not from I" bits (bits 3, 2).
                const uint32_t x3 = pk_sub_sat(H, S), x2 = pk_sub_sat(Iv[r], S);
                const uint32_t x1 = pk_sub_sat(U, pk_sub(Iv[r], e2)), x0 = pk_sub_sat(U, pk_sub(Dv[r], e2));
                const uint32_t p31 = __builtin_amdgcn_perm(x3, x1, 0x0B0A0908u);
                const uint32_t p20 = __builtin_amdgcn_perm(x2, x0, 0x0B0A0908u);
                bits[r] = (p31 & 0x08080202u) | (p20 & 0x04040101u);
            }
            R[r] = Rn;
            Dn[r] = Dnn;
            SN[r] = Sk;
            dmax = r == 0 ? Sk : pk_max(dmax, Sk);     // (killed halves hold DEAD)
        }
        if (PTR) {
            // the packed row order (RowHdr): cell k of the lane at bit
            // 16 * (k >> 2) + 8 * (k & 1) + 4 * ((k >> 1) & 1); the two bit
            // bytes of each cell are ORed into its nibble
            const uint32_t t = bits[0] | (bits[1] << 4);
            const uint32_t f = t | (t >> 16);               // bytes 0, 1: cells 0 | 2, 1 | 3
            if constexpr (C2 == 2) {
                word = f & 0xFFFFu;
            } else {
                const uint32_t g = bits[2] | (bits[2] >> 16);    // bytes 0, 1: cells 4, 5
                word = __builtin_amdgcn_perm(g, f, 0x05040100u);
            }
        }
        // dead-byte masks: the sign byte of each half
        if constexpr (C2 == 2) {
            m0 = __builtin_amdgcn_perm(Kd[1], Kd[0], 0x07050301u);
            m1 = 0xFFFFFFFFu;
        } else {
            m0 = __builtin_amdgcn_perm(Kd[1], Kd[0], 0x07050301u);
            m1 = __builtin_amdgcn_perm(Kd[2], Kd[2], 0x0D0D0301u);
        }
    }

    __device__ __forceinline__ void slide(int s)
    {
        while (s > 0) {
#pragma unroll
            for (int r = 0; r < C2; ++r) {
                SA[r] = (uint32_t)from_next_lane((int)SA[r], (int)PK_DEAD2);
                SB[r] = (uint32_t)from_next_lane((int)SB[r], (int)PK_DEAD2);
                R[r] = (uint32_t)from_next_lane((int)R[r], (int)PK_DEAD2);
                Dn[r] = (uint32_t)from_next_lane((int)Dn[r], (int)PK_DEAD2);
            }
            --s;
        }
        while (s < 0) {
#pragma unroll
            for (int r = 0; r < C2; ++r) {
                SA[r] = (uint32_t)from_prev_lane((int)SA[r], (int)PK_DEAD2);
                SB[r] = (uint32_t)from_prev_lane((int)SB[r], (int)PK_DEAD2);
                R[r] = (uint32_t)from_prev_lane((int)R[r], (int)PK_DEAD2);
                Dn[r] = (uint32_t)from_prev_lane((int)Dn[r], (int)PK_DEAD2);
            }
            ++s;
        }
    }

    // Move every stored value down by delta (the threshold grew by delta).
    __device__ __forceinline__ void rebase(int delta)
    {
        const uint32_t d2 = ((uint32_t)delta & 0xFFFFu) * 0x10001u;
#pragma unroll
        for (int r = 0; r < C2; ++r) {
            SA[r] = pk_sub(SA[r], d2);
            SB[r] = pk_sub(SB[r], d2);
            R[r] = pk_sub(R[r], d2);
            Dn[r] = pk_sub(Dn[r], d2);
        }
    }

    // Evaluate diagonal d; false when the side has ended before it (an
    // empty range, a band wider than the window (overflow), or, in the
    // executor, d past the best cell's diagonal).  There is no early exit:
    // an ended side runs the masked sweep over an empty range (every cell
    // dead, nothing counted) and keeps empty hulls, so that later diagonals
    // end too, and the caller leaves its loop in one place with every value
    // of the side's state defined.
    //
    // Buffers (P = 0, 1 in turn over the diagonal pairs): step<1, P> reads
    // the target codes in Ta[P] and the query codes in Qb[P ^ 1] and
    // prefetches the target codes of d + 2 into Ta[P ^ 1]; step<0, P> reads
    // Ta[P] and Qb[P] and prefetches the query codes of d + 2 into
    // Qb[P ^ 1].  After the four steps of P = 0, 1 every buffer is back in
    // its role.
    template <int DELTA, bool PTR, int P>
    __device__ __forceinline__ bool step(int d, int dstop)
    {
        int od = (d + K) >> 1;
        if (DELTA == 1) fetch(ba, ua + (od + 1), Ta[P ^ 1]);
        else fetch(bb, ub + (od - d - 1), Qb[P ^ 1]);
        int rlo = min(lo1 - DELTA, lo2);
        int rhi = max(hi1 - DELTA + 1, hi2);
        bool masked = false, live = true;
        if (((dmask - 1 - d) | rlo | (W - 1 - rhi) | (rhi - rlo) | (STOPS ? dstop - d : 0)) < 0) {
            const int vlo = max(0, d - t.n) - od, vhi = min(t.m, d) - od;
            rlo = max(rlo, vlo);
            rhi = min(rhi, STOPS && d > dstop ? rlo - 1 : vhi);
            if (rlo <= rhi && (rlo < 0 || rhi > W - 1)) {
                const int smin = floordiv(rhi - (W - 1) + C - 1, C), smax = floordiv(rlo, C);
                if (smin > smax) {
                    overflow = true;
                    rhi = rlo - 1;
                } else {
                    int s = floordiv((rlo + rhi + 1) / 2 - W / 2, C);
                    s = s < smin ? smin : (s > smax ? smax : s);
                    slide(s);
                    const int sh = s * C;
                    K += 2 * sh;
                    od += sh;
                    lo1 -= sh; hi1 -= sh; lo2 -= sh; hi2 -= sh;
                    rlo -= sh; rhi -= sh;
                    set_dmask();
                    reload<DELTA, P>(d, od);
                }
            }
            masked = (W - 1 + od > t.m) || (d - od > t.n);
            if (rlo > rhi) {
                live = false;
                masked = true;
                rlo = NONE_LO;      // no position of the window lies in [rlo, rhi]
                rhi = NONE_LO;
                lo1 = NONE_LO;      // (read above): the next diagonal's range is empty too
                hi1 = NONE_HI;
                if (!EXEC) acc_words += 1;      // the empty hull's row count below is -1
            }
        }
        uint32_t m0, m1, dmax, word = 0;
        const uint32_t(&TAc)[C2] = Ta[P];
        const uint32_t(&QBc)[C2] = Qb[DELTA == 1 ? P ^ 1 : P];
        if (masked) {
            if (DELTA == 1) cells_of<DELTA, PTR, true>(SA, TAc, QBc, rlo, rhi, m0, m1, dmax, word);
            else cells_of<DELTA, PTR, true>(SB, TAc, QBc, rlo, rhi, m0, m1, dmax, word);
        } else {
            if (DELTA == 1) cells_of<DELTA, PTR, false>(SA, TAc, QBc, rlo, rhi, m0, m1, dmax, word);
            else cells_of<DELTA, PTR, false>(SB, TAc, QBc, rlo, rhi, m0, m1, dmax, word);
        }

        // live hull of d: lanes from the ballot, positions from the edge
        // lanes' dead-byte masks
        const uint64_t anyl = ballot((m0 & m1) != 0xFFFFFFFFu);
        int lo = NONE_LO, hi = NONE_HI, llo = 0, lhi = -1;
        if (anyl) {
            llo = ctz64(anyl);
            lhi = hibit64(anyl);
            const uint32_t a0 = ~(uint32_t)__builtin_amdgcn_readlane((int)m0, llo);
            const uint32_t b0 = ~(uint32_t)__builtin_amdgcn_readlane((int)m1, llo);
            const uint32_t a1 = ~(uint32_t)__builtin_amdgcn_readlane((int)m0, lhi);
            const uint32_t b1 = ~(uint32_t)__builtin_amdgcn_readlane((int)m1, lhi);
            const int flo = a0 ? (__builtin_ctz(a0) >> 3) : 4 + (__builtin_ctz(b0) >> 3);
            const int fhi = b1 ? 4 + ((31 - __builtin_clz(b1)) >> 3) : ((31 - __builtin_clz(a1)) >> 3);
            lo = llo * C + flo;
            hi = lhi * C + fhi;
        }
        acc_cells += rhi - rlo;                 // 0 for an ended side
        bmax = max(bmax, rhi - rlo);
        const int rlane0 = PAIRED ? (llo & ~1) : llo;
        const int nl1 = PAIRED ? (lhi >> 1) - (llo >> 1) : lhi - llo;
        const int nl = nl1 + 1;
        if (!EXEC) acc_words += nl1;

        // (no cell of an ended side is live, so its best cannot move)
        const int lmax = max(pk_lo(dmax), pk_hi(dmax));
        if (ballot(lmax > ydrop)) {          // (the best score is ydrop in these terms)
            int nb = wave_max(lmax);
            // first position holding it
            int slot = C;
#pragma unroll
            for (int r = C2 - 1; r >= 0; --r) {
                const uint32_t Sv = DELTA == 1 ? SA[r] : SB[r];
                slot = pk_hi(Sv) == nb ? 2 * r + 1 : slot;
                slot = pk_lo(Sv) == nb ? 2 * r : slot;
            }
            const int fl = ctz64(ballot(slot < C));
            const int pbest = fl * C + __builtin_amdgcn_readlane(slot, fl);
            const int delta = nb - ydrop;     // the best grows by delta, and so does the threshold
            best += delta;
            rebase(delta);
            bi = pbest + od;
            bj = d - bi;
            const int n = d - dflush;
            ptr_at_best = cum_bytes + 8 * (int64_t)n + 4 * NWORD * ((int64_t)acc_words + n);
        }

        if (EXEC && live) {
            if (rowoff + (uint32_t)nl > rowcap) {
                // the recompute disagrees with the inspector's sizing
                overflow = true;
                live = false;
            } else {
                if (lane == 0) {
                    RowHdr h;
                    h.off = rowoff | (CPW == 8 ? ROW_CPW8 : 0u) | ROW_PK;
                    h.ibase = rlane0 * C + od;
                    store_hdr(hdr + d, h.off, h.ibase);
                }
                if (PAIRED) {
                    // the odd lane's 16 bits above the even lane's
                    const uint32_t odd = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)word, 0xB1, 0xF, 0xF, false);
                    if (!(lane & 1) && lane >= rlane0 && lane <= lhi)
                        gstore(rows + rowoff + ((lane - rlane0) >> 1), word | (odd << 16));
                } else if (lane >= llo && lane <= lhi) {
                    gstore(rows + rowoff + (lane - llo), word);
                }
                rowoff += (uint32_t)nl;
            }
        }

        lo2 = lo1; hi2 = hi1;
        lo1 = lo; hi1 = hi;
        return live;
    }

    __device__ __forceinline__ void flush()
    {
        const int n = dend - dflush;
        cells += (int64_t)acc_cells + n;
        cum_bytes += 8 * (int64_t)n + 4 * NWORD * ((int64_t)acc_words + n);
        acc_cells = 0;
        acc_words = 0;
        dflush = dend;
    }

    __device__ __forceinline__ int hull_width() const
    {
        const int ul = min(lo1, lo2), uh = max(hi1, hi2);
        return ul <= uh ? uh - ul : -1;
    }

    // The packed layouts switch between 256 and 384 positions; the test runs
    // every 8 diagonals, during which a union can widen by at most 16.
    static constexpr int SWITCH_EVERY = 8;
    static constexpr int NARROW_ENTER = 216;     // union hull width to enter the 256-position layout
    static constexpr int NARROW_LEAVE = 232;     // ... and to leave it (232 + 16 + 3 <= 256 - 4)

    __device__ __forceinline__ bool want_switch() const
    {
        const int w = hull_width();
        if (C2 == 3) return w >= 0 && w <= NARROW_ENTER;
        return w > NARROW_LEAVE;
    }

    // Diagonals from d (even) on until the end (-1) or a layout change
    // (returns the next d, even).
    //
    // Four diagonals per trip (the two buffer parities); a side entering at
    // d = 2 (mod 4) first takes one pair.  An ended side stays ended (its
    // hulls stay empty), so the number of live results of a trip gives the
    // last live diagonal.
    __device__ int advance(int d, int dstop)
    {
        enter();
        if (d & 2) {
            const bool a = step<1, EXEC, 0>(d, dstop);
            const bool b = step<0, EXEC, 0>(d + 1, dstop);
            if (!(a && b)) {
                dend = a ? d : d - 1;       // the last live diagonal
                return -1;
            }
            d += 2;
            swap_buffers();
        }
        for (;;) {
            // (scheduling barriers: each step's loads stay in its step, so
            // the unrolled steps do not hold each other's registers)
            const bool a = step<1, EXEC, 0>(d, dstop);
            __builtin_amdgcn_sched_barrier(0);
            const bool b = step<0, EXEC, 0>(d + 1, dstop);
            __builtin_amdgcn_sched_barrier(0);
            const bool c = step<1, EXEC, 1>(d + 2, dstop);
            __builtin_amdgcn_sched_barrier(0);
            const bool e = step<0, EXEC, 1>(d + 3, dstop);
            if (!(a && b && c && e)) {
                dend = d - 1 + (int)a + (int)b + (int)c + (int)e;
                return -1;
            }
            d += 4;
            if ((d & (SWITCH_EVERY - 1)) == 0) {
                dend = d - 1;
                flush();
                // the caller's checkpoints (out of this loop, whose
                // registers they would crowd): the inspector's hand-over
                // test, the one-pass executor's block ends
                if (at_checkpoint(d)) return d;
                if (want_switch()) return d;
            }
        }
    }

    // Hand-over through LDS, as SideDP::export_regs / adopt: absolute int32
    // scores by position (NEG for dead ones) of the union [ul, uh].
    static constexpr int XFER_W = XFER_STRIDE;
    __device__ __forceinline__ void export_regs(uint32_t *x, int ul, int uh) const
    {
        const int q0 = fresh_lane_id() * C - ul;
        const int T = best - ydrop;
        auto absval = [&](int v) -> uint32_t { return (uint32_t)(v < PK_DEAD_LIMIT ? NEG : v + T); };
#pragma unroll
        for (int r = 0; r < C2; ++r) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int q = q0 + 2 * r + h;
                if ((uint32_t)q <= (uint32_t)(uh - ul)) {
                    x[q] = absval(h ? pk_hi(SA[r]) : pk_lo(SA[r]));
                    x[XFER_W + q] = absval(h ? pk_hi(SB[r]) : pk_lo(SB[r]));
                    x[2 * XFER_W + q] = absval(h ? pk_hi(R[r]) : pk_lo(R[r]));
                    x[3 * XFER_W + q] = absval(h ? pk_hi(Dn[r]) : pk_lo(Dn[r]));
                }
            }
        }
    }

    template <class O>
    __device__ __forceinline__ void adopt(const O &o, int s, const uint32_t *x, int ul, int uh, int dlast)
    {
        K = o.K + 2 * s;
        const int T = o.best - ydrop;       // the 32-bit layouts' threshold too (ydrop is small here)
        const int q0 = fresh_lane_id() * C + s - ul;
        auto rel = [&](uint32_t v) -> uint32_t {
            const int a = (int)v;
            const int r = (a <= NEG / 2) ? PK_DEAD : max(a - T, PK_DEAD);
            return (uint32_t)r & 0xFFFFu;
        };
#pragma unroll
        for (int r = 0; r < C2; ++r) {
            uint32_t va[2], vb[2], vr[2], vd[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int q = q0 + 2 * r + h;
                const bool in = (uint32_t)q <= (uint32_t)(uh - ul);
                const int qq = in ? q : 0;
                va[h] = in ? rel(x[qq]) : (uint32_t)PK_DEAD & 0xFFFFu;
                vb[h] = in ? rel(x[XFER_W + qq]) : (uint32_t)PK_DEAD & 0xFFFFu;
                vr[h] = in ? rel(x[2 * XFER_W + qq]) : (uint32_t)PK_DEAD & 0xFFFFu;
                vd[h] = in ? rel(x[3 * XFER_W + qq]) : (uint32_t)PK_DEAD & 0xFFFFu;
            }
            SA[r] = va[0] | (va[1] << 16);
            SB[r] = vb[0] | (vb[1] << 16);
            R[r] = vr[0] | (vr[1] << 16);
            Dn[r] = vd[0] | (vd[1] << 16);
        }
        crossL = PK_DEAD2;
        crossR = PK_DEAD2;
        auto mlo = [&](int v) { return v == NONE_LO ? v : v - s; };
        auto mhi = [&](int v) { return v == NONE_HI ? v : v - s; };
        lo1 = mlo(o.lo1); hi1 = mhi(o.hi1);
        lo2 = mlo(o.lo2); hi2 = mhi(o.hi2);
        best = o.best; bi = o.bi; bj = o.bj; dend = o.dend;
        cells = o.cells; cum_bytes = o.cum_bytes; ptr_at_best = o.ptr_at_best;
        dflush = o.dflush; acc_cells = 0; acc_words = 0;
        bmax = o.bmax;
        overflow = o.overflow;
        state = 0;
        rowoff = o.rowoff; rowcap = o.rowcap; hdr = o.hdr; rows = o.rows;
        lane = fresh_lane_id();
        set_dmask();
        init_bases();
        reload_entry(dlast, (dlast + K) >> 1);
    }
};

// One side with the packed layouts: the 192-position 32-bit layout for
// diagonals 0..33 (the eager block and its pointers), then the packed
// 256-position layout, moving to the 384-position one while the band is
// wider than 232 positions and back when it narrows to 216.  The executor
// makes the same moves at the same diagonals, so its pointer rows match the
// inspector's sizing.
//
// ONEPASS (with EXEC): the one-pass executor.  No end is known (dstop is
// INT_MAX), and the rows go to blocks of OP_BLOCK anti-diagonals taken from
// the pool as the side grows; the block table's address is left in
// op_state.btab.  The side's last row is followed by a header holding the
// block's word count, as at every block's end.
template <bool EXEC, bool ONEPASS = false>
__device__ __forceinline__ SideResult run_side_pk(const SideTask &task, const Scoring &sc, int dstop,
                                                  uint32_t *eager_lds, uint32_t *xfer, uint8_t *ptr_base,
                                                  int64_t ptr_bytes)
{
    SideResult r;
    int64_t nhdr = -1;
    if constexpr (ONEPASS) {
        // the block table (a block for every flush point the side can
        // reach, up to anti-diagonal m + n + 1), then block 0
        const uint64_t nblk = (uint64_t)(((int64_t)task.m + task.n + 1) / OP_BLOCK + 1);
        // admission: a side starts only if the pool had less than its
        // admission mark taken before the side's first carve (taken in the
        // same atomic step, so sides that start together are counted one
        // after the other), so that the sides already running have room to
        // finish: a side that runs out midway was swept for nothing
        uint8_t *bt = op_alloc(0, 8 * nblk, uniform64(op_state.admit));
        uint8_t *b0 = bt ? op_alloc(((uint64_t)(uintptr_t)bt + 8 * nblk + 15) & ~(uint64_t)15, (uint64_t)OP_BLOCK_BYTES)
                         : nullptr;
        if (!b0) {
            r.best = r.bi = r.bj = r.dend = r.band = 0;
            r.cells = r.ptr_at_best = 0;
            r.overflow = false;
            r.state = SidePk<2, EXEC, ONEPASS>::END_POOL;
            return r;
        }
        op_state.btab = reinterpret_cast<uint64_t *>(bt);      // (every lane writes the same value)
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        if (fresh_lane_id() == 0) gstore64(reinterpret_cast<uint64_t *>(bt), (uint64_t)(uintptr_t)b0);
        ptr_base = reinterpret_cast<uint8_t *>(uniform64((uint64_t)(uintptr_t)b0));
        ptr_bytes = 8 * OP_HDRS + 4 * (int64_t)OP_BLOCK_WORDS;
        nhdr = OP_HDRS;
    }
    // the header after the side's last row: its row's end
    auto close_rows = [&](auto &x) {
        if constexpr (ONEPASS) {
            if (!x.overflow && fresh_lane_id() == 0) {
                RowHdr h;
                h.off = x.rowoff;
                h.ibase = 0;
                store_hdr(x.hdr + (x.dend + 1), h.off, h.ibase);
            }
        }
    };
    SideDP<3, EXEC, SUB_LUT> dn(task, sc);
    int d = dn.start(dstop, eager_lds, ptr_base, ptr_bytes, nhdr);
    // (the inspector's start runs to diagonal 33, the executor's to 1)
    while (d >= 0 && d < EAGER_ROWS + 1) {
        if (!dn.template step<1, EXEC>(d, dstop, eager_lds) || !dn.template step<0, EXEC>(d + 1, dstop, eager_lds)) {
            d = -1;
            break;
        }
        d += 2;
    }
    if (d < 0) {
        r.take(dn);
        close_rows(dn);
        return r;
    }
    SidePk<2, EXEC, ONEPASS> p4(task, sc);
    SidePk<3, EXEC, ONEPASS> p6(task, sc);
    switch_layout(p4, dn, xfer, d);
    constexpr bool CHECKPOINTS = ONEPASS || !EXEC;
    // at a checkpoint: false to end the side (its state says why); else
    // *stay when the layout does not change there
    auto checkpoint = [&](auto &p, int dd, bool &stay) -> bool {
        stay = false;
        if (!p.at_checkpoint(dd)) return true;
        if constexpr (!EXEC) {
            if (p.defer_now(dd)) {
                p.state = p.END_DEFER;
                return false;
            }
        }
        if constexpr (ONEPASS) {
            p.op_next_block(dd);
            // out of pool: the side ends at the next diagonal (its stop
            // diagonal; no exit from the sweep here) and is given back
            if (uniform(op_state.out_of_pool)) dstop = dd - 1;
        }
        stay = !p.want_switch();
        return true;
    };
    auto finish = [&](auto &p) {
        r.take(p);
        r.state = p.state;
        if (!p.state) close_rows(p);
    };
    for (;;) {
        bool stay = false;
        do {
            d = p4.advance(d, dstop);
            if (d < 0 || (CHECKPOINTS && !checkpoint(p4, d, stay))) {
                finish(p4);
                return r;
            }
        } while (CHECKPOINTS && stay);
        switch_layout(p6, p4, xfer, d);
        do {
            d = p6.advance(d, dstop);
            if (d < 0 || (CHECKPOINTS && !checkpoint(p6, d, stay))) {
                finish(p6);
                return r;
            }
        } while (CHECKPOINTS && stay);
        switch_layout(p4, p6, xfer, d);
    }
}

// One wave per side; the grid covers the work list (the hardware dispatcher
// hands waves to CUs as others retire, which balances sides of very
// different lengths).  Register budgets of the standard kernels: the
// inspector and the packed executor fit 64 VGPRs (8 waves per SIMD), the
// one-pass executor (which keeps the inspector's results and the
// executor's rows) 72 (7 waves), the 32-bit executor 72 with byte
// substitution scores and 80 (6) without; more waves let a SIMD pair one
// wave's VALU instruction with another's SALU instruction.
//
// PK: the packed layouts (fz_packed.hpp) after the eager block; the host
// launches it for scorings within their exact range (C = 6, SUB_LUT).
// ONEPASS (with EXEC and PK): the one-pass executor over a.list, the sides
// the inspector deferred; it reports like the inspector and writes the rows
// to the pool.
template <int C, bool EXEC, int SUB, int WAVES, bool PK = false, bool ONEPASS = false>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(C <= 8 ? (EXEC ? (PK ? (ONEPASS ? 7 : 8) : SUB != SUB_WIDE ? 7 : 6) : 8) : 1))) void extend_kernel(ExtendArgs a)
{
    static_assert(!ONEPASS || (EXEC && PK && WAVES == 1), "the one-pass executor runs the packed layouts, one wave per group");
    // The 1024-position kernels (the wide retry and its executor) run a
    // handful of long latency-bound waves beside the one-pass executor's
    // thousands: they take the SIMD's issue first, else each would get an
    // eighth of it and end long after the one-pass sides.
    if constexpr (C > 8) __builtin_amdgcn_s_setprio(3);
    using DP = SideDP<C, EXEC, SUB>;
    using EDP = SideDP<StartLayout<C>::value, EXEC, SUB>;     // holds the eager block
    __shared__ uint32_t eager_lds_all[WAVES][EAGER_ROWS * EDP::NEL * EDP::NWORD];
    __shared__ uint32_t xfer_all[WAVES][C == 6 ? 4 * DP::XFER_W : 1];
    const int wv = uniform((int)(threadIdx.x / 64));
    uint32_t *eager_lds = eager_lds_all[wv];
    uint32_t *xfer = xfer_all[wv];
    const int idx = (int)blockIdx.x * WAVES + wv;
    if (idx >= a.nlist) return;
    if constexpr (ONEPASS) {
        // (workgroups start in index order: the host launches the tail walk
        // once the grid's last wave runs, so that the walk's waves never
        // hold slots that executor waves still wait for)
        if (a.op_last_started && idx == a.nlist - 1 && fresh_lane_id() == 0)
            __hip_atomic_store(a.op_last_started, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    constexpr bool TWO_PASS_EXEC = EXEC && !ONEPASS;
    const int64_t item = TWO_PASS_EXEC ? a.exec_begin + idx : (int64_t)idx;
    const int sid = TWO_PASS_EXEC ? a.exec[item].side : (a.list ? a.list[item] : (int)item);
    const SideTask task = a.tasks[sid];
    SideOut *o = &a.out[sid];
    if (task.m < 0) {
        if (!EXEC && fresh_lane_id() == 0) {
            SideOut r = {};
            r.flags = SO_SKIPPED;
            *o = r;
        }
        return;
    }
    if constexpr (ONEPASS) {
        op_state.pool = a.op_pool;              // (every lane writes the same values)
        op_state.pool_bytes = a.op_pool_bytes;
        op_state.used = a.op_pool_used;
        op_state.aend = 0;
        op_state.btab = nullptr;
        op_state.admit = a.op_pool_bytes / 10 * 9;
        op_state.out_of_pool = 0;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        const SideResult x = run_side_pk<true, true>(task, a.sc, 0x7fffffff, nullptr, xfer, nullptr, 0);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        const bool pool_out = x.state != 0 || uniform(op_state.out_of_pool) != 0;
        SideOut r;
        r.score = x.best;
        r.ie = x.bi;
        r.je = x.bj;
        r.dend = x.dend;
        r.cells = x.cells;
        r.ptr_bytes = 0;        // (its rows are in the pool; a side given back is inspected again)
        r.flags = x.overflow ? SO_OVERFLOW : (pool_out ? SO_DEFERRED : SO_ONEPASS);
        r.eager_len = 0;
        r.max_band = x.band;
        r.pad_ = 0;
        const uint64_t btab = uniform64((uint64_t)(uintptr_t)op_state.btab);
        if (fresh_lane_id() == 0) {
            *o = r;
            a.op_btab[sid] = btab;
            if (x.overflow) {
                const uint32_t k = atomicAdd(a.overflow_count, 1u);
                a.overflow_list[k] = sid;
            } else if (pool_out) {
                const uint32_t k = atomicAdd(a.op_fail_count, 1u);
                a.op_fail_list[k] = sid;
            } else {
                atomicAdd((unsigned long long *)a.exec_cells, (unsigned long long)x.cells);
                const uint32_t k = atomicAdd(a.op_done_count, 1u);
                a.op_done_list[k] = sid;
            }
        }
        if (a.op_fin && !x.overflow && !pool_out) {
            // Publish the finished side to the tail walk: its rows, headers,
            // block table and result must be written back past this XCD's L2
            // before the walk reads them.  Every store of the wave is first
            // acknowledged by the L2; a side that then finds the flush not
            // begun leaves the write-back to tail_flush_kernel, which sets
            // its flag before writing back every XCD's L2 and runs before the
            // walk; a side that finds it begun writes back its own L2.
            // (the signal fences keep the compiler from moving memory
            // operations across the wait, the load and the flag store)
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_s_waitcnt(0);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            const uint32_t flushed = __hip_atomic_load(a.op_flushed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (uniform((int)flushed) != 0) {
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                // (the write-back done before the flag: the compiler's own
                // wait after it is dropped when no store is outstanding)
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if (fresh_lane_id() == 0) __hip_atomic_store(a.op_fin + idx, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        return;
    }
    if (EXEC) {
        const ExecItem it = a.exec[item];
        SideResult x;
        if constexpr (PK) x = run_side_pk<EXEC>(task, a.sc, it.dstar, nullptr, xfer,
                                                a.ptr_ws + (it.ptr_off - a.ptr_base_off), it.ptr_bytes);
        else x = run_side<C, EXEC, SUB>(task, a.sc, it.dstar, nullptr, xfer,
                                        a.ptr_ws + (it.ptr_off - a.ptr_base_off), it.ptr_bytes);
        if (fresh_lane_id() == 0) {
            atomicAdd((unsigned long long *)a.exec_cells, (unsigned long long)x.cells);
            if (x.overflow || x.best != o->score || x.bi != o->ie) atomicOr(&o->flags, SO_EXEC_MISMATCH);
        }
        return;
    }
    SideResult x;
    if constexpr (PK) x = run_side_pk<EXEC>(task, a.sc, 0x7fffffff, eager_lds, xfer, nullptr, 0);
    else x = run_side<C, EXEC, SUB>(task, a.sc, 0x7fffffff, eager_lds, xfer, nullptr, 0);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    SideOut r;
    r.score = x.best;
    r.ie = x.bi;
    r.je = x.bj;
    r.dend = x.dend;
    r.cells = x.cells;
    r.ptr_bytes = x.ptr_at_best;
    r.flags = (x.overflow ? SO_OVERFLOW : 0) | a.result_flags;
    r.eager_len = 0;
    r.max_band = x.band;
    r.pad_ = 0;
    const bool deferred = x.state == SidePk<2, false>::END_DEFER;
    if (deferred) r.flags = SO_DEFERRED;
    if (!x.overflow && !deferred && x.bi <= EAGER_EDGE && x.bj <= EAGER_EDGE) {
        // the best cell lies in the eager block, which the start layout
        // kept (no layout change happens before diagonal 34)
        EDP e(task, a.sc);
        e.bi = x.bi;
        e.bj = x.bj;
        r.flags |= SO_EAGER;
        r.eager_len = e.eager_walk(eager_lds, a.eager_ops + (int64_t)sid * EAGER_OPS);
    }
    if constexpr (C > 8 && !EXEC) {
        // (the wide retry beside the one-pass executor) a side whose seed is
        // now certain to be traced is traced at once: the executor sweeps it
        // again to its best cell in this wave, into the early workspace.  The
        // other side is final unless it is in this retry too (then the side
        // waits for the executor phase); a torn read of it only changes
        // which path traces the side, the walk takes traced sides only.
        if (a.early_items && !x.overflow && !(r.flags & SO_EAGER)) {
            const SideOut p = a.out[sid ^ 1];
            const int64_t seed_score = reinterpret_cast<const int64_t *>(a.info)[2 * (sid >> 1)];
            bool traced = (p.flags & SO_DEFERRED) != 0;
            if (!traced && !(p.flags & (SO_OVERFLOW | SO_SKIPPED)))
                traced = (int64_t)x.best + seed_score + p.score > a.min_tb;
            if (traced) {
                const uint64_t need = ((uint64_t)x.ptr_at_best + 15) & ~(uint64_t)15;
                uint64_t off = 0;
                if (fresh_lane_id() == 0) off = atomicAdd(a.early_bytes, (unsigned long long)need);
                off = uniform64(off);
                if (off + need <= a.early_cap) {
                    const SideResult e = run_side<C, true, SUB>(task, a.sc, x.bi + x.bj, nullptr, xfer,
                                                                a.early_ws + off, x.ptr_at_best);
                    r.flags |= SO_EARLY;
                    if (e.overflow || e.best != x.best || e.bi != x.bi) r.flags |= SO_EXEC_MISMATCH;
                    if (fresh_lane_id() == 0) {
                        atomicAdd((unsigned long long *)a.exec_cells, (unsigned long long)e.cells);
                        ExecItem it;
                        it.side = sid;
                        it.dstar = x.bi + x.bj;
                        it.ptr_off = (int64_t)off;
                        it.ptr_bytes = x.ptr_at_best;
                        it.batch = 0;
                        a.early_items[atomicAdd(a.early_count, 1u)] = it;
                    }
                }
            }
        }
    }
    if (fresh_lane_id() == 0) {
        *o = r;
        if (deferred) {
            const uint32_t k = atomicAdd(a.defer_count, 1u);
            a.defer_list[k] = sid;
            atomicAdd(a.defer_diags, (unsigned long long)((int64_t)task.m + task.n + 1));
        } else if (x.overflow) {
            const uint32_t k = atomicAdd(a.overflow_count, 1u);
            a.overflow_list[k] = sid;
        }
    }
}

}  // namespace fz

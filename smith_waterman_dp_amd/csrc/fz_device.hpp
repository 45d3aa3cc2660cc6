// fz_device.hpp -- records and wave64 helpers shared by the libfz kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fz {

// "Minus infinity" for scores.  Live scores stay above T_FLOOR (the library
// rejects windows whose worst-case score could reach it), so anything built
// from NEG stays below every threshold and never wraps.
constexpr int32_t NEG = -(1 << 30);
constexpr int32_t T_FLOOR = -(1 << 29);
constexpr int64_t SCORE_LIMIT = (int64_t)1 << 29;

// Padding (bases) around the packed sequences: kernels read whole window
// rows that may run past a window edge.
constexpr int64_t PAD = 4096;

// Eager traceback block of FastZ section 3.1.2: extensions whose best cell
// has i, j <= 16 are traced inside the inspector.
constexpr int EAGER_EDGE = 16;
constexpr int EAGER_ROWS = 2 * EAGER_EDGE + 1;   // anti-diagonals 0..32
constexpr int EAGER_OPS = 2 * EAGER_EDGE;

// Length bins of FastZ section 3.3: 512, 2048, 8192, 32768, then x4.
constexpr int NBINS = 8;

// How a kernel scores a base pair (its template argument):
//   SUB_WIDE    match / transition / transversion from the xor of the codes,
//               any int32 scores;
//   SUB_LUT     the same three scores as int8, one byte permute per four
//               cells (the xor of two codes, 0..3, selects the byte);
//   SUB_MATRIX  a 4x4 int8 matrix plus an N score (see matrix_scores).
enum : int { SUB_WIDE = 0, SUB_LUT = 1, SUB_MATRIX = 2 };

// Byte codes in the matrix mode.  Codes of the other modes are the bases
// 0..3 (A, C, G, T) in both sequences.  Here the target and the query are
// coded differently, so that OR-ing a target byte with a query byte gives a
// byte-permute selector into the matrix: the query byte is its base (bits
// 0-1), the target byte has its base's low bit at bit 2 and its high bit at
// bit 6, and N is bit 7 in either.
constexpr uint32_t MX_N = 0x80u;
__host__ __device__ constexpr uint32_t mx_target_code(uint32_t base) { return ((base & 1u) << 2) | ((base >> 1) << 6); }

struct Scoring {
    int32_t match, ts, tv;      // substitution scores (SUB_WIDE, SUB_LUT)
    int32_t oe, e;              // open + extend, extend
    uint32_t lut;               // int8 score per xor code (A=0,C=1,G=2,T=3): [match, tv, ts, tv]
    int32_t ydrop;              // >= 0; values >= SCORE_LIMIT act as "no pruning"
    int32_t small;              // lut usable (all three scores fit int8)
    int32_t mode;               // SUB_* the kernels are launched with
    uint32_t mrow[4];           // SUB_MATRIX: row a (target A, C, G, T), byte b = score against query base b
    uint32_t nrep;              // SUB_MATRIX: the N score in all four bytes
    int32_t nsc;                // SUB_MATRIX: the N score
    int32_t msub;               // largest |substitution score| (range checks)
};

// SUB_MATRIX: the four int8 scores of four cells from sel = target bytes |
// query bytes.  A selector byte 0..7 picks from rows A and C (one permute),
// 0x40..0x47 from rows G and T (a second permute after flipping bit 6); the
// permute returns 0xFF for any selector byte of 13 or more, so each byte is
// right in one permute and all ones in the other, and AND keeps the right
// one.  Bit 7 (N) makes both all ones; a third permute spreads each byte's
// bit 7 over the byte (selectors 8..11 copy the top bit of bytes 1, 3, 5, 7
// of the pair (sel, sel << 8), which are sel's bytes 0, 2, 1, 3), and that
// mask puts the N score in those bytes.
__device__ __forceinline__ uint32_t matrix_scores(uint32_t sel, const Scoring &sc)
{
    const uint32_t lo = __builtin_amdgcn_perm(sc.mrow[1], sc.mrow[0], sel);
    const uint32_t hi = __builtin_amdgcn_perm(sc.mrow[3], sc.mrow[2], sel ^ 0x40404040u);
    const uint32_t nmask = __builtin_amdgcn_perm(sel, sel << 8, 0x0B090A08u);
    return ((lo & hi) & ~nmask) | (sc.nrep & nmask);
}

// Score of one target code against one query code, any mode (setup and
// per-row profiles; not the per-cell path).
__host__ __device__ inline int sub_pair(uint32_t ta, uint32_t qb, const Scoring &sc)
{
    if (sc.mode == SUB_MATRIX) {
        if ((ta | qb) & MX_N) return sc.nsc;
        const uint32_t a = ((ta >> 2) & 1u) | ((ta >> 5) & 2u);
        const uint32_t row = a == 0 ? sc.mrow[0] : a == 1 ? sc.mrow[1] : a == 2 ? sc.mrow[2] : sc.mrow[3];
        return (int)(int8_t)((row >> (8 * (qb & 3u))) & 0xFFu);
    }
    const uint32_t x = ta ^ qb;
    return x == 0 ? sc.match : (x == 2 ? sc.ts : sc.tv);
}

// One side of one seed.  a_i = A[abase + i], b_j = B[bbase - j] for
// i = 1..m, j = 1..n.  A and B are padded code arrays (0..3), so every
// index a kernel forms for cells near the window stays inside them.
struct SideTask {
    const uint8_t *A;
    const uint8_t *B;
    const uint8_t *A16;         // the same sequences as 16-bit codes (packed layouts), same element index
    const uint8_t *B16;
    int64_t abase, bbase;
    int32_t m, n;               // m < 0: skip (invalid seed)
    int32_t seed, side;         // side 0 = left, 1 = right
    // The inspector hands the side to the one-pass executor when, at
    // anti-diagonal ONEPASS_AT (or AT2, AT3), its best score is at least this (its seed is
    // then traced whatever the other side scores) and still growing;
    // INT32_MAX: never.
    int32_t defer_need, pad_;
};

// SO_DEFERRED: the inspector stopped the side at a hand-over test for the one-pass
// executor (a transient state); SO_ONEPASS: the one-pass executor extended
// it and wrote its complete pointer rows (walked from its block table);
// SO_WALKED: ... and it was walked at once, its runs in the one-pass runs
// buffer (an earlier round of a batch whose one-pass rows did not all fit
// the pool at once).
// SO_EARLY: a side of the wide retry that the retry's wave also traced (its
// rows in the early workspace, an item of the early list); it is only
// walked with the other executor sides.
// SO_TAIL: a one-pass side walked while the one-pass executor still ran
// (the tail walk); its runs are in the tail buffer at op_run_off[side]
// until a round's packing moves them to the one-pass runs buffer.
enum : int32_t {
    SO_OVERFLOW = 1, SO_EAGER = 2, SO_SKIPPED = 4, SO_EXEC_MISMATCH = 8, SO_WIDE_FLAG = 16,
    SO_DEFERRED = 32, SO_ONEPASS = 64, SO_WALKED = 128, SO_EARLY = 256, SO_TAIL = 512
};

struct SideOut {
    int32_t score, ie, je, dend;
    int64_t cells;
    int64_t ptr_bytes;          // executor pointer bytes through the best anti-diagonal
    int32_t flags, eager_len;
    int32_t max_band, pad_;     // widest range R_d of the side
};

// One side queued for the executor / walker.
struct ExecItem {
    int32_t side;               // index into tasks / side outputs
    int32_t dstar;              // anti-diagonal of the best cell
    int64_t ptr_off;            // byte offset of its pointer rows (whole list; a batch subtracts its base)
    int64_t ptr_bytes;
    int64_t batch;
};

// Row header of the executor's pointer store, one per anti-diagonal.  A
// row word holds 6 or 8 consecutive positions' nibbles: 8 when off carries
// ROW_CPW8 (the 1024-position and the packed 256-position layouts), 6
// otherwise.  The 32-bit layouts put the first position in the highest
// nibble.  The packed layouts (ROW_PK) put cell k of a word (k = p % 6, or
// p % 8 with ROW_CPW8, where the odd lane of a pair fills the upper half)
// at bit 16 * (k >> 2) + 8 * (k & 1) + 4 * ((k >> 1) & 1), and store the
// PTR_DIAG and PTR_FROM_I bits inverted.
constexpr uint32_t ROW_CPW8 = 0x80000000u;
constexpr uint32_t ROW_PK = 0x40000000u;
constexpr uint32_t ROW_OFF_MASK = 0x3FFFFFFFu;
struct RowHdr {
    uint32_t off;               // dword offset of the row inside the side's row area (| format flags)
    int32_t ibase;              // i of slot 0 of the row's first lane
};

// Longest side window: keeps every position, and the walker's packed
// (position, row format) words, far inside 32 bits.
constexpr int64_t MAX_SIDE_LEN = (int64_t)1 << 28;

// One-pass executor (sides whose seed is certain to be traced once they pass
// ONEPASS_AT with a growing best): one extension that writes its pointer
// rows as it goes, without a known end.  Its rows go to blocks of OP_BLOCK
// anti-diagonals, each laid out like an executor area: OP_BLOCK + 1 row
// headers (the last one holds only the block's word count, so that every
// row's end is the next header's offset), then the rows, at most
// OP_ROW_WORDS words each, offsets relative to the block's first row word.
// A side's block table (one 64-bit address per block) and its blocks are
// carved out of per-wave arenas of OP_ARENA bytes taken from one pool.
// Hand-over tests at anti-diagonals 256, 1024 and 4096 (flush points of the
// packed layouts): a long side whose best stalls for a while near 256 and
// grows again is still handed over later, at the cost of the anti-diagonals
// the inspector swept before.
constexpr int ONEPASS_AT = 256;
constexpr int ONEPASS_AT2 = 1024;
constexpr int ONEPASS_AT3 = 4096;
constexpr int ONEPASS_RECENT = 64;          // best found at most this many anti-diagonals before
constexpr int OP_BLOCK = 64;                // anti-diagonals per block (a power of two, a multiple of 8)
constexpr int OP_HDRS = OP_BLOCK + 1;
constexpr int OP_ROW_WORDS = 64;            // widest row of the eager and packed layouts
constexpr int64_t OP_BLOCK_BYTES = ((8 * OP_HDRS + 4 * OP_BLOCK * OP_ROW_WORDS) + 15) & ~(int64_t)15;
constexpr int64_t OP_ARENA = (int64_t)256 << 10;
constexpr uint32_t OP_BLOCK_WORDS = OP_BLOCK * OP_ROW_WORDS;

// Bytes kept readable after every area of pointer rows (the pool, the
// executor's workspaces): the traceback walker loads rows in 16-byte groups
// that may run past a row's last word.
constexpr int64_t WALK_PAD = 256;

// Entries per array of the LDS hand-over between layouts (S of two
// diagonals and the two gap states of the union of the last two hulls,
// which is at most 256 positions wide when a side changes layout).
constexpr int XFER_STRIDE = 256;

// ----------------------------------------------------------- wave helpers --

// A dword in the global address space (device memory): loads through it are
// global_load instructions, which return in order.
typedef __attribute__((address_space(1))) const uint32_t GlobalU32;
typedef __attribute__((address_space(1))) const uint8_t GlobalU8;

// Stores of pointer rows and their headers, which always lie in device
// memory: global (not flat) stores whatever the pointer's provenance.
__device__ __forceinline__ void gstore(uint32_t *p, uint32_t v)
{
    *(__attribute__((address_space(1))) uint32_t *)p = v;
}
__device__ __forceinline__ void gstore64(uint64_t *p, uint64_t v)
{
    *(__attribute__((address_space(1))) uint64_t *)p = v;
}
__device__ __forceinline__ void store_hdr(RowHdr *p, uint32_t off, int32_t ibase)
{
    gstore64(reinterpret_cast<uint64_t *>(p), (uint64_t)off | ((uint64_t)(uint32_t)ibase << 32));
}

// N dwords at any byte address in device memory, as one global load
// (gfx9 and later serve unaligned global loads; the compiler emits a single
// global_load_dword{,x2,x4} for these types).
template <int N> struct Unaligned;
template <> struct Unaligned<1> { typedef uint32_t T __attribute__((aligned(1))); };
template <> struct Unaligned<2> { typedef uint32_t T __attribute__((ext_vector_type(2), aligned(1))); };
template <> struct Unaligned<4> { typedef uint32_t T __attribute__((ext_vector_type(4), aligned(1))); };

template <int N>
__device__ __forceinline__ void load_unaligned(const GlobalU8 *p, uint32_t (&out)[N])
{
    typedef typename Unaligned<N>::T V;
    const V v = *reinterpret_cast<const __attribute__((address_space(1))) V *>(p);
    if constexpr (N == 1) {
        out[0] = v;
    } else {
#pragma unroll
        for (int k = 0; k < N; ++k) out[k] = v[k];
    }
}

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// The lane id computed afresh where it is used (two VALU instructions the
// compiler cannot merge with other computations of it), so that it need not
// stay in a register, or be spilled, across a long loop that does not use it.
__device__ __forceinline__ int fresh_lane_id()
{
    int r;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(r));
    return r;
}

// Lane l receives lane l+1's value; lane 63 receives `fill`.
__device__ __forceinline__ int from_next_lane(int v, int fill)
{
    return __builtin_amdgcn_update_dpp(fill, v, 0x130 /* wave_shl:1 */, 0xF, 0xF, false);
}

// Lane l receives lane l-1's value; lane 0 receives `fill`.
__device__ __forceinline__ int from_prev_lane(int v, int fill)
{
    return __builtin_amdgcn_update_dpp(fill, v, 0x138 /* wave_shr:1 */, 0xF, 0xF, false);
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// ------------------------------------------------------ traceback pointers --
// One 4-bit pointer per cell (FastZ section 3.1.3), built by shifting bits
// into a dword, most significant first:
//   PTR_DIAG (bit 3)  S came by the diagonal move (H)
//   PTR_FROM_I (2)    S came from I (taken when not PTR_DIAG)
//   PTR_EXT_I (1)     the I handed to the right neighbour extends this I
//   PTR_EXT_D (0)     the D handed to the lower neighbour extends this D
// A lane's C cells fill ceil(C/8) dwords, eight cells each; the first cell
// of a dword ends up in its highest nibble.
enum : uint32_t { PTR_DIAG = 8, PTR_FROM_I = 4, PTR_EXT_I = 2, PTR_EXT_D = 1 };

// w * 2 + bit, with the bit taken from the lane mask of a comparison (one
// v_addc: the comparison's mask is the carry-in).
__device__ __forceinline__ uint32_t shift_in(uint32_t w, bool bit)
{
    const uint64_t m = ballot(bit);
    uint32_t r;
    asm("v_addc_co_u32_e64 %0, vcc, %1, %1, %2" : "=v"(r) : "v"(w), "s"(m) : "vcc");
    return r;
}

// Bit offset of the nibble of slot c (0 .. C-1) inside its dword.
template <int C>
__device__ __forceinline__ int ptr_shift(int c)
{
    const int n = (C - (c / 8) * 8) < 8 ? (C - (c / 8) * 8) : 8;    // cells in c's dword
    return 4 * (n - 1 - c % 8);
}

// Source of S from a pointer: 0 diagonal, 1 I, 2 D.
__device__ __forceinline__ uint32_t ptr_src(uint32_t nib)
{
    return (nib & PTR_DIAG) ? 0u : ((nib & PTR_FROM_I) ? 1u : 2u);
}

// Maximum over the wave (every lane active), by DPP moves only: within
// quads, then 8-lane halves, then 16-lane rows; then the row broadcasts
// fold rows 0-1 into row 1, rows 2-3 into row 3 and rows 0-1 into rows
// 2-3, leaving the wave's maximum in lane 63.
__device__ __forceinline__ int wave_max(int v)
{
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false));    // quad_perm [1,0,3,2]
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false));    // quad_perm [2,3,0,1]
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x141, 0xF, 0xF, false));   // row_half_mirror
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x140, 0xF, 0xF, false));   // row_mirror
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x142, 0xA, 0xF, false));   // row_bcast:15 -> rows 1, 3
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x143, 0xC, 0xF, false));   // row_bcast:31 -> rows 2, 3
    return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint64_t uniform64(uint64_t x)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ int ctz64(uint64_t x) { return __builtin_ctzll(x); }
__device__ __forceinline__ int hibit64(uint64_t x) { return 63 - __builtin_clzll(x); }

// Lanes [lo, hi] as a mask (empty when hi < lo); lo, hi clamped to 0..63.
__device__ __forceinline__ uint64_t lane_range(int lo, int hi)
{
    lo = lo < 0 ? 0 : lo;
    hi = hi > 63 ? 63 : hi;
    if (hi < lo) return 0ull;
    return (~0ull >> (63 - hi)) & (~0ull << lo);
}

__device__ __forceinline__ int floordiv(int a, int b)
{
    int q = a / b;
    return (q * b > a) ? q - 1 : q;
}

// NW little-endian dwords holding bytes p[x], p[x+1], ... built from
// dword-aligned loads (p itself is 256-byte aligned).
template <int NW>
__device__ __forceinline__ void load_bytes(const uint8_t *p, int64_t x, uint32_t (&out)[NW])
{
    const uint32_t *w = reinterpret_cast<const uint32_t *>(p + (x & ~(int64_t)3));
    const uint32_t sh = (uint32_t)(x & 3);
    uint32_t raw[NW + 1];
#pragma unroll
    for (int k = 0; k <= NW; ++k) raw[k] = w[k];
#pragma unroll
    for (int k = 0; k < NW; ++k) out[k] = __builtin_amdgcn_alignbyte(raw[k + 1], raw[k], sh);
}

}  // namespace fz

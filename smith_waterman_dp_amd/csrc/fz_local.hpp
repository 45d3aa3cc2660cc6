// fz_local.hpp -- full-window local alignment, score and end cell (gfx950).
//
// S = max(0, H, I, D) over the whole window with affine gaps, no y-drop (the
// local recurrence with a zero clamp applied last, as the DPX article's
// section 1.1 and section 3.2 give it, with FastZ's three-state gap model).
//
// One wave64 per pair.  The window's rows are cut into strips of 64 * RL
// rows; lane l owns rows l*RL .. l*RL + RL - 1 of the strip and keeps, per
// row, S of the previous column and the I handed to the next column in
// registers.  Columns are swept left to right with a one-step skew between
// lanes (lane l works on column t - l at step t), so the only values that
// cross lanes are the S and D of a lane's last row, passed down by one DPP
// move per step.  The strip's last row is spilled to memory for the next
// strip (FastZ section 3.2's strip-boundary spill).  The substitution score
// comes from a per-row profile: four int8 scores (one per query base) packed
// in one register, so a cell's score is one signed byte extract.  With a
// substitution matrix the profile is the matrix row of the row's target base
// (the N score in every byte for N), and a query N takes the N score.
//
// End cell: largest S, ties to the smallest anti-diagonal d = i + j, then
// the smallest i; (0,0) when nothing scores above 0.
#pragma once

#include "../../include/fz.h"
#include "fz_device.hpp"

namespace fz {

struct LocalArgs {
    const fz_seed *seeds;
    int64_t n;
    int64_t tlen, qlen;
    const uint8_t *Tf, *Qf;     // padded codes
    Scoring sc;
    fz_hit *hits;
    int32_t *bnd;               // strip spill: 2 * (max_n + 1) ints per wave slot
    int64_t bnd_stride;
};

template <int RL, int SUB, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void local_kernel(LocalArgs a)
{
    constexpr bool SMALL = SUB != SUB_WIDE;
    const int lane = lane_id();
    const int64_t wave = (int64_t)blockIdx.x * WAVES + threadIdx.x / 64;
    if (wave >= a.n) return;
    const fz_seed s = a.seeds[wave];
    fz_hit h = {};
    h.bin = -1;
    const bool ok = s.t_lo >= 0 && s.q_lo >= 0 && s.t_hi <= a.tlen && s.q_hi <= a.qlen && s.t_lo <= s.t_hi &&
                    s.q_lo <= s.q_hi;
    if (!ok) {
        if (lane == 0) {
            h.status = FZ_HIT_ESEED;
            a.hits[wave] = h;
        }
        return;
    }
    const int m = (int)(s.t_hi - s.t_lo), n = (int)(s.q_hi - s.q_lo);
    const Scoring &sc = a.sc;
    const int64_t msub = sc.msub;
    if ((msub + sc.e) * ((int64_t)m + n + 2) + sc.oe >= SCORE_LIMIT / 2) {
        if (lane == 0) {
            h.status = FZ_HIT_ERANGE;
            a.hits[wave] = h;
        }
        return;
    }
    const uint8_t *A = a.Tf + PAD + s.t_lo;     // a_i = A[i - 1]
    const uint8_t *B = a.Qf + PAD + s.q_lo;     // b_j = B[j - 1]
    int32_t *bndS = a.bnd + wave * a.bnd_stride;
    int32_t *bndD = bndS + (a.bnd_stride / 2);

    int best = 0, bd = 0, bi = 0;               // this lane's best and its (d, i)
    for (int row0 = 0; row0 < m; row0 += 64 * RL) {
        const bool first = row0 == 0;
        const int ilane = row0 + lane * RL;     // rows ilane+1 .. ilane+RL
        int Sl[RL], Ir[RL];
        uint32_t prof[RL];
#pragma unroll
        for (int r = 0; r < RL; ++r) {
            const int i = ilane + r + 1;
            const int ca = i <= m ? A[i - 1] : 0;
            // byte b of prof: score of a_i against query base b
            uint32_t p = 0;
            if (SUB == SUB_MATRIX) {
                // the matrix row of a_i (the N score throughout for N)
                const uint32_t ua = (uint32_t)ca;
                const uint32_t ra = ((ua >> 2) & 1u) | ((ua >> 5) & 2u);
                p = (ua & MX_N) ? sc.nrep
                                : ra == 0 ? sc.mrow[0] : ra == 1 ? sc.mrow[1] : ra == 2 ? sc.mrow[2] : sc.mrow[3];
            } else if (SMALL) {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int x = ca ^ b;
                    const int sv = x == 0 ? sc.match : (x == 2 ? sc.ts : sc.tv);
                    p |= ((uint32_t)sv & 0xFFu) << (8 * b);
                }
            } else {
                p = (uint32_t)ca;
            }
            prof[r] = p;
            Sl[r] = 0;                           // S(i, 0) = 0
            Ir[r] = -sc.oe;                      // I handed to column 1: max(-inf - E, 0 - O - E)
        }
        const bool full = ilane + RL <= m;      // all my rows inside the window
        const bool strip_full = __ballot(!full) == 0;
        int outS = 0, outD = NEG;               // my last row's S, D of the column just done
        int recv_prev = 0;                      // S(row above my first row, j - 1)
        const int steps = n + 63;
        for (int t = 0; t < steps; ++t) {
            const int j = t - lane + 1;
            const bool active = j >= 1 && j <= n;
            int fillS = 0, fillD = NEG;
            if (!first && lane == 0 && active) {
                fillS = bndS[j];
                fillD = bndD[j];
            }
            const int upS0 = from_prev_lane(outS, fillS);
            const int upD0 = from_prev_lane(outD, fillD);
            const int diag0 = recv_prev;
            recv_prev = upS0;
            int colmax = 0;
            if (active) {
                const int bj = B[j - 1];
                const uint32_t sh = 8u * ((uint32_t)bj & 3u);
                const bool colN = SUB == SUB_MATRIX && ((uint32_t)bj & MX_N);   // query base N
                int diag = diag0, uS = upS0, uD = upD0;
#pragma unroll
                for (int r = 0; r < RL; ++r) {
                    int sub;
                    if (SUB == SUB_MATRIX) {
                        sub = colN ? sc.nsc : (int)(int8_t)((prof[r] >> sh) & 0xFFu);
                    } else if (SMALL) {
                        sub = (int)(int8_t)((prof[r] >> sh) & 0xFFu);
                    } else {
                        const int x = (int)prof[r] ^ bj;
                        sub = x == 0 ? sc.match : (x == 2 ? sc.ts : sc.tv);
                    }
                    const int H = diag + sub;
                    const int I = Ir[r];
                    const int D = max(uD - sc.e, uS - sc.oe);
                    int S = max(max(max(H, I), D), 0);
                    if (!strip_full && ilane + r + 1 > m) S = 0;   // rows past the window
                    diag = Sl[r];
                    Sl[r] = S;
                    Ir[r] = max(I - sc.e, S - sc.oe);
                    uS = S;
                    uD = D;
                    colmax = max(colmax, S);
                }
                outS = uS;
                outD = uD;
                if (lane == 63 && row0 + 64 * RL < m) {
                    bndS[j] = uS;
                    bndD[j] = uD;
                }
            }
            // best cell: only when this column can beat or tie-improve the lane's best
            const bool trig = active && colmax > 0 &&
                              (colmax > best || (colmax == best && ilane + 1 + j < bd));
            if (__ballot(trig)) {
                if (trig) {
                    int rf = RL;
#pragma unroll
                    for (int r = RL - 1; r >= 0; --r)
                        if (Sl[r] == colmax) rf = r;
                    const int i = ilane + rf + 1;
                    const int dnew = i + j;
                    if (colmax > best || dnew < bd || (dnew == bd && i < bi)) {
                        best = colmax;
                        bd = dnew;
                        bi = i;
                    }
                }
            }
        }
        __threadfence();
    }
    // wave reduction: max score, then smallest d, then smallest i
    const int wb = wave_max(best);
    int kd = best == wb ? bd : 0x7fffffff;
    for (int off = 32; off >= 1; off >>= 1) kd = min(kd, __shfl_xor(kd, off));
    int ki = (best == wb && bd == kd) ? bi : 0x7fffffff;
    for (int off = 32; off >= 1; off >>= 1) ki = min(ki, __shfl_xor(ki, off));
    if (lane == 0) {
        h.score = wb;
        if (wb == 0) {
            kd = 0;
            ki = 0;
        }
        h.t_begin = s.t_lo;
        h.q_begin = s.q_lo;
        h.t_end = s.t_lo + ki;
        h.q_end = s.q_lo + (kd - ki);
        h.cells = (int64_t)m * n;
        h.score_right = wb;
        a.hits[wave] = h;
    }
}

}  // namespace fz

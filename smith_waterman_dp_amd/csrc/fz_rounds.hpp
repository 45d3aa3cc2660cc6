// fz_rounds.hpp -- covered-seed suppression by rounds (gfx950).
//
// FastZ (SC'21) section 2.1 describes LASTZ ending a seed extension that runs
// into an alignment it found earlier, and section 3.4 why FastZ drops the
// rule: it makes each extension depend on the ones before it.  The form
// built here keeps the extensions of one round independent (a batch for the
// usual pipeline) and applies the rule between rounds: a seed whose
// exact-match columns share a cell with an aligned (M) column of an
// alignment traced in an earlier round is not extended.
//
// The aligned columns of traced alignments are kept as segments on
// diagonals: one per M run, key ((t - q + query_len) << 32) | t_first and
// end t_last + 1.  After each round the segments are sorted by key and a max
// scan of (diagonal << 32) | end gives, at every index, the largest end of
// the segments up to it on its diagonal (the diagonal part never decreases
// in key order, so the maximum always carries the current diagonal).  A
// seed's columns [t, t + L) on diagonal d then meet some segment iff the
// last segment with key <= (d, t + L - 1) lies on d and that running
// maximum end exceeds t: one binary search per seed.
#pragma once

#include <stdint.h>

#include "../../include/fz.h"
#include "fz_device.hpp"

namespace fz {

// keep[k] = 1 unless seed k of the round is covered.  Seeds without
// columns, or with columns outside the sequences, are never covered.
__global__ void cover_kernel(const fz_seed *__restrict__ seeds, int64_t n, int64_t tlen, int64_t qlen,
                             const uint64_t *__restrict__ segkey, const uint64_t *__restrict__ segmax, int64_t nseg,
                             uint32_t *__restrict__ keep)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n) return;
    const fz_seed s = seeds[k];
    uint32_t kp = 1;
    if (nseg > 0 && s.seed_len >= 1 && s.t_pos >= 0 && s.q_pos >= 0 && s.t_pos + s.seed_len <= tlen &&
        s.q_pos + s.seed_len <= qlen) {
        const uint64_t dg = (uint64_t)(s.t_pos - s.q_pos + qlen);
        const uint64_t hi = (dg << 32) | (uint64_t)(s.t_pos + s.seed_len - 1);
        int64_t a = 0, b = nseg;            // first index with key > hi
        while (a < b) {
            const int64_t m = (a + b) >> 1;
            if (segkey[m] <= hi) a = m + 1;
            else b = m;
        }
        if (a > 0) {
            const uint64_t mx = segmax[a - 1];
            if ((mx >> 32) == dg && (int64_t)(mx & 0xffffffffull) > s.t_pos) kp = 0;
        }
    }
    keep[k] = kp;
}

// The kept seeds, packed in order (pos = exclusive scan of keep).
__global__ void compact_seeds_kernel(const fz_seed *__restrict__ seeds, int64_t n, const uint32_t *__restrict__ keep,
                                     const uint32_t *__restrict__ pos, fz_seed *__restrict__ out)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n || !keep[k]) return;
    out[pos[k]] = seeds[k];
}

// Every seed of the round gets its record: the extension's result (CIGAR
// offset moved past the words of earlier rounds), or the covered record.
__global__ void scatter_hits_kernel(const fz_hit *__restrict__ rhits, int64_t n, const uint32_t *__restrict__ keep,
                                    const uint32_t *__restrict__ pos, int64_t cig_base, fz_hit *__restrict__ out)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n) return;
    fz_hit h;
    if (keep[k]) {
        h = rhits[pos[k]];
        h.cigar_off += cig_base;
    } else {
        h = fz_hit{};
        h.status = FZ_HIT_COVERED;
        h.bin = -1;
    }
    out[k] = h;
}

// Number of M runs in each traced alignment's CIGAR.
__global__ void seg_count_kernel(const fz_hit *__restrict__ hits, int64_t n, const uint32_t *__restrict__ cigar,
                                 uint64_t *__restrict__ cnt)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n) return;
    const fz_hit h = hits[k];
    uint64_t c = 0;
    if (h.status & FZ_HIT_TRACED)
        for (int64_t w = 0; w < h.cigar_len; ++w) c += (cigar[h.cigar_off + w] & 15u) == 0u;
    cnt[k] = c;
}

// The M runs as segments, walking each CIGAR from (t_begin, q_begin).
__global__ void seg_emit_kernel(const fz_hit *__restrict__ hits, int64_t n, const uint32_t *__restrict__ cigar,
                                const uint64_t *__restrict__ off, int64_t qlen, uint64_t *__restrict__ key,
                                uint32_t *__restrict__ end)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n) return;
    const fz_hit h = hits[k];
    if (!(h.status & FZ_HIT_TRACED)) return;
    int64_t t = h.t_begin, q = h.q_begin;
    uint64_t o = off[k];
    for (int64_t w = 0; w < h.cigar_len; ++w) {
        const uint32_t word = cigar[h.cigar_off + w];
        const int64_t len = (int64_t)(word >> 4);
        const uint32_t op = word & 15u;
        if (op == 0u) {
            key[o] = ((uint64_t)(t - q + qlen) << 32) | (uint64_t)t;
            end[o] = (uint32_t)(t + len);
            ++o;
            t += len;
            q += len;
        } else if (op == 1u) {
            q += len;
        } else {
            t += len;
        }
    }
}

// (diagonal << 32) | end of every sorted segment, for the running maximum.
__global__ void seg_diag_end_kernel(const uint64_t *__restrict__ key, const uint32_t *__restrict__ end, int64_t n,
                                    uint64_t *__restrict__ v)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    v[i] = (key[i] & 0xffffffff00000000ull) | (uint64_t)end[i];
}

}  // namespace fz

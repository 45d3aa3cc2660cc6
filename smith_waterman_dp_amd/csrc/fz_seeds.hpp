// fz_seeds.hpp -- the seed stage on gfx950: shared k-mers of target and query
// and their diagonal dedup.
//
// FastZ (SC'21), section 2: whole-genome alignment first finds short exact
// matches (19 bases) between the two sequences as seed sites, then filters
// them, then extends the survivors with the gapped DP.  This file is the
// first step plus the plainest filter, one seed per run of hits on one
// diagonal:
//   keys    the k codes at every target start position as one base-4
//           number; k-mers holding N (which matches nothing) are dropped
//   sort    the target's (key, position) pairs by key (device radix sort)
//   index   a direct-address table over the top bits of the key: for each
//           bucket, where its keys start in the sorted array (about one key
//           per bucket, so a lookup is two table reads and a short search)
//   join    per query position, its key from the codes, then the range of
//           equal target keys through the table; counts, their exclusive
//           scan, then every hit written as one 64-bit word
//           ((t - q + query_len) << 32 | t)
//   sort    the hit words, which orders hits by diagonal and then by t
//   runs    a hit starts a run unless its word is the previous word + 1
//           (same diagonal, t one further): one seed per run
// The stage is bound by memory traffic (keys and hits through the sorts);
// nothing here is arithmetic-heavy.
#pragma once

#include <stdint.h>

#include "fz_device.hpp"

namespace fz {

// key of every start position p < nkeys: codes[p .. p+k-1], first base most
// significant (k <= 32, two bits per base); valid[p] = 0 when the k bases
// hold an N (code MX_N), which matches nothing
__global__ void kmer_keys_kernel(const uint8_t *__restrict__ codes, int64_t nkeys, int k, uint64_t *__restrict__ keys,
                                 uint32_t *__restrict__ pos, uint32_t *__restrict__ valid)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < nkeys; p += stride) {
        uint64_t key = 0;
        uint32_t any_n = 0;
        for (int i = 0; i < k; ++i) {
            const uint32_t c = codes[p + i];
            any_n |= c;
            key = (key << 2) | (uint64_t)(c & 3u);
        }
        keys[p] = key;
        pos[p] = (uint32_t)p;
        valid[p] = (any_n & MX_N) ? 0u : 1u;
    }
}

// The valid (key, position) pairs, packed in order (vpos = exclusive scan
// of valid).
__global__ void compact_keys_kernel(const uint64_t *__restrict__ keys, const uint32_t *__restrict__ pos,
                                    const uint32_t *__restrict__ valid, const uint32_t *__restrict__ vpos, int64_t n,
                                    uint64_t *__restrict__ okeys, uint32_t *__restrict__ opos)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < n; p += stride) {
        if (!valid[p]) continue;
        okeys[vpos[p]] = keys[p];
        opos[vpos[p]] = pos[p];
    }
}

// Bucket table, step 1: for each non-empty bucket b (key >> shift), one past
// the last index of its keys in the sorted array.  bend[] starts at zero.
__global__ void bucket_end_kernel(const uint64_t *__restrict__ tkeys, int64_t nt, int shift, uint32_t *__restrict__ bend)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nt; i += stride) {
        const uint64_t b = tkeys[i] >> shift;
        if (i == nt - 1 || (tkeys[i + 1] >> shift) != b) bend[b] = (uint32_t)(i + 1);
    }
}
// Step 2 (host side): off[0] = 0 and off[b + 1] = the running maximum of
// bend[0..b], so bucket b's keys are sorted[off[b] .. off[b + 1]).

// For every query position: its key (read from the codes), then where that
// key's run starts in the sorted target keys, and how long it is.
__global__ void join_count_kernel(const uint64_t *__restrict__ tkeys, int64_t nt, const uint32_t *__restrict__ off,
                                  int shift, const uint8_t *__restrict__ qcodes, int64_t nq, int k,
                                  uint32_t *__restrict__ lo_out, uint64_t *__restrict__ cnt)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < nq; q += stride) {
        uint64_t key = 0;
        uint32_t any_n = 0;
        for (int i = 0; i < k; ++i) {
            const uint32_t c = qcodes[q + i];
            any_n |= c;
            key = (key << 2) | (uint64_t)(c & 3u);
        }
        if (nt == 0 || (any_n & MX_N)) {     // no target k-mers, or an N here: no hit
            lo_out[q] = 0;
            cnt[q] = 0;
            continue;
        }
        const uint64_t b = key >> shift;
        uint32_t a = off[b], e = off[b + 1];
        if (shift) {                        // the bucket holds other keys too
            uint32_t x = a, y = e;          // first index with tkeys >= key
            while (x < y) {
                const uint32_t m = x + ((y - x) >> 1);
                if (tkeys[m] < key) x = m + 1;
                else y = m;
            }
            uint32_t u = x, v = e;          // first index with tkeys > key
            while (u < v) {
                const uint32_t m = u + ((v - u) >> 1);
                if (tkeys[m] <= key) u = m + 1;
                else v = m;
            }
            a = x;
            e = u;
        }
        lo_out[q] = a;
        cnt[q] = (uint64_t)(e - a);
    }
}

// Every hit of query position q as ((t - q + qlen) << 32) | t.
__global__ void emit_hits_kernel(const uint32_t *__restrict__ tpos, const uint32_t *__restrict__ lo,
                                 const uint64_t *__restrict__ cnt, const uint64_t *__restrict__ off, int64_t nq,
                                 int64_t qlen, uint64_t *__restrict__ hits)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < nq; q += stride) {
        const uint64_t c = cnt[q];
        const uint64_t base = off[q];
        const uint32_t l = lo[q];
        for (uint64_t i = 0; i < c; ++i) {
            const uint64_t t = tpos[l + i];
            hits[base + i] = ((t - (uint64_t)q + (uint64_t)qlen) << 32) | t;
        }
    }
}

// 1 where a hit starts a run on its diagonal (or every hit, without dedup).
__global__ void run_start_kernel(const uint64_t *__restrict__ hits, int64_t n, int dedup, uint64_t *__restrict__ flag)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        flag[i] = (!dedup || i == 0 || hits[i] != hits[i - 1] + 1) ? 1u : 0u;
}

// The selected hits as seed records, in hit order, windows +-flank clipped
// to the sequences.
__global__ void write_seeds_kernel(const uint64_t *__restrict__ hits, const uint64_t *__restrict__ flag,
                                   const uint64_t *__restrict__ rank, int64_t n, int k, int64_t flank, int64_t tlen,
                                   int64_t qlen, fz_seed *__restrict__ out)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        if (!flag[i]) continue;
        const int64_t t = (int64_t)(hits[i] & 0xffffffffull);
        const int64_t diag = (int64_t)(hits[i] >> 32) - qlen;
        const int64_t q = t - diag;
        fz_seed s;
        s.t_pos = t;
        s.q_pos = q;
        s.seed_len = k;
        s.t_lo = t - flank > 0 ? t - flank : 0;
        s.t_hi = t + k + flank < tlen ? t + k + flank : tlen;
        s.q_lo = q - flank > 0 ? q - flank : 0;
        s.q_hi = q + k + flank < qlen ? q + k + flank : qlen;
        out[rank[i]] = s;
    }
}

}  // namespace fz

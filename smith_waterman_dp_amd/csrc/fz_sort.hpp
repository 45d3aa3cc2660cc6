// fz_sort.hpp -- device-wide scans and a stable LSD radix sort for gfx950.
//
// The seed stage (keys and hit words) and the covered-seed rounds (aligned
// segments) order and count things: exclusive sums of per-element counts,
// running maxima, and sorts of 64-bit keys, alone or with a 32-bit value.
// These are memory-bound kernels; the work per element is a few integer
// operations.
//
// Scans: three launches (per-tile reduction, a one-block scan of the tile
// totals, per-tile scan with the tile's prefix), any associative operation
// with an identity, inclusive or exclusive, in place or not.
//
// Radix sort: least-significant digit first, eight bits per pass; each
// pass is a per-tile digit histogram, an exclusive scan of the histograms
// laid out digit-major (so the scan gives every (digit, tile) its first
// output slot), and a scatter.  The scatter keeps the order of equal digits
// (stability, which LSD sorting needs): each wave owns a contiguous quarter
// of the tile, taken 64 keys at a time in index order; the lanes holding the
// same digit are found with eight ballots (one per digit bit), a key's rank
// among them is the count of such lanes below it, and per-wave, per-digit
// counters in LDS supply the rest of the offset.
#pragma once

#include <stdint.h>

#include "fz_device.hpp"

namespace fz {

// ------------------------------------------------------------------ scans --
constexpr int PS_BLOCK = 256;
constexpr int PS_ITEMS = 8;
constexpr int PS_TILE = PS_BLOCK * PS_ITEMS;

struct ScanSum {
    template <class T> __device__ static T id() { return T(0); }
    template <class T> __device__ static T op(T a, T b) { return a + b; }
};
struct ScanMax {       // unsigned values: 0 is the identity
    template <class T> __device__ static T id() { return T(0); }
    template <class T> __device__ static T op(T a, T b) { return a > b ? a : b; }
};

// Inclusive scan of one value per thread over the block (Hillis-Steele in
// LDS); *total receives the block's aggregate.
template <class T, class OP>
__device__ __forceinline__ T block_inclusive(T v, T *sh, T &total)
{
    const int t = threadIdx.x;
    sh[t] = v;
    __syncthreads();
    for (int off = 1; off < PS_BLOCK; off <<= 1) {
        const T add = t >= off ? sh[t - off] : OP::template id<T>();
        __syncthreads();
        sh[t] = OP::op(add, sh[t]);
        __syncthreads();
    }
    total = sh[PS_BLOCK - 1];
    const T r = sh[t];
    __syncthreads();
    return r;
}

template <class T, class OP>
__global__ __launch_bounds__(PS_BLOCK) void pscan_reduce_kernel(const T *__restrict__ in, int64_t n,
                                                                  T *__restrict__ tile_total)
{
    __shared__ T sh[PS_BLOCK];
    const int64_t base = (int64_t)blockIdx.x * PS_TILE + (int64_t)threadIdx.x * PS_ITEMS;
    T a = OP::template id<T>();
    for (int k = 0; k < PS_ITEMS; ++k)
        if (base + k < n) a = OP::op(a, in[base + k]);
    T tot;
    block_inclusive<T, OP>(a, sh, tot);
    if (threadIdx.x == 0) tile_total[blockIdx.x] = tot;
}

// Exclusive scan of the tile totals in place, one block.
template <class T, class OP>
__global__ __launch_bounds__(PS_BLOCK) void pscan_top_kernel(T *tile_total, int64_t ntiles)
{
    __shared__ T sh[PS_BLOCK];
    T carry = OP::template id<T>();
    for (int64_t b0 = 0; b0 < ntiles; b0 += PS_BLOCK) {
        const int64_t i = b0 + threadIdx.x;
        const T v = i < ntiles ? tile_total[i] : OP::template id<T>();
        T tot;
        const T incl = block_inclusive<T, OP>(v, sh, tot);
        // exclusive = inclusive of the previous thread (carry for thread 0)
        sh[threadIdx.x] = incl;
        __syncthreads();
        const T excl = threadIdx.x == 0 ? carry : OP::op(carry, sh[threadIdx.x - 1]);
        __syncthreads();
        if (i < ntiles) tile_total[i] = excl;
        carry = OP::op(carry, tot);
    }
}

template <class T, class OP, bool INCL>
__global__ __launch_bounds__(PS_BLOCK) void pscan_apply_kernel(const T *in, int64_t n, const T *__restrict__ tile_prefix,
                                                                 T *out)
{
    __shared__ T sh[PS_BLOCK];
    const int64_t base = (int64_t)blockIdx.x * PS_TILE + (int64_t)threadIdx.x * PS_ITEMS;
    T v[PS_ITEMS];
    T a = OP::template id<T>();
    for (int k = 0; k < PS_ITEMS; ++k) {
        v[k] = base + k < n ? in[base + k] : OP::template id<T>();
        a = OP::op(a, v[k]);
    }
    T tot;
    const T incl = block_inclusive<T, OP>(a, sh, tot);
    sh[threadIdx.x] = incl;
    __syncthreads();
    T run = threadIdx.x == 0 ? tile_prefix[blockIdx.x] : OP::op(tile_prefix[blockIdx.x], sh[threadIdx.x - 1]);
    for (int k = 0; k < PS_ITEMS; ++k) {
        if (INCL) run = OP::op(run, v[k]);
        if (base + k < n) out[base + k] = run;
        if (!INCL) run = OP::op(run, v[k]);
    }
}

// ------------------------------------------------------------ radix sort --
constexpr int RS_BLOCK = 256;                    // four waves
constexpr int RS_ROUNDS = 16;                    // 256-key rounds per tile (histogram)
constexpr int RS_TILE = RS_BLOCK * RS_ROUNDS;    // 4096 keys per tile
constexpr int RS_BINS = 256;

// counts[digit * ntiles + tile] = keys of the tile whose digit (bits
// shift .. shift+7 of the key) is `digit`.
__global__ __launch_bounds__(RS_BLOCK) void rs_hist_kernel(const uint64_t *__restrict__ keys, int64_t n, int shift,
                                                          uint32_t *__restrict__ counts, int64_t ntiles)
{
    __shared__ uint32_t h[RS_BINS];
    h[threadIdx.x] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * RS_TILE;
    for (int r = 0; r < RS_ROUNDS; ++r) {
        const int64_t idx = base + (int64_t)r * RS_BLOCK + threadIdx.x;
        if (idx < n) atomicAdd(&h[(uint32_t)(keys[idx] >> shift) & (RS_BINS - 1)], 1u);
    }
    __syncthreads();
    counts[(int64_t)threadIdx.x * ntiles + blockIdx.x] = h[threadIdx.x];
}

// Stable scatter by the digit at `shift`, with offs = the exclusive scan of
// rs_hist_kernel's counts (same layout).  Wave w of the block owns keys
// [w * RS_WAVE_KEYS, (w + 1) * RS_WAVE_KEYS) of the tile and keeps them in
// registers: a first sweep counts its digits, one barrier lets every digit's
// thread turn the four waves' counts into their first output slots, and a
// second sweep scatters, each wave advancing only its own counters (the
// leader of a group of equal digits, the lowest lane, moves its counter on
// after every lane has read it), so the sweeps need no block barrier.
constexpr int RS_WAVES = RS_BLOCK / 64;
constexpr int RS_WAVE_KEYS = RS_TILE / RS_WAVES;     // 1024
constexpr int RS_WAVE_ROUNDS = RS_WAVE_KEYS / 64;    // 16

__device__ __forceinline__ uint64_t rs_peers(uint32_t digit, bool valid)
{
    uint64_t peers = ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const bool bit = (digit >> b) & 1u;
        const uint64_t m = ballot(bit);
        peers &= bit ? m : ~m;
    }
    return peers;
}

template <bool PAIRS>
__global__ __launch_bounds__(RS_BLOCK) void rs_scatter_kernel(const uint64_t *__restrict__ kin,
                                                             uint64_t *__restrict__ kout,
                                                             const uint32_t *__restrict__ vin,
                                                             uint32_t *__restrict__ vout, int64_t n, int shift,
                                                             const uint32_t *__restrict__ offs, int64_t ntiles)
{
    __shared__ uint32_t cnt[RS_WAVES][RS_BINS];
    const int t = threadIdx.x, w = t >> 6;
    const int lane = lane_id();
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int q = 0; q < RS_WAVES; ++q) cnt[q][t] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * RS_TILE + (int64_t)w * RS_WAVE_KEYS;
    uint64_t key[RS_WAVE_ROUNDS];
    uint32_t val[RS_WAVE_ROUNDS];
#pragma unroll
    for (int r = 0; r < RS_WAVE_ROUNDS; ++r) {
        const int64_t idx = base + (int64_t)r * 64 + lane;
        key[r] = idx < n ? kin[idx] : 0ull;
        if (PAIRS) val[r] = idx < n ? vin[idx] : 0u;
    }
    // sweep 1: this wave's digit counts
#pragma unroll
    for (int r = 0; r < RS_WAVE_ROUNDS; ++r) {
        const bool valid = base + (int64_t)r * 64 + lane < n;
        const uint32_t digit = (uint32_t)(key[r] >> shift) & (RS_BINS - 1);
        const uint64_t peers = rs_peers(digit, valid);
        if (valid && (peers & below) == 0) cnt[w][digit] += (uint32_t)__popcll(peers);
    }
    __syncthreads();
    // each digit's first slot for each wave
    {
        uint32_t run = offs[(int64_t)t * ntiles + blockIdx.x];
#pragma unroll
        for (int q = 0; q < RS_WAVES; ++q) {
            const uint32_t c = cnt[q][t];
            cnt[q][t] = run;
            run += c;
        }
    }
    __syncthreads();
    // sweep 2: scatter
#pragma unroll
    for (int r = 0; r < RS_WAVE_ROUNDS; ++r) {
        const bool valid = base + (int64_t)r * 64 + lane < n;
        const uint32_t digit = (uint32_t)(key[r] >> shift) & (RS_BINS - 1);
        const uint64_t peers = rs_peers(digit, valid);
        const uint32_t first = cnt[w][digit];
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        if (valid && (peers & below) == 0) cnt[w][digit] = first + (uint32_t)__popcll(peers);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        if (valid) {
            const uint32_t pos = first + (uint32_t)__popcll(peers & below);
            kout[pos] = key[r];
            if (PAIRS) vout[pos] = val[r];
        }
    }
}

}  // namespace fz

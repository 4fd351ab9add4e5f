// moe_permute.h -- grouping of up to a few thousand (token, slot) assignments by expert: by one
// wave in order (permute_wave), or, up to 1024 of them, by a whole workgroup at once
// (permute_block, below).
//
// Same result as the multi-launch grouping in moe_permute.hip (the unique stable order:
// ascending flat index within each expert).  permute_wave, for inputs small enough that one wave
// walks them in order:
//   pass 1  per 64-assignment chunk, peers with the same expert are found with one ballot per
//           bit of the expert id and the lowest peer adds the group's size to cnt[e];
//   scan    lane l owns experts [l*G, (l+1)*G): its sum, a wave exclusive scan, then the
//           experts' offsets in order; cnt[e] becomes the running slot base of expert e;
//   pass 2  per chunk in order: slot = base[e] + (lower peers in the chunk); the lowest peer
//           then advances base[e].
// One wave's LDS operations execute in order, so the per-chunk read-modify-writes need no
// barrier.  Ids outside [0, E) are skipped.
#pragma once

#include "moe_device.h"

namespace moe {

constexpr int kSmallBatch = 8;  // chunks whose ids are loaded together

// ids: n flat assignments (global or LDS); cnt: LDS scratch of E ints.  Whole wave.
__device__ __forceinline__ void permute_wave(const int32_t* ids, int n, int E, int nbits, int* cnt,
                                             int32_t* __restrict__ counts,
                                             int32_t* __restrict__ offsets,
                                             int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    const int lane = lane_id();
    for (int e = lane; e < E; e += kWave) cnt[e] = 0;
    __builtin_amdgcn_wave_barrier();
    const int chunks = (n + kWave - 1) / kWave;
    auto load_batch = [&](int c, int (&ev)[kSmallBatch]) {
#pragma unroll
        for (int b = 0; b < kSmallBatch; ++b) {
            const int f = (c + b) * kWave + lane;
            ev[b] = (c + b < chunks && f < n) ? ids[f] : -1;
        }
    };
    // pass 1: histogram
    for (int c = 0; c < chunks; c += kSmallBatch) {
        int ev[kSmallBatch];
        load_batch(c, ev);
#pragma unroll
        for (int b = 0; b < kSmallBatch; ++b) {
            const int e = ev[b];
            const bool valid = e >= 0 && e < E;
            const uint64_t peers = match_peers(e, valid, nbits);
            if (valid && lane == __ffsll((unsigned long long)peers) - 1) cnt[e] += __popcll(peers);
            __builtin_amdgcn_wave_barrier();
        }
    }
    // scan over experts: lane owns G consecutive experts
    const int G = (E + kWave - 1) / kWave;
    const int e0 = min(E, lane * G), e1 = min(E, e0 + G);
    int local = 0;
    for (int e = e0; e < e1; ++e) local += cnt[e];
    const int incl = wave_inclusive_scan(local);
    int base = incl - local;
    for (int e = e0; e < e1; ++e) {
        const int c = cnt[e];
        counts[e] = c;
        offsets[e] = base;
        cnt[e] = base;
        base += c;
    }
    if (lane == kWave - 1) offsets[E] = incl;
    __builtin_amdgcn_wave_barrier();
    // pass 2: slots
    for (int c = 0; c < chunks; c += kSmallBatch) {
        int ev[kSmallBatch];
        load_batch(c, ev);
#pragma unroll
        for (int b = 0; b < kSmallBatch; ++b) {
            const int f = (c + b) * kWave + lane;
            const int e = ev[b];
            const bool valid = e >= 0 && e < E;
            const uint64_t peers = match_peers(e, valid, nbits);
            int bse = 0;
            if (valid) {
                bse = cnt[e];
                const int pos = bse + __popcll(peers & ((1ull << lane) - 1ull));
                perm[pos] = f;
                inv[f] = pos;
            }
            // the wave's reads of cnt above are issued before this write (in-order LDS per wave)
            __builtin_amdgcn_wave_barrier();
            if (valid && lane == __ffsll((unsigned long long)peers) - 1) cnt[e] = bse + __popcll(peers);
            __builtin_amdgcn_wave_barrier();
        }
    }
}

// The same grouping by a whole workgroup of kBlockThreads threads for n <= kBlockThreads
// assignments, one a thread: per wave, peers with the same expert (one ballot per id bit) and the
// lowest peer records the wave's count of that expert; per expert, the waves' counts become
// running bases (wave order) and the experts' totals an exclusive sum (the offsets); then each
// assignment's slot is offsets[e] + (its wave's base) + (lower peers in its wave).
// ids may be in global memory or LDS; wcnt: LDS scratch of kBlockWaves * E ints, off: E + 1 ints,
// wsum: kBlockWaves ints.  Whole workgroup; E <= kBlockThreads.
constexpr int kBlockWaves = 16;
constexpr int kBlockThreads = kBlockWaves * kWave;

__device__ __forceinline__ void permute_block(const int32_t* ids, int n, int E, int nbits, int* wcnt,
                                              int* off, int* wsum, int32_t* __restrict__ counts,
                                              int32_t* __restrict__ offsets,
                                              int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    const int tid = (int)threadIdx.x, lane = lane_id(), wave = tid >> 6;
    for (int i = tid; i < kBlockWaves * E; i += kBlockThreads) wcnt[i] = 0;
    const int e = tid < n ? ids[tid] : -1;
    const bool valid = e >= 0 && e < E;
    __syncthreads();
    const uint64_t peers = match_peers(e, valid, nbits);
    if (valid && lane == __ffsll((unsigned long long)peers) - 1) wcnt[wave * E + e] = __popcll(peers);
    __syncthreads();
    int total = 0;
    if (tid < E) {
        for (int w = 0; w < kBlockWaves; ++w) {
            const int v = wcnt[w * E + tid];
            wcnt[w * E + tid] = total;
            total += v;
        }
        counts[tid] = total;
    }
    const int incl = wave_inclusive_scan(total);
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const int s = lane < kBlockWaves ? wsum[lane] : 0;
        const int si = wave_inclusive_scan(s);
        if (lane < kBlockWaves) wsum[lane] = si - s;
    }
    __syncthreads();
    if (tid < E) {
        const int excl = wsum[wave] + incl - total;
        off[tid] = excl;
        offsets[tid] = excl;
        if (tid == E - 1) offsets[E] = excl + total;
    }
    __syncthreads();
    if (valid) {
        const int pos = off[e] + wcnt[wave * E + e] + __popcll(peers & ((1ull << lane) - 1ull));
        perm[pos] = tid;
        inv[tid] = pos;
    }
}

}  // namespace moe

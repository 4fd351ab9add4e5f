// moe_permute.h -- grouping of a few thousand (token, slot) assignments by expert, by one wave.
//
// Same result as the workgroup-wide kernel in moe_permute.hip (the unique stable order: ascending
// flat index within each expert), for inputs small enough that one wave walks them in order:
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

}  // namespace moe

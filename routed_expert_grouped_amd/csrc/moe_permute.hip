// moe_permute.hip -- grouping of the (token, slot) assignments by expert.
//
// Tokens that hit the same expert are gathered so that each expert runs one GEMM over all of
// them (KTransformers article, 2.2); in the expert-parallel flow this is the "sorting" after
// gating (OSDI'26 hybrid-inference article, DSLP section).
//
// One workgroup of 16 waves does the whole job, so the order is decided without atomics:
//   pass 1  each wave walks its contiguous run of 64-assignment chunks (the ids of 8 chunks
//           are loaded together, so the loads overlap) and counts, per expert, its own
//           assignments (peers with the same expert are found with one ballot per bit of the
//           expert id; the lowest peer adds the group's size to the wave's LDS row);
//   scan    per expert: exclusive sum over the waves (in wave order) and the total; then an
//           exclusive sum of the totals over experts gives `offsets`;
//   pass 2  each wave walks its chunks again in order; an assignment's slot is
//           offsets[e] + (earlier waves' count of e) + (count of e in this wave's earlier
//           chunks) + (lower peers in its chunk).
// The result is the stable order by construction (ascending flat index within each expert).
// Up to kSmallN assignments one wave does the same in order (moe_permute.h).
#include "libmoe.h"
#include "moe_device.h"
#include "moe_host.h"
#include "moe_permute.h"

namespace moe {

constexpr int kPermWaves = 16;
constexpr int kBatch = 8;  // 64-assignment chunks whose ids are loaded together

__global__ __launch_bounds__(kPermWaves * kWave) void permute_kernel(
    const int32_t* __restrict__ ids, int n, int E, int nbits, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    __shared__ int rowbase[kPermWaves * MOE_MAX_EXPERTS];  // [wave][expert]
    __shared__ int start[MOE_MAX_EXPERTS];                  // offsets[e]
    __shared__ int wsum[kPermWaves];
    const int tid = (int)threadIdx.x, lane = lane_id(), wave = tid >> 6;

    for (int i = tid; i < kPermWaves * E; i += kPermWaves * kWave) rowbase[i] = 0;
    __syncthreads();

    const int chunks = (n + kWave - 1) / kWave;
    const int c0 = (int)((int64_t)wave * chunks / kPermWaves);
    const int c1 = (int)((int64_t)(wave + 1) * chunks / kPermWaves);
    int* myrow = rowbase + wave * E;

    // ids of kBatch chunks are loaded together (independent loads), then walked in order
    auto load_batch = [&](int c, int (&ev)[kBatch]) {
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int f = (c + b) * kWave + lane;
            ev[b] = (c + b < c1 && f < n) ? ids[f] : -1;
        }
    };

    // pass 1: per-wave histogram
    for (int c = c0; c < c1; c += kBatch) {
        int ev[kBatch];
        load_batch(c, ev);
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int e = ev[b];
            const bool valid = e >= 0 && e < E;
            const uint64_t peers = match_peers(e, valid, nbits);
            if (valid && lane == __ffsll((unsigned long long)peers) - 1) myrow[e] += __popcll(peers);
        }
    }
    __syncthreads();

    // per-expert exclusive sum over waves; totals
    int total = 0;
    if (tid < E) {
        for (int w = 0; w < kPermWaves; ++w) {
            const int v = rowbase[w * E + tid];
            rowbase[w * E + tid] = total;
            total += v;
        }
        counts[tid] = total;
    }
    // exclusive sum of the totals over experts (E <= 1024 = one expert per thread)
    const int incl = wave_inclusive_scan(total);
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const int s = lane < kPermWaves ? wsum[lane] : 0;
        const int si = wave_inclusive_scan(s);
        if (lane < kPermWaves) wsum[lane] = si - s;
    }
    __syncthreads();
    if (tid < E) {
        const int excl = wsum[wave] + incl - total;
        start[tid] = excl;
        offsets[tid] = excl;
        if (tid == E - 1) offsets[E] = excl + total;
    }
    __syncthreads();
    for (int i = tid; i < kPermWaves * E; i += kPermWaves * kWave) rowbase[i] += start[i % E];
    __syncthreads();

    // pass 2: slots
    for (int c = c0; c < c1; c += kBatch) {
        int ev[kBatch];
        load_batch(c, ev);
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int f = (c + b) * kWave + lane;
            const int e = ev[b];
            const bool valid = e >= 0 && e < E;
            const uint64_t peers = match_peers(e, valid, nbits);
            int base = 0;
            if (valid) {
                base = myrow[e];
                const int pos = base + __popcll(peers & ((1ull << lane) - 1ull));
                perm[pos] = f;
                inv[f] = pos;
            }
            // the wave's reads of myrow above are issued before this write (in-order LDS per wave)
            __builtin_amdgcn_wave_barrier();
            if (valid && lane == __ffsll((unsigned long long)peers) - 1) myrow[e] = base + __popcll(peers);
            __builtin_amdgcn_wave_barrier();
        }
    }
}

constexpr int kSmallN = 2048;  // assignments up to which one wave groups them

__global__ __launch_bounds__(kWave) void permute_small_kernel(
    const int32_t* __restrict__ ids, int n, int E, int nbits, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    __shared__ int cnt[MOE_MAX_EXPERTS];
    permute_wave(ids, n, E, nbits, cnt, counts, offsets, perm, inv);
}

static moe_status check_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                         const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                         const int32_t* inv) {
    if (T < 0 || k < 1 || E < 1) return MOE_ERR_INVALID_ARG;
    if (E > MOE_MAX_EXPERTS || (int64_t)T * k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!topk_ids || !counts || !offsets || !perm || !inv) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

static moe_status launch_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* inv, hipStream_t st) {
    const int n = T * k;
    const int nbits = ceil_log2(E) > 0 ? ceil_log2(E) : 1;
    if (n <= kSmallN)
        permute_small_kernel<<<dim3(1), dim3(kWave), 0, st>>>(topk_ids, n, E, nbits, counts, offsets,
                                                               perm, inv);
    else
        permute_kernel<<<dim3(1), dim3(kPermWaves * kWave), 0, st>>>(topk_ids, n, E, nbits, counts,
                                                                     offsets, perm, inv);
    return launch_status();
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                                  int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                                  void* stream) {
    const moe_status s = check_permute(topk_ids, T, k, E, counts, offsets, perm, inv);
    if (s != MOE_OK || T == 0) return s;
    return launch_permute(topk_ids, T, k, E, counts, offsets, perm, inv, as_stream(stream));
}

// moe_permute.hip -- grouping of the (token, slot) assignments by expert.
//
// Tokens that hit the same expert are gathered so that each expert runs one GEMM over all of
// them (KTransformers article, 2.2); in the expert-parallel flow this is the "sorting" after
// gating (OSDI'26 hybrid-inference article, DSLP section).
//
// Above kSmallN assignments the work is spread over the chip in four launches, and still no
// atomics decide an order:
//   hist    block b (kBlockN consecutive assignments) counts its ids per expert in LDS and writes
//           the counts to row b of a table [B][E];
//   scan    one workgroup turns every expert's column into exclusive per-block bases (block
//           order), writes `counts`, and `offsets` as the exclusive sum of the counts;
//   place   block b walks its 64-assignment chunks in order, 16 waves each taking a contiguous
//           run: pass 1 counts per wave and expert (peers with the same expert are found with one
//           ballot per bit of the expert id), then per expert the waves' counts become running
//           bases from offsets[e] + table[b][e]; pass 2 gives an assignment the slot
//           base + (lower peers in its chunk), and perm[slot] = its flat index;
//   invert  inv[perm[p]] = p.
// The result is the stable order by construction (ascending flat index within each expert).
// The table, B = ceil(n / kBlockN) rows of E ints, is the caller's workspace
// (moe_permute_workspace_size); every entry is written by the hist launch before it is read, so
// the workspace needs no clearing.
// Up to kBlockThreads (1024) assignments one workgroup places them all at once, one a thread,
// and up to kSmallN one wave walks them in order (both in moe_permute.h).
#include <mutex>

#include "libmoe.h"
#include "moe_device.h"
#include "moe_host.h"
#include "moe_permute.h"

namespace moe {

constexpr int kPlaceWaves = 16;
constexpr int kBlockChunks = 32;                 // 64-assignment chunks per block
constexpr int kBlockN = kBlockChunks * kWave;    // 2048 assignments per block
constexpr int kWaveChunks = kBlockChunks / kPlaceWaves;
constexpr int kHistThreads = 256;

__global__ __launch_bounds__(kHistThreads) void permute_hist_kernel(const int32_t* __restrict__ ids,
                                                                    int n, int E,
                                                                    int32_t* __restrict__ table) {
    __shared__ int hist[MOE_MAX_EXPERTS];
    const int tid = (int)threadIdx.x, b = (int)blockIdx.x;
    for (int e = tid; e < E; e += kHistThreads) hist[e] = 0;
    __syncthreads();
    const int f0 = b * kBlockN, f1 = min(n, f0 + kBlockN);
    constexpr int kPer = kBlockN / kHistThreads;
    int ev[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {  // loads first, so they overlap
        const int f = f0 + i * kHistThreads + tid;
        ev[i] = f < f1 ? ids[f] : -1;
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        if (ev[i] >= 0 && ev[i] < E) atomicAdd(&hist[ev[i]], 1);  // counts only: order-free
    __syncthreads();
    for (int e = tid; e < E; e += kHistThreads) table[(size_t)b * E + e] = hist[e];
}

// One workgroup, one thread per expert (E <= 1024).
__global__ __launch_bounds__(1024) void permute_scan_kernel(int32_t* __restrict__ table, int B, int E,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets) {
    __shared__ int wsum[16];
    const int tid = (int)threadIdx.x, lane = lane_id(), wave = tid >> 6;
    int total = 0;
    if (tid < E) {
        int b = 0;
        for (; b + 8 <= B; b += 8) {  // eight independent loads per trip
            int v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = table[(size_t)(b + i) * E + tid];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                table[(size_t)(b + i) * E + tid] = total;
                total += v[i];
            }
        }
        for (; b < B; ++b) {
            const int v = table[(size_t)b * E + tid];
            table[(size_t)b * E + tid] = total;
            total += v;
        }
        counts[tid] = total;
    }
    const int incl = wave_inclusive_scan(total);
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const int s = lane < 16 ? wsum[lane] : 0;
        const int si = wave_inclusive_scan(s);
        if (lane < 16) wsum[lane] = si - s;
    }
    __syncthreads();
    if (tid < E) {
        const int excl = wsum[wave] + incl - total;
        offsets[tid] = excl;
        if (tid == E - 1) offsets[E] = excl + total;
    }
}

__global__ __launch_bounds__(kPlaceWaves * kWave) void permute_place_kernel(
    const int32_t* __restrict__ ids, int n, int E, int nbits, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ table, int32_t* __restrict__ perm) {
    __shared__ int rowbase[kPlaceWaves * MOE_MAX_EXPERTS];  // [wave][expert]
    const int tid = (int)threadIdx.x, lane = lane_id(), wave = tid >> 6, b = (int)blockIdx.x;
    for (int i = tid; i < kPlaceWaves * E; i += kPlaceWaves * kWave) rowbase[i] = 0;
    __syncthreads();
    const int chunks = (n + kWave - 1) / kWave;
    const int c0 = b * kBlockChunks + wave * kWaveChunks;
    const int c1 = min(chunks, c0 + kWaveChunks);
    int* myrow = rowbase + wave * E;
    int ev[kWaveChunks];
#pragma unroll
    for (int i = 0; i < kWaveChunks; ++i) {
        const int f = (c0 + i) * kWave + lane;
        ev[i] = (c0 + i < c1 && f < n) ? ids[f] : -1;
    }
    // pass 1: this wave's count per expert
#pragma unroll
    for (int i = 0; i < kWaveChunks; ++i) {
        const int e = ev[i];
        const bool valid = e >= 0 && e < E;
        const uint64_t peers = match_peers(e, valid, nbits);
        if (valid && lane == __ffsll((unsigned long long)peers) - 1) myrow[e] += __popcll(peers);
    }
    __syncthreads();
    // running bases per expert over the waves, from the block's base
    for (int e = tid; e < E; e += kPlaceWaves * kWave) {
        int base = offsets[e] + table[(size_t)b * E + e];
        for (int w = 0; w < kPlaceWaves; ++w) {
            const int v = rowbase[w * E + e];
            rowbase[w * E + e] = base;
            base += v;
        }
    }
    __syncthreads();
    // pass 2: slots
#pragma unroll
    for (int i = 0; i < kWaveChunks; ++i) {
        const int f = (c0 + i) * kWave + lane;
        const int e = ev[i];
        const bool valid = e >= 0 && e < E;
        const uint64_t peers = match_peers(e, valid, nbits);
        int base = 0;
        if (valid) {
            base = myrow[e];
            perm[base + __popcll(peers & ((1ull << lane) - 1ull))] = f;
        }
        // the wave's reads of myrow above are issued before this write (in-order LDS per wave)
        __builtin_amdgcn_wave_barrier();
        if (valid && lane == __ffsll((unsigned long long)peers) - 1) myrow[e] = base + __popcll(peers);
        __builtin_amdgcn_wave_barrier();
    }
}

// inv[perm[p]] = p over the offsets[E] slots that were filled
__global__ __launch_bounds__(256) void permute_invert_kernel(const int32_t* __restrict__ perm, int n,
                                                             const int32_t* __restrict__ offsets,
                                                             int E, int32_t* __restrict__ inv) {
    const int p = (int)(blockIdx.x * 256 + threadIdx.x);
    if (p >= min(n, offsets[E])) return;
    const int f = perm[p];
    if (f >= 0 && f < n) inv[f] = p;
}

constexpr int kSmallN = 2048;  // assignments up to which one wave groups them

__global__ __launch_bounds__(kBlockThreads) void permute_block_kernel(
    const int32_t* __restrict__ ids, int n, int E, int nbits, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    __shared__ int wcnt[kBlockWaves * MOE_MAX_EXPERTS];
    __shared__ int off[MOE_MAX_EXPERTS + 1];
    __shared__ int wsum[kBlockWaves];
    permute_block(ids, n, E, nbits, wcnt, off, wsum, counts, offsets, perm, inv);
}

__global__ __launch_bounds__(kWave) void permute_small_kernel(
    const int32_t* __restrict__ ids, int n, int E, int nbits, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    __shared__ int cnt[MOE_MAX_EXPERTS];
    permute_wave(ids, n, E, nbits, cnt, counts, offsets, perm, inv);
}

// Bytes of the count table [B][E] for n assignments (0 when one workgroup groups them all).
static size_t permute_table_bytes(int64_t n, int E) {
    if (n <= kSmallN) return 0;
    const int64_t B = (n + kBlockN - 1) / kBlockN;
    return (size_t)B * (size_t)E * sizeof(int32_t);
}

static moe_status check_permute_sizes(int32_t T, int32_t k, int32_t E) {
    if (T < 0 || k < 1 || E < 1) return MOE_ERR_INVALID_ARG;
    if (E > MOE_MAX_EXPERTS || (int64_t)T * k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

static moe_status check_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                         const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                         const int32_t* inv) {
    const moe_status s = check_permute_sizes(T, k, E);
    if (s != MOE_OK || T == 0) return s;
    if (!topk_ids || !counts || !offsets || !perm || !inv) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

// `table` holds permute_table_bytes(T * k, E) bytes (unused, may be NULL, up to kSmallN).
static moe_status launch_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* table,
                          hipStream_t st) {
    const int n = T * k;
    const int nbits = ceil_log2(E) > 0 ? ceil_log2(E) : 1;
    if (n <= kBlockThreads) {
        permute_block_kernel<<<dim3(1), dim3(kBlockThreads), 0, st>>>(topk_ids, n, E, nbits, counts,
                                                                      offsets, perm, inv);
        return launch_status();
    }
    if (n <= kSmallN) {
        permute_small_kernel<<<dim3(1), dim3(kWave), 0, st>>>(topk_ids, n, E, nbits, counts, offsets,
                                                               perm, inv);
        return launch_status();
    }
    const int B = (int)(((int64_t)n + kBlockN - 1) / kBlockN);
    permute_hist_kernel<<<dim3(B), dim3(kHistThreads), 0, st>>>(topk_ids, n, E, table);
    permute_scan_kernel<<<dim3(1), dim3(1024), 0, st>>>(table, B, E, counts, offsets);
    permute_place_kernel<<<dim3(B), dim3(kPlaceWaves * kWave), 0, st>>>(topk_ids, n, E, nbits,
                                                                       offsets, table, perm);
    permute_invert_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(perm, n, offsets,
                                                                                  E, inv);
    return launch_status();
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_permute_workspace_size(int32_t T, int32_t k, int32_t E, size_t* bytes) {
    if (!bytes) return MOE_ERR_INVALID_ARG;
    const moe_status s = check_permute_sizes(T, k, E);
    if (s != MOE_OK) return s;
    *bytes = permute_table_bytes((int64_t)T * k, E);
    return MOE_OK;
}

extern "C" moe_status moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                                  int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                                  void* ws, size_t ws_bytes, void* stream) {
    const moe_status s = check_permute(topk_ids, T, k, E, counts, offsets, perm, inv);
    if (s != MOE_OK || T == 0) return s;
    const size_t need = permute_table_bytes((int64_t)T * k, E);
    if (need > 0 && (!ws || ws_bytes < need)) return MOE_ERR_WORKSPACE;
    if (need > 0 && !aligned16(ws)) return MOE_ERR_INVALID_ARG;
    return launch_permute(topk_ids, T, k, E, counts, offsets, perm, inv,
                          static_cast<int32_t*>(ws), as_stream(stream));
}

// ------------------------------------------------------------------ no-allocation variant
//
// moe_permute_noalloc keeps the count table in `scratch`, a static device array of this library
// (each GPU the library runs on holds its own copy until the process ends).  In host code the
// array's name is not a device address: the address is looked up once per device, with that
// device current, and only the looked-up pointer is ever handed to kernels.
static __device__ __align__(256) int32_t scratch[MOE_PERMUTE_NOALLOC_MAX_BYTES / sizeof(int32_t)];

namespace moe {

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mutex;
static int32_t* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first call there), which
// must be the device `stream` belongs to (else INVALID_ARG: the kernels would run on the
// stream's device with another device's address).
static moe_status scratch_on_current_device(hipStream_t stream, int32_t** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_DEVICE;
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    if (stream != nullptr) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return MOE_ERR_DEVICE;
        if (sdev != dev) return MOE_ERR_INVALID_ARG;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return MOE_ERR_DEVICE;
        g_scratch[dev] = static_cast<int32_t*>(p);
    }
    *out = g_scratch[dev];
    return MOE_OK;
}

}  // namespace moe

extern "C" moe_status moe_permute_noalloc(const int32_t* topk_ids, int32_t T, int32_t k,
                                          int32_t E, int32_t* counts, int32_t* offsets,
                                          int32_t* perm, int32_t* inv, void* stream) {
    const moe_status s = check_permute(topk_ids, T, k, E, counts, offsets, perm, inv);
    if (s != MOE_OK || T == 0) return s;
    if (permute_table_bytes((int64_t)T * k, E) > MOE_PERMUTE_NOALLOC_MAX_BYTES)
        return MOE_ERR_UNSUPPORTED;
    int32_t* table = nullptr;
    const moe_status a = scratch_on_current_device(as_stream(stream), &table);
    if (a != MOE_OK) return a;
    return launch_permute(topk_ids, T, k, E, counts, offsets, perm, inv, table,
                          as_stream(stream));
}

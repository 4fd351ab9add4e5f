// moe_route.hip -- top-k routing: one wave64 per token (the routine is in moe_route.h); and,
// for decode-sized batches, routing and grouping in one launch (moe_permute.h's wave walk).
#include "libmoe.h"
#include "moe_device.h"
#include "moe_host.h"
#include "moe_permute.h"
#include "moe_route.h"

namespace moe {

template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ scores, int T, int E,
                                                    int k, int score_fn, int renorm,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ wts) {
    const int t = (int)(blockIdx.x * 4 + (threadIdx.x >> 6));
    if (t >= T) return;  // whole waves leave together
    route_token<VPL>(scores + (size_t)t * E, E, k, score_fn, renorm, ids + (size_t)t * k,
                     wts + (size_t)t * k);
}

// Routing then grouping in one workgroup: its waves route the tokens (a wave per token), and
// after the barrier the workgroup groups the T*k assignments: up to kBlockThreads of them all its
// threads, one assignment each, from the ids the routing also left in LDS (permute_block); above
// that wave 0 walks them in order from the ids just written (the barrier makes the workgroup's
// global writes visible to all its waves).
constexpr int kFusedN = 2048;  // assignments up to which one workgroup routes and groups
constexpr int kFusedWaves = 16;

template <int VPL>
__global__ __launch_bounds__(kFusedWaves * 64) void route_permute_kernel(
    const float* __restrict__ scores, int T, int E, int k, int score_fn, int renorm, int nbits,
    int32_t* __restrict__ ids, float* __restrict__ wts, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    static_assert(kFusedWaves == kBlockWaves, "the grouping runs on the routing workgroup");
    __shared__ int wcnt[kBlockWaves * MOE_MAX_EXPERTS];  // (one wave: its first E ints)
    __shared__ int off[MOE_MAX_EXPERTS + 1];
    __shared__ int wsum[kBlockWaves];
    __shared__ int sids[kBlockThreads];
    const int wave = (int)(threadIdx.x >> 6);
    const int n = T * k;
    const bool block = n <= kBlockThreads;
    for (int t = wave; t < T; t += kFusedWaves)
        route_token<VPL>(scores + (size_t)t * E, E, k, score_fn, renorm, ids + (size_t)t * k,
                         wts + (size_t)t * k, block ? sids + t * k : nullptr);
    __syncthreads();
    if (block)
        permute_block(sids, n, E, nbits, wcnt, off, wsum, counts, offsets, perm, inv);
    else if (wave == 0)
        permute_wave(ids, n, E, nbits, wcnt, counts, offsets, perm, inv);
}

static moe_status check_route(const float* scores, int32_t T, int32_t E, int32_t k, int32_t score_fn,
                       const int32_t* topk_ids, const float* topk_w) {
    if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
    if (score_fn != MOE_SCORE_SOFTMAX && score_fn != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
    if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!scores || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

static moe_status launch_route(const float* scores, int32_t T, int32_t E, int32_t k, int32_t score_fn,
                        int32_t renorm, int32_t* topk_ids, float* topk_w, hipStream_t st) {
    const dim3 grid((unsigned)((T + 3) / 4)), block(256);
    switch (route_vpl(E)) {
#define MOE_ROUTE(V) \
    case V: route_kernel<V><<<grid, block, 0, st>>>(scores, T, E, k, score_fn, renorm, topk_ids, topk_w); break;
        MOE_ROUTE(1) MOE_ROUTE(2) MOE_ROUTE(4) MOE_ROUTE(8) MOE_ROUTE(16)
#undef MOE_ROUTE
    }
    return launch_status();
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_route_permute(const float* scores, int32_t T, int32_t E, int32_t k,
                                        int32_t score_fn, int32_t renorm, int32_t* topk_ids,
                                        float* topk_w, int32_t* counts, int32_t* offsets,
                                        int32_t* perm, int32_t* inv, void* stream) {
    moe_status s = check_route(scores, T, E, k, score_fn, topk_ids, topk_w);
    if (s != MOE_OK) return s;
    if (T > 0 && (!counts || !offsets || !perm || !inv)) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if ((int64_t)T * k > kFusedN) return MOE_ERR_UNSUPPORTED;
    const int nbits = ceil_log2(E) > 0 ? ceil_log2(E) : 1;
    const dim3 grid(1), block(kFusedWaves * 64);
    hipStream_t st = as_stream(stream);
    switch (route_vpl(E)) {
#define MOE_FUSED(V)                                                                          \
    case V:                                                                                   \
        route_permute_kernel<V><<<grid, block, 0, st>>>(scores, T, E, k, score_fn, renorm,     \
                                                        nbits, topk_ids, topk_w, counts,       \
                                                        offsets, perm, inv);                   \
        break;
        MOE_FUSED(1) MOE_FUSED(2) MOE_FUSED(4) MOE_FUSED(8) MOE_FUSED(16)
#undef MOE_FUSED
    }
    return launch_status();
}

extern "C" moe_status moe_route(const float* scores, int32_t T, int32_t E, int32_t k,
                                int32_t score_fn, int32_t renorm, int32_t* topk_ids, float* topk_w,
                                void* stream) {
    const moe_status s = check_route(scores, T, E, k, score_fn, topk_ids, topk_w);
    if (s != MOE_OK || T == 0) return s;
    return launch_route(scores, T, E, k, score_fn, renorm, topk_ids, topk_w, as_stream(stream));
}

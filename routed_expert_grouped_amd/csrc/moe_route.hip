// moe_route.hip -- top-k routing: one wave64 per token (the routine is in moe_route.h).
#include "libmoe.h"
#include "moe_device.h"
#include "moe_host.h"
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

extern "C" moe_status moe_route(const float* scores, int32_t T, int32_t E, int32_t k,
                                int32_t score_fn, int32_t renorm, int32_t* topk_ids, float* topk_w,
                                void* stream) {
    const moe_status s = check_route(scores, T, E, k, score_fn, topk_ids, topk_w);
    if (s != MOE_OK || T == 0) return s;
    return launch_route(scores, T, E, k, score_fn, renorm, topk_ids, topk_w, as_stream(stream));
}

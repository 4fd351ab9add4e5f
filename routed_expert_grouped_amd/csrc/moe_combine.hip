// moe_combine.hip -- weighted combine of the expert outputs plus the shared expert.
//
// After the experts, each token's k outputs are summed with the gate weights ("weighted
// reduction" closing the expert-parallel flow: OSDI'26 hybrid-inference article, DSLP section)
// and the always-active shared expert is added with weight 1 (DeepSeek-V3 has one shared expert
// next to its 256 routed ones: KTransformers article, 1.2).
//
// Gather form: one thread owns 8 consecutive columns of one token and reads the token's k rows
// of y through inv (16-byte loads), so every output element is written once, in a fixed order,
// with no atomics.  HBM-bound: it reads T*k*H*2 + T*H*2 bytes and writes T*H*2 bytes.
//
// Under expert parallelism each rank reduces only its own experts' outputs to a partial T x H
// (the local weighted partial reduction of the article's SmallEP section); kRange skips the
// assignments whose expert is outside [e_begin, e_end) without reading their rows of y.
#include "libmoe.h"
#include "moe_device.h"
#include "moe_host.h"

namespace moe {

constexpr int kCombineThreads = 256;
constexpr int kCombineCols = kCombineThreads * 8;

template <bool kRange>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const uint16_t* __restrict__ y, const int32_t* __restrict__ inv, const float* __restrict__ w,
    const int32_t* __restrict__ ids, int e_begin, int e_end, const uint16_t* __restrict__ S,
    int k, int H, int cblocks, uint16_t* __restrict__ out) {
    const int t = (int)(blockIdx.x / cblocks);
    const int c = (int)((blockIdx.x % cblocks) * kCombineCols + threadIdx.x * 8);
    if (c >= H) return;
    float acc[8];
    if (S) {
        const uint4 v = *(const uint4*)(S + (size_t)t * H + c);
        const uint16_t* b = (const uint16_t*)&v;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = bf16_to_f32(b[i]);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    }
    for (int j = 0; j < k; ++j) {
        if (kRange) {
            const int e = ids[(size_t)t * k + j];
            if (e < e_begin || e >= e_end) continue;
        }
        const int p = inv[(size_t)t * k + j];
        const float wj = w[(size_t)t * k + j];
        const uint4 v = *(const uint4*)(y + (size_t)p * H + c);
        const uint16_t* b = (const uint16_t*)&v;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, bf16_to_f32(b[i]), acc[i]);
    }
    uint4 o;
    uint16_t* ob = (uint16_t*)&o;
#pragma unroll
    for (int i = 0; i < 8; ++i) ob[i] = f32_to_bf16(acc[i]);
    *(uint4*)(out + (size_t)t * H + c) = o;
}

}  // namespace moe

using namespace moe;

static moe_status combine(const uint16_t* y, const int32_t* inv, const int32_t* ids,
                          const float* topk_w, int32_t e_begin, int32_t e_end,
                          const uint16_t* shared_y, int32_t T, int32_t k, int32_t H,
                          uint16_t* out, void* stream, bool range) {
    if (T < 0 || k < 1 || H < 1) return MOE_ERR_INVALID_ARG;
    if (range && e_begin > e_end) return MOE_ERR_INVALID_ARG;
    if (H % 8 != 0) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!y || !inv || !topk_w || !out || (range && !ids)) return MOE_ERR_INVALID_ARG;
    if (!aligned16(y) || !aligned16(out) || (shared_y && !aligned16(shared_y)))
        return MOE_ERR_INVALID_ARG;
    const int cblocks = (H + kCombineCols - 1) / kCombineCols;
    const int64_t wgs = (int64_t)T * cblocks;
    if (wgs > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)wgs), block(kCombineThreads);
    if (range)
        combine_kernel<true><<<grid, block, 0, as_stream(stream)>>>(
            y, inv, topk_w, ids, e_begin, e_end, shared_y, k, H, cblocks, out);
    else
        combine_kernel<false><<<grid, block, 0, as_stream(stream)>>>(
            y, inv, topk_w, nullptr, 0, 0, shared_y, k, H, cblocks, out);
    return launch_status();
}

extern "C" moe_status moe_combine(const uint16_t* y, const int32_t* inv, const float* topk_w,
                                  const uint16_t* shared_y, int32_t T, int32_t k, int32_t H,
                                  uint16_t* out, void* stream) {
    return combine(y, inv, nullptr, topk_w, 0, 0, shared_y, T, k, H, out, stream, false);
}

extern "C" moe_status moe_combine_partial(const uint16_t* y, const int32_t* inv, const int32_t* ids,
                                          const float* topk_w, int32_t e_begin, int32_t e_end,
                                          const uint16_t* shared_y, int32_t T, int32_t k, int32_t H,
                                          uint16_t* out, void* stream) {
    return combine(y, inv, ids, topk_w, e_begin, e_end, shared_y, T, k, H, out, stream, true);
}

extern "C" const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
        case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
    }
    return "MOE_ERR_UNKNOWN";
}

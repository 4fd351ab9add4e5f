// moe_combine.hip -- weighted combine of the expert outputs plus the shared expert.
//
// After the experts, each token's k outputs are summed with the gate weights ("weighted
// reduction" closing the expert-parallel flow: OSDI'26 hybrid-inference article, DSLP section)
// and the always-active shared expert is added with weight 1 (DeepSeek-V3 has one shared expert
// next to its 256 routed ones: KTransformers article, 1.2).
//
// Gather form: one thread owns 8 consecutive columns of one token and reads the token's k rows
// of y through inv (16-byte loads), so every output element is written once, in a fixed order,
// with no atomics.  One workgroup covers a whole token row (up to 1024 threads, H <= 8192), so
// a launch has T workgroups that each read k + 1 full rows.  HBM-bound: it reads T*k*H*2 +
// T*H*2 bytes and writes T*H*2 bytes.
//
// Under expert parallelism each rank reduces only its own experts' outputs to a partial T x H
// (the local weighted partial reduction of the article's SmallEP section); kRange skips the
// assignments whose expert is outside [e_begin, e_end) without reading their rows of y.
#include "libmoe.h"
#include "moe_device.h"
#include "moe_host.h"

#include <type_traits>

namespace moe {

constexpr int kCombineMaxThreads = 1024;

// y, the shared row and out are each touched once: loads and the store carry the non-temporal
// hint (measured 10% faster at 32768 tokens x 7168 columns than plain ones)
__device__ __forceinline__ u32x4 stream_load(const uint16_t* p) {
    return __builtin_nontemporal_load((const u32x4*)p);
}

template <bool kRange>
__global__ __launch_bounds__(kCombineMaxThreads) void combine_kernel(
    const uint16_t* __restrict__ y, const int32_t* __restrict__ inv, const float* __restrict__ w,
    const int32_t* __restrict__ ids, int e_begin, int e_end, const uint16_t* __restrict__ S,
    int k, int H, int cblocks, uint16_t* __restrict__ out) {
    const int t = (int)(blockIdx.x / cblocks);
    const int c = (int)(((blockIdx.x % cblocks) * blockDim.x + threadIdx.x) * 8);
    if (c >= H) return;
    const int32_t* it = inv + (size_t)t * k;
    const float* wt = w + (size_t)t * k;
    float acc[8];
    auto init = [&](u32x4 sv) {
        const uint16_t* b = (const uint16_t*)&sv;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = bf16_to_f32(b[i]);
    };
    auto add = [&](float wj, u32x4 v) {
        const uint16_t* b = (const uint16_t*)&v;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, bf16_to_f32(b[i]), acc[i]);
    };
    if constexpr (kRange) {
        u32x4 sv = {0u, 0u, 0u, 0u};
        if (S) sv = stream_load(S + (size_t)t * H + c);
        init(sv);
        for (int j = 0; j < k; ++j) {
            const int e = ids[(size_t)t * k + j];
            if (e < e_begin || e >= e_end) continue;
            add(wt[j], stream_load(y + (size_t)it[j] * H + c));
        }
    } else {
        // The k rows are read in batches of eight (then four, then one) independent 16-byte
        // loads, all issued before the first is used; the sum still runs over j in ascending
        // order.  The shared row is loaded unconditionally (without one, the first assignment's
        // row, masked to zeros) and converted after the first batch is in flight, so that its
        // load overlaps theirs.
        const u32x4 sv = stream_load((S ? S + (size_t)t * H : y + (size_t)it[0] * H) + c);
        const uint32_t smask = S ? ~0u : 0u;
        auto batch = [&](int j0, auto n_tag) {
            constexpr int N = decltype(n_tag)::value;
            u32x4 v[N];
#pragma unroll
            for (int u = 0; u < N; ++u) v[u] = stream_load(y + (size_t)it[j0 + u] * H + c);
            if (j0 == 0) {
                // an empty asm ties the conversion to this point, after the batch's loads (the
                // compiler would otherwise hoist it, and the wait for the shared row, above them)
                u32x4 s = sv;
                asm volatile("" : "+v"(s));
                init(s & smask);
            }
#pragma unroll
            for (int u = 0; u < N; ++u) add(wt[j0 + u], v[u]);
        };
        int j = 0;
        for (; j + 8 <= k; j += 8) batch(j, std::integral_constant<int, 8>{});
        if (j + 4 <= k) {
            batch(j, std::integral_constant<int, 4>{});
            j += 4;
        }
        for (; j < k; ++j) batch(j, std::integral_constant<int, 1>{});
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = f32x2_to_bf16x2(acc[2 * i], acc[2 * i + 1]);
    __builtin_nontemporal_store(o, (u32x4*)(out + (size_t)t * H + c));
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
    // a workgroup covers a whole token row when H <= 8192 (8 columns a thread)
    const int chunks = H / 8;
    const int cblocks = (chunks + kCombineMaxThreads - 1) / kCombineMaxThreads;
    const int threads = ((chunks + cblocks - 1) / cblocks + kWave - 1) / kWave * kWave;
    const int64_t wgs = (int64_t)T * cblocks;
    if (wgs > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)wgs), block(threads);
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

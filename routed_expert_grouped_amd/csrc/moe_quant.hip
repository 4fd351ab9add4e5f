// moe_quant.hip -- FP8 activation quantisation for the FP8 MFMA mode, and the mode's FFN call.
//
// The pages quantise weights to E4M3FN in 128-blocks with one scale per block (OSDI'26
// hybrid-inference article, "native FP8 GEMV").  In the FP8 MFMA mode activations are quantised
// the same way along the input dimension: per row, per 128 consecutive values, a power-of-two
// scale 2^e (e the smallest integer with amax <= 448 * 2^e, clamped to [-127, 127]) and codes =
// E4M3FN round-to-nearest-even of x * 2^-e in fp32.  Power-of-two scales are E8M0 numbers, the
// block scales the gfx950 FP8 matrix instructions apply themselves, and dividing by them is
// exact.
#include "libmoe.h"
#include "moe_device.h"
#include "moe_ffn.h"
#include "moe_host.h"

namespace moe {

// exponent e of the block scale for largest magnitude amax (see the file comment)
__device__ __forceinline__ int act_scale_exp(float amax) {
    if (!(amax > 0.0f)) return 0;
    int e2;
    const float m = frexpf(amax, &e2);  // amax = m 2^e2, m in [0.5, 1)
    int e = (m <= 0.875f) ? e2 - 9 : e2 - 8;
    return min(127, max(-127, e));
}

// One wave per (row, 128-block): lane l holds values 2l and 2l+1.  Writes the codes and the
// exponent (either may be null) and, if deq is not null, the dequantised values as bf16 (exact:
// a 4-bit significand times a power of two).
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ x, int rows,
                                                       int K, uint8_t* __restrict__ codes,
                                                       int8_t* __restrict__ exps,
                                                       uint16_t* __restrict__ deq) {
    const uint32_t nb = (uint32_t)K / 128;  // the launch keeps rows * nb below 2^31
    const uint32_t blk = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (blk >= (uint32_t)rows * nb) return;  // whole waves leave together
    const int lane = lane_id();
    const uint32_t r = blk / nb, b = blk - r * nb;
    const size_t at = (size_t)r * K + (size_t)b * 128 + 2 * lane;
    const uint32_t pair = *(const uint32_t*)(x + at);
    const float v0 = bf16_to_f32((uint16_t)pair), v1 = bf16_to_f32((uint16_t)(pair >> 16));
    float amax = fmaxf(fabsf(v0), fabsf(v1));
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
    const int e = act_scale_exp(amax);
    const int c2 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v0, -e), ldexpf(v1, -e), 0, false);
    if (codes) *(uint16_t*)(codes + at) = (uint16_t)c2;
    if (exps && lane == 0) exps[(size_t)r * nb + b] = (int8_t)e;
    if (deq) {
        const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c2, ldexpf(1.0f, e), false);
        *(bf16x2*)(deq + at) = d;
    }
}

moe_status launch_quantize(const uint16_t* x, int64_t rows, int K, uint8_t* codes, int8_t* exps,
                           uint16_t* deq, hipStream_t st) {
    const int64_t blocks = rows * (K / 128);
    if (blocks > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    quantize_kernel<<<dim3((unsigned)((blocks + 3) / 4)), dim3(256), 0, st>>>(x, (int)rows, K, codes,
                                                                              exps, deq);
    return launch_status();
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_quantize_act(const uint16_t* x, int32_t rows, int32_t K, uint8_t* codes,
                                       int8_t* exps, void* stream) {
    if (rows < 0 || K < 1) return MOE_ERR_INVALID_ARG;
    if (K % 128 != 0) return MOE_ERR_UNSUPPORTED;
    if (rows == 0) return MOE_OK;
    if ((int64_t)rows * (K / 128) > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (!x || !codes || !exps || !aligned16(x) || !aligned16(codes) || !aligned16(exps))
        return MOE_ERR_INVALID_ARG;
    return launch_quantize(x, rows, K, codes, exps, nullptr, as_stream(stream));
}

// Workspace of moe_expert_ffn_a8: dequantised x [T][H] bf16, h [T*k][I] bf16, dequantised h
// [T*k][I] bf16, each part 256-byte aligned.
static size_t a8_part(size_t bytes) { return (bytes + 255) & ~size_t(255); }

extern "C" moe_status moe_expert_ffn_a8_workspace_size(int32_t T, int32_t k,
                                                       const moe_expert_weights* w, size_t* bytes) {
    if (!bytes) return MOE_ERR_INVALID_ARG;
    moe_status s = check_weights(w);
    if (s != MOE_OK) return s;
    if (T < 0 || k < 1) return MOE_ERR_INVALID_ARG;
    const size_t rows = (size_t)T * k;
    *bytes = a8_part((size_t)T * w->H * 2) + 2 * a8_part(rows * w->I * 2);
    return MOE_OK;
}

extern "C" moe_status moe_expert_ffn_a8(const uint16_t* x, int32_t T, int32_t k, const int32_t* perm,
                                        const int32_t* offsets, const moe_expert_weights* w,
                                        uint16_t* y, void* ws, size_t ws_bytes, void* stream) {
    if (T < 0 || k < 1) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    size_t need = 0;
    moe_status s = moe_expert_ffn_a8_workspace_size(T, k, w, &need);
    if (s != MOE_OK) return s;
    if (w->dtype != MOE_W_FP8_E4M3_B128) return MOE_ERR_UNSUPPORTED;
    if ((s = check_grouping(T, k, perm, offsets, w, true)) != MOE_OK) return s;
    if (!x || !y || !aligned16(x) || !aligned16(y)) return MOE_ERR_INVALID_ARG;
    if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
    if (!aligned16(ws)) return MOE_ERR_INVALID_ARG;
    const int64_t rows = (int64_t)T * k;
    if (rows * (w->I / 128) > INT32_MAX || (int64_t)T * (w->H / 128) > INT32_MAX)
        return MOE_ERR_UNSUPPORTED;
    hipStream_t st = as_stream(stream);
    uint8_t* p = static_cast<uint8_t*>(ws);
    uint16_t* xq = reinterpret_cast<uint16_t*>(p);
    p += a8_part((size_t)T * w->H * 2);
    uint16_t* h = reinterpret_cast<uint16_t*>(p);
    p += a8_part((size_t)rows * w->I * 2);
    uint16_t* hq = reinterpret_cast<uint16_t*>(p);
    if ((s = launch_quantize(x, T, w->H, nullptr, nullptr, xq, st)) != MOE_OK) return s;
    if ((s = moe_expert_gate_up(xq, T, k, perm, offsets, w, h, stream)) != MOE_OK) return s;
    if ((s = launch_quantize(h, rows, w->I, nullptr, nullptr, hq, st)) != MOE_OK) return s;
    return moe_expert_down(hq, T, k, offsets, w, y, stream);
}

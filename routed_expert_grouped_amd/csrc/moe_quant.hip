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

// One row of 16 lanes per (row, 128-block), four blocks a wave: lane l of the row holds values
// 8l .. 8l + 7 (one 16-byte load), the block maximum is taken over the row with DPP row
// operations (no cross-row traffic), and every lane converts its own eight values.  Writes any
// of: the codes, the exponent (exps[r * exp_pitch + b], by the row's first lane) and the
// dequantised values as bf16 (exact: a 4-bit significand times a power of two).
constexpr int kQuantThreads = 256;
constexpr int64_t kQuantMaxBlocks = int64_t(1) << 27;  // 16 lanes a block: 32-bit thread ids

__global__ __launch_bounds__(kQuantThreads) void quantize_kernel(const uint16_t* __restrict__ x,
                                                                 int rows, int K,
                                                                 uint8_t* __restrict__ codes,
                                                                 int8_t* __restrict__ exps,
                                                                 int exp_pitch,
                                                                 uint16_t* __restrict__ deq) {
    const uint32_t nb = (uint32_t)K / 128;  // the launch keeps rows * nb * 16 below 2^32
    const uint32_t blk = (blockIdx.x * kQuantThreads + threadIdx.x) >> 4;
    if (blk >= (uint32_t)rows * nb) return;  // whole rows of 16 lanes leave together
    const int sub = (int)(threadIdx.x & 15);
    const uint32_t r = blk / nb, b = blk - r * nb;
    const size_t at = (size_t)r * K + (size_t)b * 128 + 8 * sub;
    const u32x4 raw = *(const u32x4*)(x + at);
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_to_f32((uint16_t)raw[i]);
        v[2 * i + 1] = bf16_to_f32((uint16_t)(raw[i] >> 16));
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    // non-negative floats order as their bit patterns
    amax = __uint_as_float(row16_max_u32(__float_as_uint(amax)));
    const int e = act_scale_exp(amax);
    uint32_t c[2];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * w], -e), ldexpf(v[4 * w + 1], -e), 0, false);
        c[w] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * w + 2], -e), ldexpf(v[4 * w + 3], -e), lo, true);
    }
    if (codes) *(uint2*)(codes + at) = make_uint2(c[0], c[1]);
    if (exps && sub == 0) exps[(size_t)r * exp_pitch + b] = (int8_t)e;
    if (deq) {
        const float sc = ldexpf(1.0f, e);
        bf16x2 d[4];
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            d[2 * w] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c[w], sc, false);
            d[2 * w + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c[w], sc, true);
        }
        *(u32x4*)(deq + at) = __builtin_bit_cast(u32x4, d);
    }
}

moe_status launch_quantize(const uint16_t* x, int64_t rows, int K, uint8_t* codes, int8_t* exps,
                           int exp_pitch, uint16_t* deq, hipStream_t st) {
    const int64_t blocks = rows * (K / 128);
    if (blocks > kQuantMaxBlocks) return MOE_ERR_UNSUPPORTED;
    const int64_t threads = blocks * 16;
    quantize_kernel<<<dim3((unsigned)((threads + kQuantThreads - 1) / kQuantThreads)),
                      dim3(kQuantThreads), 0, st>>>(x, (int)rows, K, codes, exps, exp_pitch, deq);
    return launch_status();
}

// The FP8 activation mode's expert FFN.  Each phase runs the FP8-code GEMM when its shape fits
// (moe_gemm_a8.hip); otherwise (few rows per expert, or shapes outside that kernel) the
// activations are dequantised exactly to bf16 and the bf16-operand kernels run, which gives the
// same values up to the order of the fp32 sums.
struct A8Plan {
    int T, k, H, I;
    bool fp8_1, fp8_2;   // phase runs on FP8 codes
    int pitch_h, pitch_i;  // exponent row pitches (bytes)
    size_t h, x1, x1e, h2, h2e, size;  // workspace offsets and total
};

static size_t a8_part(size_t bytes) { return (bytes + 255) & ~size_t(255); }

static GemmArgs a8_args(int phase, int T, int k, const moe_expert_weights* w) {
    GemmArgs a{};
    a.k = k;
    a.rows = T * k;
    a.n_groups = w->n_groups;
    a.N = phase == 1 ? w->I : w->H;
    a.K = phase == 1 ? w->H : w->I;
    a.fp8 = w->dtype == MOE_W_FP8_E4M3_B128;
    a.fp4 = w->dtype == MOE_W_MXFP4_G32;
    a.aexp_pitch = (a.K / 128 + 15) & ~15;
    return a;
}

static A8Plan a8_plan(int T, int k, const moe_expert_weights* w) {
    A8Plan p{};
    p.T = T, p.k = k, p.H = w->H, p.I = w->I;
    const GemmArgs a1 = a8_args(1, T, k, w), a2 = a8_args(2, T, k, w);
    p.fp8_1 = a8_gemm_fits(1, a1);
    p.fp8_2 = a8_gemm_fits(2, a2);
    p.pitch_h = a1.aexp_pitch;
    p.pitch_i = a2.aexp_pitch;
    const size_t rows = (size_t)T * k;
    size_t at = 0;
    p.h = at;
    at += a8_part(rows * w->I * 2);
    p.x1 = at;  // x as codes (+ exponents) or as dequantised bf16
    at += p.fp8_1 ? a8_part((size_t)T * w->H) : a8_part((size_t)T * w->H * 2);
    p.x1e = at;
    at += p.fp8_1 ? a8_part((size_t)T * p.pitch_h) : 0;
    p.h2 = at;  // h as codes (+ exponents) or as dequantised bf16
    at += p.fp8_2 ? a8_part(rows * w->I) : a8_part(rows * w->I * 2);
    p.h2e = at;
    at += p.fp8_2 ? a8_part(rows * p.pitch_i) : 0;
    p.size = at;
    return p;
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_quantize_act(const uint16_t* x, int32_t rows, int32_t K, uint8_t* codes,
                                       int8_t* exps, int32_t exp_pitch, void* stream) {
    if (rows < 0 || K < 1) return MOE_ERR_INVALID_ARG;
    if (K % 128 != 0) return MOE_ERR_UNSUPPORTED;
    if (exp_pitch < K / 128) return MOE_ERR_INVALID_ARG;
    if (rows == 0) return MOE_OK;
    if ((int64_t)rows * (K / 128) > kQuantMaxBlocks) return MOE_ERR_UNSUPPORTED;
    if (!x || !codes || !exps || !aligned16(x) || !aligned16(codes) || !aligned16(exps))
        return MOE_ERR_INVALID_ARG;
    return launch_quantize(x, rows, K, codes, exps, exp_pitch, nullptr, as_stream(stream));
}

extern "C" moe_status moe_expert_ffn_a8_workspace_size(int32_t T, int32_t k,
                                                       const moe_expert_weights* w, size_t* bytes) {
    if (!bytes) return MOE_ERR_INVALID_ARG;
    moe_status s = check_weights(w);
    if (s != MOE_OK) return s;
    if (T < 0 || k < 1) return MOE_ERR_INVALID_ARG;
    if ((int64_t)T * k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    *bytes = a8_plan(T, k, w).size;
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
    if (w->dtype != MOE_W_FP8_E4M3_B128 && w->dtype != MOE_W_MXFP4_G32) return MOE_ERR_UNSUPPORTED;
    if ((s = check_grouping(T, k, perm, offsets, w, true)) != MOE_OK) return s;
    if (!x || !y || !aligned16(x) || !aligned16(y)) return MOE_ERR_INVALID_ARG;
    if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
    if (!aligned16(ws)) return MOE_ERR_INVALID_ARG;
    const int64_t rows = (int64_t)T * k;
    if (rows * (w->I / 128) > INT32_MAX || (int64_t)T * (w->H / 128) > INT32_MAX)
        return MOE_ERR_UNSUPPORTED;
    const A8Plan p = a8_plan(T, k, w);
    hipStream_t st = as_stream(stream);
    uint8_t* base = static_cast<uint8_t*>(ws);
    uint16_t* h = reinterpret_cast<uint16_t*>(base + p.h);
    // phase 1: x -> h
    if (p.fp8_1) {
        uint8_t* codes = base + p.x1;
        int8_t* e = reinterpret_cast<int8_t*>(base + p.x1e);
        if ((s = launch_quantize(x, T, w->H, codes, e, p.pitch_h, nullptr, st)) != MOE_OK) return s;
        s = moe_expert_gate_up_a8(codes, e, p.pitch_h, T, k, perm, offsets, w, h, stream);
    } else {
        uint16_t* xq = reinterpret_cast<uint16_t*>(base + p.x1);
        if ((s = launch_quantize(x, T, w->H, nullptr, nullptr, 0, xq, st)) != MOE_OK) return s;
        s = moe_expert_gate_up(xq, T, k, perm, offsets, w, h, stream);
    }
    if (s != MOE_OK) return s;
    // phase 2: h -> y
    if (p.fp8_2) {
        uint8_t* codes = base + p.h2;
        int8_t* e = reinterpret_cast<int8_t*>(base + p.h2e);
        if ((s = launch_quantize(h, rows, w->I, codes, e, p.pitch_i, nullptr, st)) != MOE_OK)
            return s;
        return moe_expert_down_a8(codes, e, p.pitch_i, T, k, offsets, w, y, stream);
    }
    uint16_t* hq = reinterpret_cast<uint16_t*>(base + p.h2);
    if ((s = launch_quantize(h, rows, w->I, nullptr, nullptr, 0, hq, st)) != MOE_OK) return s;
    return moe_expert_down(hq, T, k, offsets, w, y, stream);
}

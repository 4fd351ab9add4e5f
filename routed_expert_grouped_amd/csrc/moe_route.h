// moe_route.h -- device routine of top-k routing for one token, run by one wave64.
//
// The router keeps, per token, the k experts with the largest score and turns their scores into
// normalised gate weights (sparse MoE FFN with a few active experts per token: CMU 11-868
// appendix A2 notes, 4.1; DeepSeek-V3 routes each token to 8 of 256 experts: KTransformers
// article, 1.2; "gating" opens the expert-parallel flow in the OSDI'26 hybrid-inference article,
// DSLP section).
//
// Each lane holds the scores e = lane + 64*i (coalesced loads) as order-preserving 32-bit keys
// (-0 is taken as +0, so equal scores have equal keys).  The k winners are found by k rounds:
// every lane offers its best untaken key (the lowest i among equal keys), the wave maximum is
// taken with DPP row operations and four lane reads, and among the lanes that hold it the lowest
// expert id wins (the lowest i, then the lowest lane: one ballot per i).  The comparisons are
// exact, so the selection is bit-identical to any correct top-k with the same tie rule (lower id
// wins; -0 == +0).  Slot j of the result ends up in lane j, which computes its weight in double.
#pragma once

#include "libmoe.h"
#include "moe_device.h"

namespace moe {

// Order-preserving key of a finite float: a > b  <=>  key(a) > key(b); key(-0) == key(+0).
// Every finite score has a key >= 0x00800000, so 0 marks "no candidate".
__device__ __forceinline__ uint32_t score_key(float f) {
    const uint32_t u = f == 0.0f ? 0u : __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Maximum of v over the 64 lanes (wave-uniform result): within each row of 16 lanes by DPP,
// then over the four rows.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = row16_max_u32(v);
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(r0, r1), max(r2, r3));
}

// Sum of x over the 64 lanes (wave-uniform result), in a fixed order: within each row of 16
// lanes by the DPP steps of row16_max_u32 (on both halves of the double), then the four row sums
// in row order.
template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double x) {
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, kCtrl, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), kCtrl, 0xF, 0xF, false);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double wave_sum_f64(double x) {
    x += dpp_f64<0xB1>(x);
    x += dpp_f64<0x4E>(x);
    x += dpp_f64<0x141>(x);
    x += dpp_f64<0x140>(x);
    auto lane_value = [&](int l) {
        const uint64_t u = (uint64_t)__double_as_longlong(x);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
        return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
    };
    return ((lane_value(0) + lane_value(16)) + lane_value(32)) + lane_value(48);
}

// Routes one token: s = its E scores; writes ids[0..k) and w[0..k) (and the ids to lds_ids too,
// when it is not null).  Must be called by a whole wave.
template <int VPL>
__device__ __forceinline__ void route_token(const float* __restrict__ s, int E, int k, int score_fn,
                                            int renorm, int32_t* __restrict__ ids,
                                            float* __restrict__ wts, int* lds_ids = nullptr) {
    const int lane = lane_id();
    float v[VPL];
    uint32_t key[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e = lane + kWave * i;
        v[i] = e < E ? s[e] : 0.0f;
        key[i] = e < E ? score_key(v[i]) : 0u;
    }
    int my_id = -1;
    float my_s = 0.0f;
    for (int j = 0; j < k; ++j) {
        uint32_t kb = 0u;  // this lane's best untaken key and its i (the lowest i on equal keys)
        int ib = 0;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (key[i] > kb) {
                kb = key[i];
                ib = i;
            }
        const uint32_t m = wave_max_u32(kb);
        int wi = 0, wl = 0;  // the winner: i, then lane
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const uint64_t b = __ballot(kb == m && ib == i);
            if (b) {
                wi = i;
                wl = __ffsll((unsigned long long)b) - 1;
                break;
            }
        }
        float vw = v[0];
#pragma unroll
        for (int i = 1; i < VPL; ++i)
            if (i == wi) vw = v[i];
        const float sw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vw), wl));
        if (lane == wl) {
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                if (i == wi) key[i] = 0u;  // taken
        }
        if (lane == j) {
            my_id = wl + kWave * wi;
            my_s = sw;
        }
    }
    // gate weights, in double
    const bool slot = lane < k;
    double num = 0.0, den_part = 0.0;
    if (score_fn == MOE_SCORE_SOFTMAX) {
        const double mx = (double)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), 0));  // slot 0: the maximum
        if (slot) num = exp((double)my_s - mx);
        if (renorm) {
            den_part = num;
        } else {
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                if (lane + kWave * i < E) den_part += exp((double)v[i] - mx);
        }
    } else {
        if (slot) num = 1.0 / (1.0 + exp(-(double)my_s));
        den_part = renorm ? num : 0.0;
    }
    double den = wave_sum_f64(den_part);
    if (score_fn == MOE_SCORE_SIGMOID && !renorm) den = 1.0;
    if (slot) {
        ids[lane] = my_id;
        wts[lane] = (float)(num / den);
        if (lds_ids) lds_ids[lane] = my_id;
    }
}

// VPL (scores per lane) for E experts: the smallest of 1, 2, 4, 8, 16 with 64 * VPL >= E.
inline int route_vpl(int E) {
    const int v = (E + kWave - 1) / kWave;
    return v <= 1 ? 1 : v <= 2 ? 2 : v <= 4 ? 4 : v <= 8 ? 8 : 16;
}

}  // namespace moe

// moe_route.h -- device routine of top-k routing for one token, run by one wave64.
//
// The router keeps, per token, the k experts with the largest score and turns their scores into
// normalised gate weights (sparse MoE FFN with a few active experts per token: CMU 11-868
// appendix A2 notes, 4.1; DeepSeek-V3 routes each token to 8 of 256 experts: KTransformers
// article, 1.2; "gating" opens the expert-parallel flow in the OSDI'26 hybrid-inference article,
// DSLP section).
//
// Each lane holds the scores e = lane + 64*i (coalesced loads).  The k winners are found by k
// rounds of a wave-wide arg-max over (score, -id) -- exact fp32 comparisons, so the selection
// is bit-identical to any correct top-k with the same tie rule (lower id wins; -0 == +0).
// Slot j of the result ends up in lane j, which computes its weight in double.
#pragma once

#include "libmoe.h"
#include "moe_device.h"

namespace moe {

__device__ __forceinline__ bool better(float va, int ea, float vb, int eb) {
    // is candidate a ranked before candidate b?  (an id < 0 marks "no candidate")
    if (ea < 0) return false;
    if (eb < 0) return true;
    return va > vb || (va == vb && ea < eb);
}

// Routes one token: s = its E scores; writes ids[0..k) and w[0..k).  Must be called by a whole
// wave.
template <int VPL>
__device__ __forceinline__ void route_token(const float* __restrict__ s, int E, int k, int score_fn,
                                            int renorm, int32_t* __restrict__ ids,
                                            float* __restrict__ wts) {
    const int lane = lane_id();
    float v[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e = lane + kWave * i;
        v[i] = e < E ? s[e] : 0.0f;
    }
    uint32_t taken = 0;
    int my_id = -1;
    float my_s = 0.0f;
    for (int j = 0; j < k; ++j) {
        float bv = 0.0f;
        int be = -1;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int e = lane + kWave * i;
            if (e < E && !((taken >> i) & 1u) && better(v[i], e, bv, be)) {
                bv = v[i];
                be = e;
            }
        }
#pragma unroll
        for (int off = kWave / 2; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off, kWave);
            const int oe = __shfl_xor(be, off, kWave);
            if (better(ov, oe, bv, be)) {
                bv = ov;
                be = oe;
            }
        }
        if ((be & (kWave - 1)) == lane) taken |= 1u << (be >> 6);
        if (lane == j) {
            my_id = be;
            my_s = bv;
        }
    }
    // gate weights, in double
    const bool slot = lane < k;
    double num = 0.0, den_part = 0.0;
    if (score_fn == MOE_SCORE_SOFTMAX) {
        const double mx = (double)__shfl(my_s, 0, kWave);  // slot 0 holds the maximum
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
    double den = den_part;
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) den += __shfl_xor(den, off, kWave);
    if (score_fn == MOE_SCORE_SIGMOID && !renorm) den = 1.0;
    if (slot) {
        ids[lane] = my_id;
        wts[lane] = (float)(num / den);
    }
}

// VPL (scores per lane) for E experts: the smallest of 1, 2, 4, 8, 16 with 64 * VPL >= E.
inline int route_vpl(int E) {
    const int v = (E + kWave - 1) / kWave;
    return v <= 1 ? 1 : v <= 2 ? 2 : v <= 4 ? 4 : v <= 8 ? 8 : 16;
}

}  // namespace moe

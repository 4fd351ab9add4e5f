// moe_ffn.hip -- grouped expert projections (gate/up with SiLU*up, then down).
//
// Every expert is gate, up and down; gate and up feed SiLU(gate)*up, which feeds down, and the
// layer synchronises once after gate/up and once after down (OSDI'26 hybrid-inference article,
// "CPU fine-grained parallelism" section).  Tokens are grouped by expert so that each expert's
// projection is a GEMM over all of its tokens (KTransformers article, 2.2).  Weights are E4M3FN
// with one fp32 scale per 128x128 block; as in the article's FP8 GEMV (section "native FP8
// GEMV", Figures 9-10) the FP8 codes are expanded exactly to bf16, multiplied with bf16
// activations into fp32, and each 128-long partial sum is multiplied by its block scale.
//
// On gfx950 the bf16 x bf16 -> fp32 products run on the matrix cores (MFMA); the per-128-block
// partial sum is one chain of MFMAs whose result is scaled into the running accumulator.
//
// Two kernel shapes:
//   gemv  (few rows per expert, decode): m-tiles of 16 rows, MFMA 16x16x32; each wave streams
//         its weight rows straight from HBM (32 bytes per lane per 128-block, 128 contiguous
//         bytes per row per 4 lanes) and reads its 16 activation rows from L2.
//   gemm  (many rows per expert, prefill): see moe_gemm.hip.
#include "libmoe.h"
#include "moe_device.h"
#include "moe_ffn.h"
#include "moe_host.h"

namespace moe {

// One workgroup = 4 waves; each wave owns two 16-row weight groups (phase 1: the same 16 rows
// of gate and of up; phase 2: 32 consecutive rows of down) over the full K, for one m-tile of
// up to 16 grouped rows.  kGrouped = false is the identity grouping (shared expert).
template <bool kFP8, int kPhase, bool kGrouped>
__global__ __launch_bounds__(256) void gemv_kernel(GemmArgs a) {
    Tile tile;
    const int n_tiles = a.N / (kPhase == 1 ? kGemvColsP1 : kGemvColsP2);
    if (!find_tile(kGrouped ? a.offsets : nullptr, a.n_groups, a.rows, kGemvBM, n_tiles, tile))
        return;

    const int lane = lane_id(), wave = (int)(threadIdx.x >> 6);
    const int m = lane & 15, kq = lane >> 4;
    const int K = a.K;
    const int e = tile.group;
    const int p = tile.row0 + m;
    const bool valid = p < tile.row1;

    // activation row of this lane's M index
    const uint16_t* arow = nullptr;
    if (valid) {
        if (kPhase == 1) {
            const int tok = kGrouped ? a.perm[p] / a.k : p;
            arow = a.act + (size_t)tok * K;
        } else {
            arow = a.act + (size_t)p * K;
        }
    }
    // weight rows of this lane's N index, in both groups
    const int n0 = tile.nt * (kPhase == 1 ? kGemvColsP1 : kGemvColsP2) +
                   wave * (kPhase == 1 ? 16 : 32);
    const size_t esz = kFP8 ? 1 : 2;
    const uint8_t* w0;
    const uint8_t* w1;
    const float* s0 = nullptr;
    const float* s1 = nullptr;
    const int kblocks = K / 128;
    if (kPhase == 1) {
        w0 = (const uint8_t*)a.w0 + ((size_t)e * a.N + n0 + m) * K * esz;
        w1 = (const uint8_t*)a.w1 + ((size_t)e * a.N + n0 + m) * K * esz;
        if (kFP8) {
            s0 = a.s0 + ((size_t)e * (a.N / 128) + n0 / 128) * kblocks;
            s1 = a.s1 + ((size_t)e * (a.N / 128) + n0 / 128) * kblocks;
        }
    } else {
        w0 = (const uint8_t*)a.w0 + ((size_t)e * a.N + n0 + m) * K * esz;
        w1 = (const uint8_t*)a.w0 + ((size_t)e * a.N + n0 + 16 + m) * K * esz;
        if (kFP8) {
            s0 = a.s0 + ((size_t)e * (a.N / 128) + n0 / 128) * kblocks;
            s1 = s0;
        }
    }

    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    constexpr int kWVec = kFP8 ? 2 : 4;  // 16-byte vectors of weights per lane per 128-block
    u32x4 b0[kWVec], b1[kWVec], xa[4];
    auto load = [&](int kb) {
        const int k0 = kb * 128 + kq * 32;  // this lane's 32 K values of the block
        const u32x4* q0 = (const u32x4*)(w0 + (size_t)k0 * esz);
        const u32x4* q1 = (const u32x4*)(w1 + (size_t)k0 * esz);
#pragma unroll
        for (int i = 0; i < kWVec; ++i) {
            b0[i] = __builtin_nontemporal_load(q0 + i);
            b1[i] = __builtin_nontemporal_load(q1 + i);
        }
        if (valid) {
            const u32x4* xr = (const u32x4*)(arow + k0);
#pragma unroll
            for (int i = 0; i < 4; ++i) xa[i] = xr[i];
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) xa[i] = u32x4{0u, 0u, 0u, 0u};
        }
    };
    load(0);
    for (int kb = 0; kb < kblocks; ++kb) {
        u32x4 cb0[kWVec], cb1[kWVec], cx[4];
#pragma unroll
        for (int i = 0; i < kWVec; ++i) {
            cb0[i] = b0[i];
            cb1[i] = b1[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) cx[i] = xa[i];
        if (kb + 1 < kblocks) load(kb + 1);
        f32x4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bf16x8 g0, g1;
            if (kFP8) {
                const uint32_t* u0 = (const uint32_t*)cb0;
                const uint32_t* u1 = (const uint32_t*)cb1;
                g0 = fp8x8_to_bf16x8(u0[2 * i], u0[2 * i + 1]);
                g1 = fp8x8_to_bf16x8(u1[2 * i], u1[2 * i + 1]);
            } else {
                g0 = as_bf16x8(cb0[i]);
                g1 = as_bf16x8(cb1[i]);
            }
            const bf16x8 xv = as_bf16x8(cx[i]);
            p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, g0, p0, 0, 0, 0);
            p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, g1, p1, 0, 0, 0);
        }
        if (kFP8) {
            const float sc0 = s0[kb], sc1 = s1[kb];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                acc0[r] = fmaf(p0[r], sc0, acc0[r]);
                acc1[r] = fmaf(p1[r], sc1, acc1[r]);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                acc0[r] += p0[r];
                acc1[r] += p1[r];
            }
        }
    }

    // D layout of the 16x16 MFMA: lane holds rows 4*(lane/16)+r (grouped rows), column lane%16
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = tile.row0 + kq * 4 + r;
        if (row >= tile.row1) continue;
        if (kPhase == 1) {
            const float g = acc0[r], u = acc1[r];
            const float hval = g / (1.0f + __expf(-g)) * u;
            a.out[(size_t)row * a.N + n0 + m] = f32_to_bf16(hval);
        } else {
            a.out[(size_t)row * a.N + n0 + m] = f32_to_bf16(acc0[r]);
            a.out[(size_t)row * a.N + n0 + 16 + m] = f32_to_bf16(acc1[r]);
        }
    }
}

static int max_mtiles(int rows, int n_groups, int BM) {
    const int64_t bound = ((int64_t)rows + BM - 1) / BM + std::min<int64_t>(n_groups, rows);
    return (int)bound;
}

// Launch one phase.  rows = grouped rows (T*k).
static moe_status launch_phase(int phase, const GemmArgs& a, int rows_per_group_hint,
                               hipStream_t st) {
    const bool fp8 = a.fp8;
    const bool gemv = use_gemv(a.rows, a.n_groups);
    (void)rows_per_group_hint;
    if (!gemv) return launch_gemm(phase, a, st);
    const int cols = phase == 1 ? kGemvColsP1 : kGemvColsP2;
    const int64_t wgs = (int64_t)max_mtiles(a.rows, a.offsets ? a.n_groups : 1, kGemvBM) * (a.N / cols);
    const dim3 grid((unsigned)((wgs + 7) & ~int64_t(7))), block(256);
#define MOE_GEMV(F, P, G) gemv_kernel<F, P, G><<<grid, block, 0, st>>>(a)
    const bool g = a.offsets != nullptr;
    if (phase == 1) {
        if (fp8) g ? MOE_GEMV(true, 1, true) : MOE_GEMV(true, 1, false);
        else g ? MOE_GEMV(false, 1, true) : MOE_GEMV(false, 1, false);
    } else {
        if (fp8) g ? MOE_GEMV(true, 2, true) : MOE_GEMV(true, 2, false);
        else g ? MOE_GEMV(false, 2, true) : MOE_GEMV(false, 2, false);
    }
#undef MOE_GEMV
    return launch_status();
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_expert_gate_up(const uint16_t* x, int32_t T, int32_t k,
                                         const int32_t* perm, const int32_t* offsets,
                                         const moe_expert_weights* w, uint16_t* h, void* stream) {
    if (T < 0 || k < 1) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!x || !h) return MOE_ERR_INVALID_ARG;
    moe_status s = check_weights(w);
    if (s != MOE_OK) return s;
    if ((s = check_grouping(T, k, perm, offsets, w, true)) != MOE_OK) return s;
    GemmArgs a{};
    a.act = x;
    a.perm = perm;
    a.offsets = offsets;
    a.k = k;
    a.rows = T * k;
    a.n_groups = w->n_groups;
    a.N = w->I;
    a.K = w->H;
    a.w0 = w->w_gate;
    a.w1 = w->w_up;
    a.s0 = w->s_gate;
    a.s1 = w->s_up;
    a.fp8 = w->dtype == MOE_W_FP8_E4M3_B128;
    a.out = h;
    return launch_phase(1, a, 0, as_stream(stream));
}

extern "C" moe_status moe_expert_down(const uint16_t* h, int32_t T, int32_t k,
                                      const int32_t* offsets, const moe_expert_weights* w,
                                      uint16_t* y, void* stream) {
    if (T < 0 || k < 1) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!h || !y) return MOE_ERR_INVALID_ARG;
    moe_status s = check_weights(w);
    if (s != MOE_OK) return s;
    if ((s = check_grouping(T, k, nullptr, offsets, w, false)) != MOE_OK) return s;
    GemmArgs a{};
    a.act = h;
    a.perm = nullptr;
    a.offsets = offsets;
    a.k = k;
    a.rows = T * k;
    a.n_groups = w->n_groups;
    a.N = w->H;
    a.K = w->I;
    a.w0 = w->w_down;
    a.w1 = nullptr;
    a.s0 = w->s_down;
    a.s1 = nullptr;
    a.fp8 = w->dtype == MOE_W_FP8_E4M3_B128;
    a.out = y;
    return launch_phase(2, a, 0, as_stream(stream));
}

extern "C" moe_status moe_expert_ffn_workspace_size(int32_t T, int32_t k,
                                                    const moe_expert_weights* w, size_t* bytes) {
    if (!bytes || !w || T < 0 || k < 1 || w->I < 1) return MOE_ERR_INVALID_ARG;
    *bytes = (size_t)T * (size_t)k * (size_t)w->I * 2u;
    return MOE_OK;
}

extern "C" moe_status moe_expert_ffn(const uint16_t* x, int32_t T, int32_t k, const int32_t* perm,
                                     const int32_t* offsets, const moe_expert_weights* w,
                                     uint16_t* y, void* ws, size_t ws_bytes, void* stream) {
    if (T < 0 || k < 1) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    size_t need = 0;
    moe_status s = moe_expert_ffn_workspace_size(T, k, w, &need);
    if (s != MOE_OK) return s;
    if (!x || !y) return MOE_ERR_INVALID_ARG;
    if ((s = check_weights(w)) != MOE_OK) return s;
    if ((s = check_grouping(T, k, perm, offsets, w, true)) != MOE_OK) return s;
    if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
    uint16_t* h = static_cast<uint16_t*>(ws);
    if ((s = moe_expert_gate_up(x, T, k, perm, offsets, w, h, stream)) != MOE_OK) return s;
    return moe_expert_down(h, T, k, offsets, w, y, stream);
}

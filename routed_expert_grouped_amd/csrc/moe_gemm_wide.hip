// moe_gemm_wide.hip -- grouped expert GEMM for FP8 weights and bf16 activations with 160-row x
// 512-weight-row tiles.
//
// Same arithmetic as the 256 x 256 kernel of moe_gemm.hip: tokens grouped by expert so that
// each expert's projection is a GEMM (KTransformers article, 2.2); FP8 codes expanded exactly to
// bf16 as they leave LDS, MFMA 32x32x16 with fp32 accumulation, and each 128-long block's sum
// multiplied by its block scale (the OSDI'26 article's post-scaling, section "native FP8 GEMV",
// Figures 9-10), kept in units of the current block's scale as in moe_gemm.hip.
//
// Why this shape: the direct-to-LDS loads of a stage, not HBM or the matrix cores, bound these
// GEMMs, and each m-tile's activations are loaded once per weight tile.  A 160 x 512 tile loads
// 20 KB of activations + 32 KB of codes per 64-long stage for 160 x 512 outputs, against 32 + 16 KB
// for 256 x 256 in the other kernel: about a quarter fewer bytes per output at 128 rows per expert
// (the mean at T = 4096, DeepSeek-V3 shapes), and a 160-row m-tile still holds a whole expert
// there (95-160 rows).  The 3-stage ring takes 156 KB of LDS.
//
// Waves: 8, each owning 64 weight rows (phase 1: 32 gate + the same 32 up rows -> 32 h columns;
// phase 2: 64 y columns) against all five 32-row m-subtiles.  Activation loads: waves 0-3 load
// three 8-row instructions of each stage, waves 4-7 two (160 rows); code loads: four 16-row
// instructions per wave.  A wave whose activation rows all lie past the m-tile loads none of
// them; its hand-counted waits follow from its own load count.
#include "libmoe.h"
#include "moe_device.h"
#include "moe_ffn.h"
#include "moe_host.h"
#include "moe_lds.h"

#include <type_traits>

namespace moe {

constexpr int kWM = 160;        // rows per m-tile (5 subtiles of 32)
constexpr int kWN = 512;        // weight rows per tile
constexpr int kWK = 64;         // K per stage (half a scale block)
constexpr int kWStages = 3;
constexpr int kWMaxKBlocks = MOE_MAX_DIM / 128;

template <int kPhase, bool kGrouped>
__global__ __launch_bounds__(512, 1) void gemm_fp8_wide_kernel(GemmArgs a) {
    constexpr int kAStage = kWM * kWK * 2;  // 20 KB
    constexpr int kBStage = kWN * kWK;      // 32 KB
    __shared__ __attribute__((aligned(1024))) uint8_t sA[kWStages][kAStage];
    __shared__ __attribute__((aligned(1024))) uint8_t sB[kWStages][kBStage];
    __shared__ float sScale[4][kWMaxKBlocks];  // the tile's four 128-row block-rows

    constexpr int kCols = kPhase == 1 ? kWN / 2 : kWN;
    Tile tile;
    if (!find_tile(kGrouped ? a.offsets : nullptr, a.n_groups, a.rows, kWM, a.N / kCols, tile))
        return;

    const int tid = (int)threadIdx.x, lane = lane_id(), wave = uniform(tid >> 6);
    const int e = tile.group;
    const int c0 = tile.nt * kCols;
    const int K = a.K, kblocks = K / 128, nq = 2 * kblocks;
    const int fr = lane & 31, half = lane >> 5;

    // activation loads: waves 0-3 fill stage rows 24 w + 8 i + lane / 8 (i < 3), waves 4-7 rows
    // 96 + 16 (w - 4) + 8 i + lane / 8 (i < 2); slot lane % 8 holds chunk slot ^ ((row >> 1) & 7);
    // rows past the m-tile load its first row (never stored)
    const int arow0 = wave < 4 ? 24 * wave : 96 + 16 * (wave - 4);
    uint32_t aoff[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int r = min(arow0 + 8 * i + (lane >> 3), kWM - 1);
        const int p = tile.row0 + r < tile.row1 ? tile.row0 + r : tile.row0;
        const uint32_t src = (kPhase == 1 && kGrouped) ? (uint32_t)(a.perm[p] / a.k) : (uint32_t)p;
        aoff[i] = src * (uint32_t)(K / 8) + (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
    }
    // code loads: instruction i (0..3) of wave w fills stage rows 64 w + 16 i + lane / 4, slot
    // lane % 4 holding chunk slot ^ ((row >> 2) & 3); phase 1 rows 0..255 gate, 256..511 up
    const uint8_t* bsrc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 64 * wave + 16 * i + (lane >> 2);
        const uint8_t* base;
        int wr;
        if (kPhase == 1) {
            base = (const uint8_t*)(r < 256 ? a.w0 : a.w1);
            wr = c0 + (r & 255);
        } else {
            base = (const uint8_t*)a.w0;
            wr = c0 + r;
        }
        bsrc[i] = base + ((size_t)e * a.N + wr) * (size_t)K + (((lane & 3) ^ ((r >> 2) & 3)) << 4);
    }
    const bool load_a = arow0 < tile.row1 - tile.row0;
    auto issue = [&](int q, int st, auto ai_tag, auto a_tag) {
        constexpr int AI = decltype(ai_tag)::value;
        if (decltype(a_tag)::value) {
            const uint8_t* act = (const uint8_t*)a.act + (size_t)q * (kWK * 2);
#pragma unroll
            for (int i = 0; i < AI; ++i)
                lds_dma16(act + (size_t)aoff[i] * 16, &sA[st][(arow0 + 8 * i) * kWK * 2]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            lds_dma16(bsrc[i] + (size_t)q * kWK, &sB[st][(64 * wave + 16 * i) * kWK]);
    };

    // block scales of the tile's rows: phase 1 [0], [1] gate block-rows c0/128, +1, [2], [3] the
    // same up block-rows; phase 2 the four block-rows from c0/128
    for (int i = tid; i < 4 * kblocks; i += 512) {
        const int br = i / kblocks, b = i - br * kblocks;
        const float* s = kPhase == 1 ? (br < 2 ? a.s0 : a.s1) : a.s0;
        const int row = kPhase == 1 ? c0 / 128 + (br & 1) : c0 / 128 + br;
        sScale[br][b] = s[((size_t)e * (a.N / 128) + row) * kblocks + b];
    }
    // this wave's weight subtiles ni = 0, 1: phase 1 gate / up rows 32 w .. 32 w + 31 (block-rows
    // w / 4 and 2 + w / 4); phase 2 rows 64 w + 32 ni (block-row w / 2)
    const int sg0 = kPhase == 1 ? (wave >> 2) : (wave >> 1);
    const int sg1 = kPhase == 1 ? 2 + (wave >> 2) : (wave >> 1);

    const int mine = (tile.row1 - tile.row0 + 31) >> 5;  // filled 32-row subtiles (1..5)
    int aaddr[4], baddr[2][2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // subtile 0; subtile mi adds mi * 32 rows (same swizzle)
        const int c = 4 * (q >> 1) + 2 * half + (q & 1);
        aaddr[q] = fr * (kWK * 2) + ((c ^ ((fr >> 1) & 7)) << 4);
    }
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        const int r = (kPhase == 1 ? ni * 256 + wave * 32 : wave * 64 + ni * 32) + fr;
#pragma unroll
        for (int j = 0; j < 2; ++j) baddr[ni][j] = r * kWK + (((2 * j + half) ^ ((r >> 2) & 3)) << 4);
    }
    bool any_zero = false;
    __syncthreads();  // scales staged
    for (int b = lane; b < kblocks; b += kWave)
        any_zero |= sScale[sg0][b] == 0.0f || sScale[sg1][b] == 0.0f;
    any_zero = __ballot(any_zero) != 0;

    f32x16 acc[5][2];
#pragma unroll
    for (int mi = 0; mi < 5; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int x = 0; x < 16; ++x) acc[mi][ni][x] = 0.0f;

    // block scales as in moe_gemm.hip: the accumulator is kept in units of the current block's
    // scale; a zero scale keeps the units and masks the block's codes
    float u0 = 0.0f, u1 = 0.0f;
    uint32_t m0 = ~0u, m1 = ~0u;
    auto rescale = [&](float r0, float r1, auto ns_tag) {
        constexpr int NS = decltype(ns_tag)::value;
#pragma unroll
        for (int mi = 0; mi < NS; ++mi)
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                acc[mi][0][x] *= r0;
                acc[mi][1][x] *= r1;
            }
    };
    // one 64-long stage from ring slot ST with NS filled m-subtiles.  Stage q needs the loads
    // issued two stages earlier; the ones of the stage in between stay in flight.
    auto stage = [&](int q, auto st_tag, auto ns_tag, auto mask_tag, auto ai_tag, auto a_tag) {
        constexpr int ST = decltype(st_tag)::value, NS = decltype(ns_tag)::value;
        constexpr bool kMask = decltype(mask_tag)::value;
        constexpr int kIssued = (decltype(a_tag)::value ? decltype(ai_tag)::value : 0) + 4;
        if (q + 1 < nq)
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(kIssued));
        else
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();
        if (q + 2 < nq) issue(q + 2, (ST + 2) % kWStages, ai_tag, a_tag);
        if (NS == 0) return;
        if ((q & 1) == 0) {  // first half of scale block q / 2
            const int kb = q >> 1;
            const float s0 = sScale[sg0][kb], s1 = sScale[sg1][kb];
            if (kMask) {
                const bool z0 = s0 == 0.0f, z1 = s1 == 0.0f;
                const float r0 = z0 ? 1.0f : u0 * __builtin_amdgcn_rcpf(s0);
                const float r1 = z1 ? 1.0f : u1 * __builtin_amdgcn_rcpf(s1);
                u0 = z0 ? u0 : s0;
                u1 = z1 ? u1 : s1;
                m0 = z0 ? 0u : ~0u;
                m1 = z1 ? 0u : ~0u;
                rescale(r0, r1, ns_tag);
            } else {
                rescale(u0 * __builtin_amdgcn_rcpf(s0), u1 * __builtin_amdgcn_rcpf(s1), ns_tag);
                u0 = s0;
                u1 = s1;
            }
        }
        const uint8_t* A = sA[ST];
        const uint8_t* B = sB[ST];
#pragma unroll
        for (int j = 0; j < kWK / 32; ++j) {
            u32x4 fbq[2];
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                fbq[ni] = *(const u32x4*)&B[baddr[ni][j]];
                if (kMask) fbq[ni] &= ni == 0 ? m0 : m1;
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                bf16x8 fa[NS];
#pragma unroll
                for (int mi = 0; mi < NS; ++mi)
                    fa[mi] = *(const bf16x8*)&A[aaddr[2 * j + t] + mi * 32 * kWK * 2];
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) {
                    const bf16x8 fb = fp8x8_to_bf16x8(fbq[ni][2 * t], fbq[ni][2 * t + 1]);
#pragma unroll
                    for (int mi = 0; mi < NS; ++mi)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb, acc[mi][ni], 0, 0, 0);
                }
            }
        }
    };
    auto run = [&](auto ns_tag, auto mask_tag, auto ai_tag, auto a_tag) {
        using S0 = std::integral_constant<int, 0>;
        using S1 = std::integral_constant<int, 1>;
        using S2 = std::integral_constant<int, 2>;
        issue(0, 0, ai_tag, a_tag);
        issue(1, 1, ai_tag, a_tag);  // nq >= 2
        for (int q = 0; q < nq; q += 3) {
            stage(q, S0{}, ns_tag, mask_tag, ai_tag, a_tag);
            if (q + 1 < nq) stage(q + 1, S1{}, ns_tag, mask_tag, ai_tag, a_tag);
            if (q + 2 < nq) stage(q + 2, S2{}, ns_tag, mask_tag, ai_tag, a_tag);
        }
    };
    using MY = std::integral_constant<bool, true>;
    using MN = std::integral_constant<bool, false>;
    auto by_ns = [&](auto mask_tag, auto ai_tag, auto a_tag) {
        if (mine >= 5) run(std::integral_constant<int, 5>{}, mask_tag, ai_tag, a_tag);
        else if (mine == 4) run(std::integral_constant<int, 4>{}, mask_tag, ai_tag, a_tag);
        else if (mine == 3) run(std::integral_constant<int, 3>{}, mask_tag, ai_tag, a_tag);
        else if (mine == 2) run(std::integral_constant<int, 2>{}, mask_tag, ai_tag, a_tag);
        else run(std::integral_constant<int, 1>{}, mask_tag, ai_tag, a_tag);
    };
    // the K loop for this wave's activation load count (3 or 2, or none past the m-tile) and
    // the filled-subtile count; a tile with a zero block scale takes the masked path
    auto by_loads = [&](auto ai_tag) {
        if (!load_a) {
            if (any_zero) run(std::integral_constant<int, 5>{}, MY{}, ai_tag, std::false_type{});
            else by_ns(MN{}, ai_tag, std::false_type{});
        } else {
            if (any_zero) run(std::integral_constant<int, 5>{}, MY{}, ai_tag, std::true_type{});
            else by_ns(MN{}, ai_tag, std::true_type{});
        }
    };
    if (wave < 4)
        by_loads(std::integral_constant<int, 3>{});
    else
        by_loads(std::integral_constant<int, 2>{});
    rescale(u0, u1, std::integral_constant<int, 5>{});

    // D layout of the 32x32 MFMA: value x of a lane is row 8*(x/4) + 4*(lane/32) + x%4 of the
    // subtile, column lane%32
#pragma unroll
    for (int mi = 0; mi < 5; ++mi) {
        if (mi >= mine) break;
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            const int p = tile.row0 + mi * 32 + 8 * (x >> 2) + 4 * half + (x & 3);
            if (p >= tile.row1) continue;
            uint16_t* o = a.out + (size_t)p * a.N + c0 + fr;
            if (kPhase == 1) {
                const float g = acc[mi][0][x], u = acc[mi][1][x];
                o[wave * 32] = f32_to_bf16(silu_mul(g, u));
            } else {
                const uint32_t b = f32x2_to_bf16x2(acc[mi][0][x], acc[mi][1][x]);
                o[wave * 64] = (uint16_t)b;
                o[wave * 64 + 32] = (uint16_t)(b >> 16);
            }
        }
    }
}

bool wide_gemm_fits(int phase, const GemmArgs& a) {
    if (!a.fp8 || a.K / 128 > kWMaxKBlocks) return false;
    if (a.N % (phase == 1 ? kWN / 2 : kWN) != 0) return false;
    // activation rows are addressed by 32-bit 16-byte chunk indices
    return (int64_t)a.rows * (a.K / 8) < (int64_t(1) << 32);
}

moe_status launch_gemm_wide(int phase, const GemmArgs& a, hipStream_t st) {
    if (!wide_gemm_fits(phase, a)) return MOE_ERR_UNSUPPORTED;
    const int cols = phase == 1 ? kWN / 2 : kWN;
    const int groups = a.offsets ? a.n_groups : 1;
    const int64_t mt = ((int64_t)a.rows + kWM - 1) / kWM + std::min<int64_t>(groups, a.rows);
    const int64_t wgs = mt * (a.N / cols);
    if (wgs > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)((wgs + 7) & ~int64_t(7))), block(512);
    const bool g = a.offsets != nullptr;
    if (phase == 1) {
        if (g) gemm_fp8_wide_kernel<1, true><<<grid, block, 0, st>>>(a);
        else gemm_fp8_wide_kernel<1, false><<<grid, block, 0, st>>>(a);
    } else {
        if (g) gemm_fp8_wide_kernel<2, true><<<grid, block, 0, st>>>(a);
        else gemm_fp8_wide_kernel<2, false><<<grid, block, 0, st>>>(a);
    }
    return launch_status();
}

}  // namespace moe

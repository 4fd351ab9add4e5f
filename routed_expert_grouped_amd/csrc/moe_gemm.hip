// moe_gemm.hip -- grouped expert GEMMs for many rows per expert (prefill shapes).
//
// Tokens that hit the same expert are batched so that the expert's projection is a GEMM
// (KTransformers article, 2.2).  Each expert's rows are cut into m-tiles; a workgroup computes
// one m-tile against a tile of weight rows over the whole K:
//   phase 1: gate rows + the same up rows -> columns of h = SiLU(gate) * up
//   phase 2: down rows -> columns of y
// Weights are expanded exactly from FP8 to bf16 as they leave LDS and multiplied on MFMA
// 32x32x16 (bf16 in, fp32 accumulate); each 128-long K block is one FP8 scale block, applied to
// that block's MFMA sum (the post-scaling of the OSDI'26 article's FP8 GEMV, section "native
// FP8 GEMV", Figures 9-10).
//
// Kernels, picked by launch_gemm:
//   gemm_fp8_wide_kernel  (moe_gemm_wide.hip) FP8 weights, at most 160 rows per expert on
//                         average: 160-row m-tiles x 512 weight rows;
//   gemm_fp8_q256_kernel  FP8 weights, H a multiple of 256: one 8-wave workgroup per CU,
//                         256-row m-tiles x 256 weight rows, all loads direct to LDS;
//   gemm_kernel           bf16 weights and the other FP8 shapes (H an odd multiple of 128, or
//                         more than 64 GB of activations): register-staged 128 x 128 tiles.
// A wave owns interleaved 32-row m-subtiles (so a partly filled tile still spreads over both
// wave rows) and 2 32-row weight subtiles (phase 1: matching gate and up rows, so SiLU(gate)*up
// is formed in registers); subtiles past the last row are skipped.
#include "libmoe.h"
#include "moe_device.h"
#include "moe_ffn.h"
#include "moe_host.h"
#include "moe_lds.h"

#include <type_traits>

namespace moe {

constexpr int kBM = 128;            // rows per m-tile
constexpr int kBN = 128;            // weight rows per tile
constexpr int kBK = 128;            // K per block (one scale block)
constexpr int kLDA = kBK * 2 + 16;  // A row stride in LDS (bytes): 16-lane b128 reads hit distinct banks
constexpr int kMaxKBlocks = 128;    // K <= 16384 (block scales are staged in LDS)
constexpr int kWideRows = 160;      // m-tile rows of the 160 x 512 kernel (moe_gemm_wide.hip)

template <bool kFP8, int kPhase, bool kGrouped>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmArgs a) {
    constexpr int kRowB = kFP8 ? kBK : kBK * 2;    // bytes of one weight row per block
    constexpr int kLDB = kRowB + 16;               // B row stride (bytes): 16-aligned, conflict-free b128
    constexpr int kBLanes = kRowB / 16;            // threads per weight row
    constexpr int kBPer = kBN * kBLanes / 256;     // 16-byte B chunks per thread
    __shared__ __attribute__((aligned(16))) uint8_t sA[kBM * kLDA];
    __shared__ __attribute__((aligned(16))) uint8_t sB[kBN * kLDB];
    __shared__ float sScale[2][kMaxKBlocks];

    constexpr int kCols = kPhase == 1 ? kBN / 2 : kBN;  // output columns per tile
    Tile tile;
    const int n_tiles = a.N / kCols;
    if (!find_tile(kGrouped ? a.offsets : nullptr, a.n_groups, a.rows, kBM, n_tiles, tile)) return;

    const int tid = (int)threadIdx.x, lane = lane_id(), wave = uniform(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int e = tile.group;
    const int c0 = tile.nt * kCols;
    const int K = a.K, kblocks = K / kBK;
    const int fr = lane & 31, half = lane >> 5;

    // ---- activation staging: thread -> 16-byte chunk (tid % 16) of rows tid/16 + 16i.
    // Rows past the end of the m-tile load the tile's first row (never stored), so the loads
    // are unconditional.
    uint32_t arow[8];  // source row (token, or grouped row) of each staged row
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int p0 = tile.row0 + (tid >> 4) + 16 * i;
        const int p = p0 < tile.row1 ? p0 : tile.row0;
        arow[i] = (uint32_t)((kPhase == 1 && kGrouped) ? a.perm[p] / a.k : p);
    }
    const uint16_t* abase = a.act + (tid & 15) * 8;
    // ---- weight staging: thread -> 16-byte chunk (tid % kBLanes) of LDS rows tid/kBLanes + ...
    const uint8_t* brow[kBPer];
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
        const int r = tid / kBLanes + (256 / kBLanes) * i;  // LDS row 0..127
        const uint8_t* base;
        int wr;
        if (kPhase == 1) {
            base = (const uint8_t*)(r < 64 ? a.w0 : a.w1);
            wr = c0 + (r & 63);
        } else {
            base = (const uint8_t*)a.w0;
            wr = c0 + r;
        }
        brow[i] = base + ((size_t)e * a.N + wr) * (size_t)K * (kFP8 ? 1 : 2) + (tid % kBLanes) * 16;
    }
    // ---- block scales of this tile, staged once: gate and up (phase 1) or down (phase 2)
    if (kFP8 && tid < kblocks) {
        const size_t srow = ((size_t)e * (a.N / 128) + c0 / 128) * kblocks;
        sScale[0][tid] = a.s0[srow + tid];
        sScale[1][tid] = kPhase == 1 ? a.s1[srow + tid] : a.s0[srow + tid];
    }

    u32x4 ra[8], rb[kBPer];
    auto load = [&](int kb) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            ra[i] = *(const u32x4*)(abase + (size_t)arow[i] * K + kb * kBK);
#pragma unroll
        for (int i = 0; i < kBPer; ++i)
            rb[i] = __builtin_nontemporal_load((const u32x4*)(brow[i] + (size_t)kb * kRowB));
    };
    auto store = [&]() {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *(u32x4*)&sA[((tid >> 4) + 16 * i) * kLDA + (tid & 15) * 16] = ra[i];
#pragma unroll
        for (int i = 0; i < kBPer; ++i) {
            uint8_t* dst = &sB[(tid / kBLanes + (256 / kBLanes) * i) * kLDB + (tid % kBLanes) * 16];
            *(u32x4*)dst = rb[i];
        }
    };

    // subtiles of this wave: m-subtiles wm and wm + 2 (32 rows each); weight subtiles:
    // phase 1 gate rows wn*32.. and up rows 64 + wn*32..; phase 2 rows wn*64.. and wn*64 + 32..
    const int nvalid = (tile.row1 - tile.row0 + 31) >> 5;  // filled 32-row subtiles (1..4)
    const int mine = (nvalid > wm) + (nvalid > wm + 2);     // this wave's filled subtiles (0..2)
    int bsub[2];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) bsub[ni] = kPhase == 1 ? ni * 64 + wn * 32 : wn * 64 + ni * 32;

    f32x16 acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

    // weight subtile 0 uses scale 0 and subtile 1 scale 1 (phase 2 staged both equal)
    auto compute = [&](int kb, auto nsub_tag) {
        constexpr int NS = decltype(nsub_tag)::value;  // m-subtiles to compute (1 or 2)
        f32x16 part[NS][2];
#pragma unroll
        for (int mi = 0; mi < NS; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                for (int r = 0; r < 16; ++r) part[mi][ni][r] = 0.0f;
        // k-steps in pairs: for pair j, lane half h covers K elements [32j + 16h, +16) (first 8
        // for step 2j, next 8 for step 2j+1) on both operands, so one b128 weight read feeds two
        // MFMAs
        constexpr int KP = kBK / 32;
#pragma unroll
        for (int j = 0; j < KP; ++j) {
            bf16x8 fa[2][NS];
            u32x4 fbq[2];
            bf16x8 fbh[2][2];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int mi = 0; mi < NS; ++mi)
                    fa[t][mi] = *(const bf16x8*)&sA[((wm + 2 * mi) * 32 + fr) * kLDA + (32 * j + 16 * half + 8 * t) * 2];
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                const uint8_t* q = &sB[(bsub[ni] + fr) * kLDB];
                if (kFP8) {
                    fbq[ni] = *(const u32x4*)(q + 32 * j + 16 * half);
                } else {
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        fbh[t][ni] = *(const bf16x8*)(q + (32 * j + 16 * half + 8 * t) * 2);
                }
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                bf16x8 fb[2];
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    fb[ni] = kFP8 ? fp8x8_to_bf16x8(fbq[ni][2 * t], fbq[ni][2 * t + 1]) : fbh[t][ni];
#pragma unroll
                for (int mi = 0; mi < NS; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni)
                        part[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            fa[t][mi], fb[ni], part[mi][ni], 0, 0, 0);
            }
        }
        const float s0 = kFP8 ? sScale[0][kb] : 1.0f;
        const float s1 = kFP8 ? sScale[1][kb] : 1.0f;
#pragma unroll
        for (int mi = 0; mi < NS; ++mi)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                acc[mi][0][r] = fmaf(part[mi][0][r], s0, acc[mi][0][r]);
                acc[mi][1][r] = fmaf(part[mi][1][r], s1, acc[mi][1][r]);
            }
    };

    load(0);
    for (int kb = 0; kb < kblocks; ++kb) {
        __syncthreads();  // every wave is done reading the previous block (and the scales are in)
        store();
        __syncthreads();
        if (kb + 1 < kblocks) load(kb + 1);
        if (mine == 2)
            compute(kb, std::integral_constant<int, 2>{});
        else if (mine == 1)
            compute(kb, std::integral_constant<int, 1>{});
    }

    // D layout of the 32x32 MFMA: value r of a lane is row 8*(r/4) + 4*(lane/32) + r%4 of the
    // subtile, column lane%32
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
        if (mi >= mine) break;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int p = tile.row0 + (wm + 2 * mi) * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (p >= tile.row1) continue;
            uint16_t* o = a.out + (size_t)p * a.N + c0 + fr;
            if (kPhase == 1) {
                const float g = acc[mi][0][r], u = acc[mi][1][r];
                o[wn * 32] = f32_to_bf16(silu_mul(g, u));
            } else {
                const uint32_t b = f32x2_to_bf16x2(acc[mi][0][r], acc[mi][1][r]);
                o[wn * 64] = (uint16_t)b;
                o[wn * 64 + 32] = (uint16_t)(b >> 16);
            }
        }
    }
}

constexpr int kHK = 64;  // K per stage of the direct-to-LDS kernel (half a scale block)

// ------------------------------------------------------------------ FP8 weights, 256 x 256 tiles
//
// One workgroup of 8 waves per CU computes a 256-row m-tile against 256 weight rows (phase 1:
// 128 gate + the same 128 up rows -> 128 h columns; phase 2: 256 y columns).  Tiles of 256 rows
// cover a whole expert at prefill sizes (about 128 rows per expert at T = 4096), so an expert's
// weights are streamed once instead of once more for a short tail tile.  K goes in 64-long
// stages through a 3-stage ring (32 KB activations + 16 KB FP8 codes per stage), loaded directly
// to LDS two stages ahead.  Waves: 2 (rows) x 4 (weight rows); a wave owns the interleaved
// m-subtiles wm, wm + 2, wm + 4, wm + 6 and 2 weight subtiles (phase 1: matching gate and up).
constexpr int kQM = 256;  // rows per m-tile
constexpr int kQN = 256;  // weight rows per tile

template <int kPhase, bool kGrouped>
__global__ __launch_bounds__(512, 1) void gemm_fp8_q256_kernel(GemmArgs a) {
    constexpr int kAStage = kQM * kHK * 2;  // 32 KB
    constexpr int kBStage = kQN * kHK;      // 16 KB
    constexpr int kStages = 3;
    __shared__ __attribute__((aligned(1024))) uint8_t sA[kStages][kAStage];
    __shared__ __attribute__((aligned(1024))) uint8_t sB[kStages][kBStage];
    __shared__ float sScale[2][kMaxKBlocks];

    constexpr int kCols = kPhase == 1 ? kQN / 2 : kQN;
    Tile tile;
    const int n_tiles = a.N / kCols;
    if (!find_tile(kGrouped ? a.offsets : nullptr, a.n_groups, a.rows, kQM, n_tiles, tile)) return;

    const int tid = (int)threadIdx.x, lane = lane_id(), wave = uniform(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int e = tile.group;
    const int c0 = tile.nt * kCols;
    const int K = a.K, kblocks = K / kBK, nq = 2 * kblocks;
    const int fr = lane & 31, half = lane >> 5;

    // activation loads: instruction i (0..3) of wave w fills stage rows 8 (4 w + i) + lane / 8,
    // slot lane % 8 holding chunk slot ^ ((row >> 1) & 7); rows past the m-tile load its first
    // row (never stored)
    uint32_t aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 8 * (4 * wave + i) + (lane >> 3);
        const int p = tile.row0 + r < tile.row1 ? tile.row0 + r : tile.row0;
        const uint32_t src = (kPhase == 1 && kGrouped) ? (uint32_t)(a.perm[p] / a.k) : (uint32_t)p;
        aoff[i] = src * (uint32_t)(K / 8) + (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
    }
    // weight loads: instruction i (0..1) of wave w fills stage rows 16 (2 w + i) + lane / 4, slot
    // lane % 4 holding chunk slot ^ ((row >> 2) & 3); phase 1 rows 0..127 gate, 128..255 up
    const uint8_t* bsrc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = 16 * (2 * wave + i) + (lane >> 2);
        const uint8_t* base;
        int wr;
        if (kPhase == 1) {
            base = (const uint8_t*)(r < 128 ? a.w0 : a.w1);
            wr = c0 + (r & 127);
        } else {
            base = (const uint8_t*)a.w0;
            wr = c0 + r;
        }
        bsrc[i] = base + ((size_t)e * a.N + wr) * (size_t)K + (((lane & 3) ^ ((r >> 2) & 3)) << 4);
    }
    // A wave whose 32 activation rows all lie past the m-tile's last row loads no activations
    // (no filled m-subtile reads them); the load counts its waits assume follow from kA.
    const bool load_a = 32 * wave < tile.row1 - tile.row0;
    auto issue = [&](int q, int st, auto a_tag) {
        if (decltype(a_tag)::value) {
            const uint8_t* act = (const uint8_t*)a.act + (size_t)q * (kHK * 2);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                lds_dma16(act + (size_t)aoff[i] * 16, &sA[st][8 * (4 * wave + i) * kHK * 2]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
            lds_dma16(bsrc[i] + (size_t)q * kHK, &sB[st][16 * (2 * wave + i) * kHK]);
    };

    // block scales: phase 1 [0] gate, [1] up of block-row c0/128; phase 2 block-rows c0/128 and
    // c0/128 + 1 (the tile's 256 rows)
    if (tid < kblocks) {
        const size_t srow = ((size_t)e * (a.N / 128) + c0 / 128) * kblocks;
        sScale[0][tid] = a.s0[srow + tid];
        sScale[1][tid] = kPhase == 1 ? a.s1[srow + tid] : a.s0[srow + kblocks + tid];
    }
    const int sg0 = kPhase == 1 ? 0 : (wn >> 1);
    const int sg1 = kPhase == 1 ? 1 : (wn >> 1);

    const int nvalid = (tile.row1 - tile.row0 + 31) >> 5;  // filled 32-row subtiles (1..8)
    const int mine = (nvalid > wm) + (nvalid > wm + 2) + (nvalid > wm + 4) + (nvalid > wm + 6);
    int aaddr[4][4], baddr[2][2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int r = (wm + 2 * mi) * 32 + fr;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = 4 * (q >> 1) + 2 * half + (q & 1);
            aaddr[mi][q] = r * (kHK * 2) + ((c ^ ((r >> 1) & 7)) << 4);
        }
    }
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        const int r = (kPhase == 1 ? ni * 128 + wn * 32 : wn * 64 + ni * 32) + fr;
#pragma unroll
        for (int j = 0; j < 2; ++j) baddr[ni][j] = r * kHK + (((2 * j + half) ^ ((r >> 2) & 3)) << 4);
    }
    bool any_zero = false;
    __syncthreads();  // scales staged
    for (int b = lane; b < kblocks; b += kWave)
        any_zero |= sScale[sg0][b] == 0.0f || sScale[sg1][b] == 0.0f;
    any_zero = __ballot(any_zero) != 0;

    f32x16 acc[4][2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int x = 0; x < 16; ++x) acc[mi][ni][x] = 0.0f;

    // Block scales are applied by keeping each accumulator in units of the scale of the block
    // being multiplied: before block b it is multiplied by u / s_b (u = the scale of the last
    // block with a nonzero scale), the block's MFMAs add into it, and the end multiplies by u.
    // This is the post-scaling sum  sum_b s_b * P_b  with one extra fp32 rounding per block and
    // no separate partial sums.  A zero scale keeps the units and masks that block's codes, so
    // the block adds exactly nothing.
    float u0 = 0.0f, u1 = 0.0f;
    uint32_t m0 = ~0u, m1 = ~0u;
    // rescales the accumulators of the first NS m-subtiles (the others are never stored)
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
    // one 64-long stage from ring slot ST with NS filled m-subtiles
    auto stage = [&](int q, auto st_tag, auto ns_tag, auto mask_tag, auto a_tag) {
        constexpr int ST = decltype(st_tag)::value, NS = decltype(ns_tag)::value;
        constexpr bool kMask = decltype(mask_tag)::value;
        constexpr int kIssued = decltype(a_tag)::value ? 6 : 2;  // direct loads per thread per stage
        if (q + 1 < nq)
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(kIssued));
        else
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();
        if (q + 2 < nq) issue(q + 2, (ST + 2) % kStages, a_tag);
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
        for (int j = 0; j < kHK / 32; ++j) {
            u32x4 fbq[2];
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                fbq[ni] = *(const u32x4*)&B[baddr[ni][j]];
                if (kMask) fbq[ni] &= ni == 0 ? m0 : m1;
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                bf16x8 fa[NS > 0 ? NS : 1];
#pragma unroll
                for (int mi = 0; mi < NS; ++mi) fa[mi] = *(const bf16x8*)&A[aaddr[mi][2 * j + t]];
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
    auto run = [&](auto ns_tag, auto mask_tag, auto a_tag) {
        using S0 = std::integral_constant<int, 0>;
        using S1 = std::integral_constant<int, 1>;
        using S2 = std::integral_constant<int, 2>;
        issue(0, 0, a_tag);
        issue(1, 1, a_tag);  // nq >= 2
        for (int q = 0; q < nq; q += 3) {
            stage(q, S0{}, ns_tag, mask_tag, a_tag);
            if (q + 1 < nq) stage(q + 1, S1{}, ns_tag, mask_tag, a_tag);
            if (q + 2 < nq) stage(q + 2, S2{}, ns_tag, mask_tag, a_tag);
        }
    };
    using MY = std::integral_constant<bool, true>;
    using MN = std::integral_constant<bool, false>;
    // the K loop for this wave's filled-subtile count, zero-scale masking and activation loads
    auto dispatch = [&](auto a_tag) {
        if (any_zero && mine > 0)
            run(std::integral_constant<int, 4>{}, MY{}, a_tag);  // rare: all 4 subtiles (unfilled ones are never stored)
        else if (mine == 4)
            run(std::integral_constant<int, 4>{}, MN{}, a_tag);
        else if (mine == 3)
            run(std::integral_constant<int, 3>{}, MN{}, a_tag);
        else if (mine == 2)
            run(std::integral_constant<int, 2>{}, MN{}, a_tag);
        else if (mine == 1)
            run(std::integral_constant<int, 1>{}, MN{}, a_tag);
        else
            run(std::integral_constant<int, 0>{}, MN{}, a_tag);
    };
    if (load_a)
        dispatch(std::true_type{});
    else
        dispatch(std::false_type{});
    rescale(u0, u1, std::integral_constant<int, 4>{});

    // D layout of the 32x32 MFMA: value x of a lane is row 8*(x/4) + 4*(lane/32) + x%4 of the
    // subtile, column lane%32
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        if (mi >= mine) break;
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            const int p = tile.row0 + (wm + 2 * mi) * 32 + 8 * (x >> 2) + 4 * half + (x & 3);
            if (p >= tile.row1) continue;
            uint16_t* o = a.out + (size_t)p * a.N + c0 + fr;
            if (kPhase == 1) {
                const float g = acc[mi][0][x], u = acc[mi][1][x];
                o[wn * 32] = f32_to_bf16(silu_mul(g, u));
            } else {
                const uint32_t b = f32x2_to_bf16x2(acc[mi][0][x], acc[mi][1][x]);
                o[wn * 64] = (uint16_t)b;
                o[wn * 64 + 32] = (uint16_t)(b >> 16);
            }
        }
    }
}

static moe_status launch_q256(int phase, const GemmArgs& a, hipStream_t st) {
    const int cols = phase == 1 ? kQN / 2 : kQN;
    const int groups = a.offsets ? a.n_groups : 1;
    const int64_t mt = ((int64_t)a.rows + kQM - 1) / kQM + std::min<int64_t>(groups, a.rows);
    const int64_t wgs = mt * (a.N / cols);
    if (wgs > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)((wgs + 7) & ~int64_t(7))), block(512);
    const bool g = a.offsets != nullptr;
    if (phase == 1) {
        if (g) gemm_fp8_q256_kernel<1, true><<<grid, block, 0, st>>>(a);
        else gemm_fp8_q256_kernel<1, false><<<grid, block, 0, st>>>(a);
    } else {
        if (g) gemm_fp8_q256_kernel<2, true><<<grid, block, 0, st>>>(a);
        else gemm_fp8_q256_kernel<2, false><<<grid, block, 0, st>>>(a);
    }
    return launch_status();
}

moe_status launch_gemm(int phase, const GemmArgs& a, hipStream_t st) {
    if (a.K / kBK > kMaxKBlocks) return MOE_ERR_UNSUPPORTED;
    // the direct-to-LDS kernel addresses activation rows by 32-bit 16-byte chunk indices (up to
    // 64 GB of activations); beyond that, and for H an odd multiple of 128, the register-staged
    // kernel runs
    const bool chunk32 = (int64_t)a.rows * (a.K / 8) < (int64_t(1) << 32);
    // 160 x 512 tiles when an average expert fits one 160-row m-tile (measured 4% faster at
    // 128 rows per expert; at 170 rows most experts need a second m-tile, which streams the
    // weights again, and the 256 x 256 tiles are faster)
    const int64_t n_exp = a.offsets ? a.n_groups : 1;
    if (wide_gemm_fits(phase, a) && a.rows <= kWideRows * n_exp) return launch_gemm_wide(phase, a, st);
    if (a.fp8 && chunk32 && a.N % (phase == 1 ? kQN / 2 : kQN) == 0) return launch_q256(phase, a, st);
    const int cols = phase == 1 ? kBN / 2 : kBN;
    const int groups = a.offsets ? a.n_groups : 1;
    const int64_t mt = ((int64_t)a.rows + kBM - 1) / kBM + std::min<int64_t>(groups, a.rows);
    const int64_t wgs = mt * (a.N / cols);
    if (wgs > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)((wgs + 7) & ~int64_t(7))), block(256);
    const bool g = a.offsets != nullptr;
#define MOE_GEMM(F, P, G) gemm_kernel<F, P, G><<<grid, block, 0, st>>>(a)
    if (phase == 1) {
        if (a.fp8) g ? MOE_GEMM(true, 1, true) : MOE_GEMM(true, 1, false);
        else g ? MOE_GEMM(false, 1, true) : MOE_GEMM(false, 1, false);
    } else {
        if (a.fp8) g ? MOE_GEMM(true, 2, true) : MOE_GEMM(true, 2, false);
        else g ? MOE_GEMM(false, 2, true) : MOE_GEMM(false, 2, false);
    }
#undef MOE_GEMM
    return launch_status();
}

}  // namespace moe

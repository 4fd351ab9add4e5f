// moe_gemm.hip -- grouped expert GEMM for many rows per expert (prefill shapes).
//
// Tokens that hit the same expert are batched so that the expert's projection is a GEMM
// (KTransformers article, 2.2).  Each expert's rows are cut into 128-row m-tiles; a workgroup
// computes one m-tile against 128 weight rows over the whole K:
//   phase 1: 64 gate rows + the same 64 up rows -> 64 columns of h = SiLU(gate) * up
//   phase 2: 128 down rows -> 128 columns of y
//
// Per 128-long K block (= one FP8 scale block) the workgroup stages in LDS the activation tile
// (128 rows x 128 bf16, gathered through the grouping in phase 1) and the weight tile (128 rows
// x 128 FP8 codes, kept as codes), both loaded as whole 128-byte lines.  Four waves (2 x 2) then
// run MFMA 32x32x16 chains: each wave owns 2 of the 4 32-row m-subtiles (interleaved, so a
// partly filled tile still spreads over both wave rows) and 2 32-row weight subtiles (phase 1:
// matching gate and up rows, so SiLU(gate)*up is formed in registers).  k-steps go in pairs
// whose lane halves cover 16 consecutive K each, so one 16-byte LDS read of FP8 codes feeds two
// MFMAs.  Weight fragments are expanded exactly from FP8 to bf16 as they leave LDS (the row
// stride of 144 bytes keeps those reads free of bank conflicts); each block's chain goes into a partial
// sum that is multiplied by the block's scale into the fp32 accumulator (the post-scaling of
// the OSDI'26 article's FP8 GEMV, section "native FP8 GEMV", Figures 9-10).  Subtiles past the
// last row are skipped.  Two workgroups share a CU, so one computes while the other stages.
#include "libmoe.h"
#include "moe_device.h"
#include "moe_ffn.h"
#include "moe_host.h"

#include <type_traits>

namespace moe {

constexpr int kBM = 128;            // rows per m-tile
constexpr int kBN = 128;            // weight rows per tile
constexpr int kBK = 128;            // K per block (one scale block)
constexpr int kLDA = kBK * 2 + 16;  // A row stride in LDS (bytes): 16-lane b128 reads hit distinct banks
constexpr int kMaxKBlocks = 128;    // K <= 16384 (block scales are staged in LDS)

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
                o[wn * 32] = f32_to_bf16(g / (1.0f + __expf(-g)) * u);
            } else {
                o[wn * 64] = f32_to_bf16(acc[mi][0][r]);
                o[wn * 64 + 32] = f32_to_bf16(acc[mi][1][r]);
            }
        }
    }
}

// ------------------------------------------------------------------ FP8 weights
//
// Same tile and wave layout, with the loads restructured so that the HBM weight stream runs
// two blocks ahead of the MFMAs and the activation rows one block ahead:
//   * activations go global -> LDS directly (16 bytes per lane per instruction, whole 256-byte
//     row slices) into a 2-stage ring; no registers, no LDS store instructions;
//   * weights (FP8 codes) go through two alternating register sets into one LDS tile.
// LDS: 2 x 32 KB activations + 16 KB weights = 80 KB, so two workgroups share a CU.  Both
// tiles are unpadded; a 16-byte chunk sits at a slot XORed with a function of its row, which
// keeps the 16-byte fragment reads free of bank conflicts.
//
// Wait counts.  Per iteration each thread issues, in this order: the block's scale loads, the
// activation loads of the next block (inline assembly, so the compiler's own wait counting
// does not see them and never waits for them before LDS reads), and exactly kBPer weight loads
// for two blocks ahead.  At the top of the next iteration `vmcnt(kBPer)` therefore means that
// everything but those weight loads has landed.

constexpr int kBPer8 = kBN * kBK / 256 / 16;  // 16-byte weight chunks per thread per block (4)

// s_waitcnt immediate that waits until at most n vector-memory loads are outstanding (gfx9
// encoding: vmcnt in bits 3:0 and 15:14; expcnt 6:4 and lgkmcnt 11:8 left at "no wait").
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// One direct global -> LDS load of 16 bytes per lane: lane l's bytes land at lds + 16 * l.
__device__ __forceinline__ void lds_dma16(const void* src, const void* lds) {
    const uint32_t addr = (uint32_t)(size_t)(const __attribute__((address_space(3))) void*)lds;
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(__builtin_amdgcn_readfirstlane(addr))
                 : "memory", "m0");
}

template <int kPhase, bool kGrouped>
__global__ __launch_bounds__(256, 2) void gemm_fp8_kernel(GemmArgs a) {
    constexpr int kAStage = kBM * kBK * 2;  // 32 KB
    __shared__ __attribute__((aligned(1024))) uint8_t sA[2][kAStage];
    __shared__ __attribute__((aligned(1024))) uint8_t sB[kBN * kBK];

    constexpr int kCols = kPhase == 1 ? kBN / 2 : kBN;
    Tile tile;
    const int n_tiles = a.N / kCols;
    if (!find_tile(kGrouped ? a.offsets : nullptr, a.n_groups, a.rows, kBM, n_tiles, tile)) return;

    const int tid = (int)threadIdx.x, lane = lane_id(), wave = uniform(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int e = tile.group;
    const int c0 = tile.nt * kCols;
    const int K = a.K, kblocks = K / kBK;
    const int fr = lane & 31, half = lane >> 5;

    // ---- activation loads: instruction i (0..7) of wave w fills tile rows 4 (8 w + i) + lane/16,
    // slot lane % 16 of the row holding logical chunk slot ^ (row & 15).  Rows past the end of
    // the m-tile load the tile's first row (never stored), so every load is in bounds.
    uint32_t aoff[8];  // 16-byte chunk index of each loaded row slice (rows * K / 8 < 2^32)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = 4 * (8 * wave + i) + (lane >> 4);
        const int p = tile.row0 + r < tile.row1 ? tile.row0 + r : tile.row0;
        const uint32_t src = (kPhase == 1 && kGrouped) ? (uint32_t)(a.perm[p] / a.k) : (uint32_t)p;
        aoff[i] = src * (uint32_t)(K / 8) + (uint32_t)((lane & 15) ^ (r & 15));
    }
    auto dma_a = [&](int kb, int st) {
        const uint8_t* act = (const uint8_t*)a.act + (size_t)kb * (kBK * 2);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            lds_dma16(act + (size_t)aoff[i] * 16, &sA[st][4 * (8 * wave + i) * kBK * 2]);
    };
    // ---- weight loads: chunk tid % 8 of tile rows tid / 8 + 32 i; phase 1 rows 0..63 gate,
    // 64..127 up.  Every row of a thread has the same swizzle ((row >> 1) & 7 = (tid >> 4) & 7).
    const uint8_t* bsrc0;
    const uint8_t* bsrc1;
    {
        const size_t row = (size_t)e * a.N + c0 + (tid >> 3);
        bsrc0 = (const uint8_t*)a.w0 + row * K + (tid & 7) * 16;
        bsrc1 = (kPhase == 1 ? (const uint8_t*)a.w1 + row * K : bsrc0 + (size_t)64 * K) + (kPhase == 1 ? (tid & 7) * 16 : 0);
    }
    const int bdst = (tid >> 3) * kBK + (((tid & 7) ^ ((tid >> 4) & 7)) << 4);
    u32x4 rb0[kBPer8], rb1[kBPer8];
    auto load_b = [&](int kb, u32x4 (&rb)[kBPer8]) {
        const size_t o = (size_t)kb * kBK, step = (size_t)32 * K;
        rb[0] = __builtin_nontemporal_load((const u32x4*)(bsrc0 + o));
        rb[1] = __builtin_nontemporal_load((const u32x4*)(bsrc0 + o + step));
        rb[2] = __builtin_nontemporal_load((const u32x4*)(bsrc1 + o));
        rb[3] = __builtin_nontemporal_load((const u32x4*)(bsrc1 + o + step));
    };
    auto store_b = [&](const u32x4 (&rb)[kBPer8]) {
#pragma unroll
        for (int i = 0; i < kBPer8; ++i) *(u32x4*)&sB[bdst + i * 32 * kBK] = rb[i];
    };
    // block scales of the tile's weight rows: phase 1 gate and up of block-row c0/128; phase 2
    // one block-row (the 128 rows of the tile)
    const size_t srow = ((size_t)e * (a.N / 128) + c0 / 128) * kblocks;
    const float* sc0 = a.s0 + srow;
    const float* sc1 = (kPhase == 1 ? a.s1 : a.s0) + srow;

    const int nvalid = (tile.row1 - tile.row0 + 31) >> 5;
    const int mine = (nvalid > wm) + (nvalid > wm + 2);
    // fragment addresses: chunk c of row r sits at slot c ^ swz(r), so a read address is a
    // per-lane base XOR a per-step constant
    int abase[2], bbase[2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
        const int r = (wm + 2 * mi) * 32 + fr;
        abase[mi] = r * (kBK * 2) + (((r & 15) << 4) ^ (half << 5));
    }
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        const int r = (kPhase == 1 ? ni * 64 + wn * 32 : wn * 64 + ni * 32) + fr;
        bbase[ni] = r * kBK + ((((r >> 1) & 7) ^ half) << 4);
    }

    f32x16 acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

    // Block scales are applied by keeping each accumulator in units of the scale of the block
    // being multiplied: before block b it is multiplied by u / s_b (u = the scale of the last
    // block with a nonzero scale), the block's MFMAs add into it, and the end multiplies by u.
    // This is the post-scaling sum  sum_b s_b * P_b  with one extra fp32 rounding per block and
    // no separate partial sums.  A zero scale keeps the units and masks that block's codes, so
    // the block adds exactly nothing.
    float u0 = 0.0f, u1 = 0.0f;
    auto compute = [&](int st, uint32_t m0, uint32_t m1, auto nsub_tag) {
        constexpr int NS = decltype(nsub_tag)::value;
        const uint8_t* A = sA[st];
        // k-steps in pairs: for pair j, lane half h covers K elements [32j + 16h, +16) on both
        // operands, so one 16-byte read of FP8 codes feeds two MFMAs
#pragma unroll
        for (int j = 0; j < kBK / 32; ++j) {
            bf16x8 fa[2][NS];
            u32x4 fbq[2];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int mi = 0; mi < NS; ++mi)
                    fa[t][mi] = *(const bf16x8*)&A[abase[mi] ^ ((4 * j + t) << 4)];
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) fbq[ni] = *(const u32x4*)&sB[bbase[ni] ^ (j << 5)];
            fbq[0] &= m0;
            fbq[1] &= m1;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                bf16x8 fb[2];
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) fb[ni] = fp8x8_to_bf16x8(fbq[ni][2 * t], fbq[ni][2 * t + 1]);
#pragma unroll
                for (int mi = 0; mi < NS; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            fa[t][mi], fb[ni], acc[mi][ni], 0, 0, 0);
            }
        }
    };
    auto rescale = [&](float r0, float r1) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                acc[mi][0][q] *= r0;
                acc[mi][1][q] *= r1;
            }
    };

    // One block.  kMode 2: the loads of block kb + 1 (scales, activations) and the weights of
    // kb + 2 are issued; 1: only those of kb + 1 (the last weights are already in flight); 0:
    // nothing (last block).  kWait: vmcnt at the top, kBPer8 while the weight loads of kb + 1
    // may still be in flight, else 0.  Each call site has constant modes, so the loads are
    // unconditional and the compiler's own wait counting stays exact.
    float sn0 = sc0[0], sn1 = sc1[0];  // scales of the next block to multiply
    auto iter = [&](int kb, u32x4 (&rb)[kBPer8], auto mode_tag, auto wait_tag) {
        constexpr int kMode = decltype(mode_tag)::value;
        constexpr int kWait = decltype(wait_tag)::value;
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kWait));
        __syncthreads();
        store_b(rb);
        const float s0 = sn0, s1 = sn1;
        if (kMode >= 1) {
            sn0 = sc0[kb + 1];
            sn1 = sc1[kb + 1];
            dma_a(kb + 1, (kb + 1) & 1);
        }
        if (kMode == 2) load_b(kb + 2, rb);
        __syncthreads();
        if (mine == 0) return;
        const bool z0 = s0 == 0.0f, z1 = s1 == 0.0f;
        const float r0 = z0 ? 1.0f : u0 / s0, r1 = z1 ? 1.0f : u1 / s1;
        u0 = z0 ? u0 : s0;
        u1 = z1 ? u1 : s1;
        rescale(r0, r1);
        const uint32_t m0 = z0 ? 0u : ~0u, m1 = z1 ? 0u : ~0u;
        if (mine == 2)
            compute(kb & 1, m0, m1, std::integral_constant<int, 2>{});
        else
            compute(kb & 1, m0, m1, std::integral_constant<int, 1>{});
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using IW = std::integral_constant<int, kBPer8>;

    // prologue: weights of block 0, activations of block 0, weights of block 1 (this order, so
    // that the first wait leaves only the last in flight)
    // (with one block the second load re-reads block 0 into registers nobody uses: unconditional
    // loads keep the compiler's wait counting exact)
    load_b(0, rb0);
    dma_a(0, 0);
    load_b(kblocks > 1 ? 1 : 0, rb1);
    int kb = 0;
    for (; kb + 3 < kblocks; kb += 2) {
        iter(kb, rb0, I2{}, IW{});
        iter(kb + 1, rb1, I2{}, IW{});
    }
    // 1 to 3 blocks left; kb is even, so block kb's weights are in rb0
    const int rem = kblocks - kb;
    if (rem == 3) {
        iter(kb, rb0, I2{}, IW{});
        iter(kb + 1, rb1, I1{}, IW{});
        iter(kb + 2, rb0, I0{}, I0{});
    } else if (rem == 2) {
        iter(kb, rb0, I1{}, IW{});
        iter(kb + 1, rb1, I0{}, I0{});
    } else {
        iter(kb, rb0, I0{}, I0{});
    }
    rescale(u0, u1);

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
                o[wn * 32] = f32_to_bf16(g / (1.0f + __expf(-g)) * u);
            } else {
                o[wn * 64] = f32_to_bf16(acc[mi][0][r]);
                o[wn * 64 + 32] = f32_to_bf16(acc[mi][1][r]);
            }
        }
    }
}

moe_status launch_gemm(int phase, const GemmArgs& a, hipStream_t st) {
    const int cols = phase == 1 ? kBN / 2 : kBN;
    const int groups = a.offsets ? a.n_groups : 1;
    const int64_t mt = ((int64_t)a.rows + kBM - 1) / kBM + std::min<int64_t>(groups, a.rows);
    const int64_t wgs = mt * (a.N / cols);
    if (wgs > INT32_MAX || a.K / kBK > kMaxKBlocks) return MOE_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)((wgs + 7) & ~int64_t(7))), block(256);
    const bool g = a.offsets != nullptr;
#define MOE_GEMM(F, P, G) gemm_kernel<F, P, G><<<grid, block, 0, st>>>(a)
#define MOE_GEMM8(P, G) gemm_fp8_kernel<P, G><<<grid, block, 0, st>>>(a)
    // the FP8 kernel addresses activation rows by 32-bit 16-byte chunk indices (up to 64 GB of
    // activations); beyond that the register-staged kernel, which uses 64-bit offsets, runs
    const bool chunk32 = (int64_t)a.rows * (a.K / 8) < (int64_t(1) << 32);
    if (phase == 1) {
        if (a.fp8 && chunk32) g ? MOE_GEMM8(1, true) : MOE_GEMM8(1, false);
        else if (a.fp8) g ? MOE_GEMM(true, 1, true) : MOE_GEMM(true, 1, false);
        else g ? MOE_GEMM(false, 1, true) : MOE_GEMM(false, 1, false);
    } else {
        if (a.fp8 && chunk32) g ? MOE_GEMM8(2, true) : MOE_GEMM8(2, false);
        else if (a.fp8) g ? MOE_GEMM(true, 2, true) : MOE_GEMM(true, 2, false);
        else g ? MOE_GEMM(false, 2, true) : MOE_GEMM(false, 2, false);
    }
#undef MOE_GEMM
#undef MOE_GEMM8
    return launch_status();
}

}  // namespace moe

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

moe_status launch_gemm(int phase, const GemmArgs& a, hipStream_t st) {
    const int cols = phase == 1 ? kBN / 2 : kBN;
    const int groups = a.offsets ? a.n_groups : 1;
    const int64_t mt = ((int64_t)a.rows + kBM - 1) / kBM + std::min<int64_t>(groups, a.rows);
    const int64_t wgs = mt * (a.N / cols);
    if (wgs > INT32_MAX || a.K / kBK > kMaxKBlocks) return MOE_ERR_UNSUPPORTED;
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

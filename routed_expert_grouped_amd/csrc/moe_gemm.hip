// moe_gemm.hip -- grouped expert GEMM for many rows per expert (prefill shapes).
//
// Tokens that hit the same expert are batched so that the expert's projection is a GEMM
// (KTransformers article, 2.2).  Each expert's rows are cut into 128-row m-tiles; a workgroup
// computes one m-tile against 128 weight rows over the whole K:
//   phase 1: 64 gate rows + the same 64 up rows -> 64 columns of h = SiLU(gate) * up
//   phase 2: 128 down rows -> 128 columns of y
// Per 128-long K block (one FP8 scale block) the workgroup stages the activation tile (gathered
// through the grouping for phase 1) and the weight tile in LDS -- the FP8 codes expanded exactly
// to bf16 on the way in -- then 4 waves (2 x 2, 64 x 64 each) run MFMA 32x32x16 chains into a
// per-block partial that is multiplied by the block's scale into the fp32 accumulator (the
// post-scaling of the OSDI'26 article's FP8 GEMV, section "native FP8 GEMV", Figures 9-10).
// The next block's global loads are issued before the current block's MFMAs, and two
// workgroups share a CU (69.6 KB of LDS each) so one computes while the other waits at a
// barrier.
#include "libmoe.h"
#include "moe_device.h"
#include "moe_ffn.h"
#include "moe_host.h"

namespace moe {

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBK = 128;
constexpr int kLD = kBK + 8;  // LDS row stride (bf16 elements): 272 B keeps 16-lane reads conflict-free

template <bool kFP8, int kPhase, bool kGrouped>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[kBM * kLD];
    __shared__ __attribute__((aligned(16))) uint16_t sB[kBN * kLD];

    constexpr int kCols = kPhase == 1 ? kBN / 2 : kBN;  // output columns per tile
    Tile tile;
    const int n_tiles = a.N / kCols;
    if (!find_tile(kGrouped ? a.offsets : nullptr, a.n_groups, a.rows, kBM, n_tiles, tile)) return;

    const int tid = (int)threadIdx.x, lane = lane_id(), wave = uniform(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int e = tile.group;
    const int c0 = tile.nt * kCols;
    const int K = a.K, kblocks = K / kBK;
    const size_t esz = kFP8 ? 1 : 2;

    // ---- staging assignment: A chunk i -> row tid/16 + 16i, 8 bf16 at column (tid%16)*8
    const uint16_t* arow[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int p = tile.row0 + (tid >> 4) + 16 * i;
        arow[i] = nullptr;
        if (p < tile.row1) {
            const int r = (kPhase == 1 && kGrouped) ? a.perm[p] / a.k : p;
            arow[i] = a.act + (size_t)r * K + (tid & 15) * 8;
        }
    }
    // B chunks: fp8 -> row tid/8 + 32i, 16 codes at (tid%8)*16; bf16 -> row tid/16 + 16i, 8 at (tid%16)*8
    constexpr int kBChunks = kFP8 ? 4 : 8;
    const uint8_t* brow[kBChunks];
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) {
        const int r = kFP8 ? (tid >> 3) + 32 * i : (tid >> 4) + 16 * i;  // LDS row 0..127
        const int col = kFP8 ? (tid & 7) * 16 : (tid & 15) * 8;
        const uint8_t* base;
        int wr;
        if (kPhase == 1) {
            base = (const uint8_t*)(r < 64 ? a.w0 : a.w1);
            wr = c0 + (r & 63);
        } else {
            base = (const uint8_t*)a.w0;
            wr = c0 + r;
        }
        brow[i] = base + (((size_t)e * a.N + wr) * K + col) * esz;
    }

    u32x4 ra[8], rb[kBChunks];
    auto load = [&](int kb) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            ra[i] = arow[i] ? *(const u32x4*)(arow[i] + kb * kBK) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < kBChunks; ++i)
            rb[i] = __builtin_nontemporal_load((const u32x4*)(brow[i] + (size_t)kb * kBK * esz));
    };
    auto store = [&]() {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *(u32x4*)&sA[((tid >> 4) + 16 * i) * kLD + (tid & 15) * 8] = ra[i];
#pragma unroll
        for (int i = 0; i < kBChunks; ++i) {
            if (kFP8) {
                const int r = (tid >> 3) + 32 * i, col = (tid & 7) * 16;
                const bf16x8 lo = fp8x8_to_bf16x8(rb[i][0], rb[i][1]);
                const bf16x8 hi = fp8x8_to_bf16x8(rb[i][2], rb[i][3]);
                *(bf16x8*)&sB[r * kLD + col] = lo;
                *(bf16x8*)&sB[r * kLD + col + 8] = hi;
            } else {
                const int r = (tid >> 4) + 16 * i, col = (tid & 15) * 8;
                *(u32x4*)&sB[r * kLD + col] = rb[i];
            }
        }
    };

    // per-lane fragment rows in LDS
    const int fr = lane & 31, fk = (lane >> 5) * 8;
    int brow_l[2];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
        brow_l[ni] = kPhase == 1 ? ni * 64 + wn * 32 + fr : wn * 64 + ni * 32 + fr;

    // block scales of this tile (phase 1: gate / up of block c0/128; phase 2: down of c0/128)
    const float* sc0 = nullptr;
    const float* sc1 = nullptr;
    if (kFP8) {
        const size_t srow = ((size_t)e * (a.N / 128) + c0 / 128) * kblocks;
        sc0 = a.s0 + srow;
        sc1 = kPhase == 1 ? a.s1 + srow : sc0;
    }

    f32x16 acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

    load(0);
    for (int kb = 0; kb < kblocks; ++kb) {
        __syncthreads();  // every wave is done reading the previous block
        store();
        __syncthreads();
        if (kb + 1 < kblocks) load(kb + 1);
        f32x16 part[2][2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                for (int r = 0; r < 16; ++r) part[mi][ni][r] = 0.0f;
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            bf16x8 fa[2], fb[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                fa[mi] = *(const bf16x8*)&sA[(wm * 64 + mi * 32 + fr) * kLD + kk * 16 + fk];
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                fb[ni] = *(const bf16x8*)&sB[brow_l[ni] * kLD + kk * 16 + fk];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    part[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni],
                                                                           part[mi][ni], 0, 0, 0);
        }
        const float s0 = kFP8 ? sc0[kb] : 1.0f;
        const float s1 = kFP8 ? sc1[kb] : 1.0f;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                acc[mi][0][r] = fmaf(part[mi][0][r], s0, acc[mi][0][r]);
                acc[mi][1][r] = fmaf(part[mi][1][r], s1, acc[mi][1][r]);
            }
    }

    // D layout of the 32x32 MFMA: value r of a lane is row 8*(r/4) + 4*(lane/32) + r%4 of the
    // fragment, column lane%32
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const int p = tile.row0 + m;
            if (p >= tile.row1) continue;
            if (kPhase == 1) {
                const float g = acc[mi][0][r], u = acc[mi][1][r];
                a.out[(size_t)p * a.N + c0 + wn * 32 + fr] = f32_to_bf16(g / (1.0f + __expf(-g)) * u);
            } else {
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    a.out[(size_t)p * a.N + c0 + wn * 64 + ni * 32 + fr] = f32_to_bf16(acc[mi][ni][r]);
            }
        }
}

moe_status launch_gemm(int phase, const GemmArgs& a, hipStream_t st) {
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

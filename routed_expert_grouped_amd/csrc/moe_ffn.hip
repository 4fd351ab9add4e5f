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
#include "moe_lds.h"

namespace moe {

// One workgroup = kWaves waves; each wave owns kG 16-row weight groups (phase 1: the same
// 8 kG rows of gate and of up; phase 2: 16 kG consecutive rows of down) over the full K, for one
// m-tile of up to 16 grouped rows.  kGrouped = false is the identity grouping (shared expert).
// Every activation fragment a lane loads feeds kG MFMAs, so kG = 4 halves the activation loads
// per weight byte; MXFP4 weights (twice the K values per weight byte of FP8) take it where the
// shape allows.
//
// kSplit > 1 (gate/up: FP8, and MXFP4 with four groups a wave): the workgroup's waves own
// kWaves / kSplit column groups, each over kSplit consecutive parts of K; after the K loop the
// other parts' fp32 sums are added to part 0's, in part order, through LDS.  A workgroup then streams 1/kSplit of the bytes, so the launch
// has kSplit times more, shorter workgroups and its ramp-down at the end (the last workgroups
// running on a few CUs) is that much shorter.  At the DeepSeek-V3 decode shape the unsplit
// launch is 3168 workgroups for 1024 resident slots.
//
// HBM access: a wave's load instruction covers 8 weight rows x 128 contiguous bytes (whole
// cache lines; 16 rows x 64 B per instruction, the MFMA operand layout, reaches only ~75% of the
// bandwidth).  Each block goes through the wave's private LDS rows once to change from that
// load layout to the MFMA operand layout (no workgroup barrier: a wave's LDS operations
// complete in order).  The K loop keeps two 128-blocks of loads in flight (2-stage ring).
//
// Weight formats (kFmt): kBF16, kFP8 (E4M3FN + fp32 128x128 block scales, post-scaled per block)
// and kMXFP4 (E2M1 codes, two a byte, + one E8M0 scale per 32 along K).  For MXFP4 the 32 K values
// a lane multiplies per block are exactly one scale group, so the lane expands its codes to bf16
// with its group's scale in the conversion instruction (exact: a power of two times a 2-bit
// significand) and nothing is post-scaled.
//
// MXFP4 scales: a wave's 32 weight rows carry K/32 scale bytes each, one dword per 128-block.
// Loaded per block they would cost a load instruction touching 16 scale rows (16 cache lines
// for 4 useful bytes each) per row group, which keeps the address unit busier than the weight
// stream itself.  Instead the wave copies its rows' scales of up to 64 blocks (a window) into
// its own LDS area with direct global -> LDS loads, coalesced along each row, before its first
// weight loads, and reads one 8-byte LDS word per row group per stage.  Rows longer than one
// window (K > 8192) are refilled at each window boundary after the wave's loads have drained.
constexpr int kBF16 = 0, kFP8 = 1, kMXFP4 = 2;
constexpr int kScaleWin = 64;    // 128-blocks of scales per window (32 rows a wave; half that for 64)
constexpr int kScaleSlot = 264;  // LDS bytes per scale load instruction (256 + 8: 8-byte reads
                                 // of 16 rows fall in distinct banks)

template <int kFmt, int kPhase, bool kGrouped, int kWaves, int kSplit, int kG>
__global__ __launch_bounds__(kWaves * 64) void gemv_kernel(GemmArgs a) {
    static_assert(kWaves % kSplit == 0, "whole column groups per workgroup");
    static_assert(kG == 2 || kG == 4, "two or four 16-row weight groups a wave");
    constexpr int kRows = 16 * kG;                    // weight rows per wave
    constexpr int kColWaves = kWaves / kSplit;        // waves per K part
    constexpr int kWaveCols = kPhase == 1 ? kRows / 2 : kRows;  // output columns per wave
    constexpr int kCols = kColWaves * kWaveCols;
    // a stage is kBPS 128-blocks, so that every format loads whole 128-byte lines per row
    constexpr int kBPS = kFmt == kMXFP4 ? 2 : 1;
    constexpr int kBB = kFmt == kFP8 ? 128 : kFmt == kMXFP4 ? 64 : 256;  // bytes of a row per block
    constexpr int kRowB = kBB * kBPS;                 // bytes of a row per stage
    constexpr int kLD = kRowB + 16;                   // LDS row stride: conflict-free reads
    constexpr int kLPR = kRowB / 16;                  // lanes per row in a load instruction
    constexpr int kRPI = 64 / kLPR;                   // rows per load instruction
    constexpr int kIns = 16 / kRPI;                   // load instructions per 16-row group
    __shared__ __attribute__((aligned(16))) uint8_t sW[kWaves][kRows * kLD];
    constexpr bool kMX = kFmt == kMXFP4;
    // MXFP4 scale window: the wave's LDS area holds kRows * kWin / 64 load slots
    constexpr int kWin = kScaleWin * 32 / kRows;
    __shared__ __attribute__((aligned(16))) uint8_t sS[kMX ? kWaves : 1][kMX ? kRows * kWin / 64 * kScaleSlot : 16];

    Tile tile;
    const int n_tiles = a.N / kCols;
    if (!find_tile(kGrouped ? a.offsets : nullptr, a.n_groups, a.rows, kGemvBM, n_tiles, tile,
                   kGrouped ? a.extra_rows : 0, a.rows))
        return;

    const int lane = lane_id(), wave = uniform((int)(threadIdx.x >> 6));
    const int cw = wave % kColWaves, kp = wave / kColWaves;  // column group, K part
    const int m = lane & 15, kq = lane >> 4;
    const int K = a.K;
    // the extra group (the shared expert): its own weights, expert index 0, row rows + t = token t
    const bool xg = kGrouped && tile.group == a.n_groups;
    const int e = xg ? 0 : tile.group;
    const void* W0 = xg ? a.xw0 : a.w0;
    const void* W1 = xg ? a.xw1 : a.w1;
    const float* S0 = xg ? a.xs0 : a.s0;
    const float* S1 = xg ? a.xs1 : a.s1;
    const int p = tile.row0 + m;
    const bool valid = p < tile.row1;
    uint8_t* lds = sW[wave];

    // activation row of this lane's M index.  Lanes past the m-tile's last row read the tile's
    // first row instead: MFMA output rows depend only on their own A row, and those rows are
    // never stored, so the loads stay unconditional (exact load counters, no branches).
    const int pa = valid ? p : tile.row0;
    const int ra = (kPhase == 1 && kGrouped) ? (xg ? pa - a.rows : a.perm[pa] / a.k) : pa;
    // this wave's K part: 128-blocks [kb0w, kb0w + kblocks) of kb_all
    const int kb_all = K / 128, kblocks = kb_all / kSplit, kb0w = kp * kblocks;
    const uint16_t* arow = a.act + (size_t)ra * K + (size_t)kb0w * 128;
    // weight rows: load layout row lrow (+ kRPI per instruction), 16-byte chunk lchunk
    const int n0 = tile.nt * kCols + cw * kWaveCols;
    const size_t row_bytes = kFmt == kFP8 ? (size_t)K : kFmt == kMXFP4 ? (size_t)K / 2 : (size_t)K * 2;
    const int nst = (kblocks + kBPS - 1) / kBPS;      // stages
    const int nb_last = kblocks - (nst - 1) * kBPS;   // blocks in the last stage
    const int lrow = lane / kLPR, lchunk = lane % kLPR;
    const size_t kofs0 = (size_t)kb0w * kBB + lchunk * 16;  // the part's first byte of a row
    // group g: phase 1 gate (g < kG / 2) or up rows n0 + 16 (g mod kG / 2); phase 2 rows n0 + 16 g
    const uint8_t* gp[kG];
#pragma unroll
    for (int g = 0; g < kG; ++g) {
        const void* W = (kPhase == 1 && g >= kG / 2) ? W1 : W0;
        const int wr = n0 + 16 * (kPhase == 1 ? g % (kG / 2) : g) + lrow;
        gp[g] = (const uint8_t*)W + ((size_t)e * a.N + wr) * row_bytes + kofs0;
    }
    const size_t ins_stride = (size_t)kRPI * row_bytes;  // bytes between a group's instructions
    const float* s0 = nullptr;
    const float* s1 = nullptr;
    if (kFmt == kFP8) {
        s0 = S0 + ((size_t)e * (a.N / 128) + n0 / 128) * kb_all + kb0w;
        s1 = kPhase == 1 ? S1 + ((size_t)e * (a.N / 128) + n0 / 128) * kb_all + kb0w : s0;
    }
    // MXFP4: E8M0 bytes [N][K/32]; the wave's scale row r (0..kRows) is weight row n0 + r of w0
    // (r < kRows / 2) and of w1 (phase 1, row n0 + r - kRows / 2) or w0 (phase 2, row n0 + r)
    // (r >= kRows / 2).  A dword per block holds the scales of its 4 groups, one per K quarter
    // kq.  A window of wdw blocks goes to the wave's LDS area with P = 2^ceil(log2 wdw) (at least
    // 2) dwords per row and 64 / P rows per load instruction, each instruction filling one
    // kScaleSlot; soff[g] is the LDS offset of this lane's compute row 16 g + m in the window.
    uint8_t* sl = sS[kMX ? wave : 0];
    int soff[kG] = {};
    auto fill_scales = [&](int w0) {
        if constexpr (kMX) {
            const int wdw = min(kWin, kblocks - w0);
            const int lgP = max(1, 32 - __builtin_clz((unsigned)(wdw - 1) | 1u));
            const int lgR = 6 - lgP;  // rows per instruction: 2^lgR (1 to 32)
            const int d = lane & ((1 << lgP) - 1), rr = lane >> lgP;
            const uint8_t* sb0 = (const uint8_t*)S0;
            const uint8_t* sb1 = (const uint8_t*)(kPhase == 1 ? S1 : S0);
            const int nins = kRows >> lgR;
            for (int i = 0; i < nins; ++i) {
                const int r = (i << lgR) + rr;  // < kRows
                const uint8_t* row = r < kRows / 2
                    ? sb0 + ((size_t)e * a.N + n0 + r) * (K / 32)
                    : sb1 + ((size_t)e * a.N + n0 + (kPhase == 1 ? r - kRows / 2 : r)) * (K / 32);
                lds_dma4(row + 4 * (kb0w + w0 + min(d, wdw - 1)), sl + i * kScaleSlot);
            }
            auto off = [&](int r) { return (r >> lgR) * kScaleSlot + ((r & ((1 << lgR) - 1)) << (lgP + 2)); };
#pragma unroll
            for (int g = 0; g < kG; ++g) soff[g] = off(16 * g + m);
        }
    };

    f32x4 acc[kG];
#pragma unroll
    for (int g = 0; g < kG; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 bw[2][kG][kIns], xa[2][kBPS][4];
    float sg0[2], sg1[2];  // FP8 block scales of the staged blocks (wave-uniform): groups below
                           // kG / 2, and the others
    auto load = [&](int s, int st) {
        const int kb0 = s * kBPS;
        sg0[st] = kFmt == kFP8 ? s0[kb0] : 1.0f;
        sg1[st] = kFmt == kFP8 ? s1[kb0] : 1.0f;
        // in a short last stage the chunks of the missing block reload the stage's first block
        // (in the row, never used)
        size_t kofs = (size_t)s * kRowB;
        if (kBPS > 1 && kb0 + 1 >= kblocks && lchunk >= kLPR / 2) kofs -= kRowB / 2;
#pragma unroll
        for (int i = 0; i < kIns; ++i)
#pragma unroll
            for (int g = 0; g < kG; ++g)
                bw[st][g][i] = __builtin_nontemporal_load((const u32x4*)(gp[g] + i * ins_stride + kofs));
#pragma unroll
        for (int b = 0; b < kBPS; ++b) {
            const int kb = min(kb0 + b, kblocks - 1);
            const u32x4* xr = (const u32x4*)(arow + kb * 128 + kq * 32);  // this lane's 32 K values
#pragma unroll
            for (int i = 0; i < 4; ++i) xa[st][b][i] = xr[i];
        }
    };
    auto compute = [&](int st, int stage, int nb) {
        // MXFP4: scales of the stage's blocks (a stage starts a window only at a multiple of
        // kScaleWin / kBPS; the first window is filled before the loop)
        uint32_t sc[kG][kBPS];
        if constexpr (kMX) {
            const int j = stage * kBPS % kWin;
            if (j == 0 && stage > 0) {
                // refill: every load of this wave has landed and every LDS read returned
                __builtin_amdgcn_s_waitcnt(0);
                fill_scales(stage * kBPS);
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            }
            static_assert(kBPS == 2, "one 8-byte LDS read per row group covers a stage");
#pragma unroll
            for (int g = 0; g < kG; ++g) {
                const uint2 v = *(const uint2*)(sl + soff[g] + 4 * j);
                sc[g][0] = v.x, sc[g][1] = v.y;
            }
        }
        // load layout -> LDS rows -> MFMA layout (lane: row m; of block b the 32 K values of
        // quarter kq, kBB / 4 bytes from byte b * kBB + kq * kBB / 4)
#pragma unroll
        for (int i = 0; i < kIns; ++i)
#pragma unroll
            for (int g = 0; g < kG; ++g)
                *(u32x4*)&lds[(16 * g + i * kRPI + lrow) * kLD + lchunk * 16] = bw[st][g][i];
#pragma unroll
        for (int b = 0; b < kBPS; ++b) {
            if (b >= nb) break;
            constexpr int kV = kBB / 64;  // 16-byte vectors per lane per block
            u32x4 rw[kG][kV];
#pragma unroll
            for (int i = 0; i < kV; ++i)
#pragma unroll
                for (int g = 0; g < kG; ++g)
                    rw[g][i] = *(const u32x4*)&lds[(16 * g + m) * kLD + b * kBB + kq * (kBB / 4) + i * 16];
            float f[kG];  // MXFP4: this lane's group scales
#pragma unroll
            for (int g = 0; g < kG; ++g) f[g] = kMX ? e8m0_to_f32((sc[g][b] >> (8 * kq)) & 255u) : 1.0f;
            f32x4 p[kG];
#pragma unroll
            for (int g = 0; g < kG; ++g) p[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bf16x8 xv = as_bf16x8(xa[st][b][i]);
#pragma unroll
                for (int g = 0; g < kG; ++g) {
                    const uint32_t* u = (const uint32_t*)rw[g];
                    const bf16x8 wv = kFmt == kFP8 ? fp8x8_to_bf16x8(u[2 * i], u[2 * i + 1])
                                    : kFmt == kMXFP4 ? fp4x8_to_bf16x8(u[i], f[g])
                                                     : as_bf16x8(rw[g][i]);
                    p[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, wv, p[g], 0, 0, 0);
                }
            }
#pragma unroll
            for (int g = 0; g < kG; ++g)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[g][r] = fmaf(p[g][r], g < kG / 2 ? sg0[st] : sg1[st], acc[g][r]);
        }
    };
    // 2-stage ring: two stages in flight.  The steady-state loop issues its loads without
    // conditions so the compiler's load counters wait only for the stage being used; the tail
    // (1 to 3 stages) is peeled.  With a single stage, stage 1 reloads stage 0 (unused).
    // (scheduling barriers keep each stage's loads after the MFMAs of the stage they replace)
    // MXFP4: the first scale window's direct loads go first; at least the 2 * kStageLoads weight
    // and activation loads of stages 0 and 1 follow them, so waiting until only stage 1's are
    // outstanding also covers them.
    constexpr int kStageLoads = kG * kIns + 4 * kBPS;
    fill_scales(0);
    load(0, 0);
    load(nst > 1 ? 1 : 0, 1);
    if constexpr (kMX) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kStageLoads));
    int s = 0;
    for (; s + 3 < nst; s += 2) {
        compute(0, s, kBPS);
        __builtin_amdgcn_sched_barrier(0);
        load(s + 2, 0);
        __builtin_amdgcn_sched_barrier(0);
        compute(1, s + 1, kBPS);
        __builtin_amdgcn_sched_barrier(0);
        load(s + 3, 1);
        __builtin_amdgcn_sched_barrier(0);
    }
    const int rest = nst - s;  // 1, 2 or 3
    compute(0, s, rest == 1 ? nb_last : kBPS);
    if (rest == 3) load(s + 2, 0);
    if (rest >= 2) compute(1, s + 1, rest == 2 ? nb_last : kBPS);
    if (rest == 3) compute(0, s + 2, nb_last);

    if constexpr (kSplit > 1) {  // the sums of K parts 1.. join part 0's, in part order
        __shared__ f32x4 red[kSplit - 1][kColWaves][kG][kWave];
        if (kp > 0) {
#pragma unroll
            for (int g = 0; g < kG; ++g) red[kp - 1][cw][g][lane] = acc[g];
        }
        __syncthreads();
        if (kp > 0) return;
#pragma unroll
        for (int q = 0; q < kSplit - 1; ++q)
#pragma unroll
            for (int g = 0; g < kG; ++g) acc[g] += red[q][cw][g][lane];
    }
    // D layout of the 16x16 MFMA: lane holds rows 4*(lane/16)+r (grouped rows), column lane%16
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = tile.row0 + kq * 4 + r;
        if (row >= tile.row1) continue;
        if (kPhase == 1) {
#pragma unroll
            for (int g = 0; g < kG / 2; ++g) {
                const float gt = acc[g][r], u = acc[g + kG / 2][r];
                const float hval = silu_mul(gt, u);
                a.out[(size_t)row * a.N + n0 + 16 * g + m] = f32_to_bf16(hval);
            }
        } else {
#pragma unroll
            for (int g = 0; g < kG; ++g)
                a.out[(size_t)row * a.N + n0 + 16 * g + m] = f32_to_bf16(acc[g][r]);
        }
    }
}

static int max_mtiles(int rows, int n_groups, int BM) {
    const int64_t bound = ((int64_t)rows + BM - 1) / BM + std::min<int64_t>(n_groups, rows);
    return (int)bound;
}

// Launch one phase.  rows = grouped rows (T*k).
static moe_status launch_phase(int phase, const GemmArgs& a, hipStream_t st) {
    // many rows per expert: the GEMMs (MXFP4 weights: the 4-bit GEMM where its shape fits); an
    // extra group is a GEMV-only feature (its callers check)
    if (a.extra_rows > 0 && !use_gemv(a.rows, a.n_groups)) return MOE_ERR_UNSUPPORTED;
    if (!use_gemv(a.rows, a.n_groups)) {
        if (!a.fp4) return launch_gemm(phase, a, st);
        if (w4_gemm_fits(phase, a)) return launch_gemm_w4(phase, a, st);
    }
    constexpr int W = kGemvWaves;
    // MXFP4: four weight groups a wave where the columns divide into whole tiles.
    // K split of gate/up: FP8 weights in 4 parts where the 128-blocks divide evenly, else 2, else
    // none (measured at the DeepSeek-V3 decode shape: 0.425 ms unsplit, 0.411 ms in 4 parts; the
    // down projection, 5544 workgroups of a quarter of the bytes, gained nothing); MXFP4 weights
    // with four groups a wave in 2 parts, so that each part's scales fit one window (0.246 ->
    // 0.229 ms; with two groups a wave, whose window already holds 64 blocks, splitting lost 28%)
    const int kb = a.K / 128;
    const int G = a.fp4 && a.N % (W * (phase == 1 ? 32 : 64)) == 0 ? 4 : 2;
    const int split = phase != 1 ? 1
                    : a.fp8      ? (kb % 4 == 0 ? 4 : kb % 2 == 0 ? 2 : 1)
                    : (a.fp4 && G == 4 && kb % 2 == 0) ? 2 : 1;
    const int cols = W / split * (phase == 1 ? 8 : 16) * G;
    // the extra group's tiles (rounded up to 8) first, then the grouped ones (find_tile)
    const int groups = a.offsets ? a.n_groups : 1;
    const int64_t xtiles = a.extra_rows > 0
        ? (((int64_t)(a.extra_rows + kGemvBM - 1) / kGemvBM * (a.N / cols) + 7) & ~int64_t(7)) : 0;
    const int64_t wgs = xtiles + (((int64_t)max_mtiles(a.rows, groups, kGemvBM) * (a.N / cols) + 7) & ~int64_t(7));
    if (wgs > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)wgs), block(W * 64);
#define MOE_GEMV(F, P, GR) gemv_kernel<F, P, GR, W, 1, 2><<<grid, block, 0, st>>>(a)
#define MOE_GEMV4(P, GR)                                                           \
    (G == 2 ? gemv_kernel<kMXFP4, P, GR, W, 1, 2><<<grid, block, 0, st>>>(a)        \
            : gemv_kernel<kMXFP4, P, GR, W, 1, 4><<<grid, block, 0, st>>>(a))
#define MOE_GEMV4_SPLIT(GR)                                                        \
    (split == 2 ? gemv_kernel<kMXFP4, 1, GR, W, 2, 4><<<grid, block, 0, st>>>(a)    \
                : MOE_GEMV4(1, GR))
#define MOE_GEMV_SPLIT(GR)                                                         \
    (split == 4   ? gemv_kernel<kFP8, 1, GR, W, 4, 2><<<grid, block, 0, st>>>(a)    \
     : split == 2 ? gemv_kernel<kFP8, 1, GR, W, 2, 2><<<grid, block, 0, st>>>(a)    \
                  : gemv_kernel<kFP8, 1, GR, W, 1, 2><<<grid, block, 0, st>>>(a))
    const bool g = a.offsets != nullptr;
    if (phase == 1) {
        if (a.fp8) g ? MOE_GEMV_SPLIT(true) : MOE_GEMV_SPLIT(false);
        else if (a.fp4) g ? MOE_GEMV4_SPLIT(true) : MOE_GEMV4_SPLIT(false);
        else g ? MOE_GEMV(kBF16, 1, true) : MOE_GEMV(kBF16, 1, false);
    } else {
        if (a.fp8) g ? MOE_GEMV(kFP8, 2, true) : MOE_GEMV(kFP8, 2, false);
        else if (a.fp4) g ? MOE_GEMV4(2, true) : MOE_GEMV4(2, false);
        else g ? MOE_GEMV(kBF16, 2, true) : MOE_GEMV(kBF16, 2, false);
    }
#undef MOE_GEMV
#undef MOE_GEMV4
#undef MOE_GEMV4_SPLIT
#undef MOE_GEMV_SPLIT
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
    a.fp4 = w->dtype == MOE_W_MXFP4_G32;
    a.out = h;
    return launch_phase(1, a, as_stream(stream));
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
    a.fp4 = w->dtype == MOE_W_MXFP4_G32;
    a.out = y;
    return launch_phase(2, a, as_stream(stream));
}

// The routed experts and the shared expert in one launch per phase (decode sizes): the shared
// expert is an extra group of T rows after the T*k grouped ones, so one grid streams both
// experts' weights and no second stream or cross-stream wait is needed.
static moe_status check_shared(const moe_expert_weights* w, const moe_expert_weights* ws) {
    const moe_status s = check_weights(ws);
    if (s != MOE_OK) return s;
    if (ws->n_groups != 1 || ws->dtype != w->dtype || ws->H != w->H || ws->I != w->I)
        return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

extern "C" moe_status moe_expert_gate_up_shared(const uint16_t* x, int32_t T, int32_t k,
                                                const int32_t* perm, const int32_t* offsets,
                                                const moe_expert_weights* w,
                                                const moe_expert_weights* ws, uint16_t* h,
                                                void* stream) {
    if (T < 0 || k < 1) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!x || !h || !perm || !offsets) return MOE_ERR_INVALID_ARG;
    moe_status s = check_weights(w);
    if (s != MOE_OK) return s;
    if ((s = check_shared(w, ws)) != MOE_OK) return s;
    if ((s = check_grouping(T, k, perm, offsets, w, true)) != MOE_OK) return s;
    if ((int64_t)T * k + T > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (!use_gemv(T * k, w->n_groups)) {  // many rows per expert: one GEMM launch each
        if ((s = moe_expert_gate_up(x, T, k, perm, offsets, w, h, stream)) != MOE_OK) return s;
        return moe_expert_gate_up(x, T, 1, nullptr, nullptr, ws, h + (size_t)T * k * w->I, stream);
    }
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
    a.fp4 = w->dtype == MOE_W_MXFP4_G32;
    a.out = h;
    a.extra_rows = T;
    a.xw0 = ws->w_gate;
    a.xw1 = ws->w_up;
    a.xs0 = ws->s_gate;
    a.xs1 = ws->s_up;
    return launch_phase(1, a, as_stream(stream));
}

extern "C" moe_status moe_expert_down_shared(const uint16_t* h, int32_t T, int32_t k,
                                             const int32_t* offsets, const moe_expert_weights* w,
                                             const moe_expert_weights* ws, uint16_t* y,
                                             void* stream) {
    if (T < 0 || k < 1) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!h || !y || !offsets) return MOE_ERR_INVALID_ARG;
    moe_status s = check_weights(w);
    if (s != MOE_OK) return s;
    if ((s = check_shared(w, ws)) != MOE_OK) return s;
    if ((s = check_grouping(T, k, nullptr, offsets, w, false)) != MOE_OK) return s;
    if ((int64_t)T * k + T > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (!use_gemv(T * k, w->n_groups)) {
        if ((s = moe_expert_down(h, T, k, offsets, w, y, stream)) != MOE_OK) return s;
        return moe_expert_down(h + (size_t)T * k * w->I, T, 1, nullptr, ws, y + (size_t)T * k * w->H,
                               stream);
    }
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
    a.s0 = w->s_down;
    a.fp8 = w->dtype == MOE_W_FP8_E4M3_B128;
    a.fp4 = w->dtype == MOE_W_MXFP4_G32;
    a.out = y;
    a.extra_rows = T;
    a.xw0 = ws->w_down;
    a.xs0 = ws->s_down;
    return launch_phase(2, a, as_stream(stream));
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

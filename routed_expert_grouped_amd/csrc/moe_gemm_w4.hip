// moe_gemm_w4.hip -- grouped expert GEMMs for many rows per expert with 4-bit MXFP4 weights and
// bf16 activations.
//
// Tokens that hit the same expert are batched so that the expert's projection is a GEMM
// (KTransformers article, 2.2), as in moe_gemm.hip.  The weights are OCP MXFP4: E2M1 codes, two
// a byte (first in the low nibble), with one E8M0 scale per 32 consecutive inputs of a row.  Each
// lane expands its codes to bf16 with its group's scale in the conversion instruction
// (v_cvt_scalef32_pk_bf16_fp4: exact, a power of two times a 2-bit significand), and the bf16
// x bf16 products accumulate in fp32 on MFMA 32x32x16; nothing is post-scaled.
//
// One 8-wave workgroup per CU computes a 256-row m-tile against 256 weight rows (phase 1: 128
// gate + the same 128 up rows -> 128 h columns; phase 2: 256 y columns).  Operands go directly to
// LDS in two rings:
//   activations  32 KB stages of 64 K (256 rows x 128 bytes), 3 slots, two stages ahead;
//   weights      16 KB slots of 128 K (256 rows x 64 bytes) plus the slot's E8M0 scales (256
//                rows x 4 bytes), 3 slots, two slots (four stages) ahead.
// Activation rows: eight 16-byte chunks, chunk c at slot c ^ ((row >> 1) & 7); weight rows: four
// chunks, chunk c at slot c ^ ((row >> 2) & 3), so the fragment reads of 32 consecutive rows
// spread over the banks.
//
// MFMA 32x32x16 operand layout: lane l supplies row (column) l % 32 and 8 K values; of the two
// 32-long halves j of a stage, step (j, t) gives lane half h = l / 32 the K values
// [32 j + 16 h + 8 t, +8).  Those 8 weights are 4 code bytes inside MX group 2 (stage % 2) + j
// of the slot, so one scale serves both t of a half.
#include "libmoe.h"
#include "moe_device.h"
#include "moe_ffn.h"
#include "moe_host.h"
#include "moe_lds.h"

#include <type_traits>

namespace moe {

constexpr int kW4M = 256;   // rows per m-tile
constexpr int kW4N = 256;   // weight rows per tile
constexpr int kW4K = 64;    // K per compute stage
constexpr int kW4BK = 128;  // K per weight slot
constexpr int kW4Ring = 3;  // slots of each ring
constexpr int kW4AL = 4;    // activation loads per wave per stage
constexpr int kW4BL = 3;    // weight loads per wave per slot (2 code + 1 scale)

template <int kPhase, bool kGrouped>
__global__ __launch_bounds__(512, 1) void gemm_w4_kernel(GemmArgs a) {
    constexpr int kAStage = kW4M * kW4K * 2;    // 32 KB
    constexpr int kBSlot = kW4N * kW4BK / 2;    // 16 KB
    constexpr int kMSlot = 8 * 256;             // 2 KB: a 256-byte area per wave (32 rows x 4 bytes used)
    __shared__ __attribute__((aligned(1024))) uint8_t sA[kW4Ring][kAStage];
    __shared__ __attribute__((aligned(1024))) uint8_t sB[kW4Ring][kBSlot];
    __shared__ __attribute__((aligned(16))) uint8_t sM[kW4Ring][kMSlot];

    constexpr int kCols = kPhase == 1 ? kW4N / 2 : kW4N;
    Tile tile;
    // phase 2 takes N = 128 mod 256 too: the last column tile's upper 128 weight rows are absent
    if (!find_tile(kGrouped ? a.offsets : nullptr, a.n_groups, a.rows, kW4M, (a.N + kCols - 1) / kCols,
                   tile))
        return;

    const int lane = lane_id(), wave = uniform((int)(threadIdx.x >> 6));
    const int wm = wave >> 2, wn = wave & 3;
    const int e = tile.group;
    const int c0 = tile.nt * kCols;
    const int K = a.K, kblocks = K / kW4BK, nq = 2 * kblocks;
    const int fr = lane & 31, half = lane >> 5;

    // activation loads: instruction i (0..3) of wave w fills stage rows 8 (4 w + i) + lane / 8,
    // slot lane % 8; rows past the m-tile load its first row (never stored), so every load is
    // unconditional
    uint32_t aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 8 * (4 * wave + i) + (lane >> 3);
        const int p = tile.row0 + r < tile.row1 ? tile.row0 + r : tile.row0;
        const uint32_t src = (kPhase == 1 && kGrouped) ? (uint32_t)(a.perm[p] / a.k) : (uint32_t)p;
        aoff[i] = src * (uint32_t)(K / 8) + (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
    }
    // weight row r of the tile (0..255): phase 1 rows 0..127 gate, 128..255 up; phase 2 down
    auto wrow = [&](int r, const void* m0, const void* m1, size_t row_bytes) {
        const uint8_t* base;
        int wr;
        if (kPhase == 1) {
            base = (const uint8_t*)(r < 128 ? m0 : m1);
            wr = c0 + (r & 127);
        } else {  // rows past N (the absent half of a last tile) read row N - 1, never stored
            base = (const uint8_t*)m0;
            wr = min(c0 + r, a.N - 1);
        }
        return base + ((size_t)e * a.N + wr) * row_bytes;
    };
    // code loads: instruction i (0..1) of wave w fills slot rows 16 (2 w + i) + lane / 4, slot
    // lane % 4
    const uint8_t* bsrc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = 16 * (2 * wave + i) + (lane >> 2);
        bsrc[i] = wrow(r, a.w0, a.w1, (size_t)K / 2) + (((lane & 3) ^ ((r >> 2) & 3)) << 4);
    }
    // scale loads: wave w's 4-byte load fills rows 32 w + lane % 32 (groups 4 kb .. 4 kb + 3) at
    // byte 256 w + 4 (lane % 32); lanes 32..63 repeat lanes 0..31 into the unused upper half
    const uint8_t* msrc = wrow(32 * wave + fr, a.s0, a.s1, (size_t)K / 32);

    // A wave whose 32 activation rows all lie past the m-tile's last row loads no activations
    // (no filled m-subtile reads them); the load counts its waits assume follow from kA.
    const bool load_a = 32 * wave < tile.row1 - tile.row0;
    auto issue_a = [&](int q) {
        const uint8_t* act = (const uint8_t*)a.act + (size_t)q * (kW4K * 2);
        uint8_t* dst = sA[q % kW4Ring];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            lds_dma16(act + (size_t)aoff[i] * 16, dst + 8 * (4 * wave + i) * kW4K * 2);
    };
    auto issue_b = [&](int kb) {
        uint8_t* dst = sB[kb % kW4Ring];
#pragma unroll
        for (int i = 0; i < 2; ++i) lds_dma16(bsrc[i] + (size_t)kb * (kW4BK / 2), dst + 16 * (2 * wave + i) * (kW4BK / 2));
        lds_dma4(msrc + (size_t)kb * 4, &sM[kb % kW4Ring][256 * wave]);
    };

    const int nvalid = (tile.row1 - tile.row0 + 31) >> 5;  // filled 32-row subtiles (1..8)
    const int mine = (nvalid > wm) + (nvalid > wm + 2) + (nvalid > wm + 4) + (nvalid > wm + 6);
    int aaddr[4][4], baddr[2][2][2], maddr[2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int r = (wm + 2 * mi) * 32 + fr;
#pragma unroll
        for (int q = 0; q < 4; ++q) {  // step (j, t) = (q / 2, q % 2): chunk 4 j + 2 half + t
            const int c = 4 * (q >> 1) + 2 * half + (q & 1);
            aaddr[mi][q] = r * (kW4K * 2) + ((c ^ ((r >> 1) & 7)) << 4);
        }
    }
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        const int r = (kPhase == 1 ? ni * 128 + wn * 32 : wn * 64 + ni * 32) + fr;
        maddr[ni] = 256 * (r >> 5) + 4 * (r & 31);
#pragma unroll
        for (int hs = 0; hs < 2; ++hs)  // stage within the slot
#pragma unroll
            for (int j = 0; j < 2; ++j)  // chunk 2 hs + j; this lane's 8 bytes at 8 half
                baddr[ni][hs][j] = r * (kW4BK / 2) + (((2 * hs + j) ^ ((r >> 2) & 3)) << 4) + 8 * half;
    }

    f32x16 acc[4][2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int x = 0; x < 16; ++x) acc[mi][ni][x] = 0.0f;

    // Loads in issue order: weight slots 0 and 1, activation stages 0 and 1 (kA); then at stage
    // q: weight slot q / 2 + 2 (q even), activation stage q + 2 (kA).  Stage q needs activation
    // stage q and weight slot q / 2; the wait leaves in flight exactly the loads issued after the
    // newest of those (with kA activation stage q: stage q + 1's, and for odd q the slot issued
    // at q - 1; without, weight slot q / 2: the next slot, and for odd q the one after).
    auto stage = [&](int q, auto st_tag, auto ns_tag, auto a_tag) {
        constexpr int ST = decltype(st_tag)::value, NS = decltype(ns_tag)::value;
        constexpr bool kA = decltype(a_tag)::value;
        constexpr int HS = ST & 1;  // stage within the weight slot (q = ST mod 6)
        const int kb = q >> 1;
        const bool b1 = kb + 1 < kblocks, b2 = kb + 2 < kblocks, a1 = q + 1 < nq;
        if (kA) {
            if (HS == 1) {
                if (b2 && a1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kW4BL + kW4AL));
                else if (b2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kW4BL));
                else if (a1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kW4AL));
                else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            } else {
                if (a1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kW4AL));
                else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            }
        } else {
            if (HS == 1 && b1 && b2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kW4BL));
            else if (b1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kW4BL));
            else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
        __syncthreads();
        if (HS == 0 && b2) issue_b(kb + 2);
        if (kA && q + 2 < nq) issue_a(q + 2);
        if (NS == 0) return;
        const uint8_t* A = sA[ST % kW4Ring];
        const uint8_t* B = sB[(ST >> 1) % kW4Ring];
        const uint8_t* M = sM[(ST >> 1) % kW4Ring];
        uint32_t sc[2];  // E8M0 scales of this stage's two groups (bytes 0, 1) per weight subtile
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) sc[ni] = *(const uint16_t*)&M[maddr[ni] + 2 * HS];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            uint2 w[2];
            float f[2];
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                w[ni] = *(const uint2*)&B[baddr[ni][HS][j]];
                f[ni] = e8m0_to_f32((sc[ni] >> (8 * j)) & 255u);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                bf16x8 fa[NS > 0 ? NS : 1];
#pragma unroll
                for (int mi = 0; mi < NS; ++mi) fa[mi] = *(const bf16x8*)&A[aaddr[mi][2 * j + t]];
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) {
                    const bf16x8 fb = fp4x8_to_bf16x8(t ? w[ni].y : w[ni].x, f[ni]);
#pragma unroll
                    for (int mi = 0; mi < NS; ++mi)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb, acc[mi][ni], 0, 0, 0);
                }
            }
        }
    };
    auto run = [&](auto ns_tag, auto a_tag) {
        issue_b(0);
        if (kblocks > 1) issue_b(1);
        if (decltype(a_tag)::value) {
            issue_a(0);
            issue_a(1);  // nq >= 2
        }
        // the slots of stage q are q % 3 (activations) and (q / 2) % 3 (weights): period 6
        for (int q = 0; q < nq; q += 6) {
            stage(q, std::integral_constant<int, 0>{}, ns_tag, a_tag);
            if (q + 1 < nq) stage(q + 1, std::integral_constant<int, 1>{}, ns_tag, a_tag);
            if (q + 2 < nq) stage(q + 2, std::integral_constant<int, 2>{}, ns_tag, a_tag);
            if (q + 3 < nq) stage(q + 3, std::integral_constant<int, 3>{}, ns_tag, a_tag);
            if (q + 4 < nq) stage(q + 4, std::integral_constant<int, 4>{}, ns_tag, a_tag);
            if (q + 5 < nq) stage(q + 5, std::integral_constant<int, 5>{}, ns_tag, a_tag);
        }
    };
    // the K loop for this wave's filled-subtile count and activation loads
    auto dispatch = [&](auto a_tag) {
        if (mine == 4) run(std::integral_constant<int, 4>{}, a_tag);
        else if (mine == 3) run(std::integral_constant<int, 3>{}, a_tag);
        else if (mine == 2) run(std::integral_constant<int, 2>{}, a_tag);
        else if (mine == 1) run(std::integral_constant<int, 1>{}, a_tag);
        else run(std::integral_constant<int, 0>{}, a_tag);
    };
    if (load_a)
        dispatch(std::true_type{});
    else
        dispatch(std::false_type{});

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
            } else if (c0 + wn * 64 < a.N) {  // a wave's 64 columns are all present or all absent
                const uint32_t b = f32x2_to_bf16x2(acc[mi][0][x], acc[mi][1][x]);
                o[wn * 64] = (uint16_t)b;
                o[wn * 64 + 32] = (uint16_t)(b >> 16);
            }
        }
    }
}

bool w4_gemm_fits(int phase, const GemmArgs& a) {
    if (!a.fp4 || use_gemv(a.rows, a.n_groups)) return false;
    // phase 1: 128 h columns a tile; phase 2: 256 y columns a tile, the last one possibly half
    if (a.K % kW4BK != 0 || a.N % (kW4N / 2) != 0) return false;
    // activation rows are addressed by 32-bit 16-byte chunk indices
    return (int64_t)a.rows * (a.K / 8) < (int64_t(1) << 32);
}

moe_status launch_gemm_w4(int phase, const GemmArgs& a, hipStream_t st) {
    if (!w4_gemm_fits(phase, a)) return MOE_ERR_UNSUPPORTED;
    const int cols = phase == 1 ? kW4N / 2 : kW4N;
    const int groups = a.offsets ? a.n_groups : 1;
    const int64_t mt = ((int64_t)a.rows + kW4M - 1) / kW4M + std::min<int64_t>(groups, a.rows);
    const int64_t wgs = mt * ((a.N + cols - 1) / cols);
    if (wgs > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)((wgs + 7) & ~int64_t(7))), block(512);
    const bool g = a.offsets != nullptr;
    if (phase == 1) {
        if (g) gemm_w4_kernel<1, true><<<grid, block, 0, st>>>(a);
        else gemm_w4_kernel<1, false><<<grid, block, 0, st>>>(a);
    } else {
        if (g) gemm_w4_kernel<2, true><<<grid, block, 0, st>>>(a);
        else gemm_w4_kernel<2, false><<<grid, block, 0, st>>>(a);
    }
    return launch_status();
}

}  // namespace moe

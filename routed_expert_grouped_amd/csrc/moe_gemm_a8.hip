// moe_gemm_a8.hip -- grouped expert GEMMs with FP8 activations, on gfx950's scaled FP8 matrix
// instruction.
//
// Both operands are E4M3FN codes.  The weights carry one fp32 scale per 128x128 block (the
// OSDI'26 hybrid-inference article, "native FP8 GEMV", Figures 9-10).  The activations carry one
// power-of-two scale 2^e per row and 128-long K block (int8 e; the E8M0 byte is 127 + e).
// v_mfma_scale_f32_32x32x64_f8f6f4 multiplies 32x64 by 64x32 codes and applies an E8M0 scale per
// row of A itself, so the activation scales cost no instructions.  The weight scales are
// applied to each 128-long block's sum as in the bf16-operand GEMM: the accumulator is kept in
// units of the current block's scale.
//
// Tiles as in the bf16-operand GEMM of moe_gemm.hip: one 8-wave workgroup per CU computes a
// 256-row m-tile against 256 weight rows (phase 1: 128 gate + the same 128 up rows -> 128 h
// columns; phase 2: 256 y columns).  K goes in 64-long compute stages.  Operands are loaded
// directly to LDS, in two rings:
//   activations  16 KB stages of 64 K (256 rows x 64 bytes), 3 slots, two stages ahead;
//   weights      32 KB slots of 128 K, one scale block (256 rows x 128 bytes: every row is read
//                in whole 128-byte lines), 3 slots, two blocks (four stages) ahead;
//   exponents    4 KB parts of 16 blocks (256 rows x 16 bytes), 2 slots, a part ahead.
//
// MFMA operand layout (32x32x64, 32 bytes a lane): lane l supplies row l % 32 of A (column
// l % 32 of B); its bytes 0-15 are K values [16 h, 16 h + 16) and bytes 16-31 are
// [32 + 16 h, 48 + 16 h) of the 64-long step, h = l / 32.  The instruction's scale operands
// apply per 32-long K group: group g of row (column) l % 32 takes the E8M0 byte of lane
// l % 32 + 32 g.
//
// Activation rows are 64 bytes in LDS, four 16-byte chunks, chunk c at slot c ^ ((row >> 2) & 3);
// weight rows are 128 bytes, eight chunks, chunk c at slot c ^ ((row >> 1) & 7), so that 16
// consecutive rows' reads of one chunk land in distinct 16-byte bank groups.
//
// MXFP4 weights with FP8 activations (W4A8) have a kernel of their own (moe_gemm_w4a8.hip); this
// launcher hands them to it.
#include "libmoe.h"
#include "moe_device.h"
#include "moe_ffn.h"
#include "moe_host.h"
#include "moe_lds.h"

#include <type_traits>

namespace moe {

typedef int i32x8 __attribute__((__vector_size__(8 * sizeof(int))));

constexpr int kA8M = 256;    // rows per m-tile
constexpr int kA8N = 256;    // weight rows per tile
constexpr int kA8K = 64;     // K per compute stage: one MFMA step, half a scale block
constexpr int kA8BK = 128;   // K per weight slot: one scale block
constexpr int kARing = 3;    // activation slots
constexpr int kBRing = 3;    // weight slots
constexpr int kEPart = 16;   // scale blocks per exponent part
constexpr int kE8M0One = 127;  // E8M0 encoding of 1.0
constexpr int kFmtFP8 = 0;   // operand format of the scaled MFMA (E4M3)

__device__ __forceinline__ i32x8 join(u32x4 lo, u32x4 hi) {
    i32x8 r = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    return r;
}

template <int kPhase, bool kGrouped>
__global__ __launch_bounds__(512, 1) void gemm_a8_kernel(GemmArgs a) {
    constexpr int kAStage = kA8M * kA8K;   // 16 KB
    constexpr int kBSlot = kA8N * 128;     // 32 KB: 128 bytes of each weight row
    constexpr int kEBytes = kA8M * 16;     // 4 KB
    constexpr int kBK = kA8BK;        // K per weight slot
    constexpr int kSPS = kBK / kA8K;  // compute stages per weight slot
    constexpr int kBL = 4;            // loads per wave per weight slot
    constexpr int kPeriod = kARing * kSPS;  // stages after which the slot pattern repeats
    __shared__ __attribute__((aligned(1024))) uint8_t sA[kARing][kAStage];
    __shared__ __attribute__((aligned(1024))) uint8_t sB[kBRing][kBSlot];
    __shared__ __attribute__((aligned(1024))) uint8_t sE[2][kEBytes];  // [row][16 blocks]
    __shared__ float sScale[2][kA8MaxPitch];

    constexpr int kCols = kPhase == 1 ? kA8N / 2 : kA8N;
    Tile tile;
    if (!find_tile(kGrouped ? a.offsets : nullptr, a.n_groups, a.rows, kA8M, a.N / kCols, tile))
        return;

    const int tid = (int)threadIdx.x, lane = lane_id(), wave = uniform(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int e = tile.group;
    const int c0 = tile.nt * kCols;
    const int K = a.K, kblocks = K / 128, nq = 2 * kblocks;
    const int nslots = K / kBK;
    const int cpr = a.aexp_pitch >> 4;  // 16-byte parts of an exponent row (1..4)
    const int fr = lane & 31, half = lane >> 5;
    const uint8_t* act = (const uint8_t*)a.act;

    // source row (token, or grouped row) of tile row r; rows past the m-tile read its first row
    // (never stored), so every load is unconditional
    auto src_row = [&](int r) -> uint32_t {
        const int p = tile.row0 + r < tile.row1 ? tile.row0 + r : tile.row0;
        return (kPhase == 1 && kGrouped) ? (uint32_t)(a.perm[p] / a.k) : (uint32_t)p;
    };
    // activation loads: instruction i (0..1) of wave w fills stage rows 16 (2 w + i) + lane / 4,
    // slot lane % 4 holding chunk slot ^ ((row >> 2) & 3); sources in 16-byte units (32 bits: the
    // host keeps the codes below 64 GB)
    uint32_t aoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = 16 * (2 * wave + i) + (lane >> 2);
        aoff[i] = src_row(r) * (uint32_t)(K / 16) + (uint32_t)((lane & 3) ^ ((r >> 2) & 3));
    }
    // weight loads: instruction i (0..3) of wave w fills slot rows 8 (4 w + i) + lane / 8, slot
    // lane % 8 holding chunk slot ^ ((row >> 1) & 7); phase 1 rows 0..127 gate, 128..255 up.
    const size_t row_bytes = (size_t)K;
    const uint8_t* bsrc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 8 * (4 * wave + i) + (lane >> 3);
        const uint8_t* base;
        int wr;
        if (kPhase == 1) {
            base = (const uint8_t*)(r < 128 ? a.w0 : a.w1);
            wr = c0 + (r & 127);
        } else {
            base = (const uint8_t*)a.w0;
            wr = c0 + r;
        }
        const int chunk = (lane & 7) ^ ((r >> 1) & 7);
        bsrc[i] = base + ((size_t)e * a.N + wr) * row_bytes + (chunk << 4);
    }
    // exponent parts: waves 0..3 each fill rows 64 w + lane (16 bytes: blocks 16 p .. 16 p + 15)
    const uint32_t eoff = src_row((64 * wave + lane) & (kA8M - 1)) * (uint32_t)cpr;

    // A wave whose 32 activation rows all lie past the m-tile's last row loads no activations
    // (no filled m-subtile reads them); the load counts its waits assume follow from kA.
    const bool load_a = 32 * wave < tile.row1 - tile.row0;
    auto issue_a = [&](int q) {
        const uint8_t* aq = act + (size_t)q * kA8K;
        uint8_t* dst = sA[q % kARing];
#pragma unroll
        for (int i = 0; i < 2; ++i) lds_dma16(aq + (size_t)aoff[i] * 16, dst + 16 * (2 * wave + i) * kA8K);
    };
    auto issue_b = [&](int sl) {  // weight slot sl (kBL loads)
        uint8_t* dst = sB[sl % kBRing];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            lds_dma16(bsrc[i] + (size_t)sl * 128, dst + 8 * (4 * wave + i) * 128);
    };
    auto issue_e = [&](int part) {  // waves 0..3 (whole waves)
        if (wave < 4)
            lds_dma16((const uint8_t*)a.aexp + ((size_t)eoff + part) * 16, &sE[part & 1][16 * 64 * wave]);
    };

    // weight block scales: phase 1 [0] gate, [1] up of block-row c0/128; phase 2 block-rows
    // c0/128 and c0/128 + 1 (the tile's 256 rows)
    if (tid < kblocks) {
        const size_t srow = ((size_t)e * (a.N / 128) + c0 / 128) * kblocks;
        sScale[0][tid] = a.s0[srow + tid];
        sScale[1][tid] = kPhase == 1 ? a.s1[srow + tid] : a.s0[srow + kblocks + tid];
    }
    const int sg0 = kPhase == 1 ? 0 : (wn >> 1);
    const int sg1 = kPhase == 1 ? 1 : (wn >> 1);

    const int nvalid = (tile.row1 - tile.row0 + 31) >> 5;  // filled 32-row subtiles (1..8)
    const int mine = (nvalid > wm) + (nvalid > wm + 2) + (nvalid > wm + 4) + (nvalid > wm + 6);
    int aaddr[4][2], baddr[2][kSPS][2], eaddr[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int r = (wm + 2 * mi) * 32 + fr;
        eaddr[mi] = r * 16;
#pragma unroll
        for (int j = 0; j < 2; ++j) aaddr[mi][j] = r * kA8K + (((2 * j + half) ^ ((r >> 2) & 3)) << 4);
    }
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        const int r = (kPhase == 1 ? ni * 128 + wn * 32 : wn * 64 + ni * 32) + fr;
#pragma unroll
        for (int hs = 0; hs < kSPS; ++hs)  // compute stage within the weight slot
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int chunk = 4 * hs + 2 * j + half;
                baddr[ni][hs][j] = r * 128 + ((chunk ^ ((r >> 1) & 7)) << 4);
            }
    }
    bool any_zero = false;
    __syncthreads();  // weight scales staged
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

    // Weight block scales by Horner (as in moe_gemm.hip): before block b the accumulator is
    // multiplied by u / s_b (u = the scale of the last block with a nonzero scale), the block's
    // MFMAs add into it, and the end multiplies by u.  A zero scale keeps the units and masks
    // that block's weight codes, so the block adds exactly nothing.
    float u0 = 0.0f, u1 = 0.0f;
    uint32_t m0 = ~0u, m1 = ~0u;
    int sc[4] = {kE8M0One, kE8M0One, kE8M0One, kE8M0One};  // E8M0 activation scales of the block
    // the E8M0 scales of four blocks per m-subtile row, read as one word every fourth block
    // (int8 e -> 127 + e in every byte: e ^ 0x80 = e + 128 is at least 1 for e >= -127, so
    // subtracting 1 from each byte borrows nothing across bytes); block kb takes byte kb % 4
    uint32_t sw[4] = {0u, 0u, 0u, 0u};
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
    // Loads in issue order: exponent part 0, weight slots 0 and 1, activation stages 0 and 1
    // (kA); then at stage q: (first stage of slot q / kSPS) exponent part q / 32 + 1 when
    // q % 32 == 0, weight slot q / kSPS + 2; activation stage q + 2 (kA).  Stage q needs
    // activation stage q and weight slot q / kSPS (and its exponent part, older than both); the
    // wait allows the loads issued after the newest of those to stay in flight: with kA the
    // newest is activation stage q, followed by stage q + 1's and, when stage q - 1 began a
    // slot, that slot's kBL weight loads; without, weight slot q / kSPS, followed by the next
    // slot's and, past the slot's first stage, the one after.  The exponent loads of waves 0..3
    // are not counted: an uncounted newer load only makes a wait stricter.
    auto stage = [&](int q, auto st_tag, auto ns_tag, auto mask_tag, auto a_tag) {
        constexpr int ST = decltype(st_tag)::value, NS = decltype(ns_tag)::value;
        constexpr bool kMask = decltype(mask_tag)::value, kA = decltype(a_tag)::value;
        constexpr int HS = ST % kSPS;  // stage within the weight slot (q = ST mod kPeriod)
        const int kb = q >> 1;         // 128-long K block: activation exponents, FP8 weight scales
        const int sl = q / kSPS;
        const bool b1 = sl + 1 < nslots, b2 = sl + 2 < nslots, a1 = q + 1 < nq;
        if (kA) {
            if (HS == 1) {
                if (b2 && a1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kBL + 2));
                else if (b2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kBL));
                else if (a1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2));
                else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            } else {
                if (a1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2));
                else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            }
        } else {
            if (HS >= 1 && b1 && b2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kBL));
            else if (b1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kBL));
            else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
        __syncthreads();
        if (HS == 0) {
            if ((q & (2 * kEPart - 1)) == 0 && kb + kEPart < kblocks) issue_e(kb / kEPart + 1);
            if (b2) issue_b(sl + 2);
        }
        if (kA && q + 2 < nq) issue_a(q + 2);
        if (NS == 0) return;
        if (HS == 0) {  // first half of scale block kb
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
        if ((ST & 1) == 0) {  // first stage of 128-long block kb: its activation exponents
            if ((kb & 3) == 0) {
                const uint8_t* E = sE[(kb / kEPart) & 1] + (kb & (kEPart - 1));
#pragma unroll
                for (int mi = 0; mi < NS; ++mi)
                    sw[mi] = (*(const uint32_t*)&E[eaddr[mi]] ^ 0x80808080u) - 0x01010101u;
            }
#pragma unroll
            for (int mi = 0; mi < NS; ++mi) sc[mi] = (int)(sw[mi] >> (8 * (kb & 3)));
        }
        const uint8_t* A = sA[ST % kARing];
        const uint8_t* B = sB[(ST / kSPS) % kBRing];
        // every fragment of the stage is read before the first MFMA
        i32x8 fb[2], fa[NS > 0 ? NS : 1];
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
            u32x4 lo = *(const u32x4*)&B[baddr[ni][HS][0]];
            u32x4 hi = *(const u32x4*)&B[baddr[ni][HS][1]];
            if (kMask) {
                lo &= ni == 0 ? m0 : m1;
                hi &= ni == 0 ? m0 : m1;
            }
            fb[ni] = join(lo, hi);
        }
#pragma unroll
        for (int mi = 0; mi < NS; ++mi)
            fa[mi] = join(*(const u32x4*)&A[aaddr[mi][0]], *(const u32x4*)&A[aaddr[mi][1]]);
#pragma unroll
        for (int mi = 0; mi < NS; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    fa[mi], fb[ni], acc[mi][ni], kFmtFP8, kFmtFP8, 0, sc[mi], 0, kE8M0One);
    };
    auto run = [&](auto ns_tag, auto mask_tag, auto a_tag) {
        issue_e(0);
        issue_b(0);
        if (nslots > 1) issue_b(1);
        if (decltype(a_tag)::value) {
            issue_a(0);
            issue_a(1);  // nq >= 2
        }
        // the slots of stage q are q % 3 (activations) and (q / kSPS) % 3 (weights): period
        // kPeriod = 6
        for (int q = 0; q < nq; q += kPeriod) {
            stage(q, std::integral_constant<int, 0>{}, ns_tag, mask_tag, a_tag);
            if (q + 1 < nq) stage(q + 1, std::integral_constant<int, 1>{}, ns_tag, mask_tag, a_tag);
            if (q + 2 < nq) stage(q + 2, std::integral_constant<int, 2>{}, ns_tag, mask_tag, a_tag);
            if (q + 3 < nq) stage(q + 3, std::integral_constant<int, 3>{}, ns_tag, mask_tag, a_tag);
            if (q + 4 < nq) stage(q + 4, std::integral_constant<int, 4>{}, ns_tag, mask_tag, a_tag);
            if (q + 5 < nq) stage(q + 5, std::integral_constant<int, 5>{}, ns_tag, mask_tag, a_tag);
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

bool a8_gemm_fits(int phase, const GemmArgs& a) {
    if (!(a.fp8 || a.fp4) || use_gemv(a.rows, a.n_groups)) return false;
    if (a.K % 128 != 0 || a.K > kA8MaxK) return false;
    if (a.N % (phase == 1 ? kA8N / 2 : kA8N) != 0) return false;
    if (a.aexp_pitch % 16 != 0 || a.aexp_pitch < a.K / 128 || a.aexp_pitch > kA8MaxPitch)
        return false;
    // activation rows: tokens (phase 1) or grouped rows (phase 2), addressed in 16-byte units
    const int64_t src_rows = phase == 1 ? a.rows / a.k : a.rows;
    return src_rows * (a.K / 16) < (int64_t(1) << 32);
}

moe_status launch_gemm_a8(int phase, const GemmArgs& a, hipStream_t st) {
    if (!a8_gemm_fits(phase, a)) return MOE_ERR_UNSUPPORTED;
    if (a.fp4) return launch_gemm_w4a8(phase, a, st);
    // the down projection takes 160 x 512 tiles when an average expert fits one 160-row m-tile
    const int64_t n_exp = a.offsets ? a.n_groups : 1;
    if (a8_wide_gemm_fits(phase, a) && a.rows <= 160 * n_exp) return launch_gemm_a8_wide(phase, a, st);
    const int cols = phase == 1 ? kA8N / 2 : kA8N;
    const int groups = a.offsets ? a.n_groups : 1;
    const int64_t mt = ((int64_t)a.rows + kA8M - 1) / kA8M + std::min<int64_t>(groups, a.rows);
    const int64_t wgs = mt * (a.N / cols);
    if (wgs > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)((wgs + 7) & ~int64_t(7))), block(512);
    const bool g = a.offsets != nullptr;
#define MOE_A8(P, G) gemm_a8_kernel<P, G><<<grid, block, 0, st>>>(a)
    if (phase == 1) g ? MOE_A8(1, true) : MOE_A8(1, false);
    else g ? MOE_A8(2, true) : MOE_A8(2, false);
#undef MOE_A8
    return launch_status();
}

}  // namespace moe

using namespace moe;

// The two public phase calls: validation, then the FP8-code GEMM.
static moe_status a8_phase(int phase, const uint8_t* codes, const int8_t* exps, int32_t pitch,
                           int32_t T, int32_t k, const int32_t* perm, const int32_t* offsets,
                           const moe_expert_weights* w, uint16_t* out, void* stream) {
    if (T < 0 || k < 1) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!codes || !exps || !out || !aligned16(codes) || !aligned16(exps) || !aligned16(out))
        return MOE_ERR_INVALID_ARG;
    moe_status s = check_weights(w);
    if (s != MOE_OK) return s;
    if (w->dtype != MOE_W_FP8_E4M3_B128 && w->dtype != MOE_W_MXFP4_G32) return MOE_ERR_UNSUPPORTED;
    if ((s = check_grouping(T, k, perm, offsets, w, phase == 1)) != MOE_OK) return s;
    GemmArgs a{};
    a.act = reinterpret_cast<const uint16_t*>(codes);
    a.aexp = exps;
    a.aexp_pitch = pitch;
    a.perm = phase == 1 ? perm : nullptr;
    a.offsets = offsets;
    a.k = k;
    a.rows = T * k;
    a.n_groups = w->n_groups;
    a.N = phase == 1 ? w->I : w->H;
    a.K = phase == 1 ? w->H : w->I;
    if (pitch < a.K / 128) return MOE_ERR_INVALID_ARG;
    a.w0 = phase == 1 ? w->w_gate : w->w_down;
    a.w1 = phase == 1 ? w->w_up : nullptr;
    a.s0 = phase == 1 ? w->s_gate : w->s_down;
    a.s1 = phase == 1 ? w->s_up : nullptr;
    a.fp8 = w->dtype == MOE_W_FP8_E4M3_B128;
    a.fp4 = w->dtype == MOE_W_MXFP4_G32;
    a.out = out;
    if (!a8_gemm_fits(phase, a)) return MOE_ERR_UNSUPPORTED;
    return launch_gemm_a8(phase, a, as_stream(stream));
}

extern "C" moe_status moe_expert_gate_up_a8(const uint8_t* x_codes, const int8_t* x_exps,
                                            int32_t exp_pitch, int32_t T, int32_t k,
                                            const int32_t* perm, const int32_t* offsets,
                                            const moe_expert_weights* w, uint16_t* h,
                                            void* stream) {
    return a8_phase(1, x_codes, x_exps, exp_pitch, T, k, perm, offsets, w, h, stream);
}

extern "C" moe_status moe_expert_down_a8(const uint8_t* h_codes, const int8_t* h_exps,
                                         int32_t exp_pitch, int32_t T, int32_t k,
                                         const int32_t* offsets, const moe_expert_weights* w,
                                         uint16_t* y, void* stream) {
    return a8_phase(2, h_codes, h_exps, exp_pitch, T, k, nullptr, offsets, w, y, stream);
}

// moe_gemm_a8_wide.hip -- the FP8-activation grouped down projection for FP8 weights with
// 160-row x 512-weight-row tiles, for layers whose average expert fits one 160-row m-tile.
//
// Arithmetic as in moe_gemm_a8.hip: E4M3FN activation codes with one power-of-two scale per row
// and 128-long K block, applied by v_mfma_scale_f32_32x32x64_f8f6f4 itself; E4M3FN weight codes
// with one fp32 scale per 128x128 block, applied to each block's sum by keeping the accumulator
// in units of the current block's scale (the OSDI'26 hybrid-inference article's post-scaling,
// "native FP8 GEMV", Figures 9-10).
//
// Why this shape: at about 128 rows per expert (T = 4096, DeepSeek-V3 shapes) a 256-row m-tile
// is half empty, so each stage of the 256 x 256 kernel carries half its MFMAs for the same weight
// loads.  A 160-row m-tile still holds a whole expert there (95-160 rows) and covers 512 weight
// rows: a 64-long stage loads 10 KB of activation codes and 32 KB of weight codes for 160 x 512
// outputs, and the down projection (K = I = 2048, short) needs half as many workgroups, each
// with its own pipeline fill and epilogue.  Measured at T = 4096: down 0.94 against 0.98 ms;
// the gate/up projection (K = 7168) was no faster this way (1.78 ms either way) and keeps the
// 256 x 256 tiles of moe_gemm_a8.hip.
//
// Waves: 8, each owning 64 y columns against all five 32-row m-subtiles, 10 MFMAs a stage.  LDS
// is a 3-slot ring of 64-long stages (activations 160 rows x 64 bytes, codes 512 rows x 64
// bytes, each row four 16-byte chunks, chunk c at slot c ^ ((row >> 2) & 3)) plus two parts of
// 16 blocks of activation exponents (192 rows x 16 bytes: rows 160-191 are padding the third
// loading wave fills).  Loads per stage: waves 0-1 two 16-row activation instructions, waves
// 2-7 one; four 16-row code instructions a wave.  A wave whose activation rows all lie past the
// m-tile loads none of them; its hand-counted waits follow from its own load count.
#include "libmoe.h"
#include "moe_device.h"
#include "moe_ffn.h"
#include "moe_host.h"
#include "moe_lds.h"

#include <type_traits>

namespace moe {

namespace {

typedef int i32x8 __attribute__((__vector_size__(8 * sizeof(int))));

constexpr int kXM = 160;       // rows per m-tile (5 subtiles of 32)
constexpr int kXN = 512;       // weight rows per tile
constexpr int kXK = 64;        // K per stage: one MFMA step, half a scale block
constexpr int kXStages = 3;    // ring slots
constexpr int kXEPart = 16;    // 128-long blocks per exponent part
constexpr int kXERows = 192;   // exponent rows per part: three whole wave loads
constexpr int kXE8M0One = 127;
constexpr int kXFmtFP8 = 0;

__device__ __forceinline__ i32x8 join8(u32x4 lo, u32x4 hi) {
    i32x8 r = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    return r;
}

}  // namespace

template <bool kGrouped>
__global__ __launch_bounds__(512, 1) void gemm_a8_wide_kernel(GemmArgs a) {
    constexpr int kAStage = kXM * kXK;  // 10 KB
    constexpr int kBStage = kXN * kXK;  // 32 KB
    __shared__ __attribute__((aligned(1024))) uint8_t sA[kXStages][kAStage];
    __shared__ __attribute__((aligned(1024))) uint8_t sB[kXStages][kBStage];
    __shared__ __attribute__((aligned(1024))) uint8_t sE[2][kXERows * 16];
    __shared__ float sScale[4][kA8MaxPitch];  // the tile's four 128-row block-rows

    Tile tile;
    if (!find_tile(kGrouped ? a.offsets : nullptr, a.n_groups, a.rows, kXM, a.N / kXN, tile))
        return;

    const int tid = (int)threadIdx.x, lane = lane_id(), wave = uniform(tid >> 6);
    const int e = tile.group;
    const int c0 = tile.nt * kXN;
    const int K = a.K, kblocks = K / 128, nq = 2 * kblocks;
    const int cpr = a.aexp_pitch >> 4;  // 16-byte parts of an exponent row
    const int fr = lane & 31, half = lane >> 5;
    const int nrows = tile.row1 - tile.row0;
    const uint8_t* act = (const uint8_t*)a.act;

    // source (grouped) row of tile row r; rows past the m-tile read its first row (never
    // stored), so every load is unconditional
    auto src_row = [&](int r) -> uint32_t {
        return (uint32_t)(tile.row0 + r < tile.row1 ? tile.row0 + r : tile.row0);
    };
    // activation loads: instruction i of wave w fills stage rows arow0 + 16 i + lane / 4, slot
    // lane % 4 holding chunk slot ^ ((row >> 2) & 3); sources in 16-byte units (32 bits: the
    // host keeps the codes below 64 GB)
    const int arow0 = wave < 2 ? 32 * wave : 64 + 16 * (wave - 2);
    uint32_t aoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = min(arow0 + 16 * i + (lane >> 2), kXM - 1);
        aoff[i] = src_row(r) * (uint32_t)(K / 16) + (uint32_t)((lane & 3) ^ ((r >> 2) & 3));
    }
    // code loads: instruction i (0..3) of wave w fills stage rows 64 w + 16 i + lane / 4, slot
    // lane % 4 holding chunk slot ^ ((row >> 2) & 3)
    const int brow0 = 64 * wave + (lane >> 2);  // weight row of instruction 0
    const uint8_t* bsrc = (const uint8_t*)a.w0 + ((size_t)e * a.N + c0 + brow0) * (size_t)K +
                          (((lane & 3) ^ ((brow0 >> 2) & 3)) << 4);
    const size_t bstep = (size_t)16 * K;  // 16 weight rows; the swizzle repeats every 16 rows
    // exponent parts: waves 0..2 fill rows 64 w + lane (16 bytes: blocks 16 p .. 16 p + 15)
    const uint32_t eoff = src_row(min(64 * wave + lane, kXM - 1)) * (uint32_t)cpr;

    const bool load_a = arow0 < nrows;
    auto issue = [&](int q, int st, auto ai_tag, auto a_tag) {
        constexpr int AI = decltype(ai_tag)::value;
        if (decltype(a_tag)::value) {
            const uint8_t* aq = act + (size_t)q * kXK;
#pragma unroll
            for (int i = 0; i < AI; ++i)
                lds_dma16(aq + (size_t)aoff[i] * 16, &sA[st][(arow0 + 16 * i) * kXK]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            lds_dma16(bsrc + i * bstep + (size_t)q * kXK, &sB[st][(64 * wave + 16 * i) * kXK]);
    };
    auto issue_e = [&](int part) {  // waves 0..2 (whole waves)
        if (wave < 3)
            lds_dma16((const uint8_t*)a.aexp + ((size_t)eoff + part) * 16,
                      &sE[part & 1][16 * 64 * wave]);
    };

    // weight block scales of the tile's four 128-row block-rows from c0/128
    for (int i = tid; i < 4 * kblocks; i += 512) {
        const int br = i / kblocks, b = i - br * kblocks;
        sScale[br][b] = a.s0[((size_t)e * (a.N / 128) + c0 / 128 + br) * kblocks + b];
    }
    // this wave's weight subtiles ni = 0, 1: rows 64 w + 32 ni, both in block-row w / 2
    const int sg = wave >> 1;

    const int mine = (nrows + 31) >> 5;  // filled 32-row subtiles (1..5)
    // fragment addresses of m-subtile 0 (subtile mi adds mi * 32 rows, the same swizzle) and of
    // weight subtile 0 (subtile 1 adds 32 rows, the same swizzle)
    int aaddr[2], baddr[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        aaddr[j] = fr * kXK + (((2 * j + half) ^ ((fr >> 2) & 3)) << 4);
        const int r = wave * 64 + fr;
        baddr[j] = r * kXK + (((2 * j + half) ^ ((r >> 2) & 3)) << 4);
    }
    constexpr int kBSub = 32 * kXK;  // weight subtile 1's offset
    const int eaddr = fr * 16;
    bool any_zero = false;
    __syncthreads();  // scales staged
    for (int b = lane; b < kblocks; b += kWave)
        any_zero |= sScale[sg][b] == 0.0f;
    any_zero = __ballot(any_zero) != 0;

    f32x16 acc[5][2];
#pragma unroll
    for (int mi = 0; mi < 5; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int x = 0; x < 16; ++x) acc[mi][ni][x] = 0.0f;

    // Weight block scales by Horner (as in moe_gemm_a8.hip): before block b the accumulator is
    // multiplied by u / s_b (u = the scale of the last block with a nonzero scale), the block's
    // MFMAs add into it, and the end multiplies by u.  A zero scale keeps the units and masks
    // that block's weight codes, so the block adds exactly nothing.  Both weight subtiles of a
    // wave share one block-row, so one scale serves them.
    float u = 0.0f;
    uint32_t m = ~0u;
    // E8M0 activation scales: one word of four blocks per m-subtile row, read every fourth block
    // (int8 e -> 127 + e in every byte: e ^ 0x80 = e + 128 is at least 1 for e >= -127, so
    // subtracting 1 from each byte borrows nothing across bytes); block kb takes byte kb % 4
    uint32_t sw[5] = {0u, 0u, 0u, 0u, 0u};
    auto rescale = [&](float r, auto ns_tag) {
        constexpr int NS = decltype(ns_tag)::value;
#pragma unroll
        for (int mi = 0; mi < NS; ++mi)
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                acc[mi][0][x] *= r;
                acc[mi][1][x] *= r;
            }
    };
    // One 64-long stage from ring slot ST with NS filled m-subtiles.  Stage q needs the loads
    // issued two stages earlier (and its exponent part, issued 32 stages before its first use);
    // the ones of the stage in between stay in flight.  The exponent loads of waves 0..2 are
    // issued before a stage's others and not counted: an uncounted older load only makes a wait
    // stricter.
    auto stage = [&](int q, auto st_tag, auto ns_tag, auto mask_tag, auto ai_tag, auto a_tag) {
        constexpr int ST = decltype(st_tag)::value, NS = decltype(ns_tag)::value;
        constexpr bool kMask = decltype(mask_tag)::value;
        constexpr int kIssued = (decltype(a_tag)::value ? decltype(ai_tag)::value : 0) + 4;
        if (q + 1 < nq)
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(kIssued));
        else
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();
        const int kb = q >> 1;  // 128-long K block: activation exponents, weight scales
        if ((q & (2 * kXEPart - 1)) == 0 && kb + kXEPart < kblocks) issue_e(kb / kXEPart + 1);
        if (q + 2 < nq) issue(q + 2, (ST + 2) % kXStages, ai_tag, a_tag);
        if (NS == 0) return;
        if ((q & 1) == 0) {  // first half of scale block kb
            const float s = sScale[sg][kb];
            if (kMask) {
                const bool z = s == 0.0f;
                rescale(z ? 1.0f : u * __builtin_amdgcn_rcpf(s), ns_tag);
                u = z ? u : s;
                m = z ? 0u : ~0u;
            } else {
                rescale(u * __builtin_amdgcn_rcpf(s), ns_tag);
                u = s;
            }
            if ((kb & 3) == 0) {
                const uint8_t* E = sE[(kb / kXEPart) & 1] + (kb & (kXEPart - 1));
#pragma unroll
                for (int mi = 0; mi < NS; ++mi)
                    sw[mi] = (*(const uint32_t*)&E[eaddr + mi * 32 * 16] ^ 0x80808080u) -
                             0x01010101u;
            }
        }
        const uint8_t* A = sA[ST];
        const uint8_t* B = sB[ST];
        i32x8 fb[2], fa[NS > 0 ? NS : 1];
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
            u32x4 lo = *(const u32x4*)&B[baddr[0] + ni * kBSub];
            u32x4 hi = *(const u32x4*)&B[baddr[1] + ni * kBSub];
            if (kMask) {
                lo &= m;
                hi &= m;
            }
            fb[ni] = join8(lo, hi);
        }
#pragma unroll
        for (int mi = 0; mi < NS; ++mi)
            fa[mi] = join8(*(const u32x4*)&A[aaddr[0] + mi * 32 * kXK],
                           *(const u32x4*)&A[aaddr[1] + mi * 32 * kXK]);
        const int sh = 8 * (kb & 3);
#pragma unroll
        for (int mi = 0; mi < NS; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    fa[mi], fb[ni], acc[mi][ni], kXFmtFP8, kXFmtFP8, 0, (int)(sw[mi] >> sh), 0,
                    kXE8M0One);
    };
    auto run = [&](auto ns_tag, auto mask_tag, auto ai_tag, auto a_tag) {
        using S0 = std::integral_constant<int, 0>;
        using S1 = std::integral_constant<int, 1>;
        using S2 = std::integral_constant<int, 2>;
        issue_e(0);
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
    // the K loop for this wave's activation load count (2 or 1, or none past the m-tile) and the
    // filled-subtile count; a tile with a zero block scale takes the masked path (all subtiles)
    auto by_loads = [&](auto ai_tag) {
        if (!load_a) {
            if (any_zero) run(std::integral_constant<int, 5>{}, MY{}, ai_tag, std::false_type{});
            else by_ns(MN{}, ai_tag, std::false_type{});
        } else {
            if (any_zero) run(std::integral_constant<int, 5>{}, MY{}, ai_tag, std::true_type{});
            else by_ns(MN{}, ai_tag, std::true_type{});
        }
    };
    if (wave < 2)
        by_loads(std::integral_constant<int, 2>{});
    else
        by_loads(std::integral_constant<int, 1>{});
    rescale(u, std::integral_constant<int, 5>{});

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
            const uint32_t b = f32x2_to_bf16x2(acc[mi][0][x], acc[mi][1][x]);
            o[wave * 64] = (uint16_t)b;
            o[wave * 64 + 32] = (uint16_t)(b >> 16);
        }
    }
}

bool a8_wide_gemm_fits(int phase, const GemmArgs& a) {
    return phase == 2 && a.fp8 && a8_gemm_fits(phase, a) && a.N % kXN == 0;
}

moe_status launch_gemm_a8_wide(int phase, const GemmArgs& a, hipStream_t st) {
    if (!a8_wide_gemm_fits(phase, a)) return MOE_ERR_UNSUPPORTED;
    const int groups = a.offsets ? a.n_groups : 1;
    const int64_t mt = ((int64_t)a.rows + kXM - 1) / kXM + std::min<int64_t>(groups, a.rows);
    const int64_t wgs = mt * (a.N / kXN);
    if (wgs > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)((wgs + 7) & ~int64_t(7))), block(512);
    if (a.offsets) gemm_a8_wide_kernel<true><<<grid, block, 0, st>>>(a);
    else gemm_a8_wide_kernel<false><<<grid, block, 0, st>>>(a);
    return launch_status();
}

}  // namespace moe

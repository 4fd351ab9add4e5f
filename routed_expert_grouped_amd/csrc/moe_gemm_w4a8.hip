// moe_gemm_w4a8.hip -- the grouped expert GEMM with FP8 activations and MXFP4 weights (W4A8),
// one wave per SIMD.
//
// E4M3FN activation codes with one power-of-two scale per row and 128-long K block (the
// FP8-activation mode's quantisation, moe_quant.hip) times E2M1 weight codes with their E8M0 scale
// per 32-long K group, both scales applied by v_mfma_scale_f32_32x32x64_f8f6f4 itself, fp32 sums.
// Nothing is rescaled (unlike FP8 weights with fp32 block scales, moe_gemm_a8.hip), so the sums
// never pass through the vector ALU until the epilogue, and the work is laid out on a CU as:
//   * 4 waves, one per SIMD, each computing 128 rows x 128 weight rows of the 256 x 256 tile:
//     16 MFMAs a 64-long stage.  The 256 fp32 sums sit in the accumulation registers, which
//     leaves the vector registers free for two sets of operand fragments.
//   * While a stage's MFMAs run, the wave reads the next stage's fragments from LDS into the
//     other set, so no MFMA waits for an LDS read.  A 128 x 128 wave tile reads 12 KB of
//     fragments a stage for 16 MFMAs (a 128 x 64 one would read 10 KB for 8).
//
// LDS (140 KB) holds every operand row as whole 128-byte lines, eight 16-byte chunks, chunk c at
// slot c ^ ((row >> 1) & 7):
//   activations  32 KB slots of 128 K (256 rows x 128 bytes: two compute stages), 2 slots;
//   weights      32 KB slots of 256 K (256 rows x 128 bytes of E2M1 codes: four stages), 2 slots,
//                each with its E8M0 scales (256 rows x 8 bytes);
//   exponents    4 KB parts of 16 blocks (256 rows x 16 bytes), 2 slots.
//
// Loads (direct to LDS, in this order within a stage; waits count them by hand).  Every wave
// issues 2 nA loads per activation slot (nA = 64-row blocks holding tile rows, the same for all
// waves), 10 per weight slot in two parts of 5, and 1 per exponent part:
//   prologue   exponent parts 0, 1 (those that exist), weight slot 0, part 0 of weight slot 1,
//              activation slots 0, 1;
//   stage q    after the barrier: exponent part q / 32 + 2 when q % 32 == 31 (if it exists);
//              part 0 of weight slot q / 4 + 2 when q % 4 == 3, part 1 of weight slot q / 4 + 1
//              when q % 4 == 0; activation slot (q + 3) / 2 when q is odd.
// Past the end of K a weight load reloads the last slot and an activation load the last slot,
// into ring slots that no stage reads again.  A ring slot is refilled in the stage after the one
// whose fragments were its last, behind the barrier that every wave passes only once it has read
// them: activation slot d + 2 two stages before its first fragments are read, weight slot s + 2
// three and four stages before.
#include "libmoe.h"
#include "moe_device.h"
#include "moe_ffn.h"
#include "moe_host.h"
#include "moe_lds.h"

#include <type_traits>

namespace moe {

namespace {

typedef int i32x8 __attribute__((__vector_size__(8 * sizeof(int))));

constexpr int kM = 256;      // rows per m-tile
constexpr int kN = 256;      // weight rows per tile
constexpr int kSK = 64;      // K per compute stage (one MFMA step)
constexpr int kAK = 128;     // K per activation slot
constexpr int kSlotK = 256;  // K per weight slot
constexpr int kSPA = kAK / kSK;      // stages per activation slot
constexpr int kSPS = kSlotK / kSK;   // stages per weight slot
constexpr int kRing = 2;             // activation and weight slots in LDS
constexpr int kEPart = 16;           // 128-long blocks per exponent part
constexpr int kBL = 10;              // loads a wave per weight slot: 8 code, 2 scale
constexpr int kBPart = kBL / 2;      // a weight slot goes out in two parts of 5 loads
constexpr int kPeriod = kRing * kSPS;  // stages after which the slot pattern repeats
// an activation exponent word covers four blocks, eight stages: one loop period
static_assert(kPeriod == 8, "the exponent words are read at the first stage of each period");
constexpr int kFmtFP8 = 0, kFmtFP4 = 4;

__device__ __forceinline__ i32x8 widen(u32x4 lo) {
    i32x8 r = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], 0, 0, 0, 0};
    return r;
}

__device__ __forceinline__ i32x8 join2(u32x4 lo, u32x4 hi) {
    i32x8 r = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    return r;
}

template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (N > 0) {
        static_for<N - 1>(f);
        f(std::integral_constant<int, N - 1>{});
    }
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(size_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
    return *(const __attribute__((address_space(3))) u32x4*)(size_t)addr;
}

__device__ __forceinline__ int lds_read_u8(uint32_t addr) {
    return *(const __attribute__((address_space(3))) uint8_t*)(size_t)addr;
}

__device__ __forceinline__ uint32_t lds_read_u32(uint32_t addr) {
    return *(const __attribute__((address_space(3))) uint32_t*)(size_t)addr;
}

// s_waitcnt vmcnt(n) for a run-time n (0..15)
__device__ __forceinline__ void wait_loads(int n) {
    switch (n) {
#define MOE_W(i) case i: __builtin_amdgcn_s_waitcnt(vmcnt_imm(i)); break;
        MOE_W(1) MOE_W(2) MOE_W(3) MOE_W(4) MOE_W(5) MOE_W(6) MOE_W(7) MOE_W(8)
        MOE_W(9) MOE_W(10) MOE_W(11) MOE_W(12) MOE_W(13) MOE_W(14) MOE_W(15)
#undef MOE_W
        default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
    }
}

}  // namespace

template <int kPhase, bool kGrouped>
__global__ __launch_bounds__(256, 1) void gemm_w4a8_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t sA[kRing][kM * 128];
    __shared__ __attribute__((aligned(1024))) uint8_t sB[kRing][kN * 128];
    __shared__ __attribute__((aligned(1024))) uint8_t sE[2][kM * 16];
    __shared__ __attribute__((aligned(16))) uint8_t sMX[kRing][kN * 8];

    constexpr int kCols = kPhase == 1 ? kN / 2 : kN;
    Tile tile;
    if (!find_tile(kGrouped ? a.offsets : nullptr, a.n_groups, a.rows, kM, a.N / kCols, tile))
        return;

    const int lane = lane_id(), wave = uniform((int)threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int e = tile.group, c0 = tile.nt * kCols;
    const int K = a.K, nq = K / kSK, nslots = (K + kSlotK - 1) / kSlotK, nd = K / kAK;
    const int nparts = (K / 128 + kEPart - 1) / kEPart;
    const bool half_last = K % kSlotK != 0;  // the last weight slot holds 128 K
    const int cpr = a.aexp_pitch >> 4;       // 16-byte parts of an exponent row
    const int fr = lane & 31, half = lane >> 5;
    const int nvalid = (tile.row1 - tile.row0 + 31) >> 5;  // filled 32-row subtiles (1..8)
    const uint8_t* act = (const uint8_t*)a.act;

    // source row (token, or grouped row) of tile row r; rows past the m-tile read its first row
    auto src_row = [&](int r) -> uint32_t {
        const int p = tile.row0 + r < tile.row1 ? tile.row0 + r : tile.row0;
        return (kPhase == 1 && kGrouped) ? (uint32_t)(a.perm[p] / a.k) : (uint32_t)p;
    };
    // activation loads: instruction i (0 .. 2 nA - 1) of every wave fills slot rows
    // 32 i + 8 wave + lane / 8, slot lane % 8, whose chunk (lane % 8) ^ ((4 wave + lane / 16) % 8)
    // does not depend on i (sources in 16-byte units: the host keeps the codes below 64 GB)
    const uint32_t achunk = (uint32_t)((lane & 7) ^ ((4 * wave + (lane >> 4)) & 7));
    uint32_t aoff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        aoff[i] = src_row(32 * i + 8 * wave + (lane >> 3)) * (uint32_t)(K / 16) + achunk;
    // weight loads: instruction i (0..7) fills slot rows 64 wave + 8 i + lane / 8, slot lane % 8
    // (phase 1: rows 0..127 gate, 128..255 up, so a wave's 64 rows lie in one matrix).  The chunk
    // of a lane, (lane % 8) ^ ((row >> 1) & 7) = (lane % 8) ^ (4 (i % 2) + lane / 16), takes two
    // patterns, so each address is a wave-uniform part plus one of two lane parts.  In a last
    // slot of 128 K the chunks past its 64 bytes reload its first half (never read).
    const size_t row_bytes = (size_t)K / 2;
    const int wrow0 = c0 + (kPhase == 1 ? 64 * (wave & 1) : 64 * wave);  // weight row of lane 0
    const uint8_t* wbase = (const uint8_t*)(kPhase == 1 && wave >= 2 ? a.w1 : a.w0) +
                           ((size_t)e * a.N + wrow0) * row_bytes;
    uint32_t boff[2], boff_part[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int chunk = (lane & 7) ^ (4 * p + (lane >> 4));
        boff[p] = (uint32_t)(lane >> 3) * (uint32_t)row_bytes + (uint32_t)(chunk << 4);
        boff_part[p] = boff[p] - (chunk >= 4 ? 64u : 0u);
    }
    // E8M0 weight scales [N][K/32]: instruction i (0..1) fills slot rows 64 wave + 32 i + lane / 2,
    // groups 4 (lane % 2) .. + 3 of the slot; in a last slot of 128 K odd lanes reload the even
    // lanes' dword
    const uint8_t* mbase = (const uint8_t*)(kPhase == 1 && wave >= 2 ? a.s1 : a.s0) +
                           ((size_t)e * a.N + wrow0) * (size_t)(K / 32);
    const uint32_t moff = (uint32_t)(lane >> 1) * (uint32_t)(K / 32) + 4u * (lane & 1);
    const uint32_t moff_part = moff - ((lane & 1) ? 4u : 0u);
    // exponent parts: every wave fills rows 64 wave + lane (16 bytes: blocks 16 p .. 16 p + 15)
    const uint32_t eoff = src_row(64 * wave + lane) * (uint32_t)cpr;

    // LDS byte addresses of this wave's load destinations (ring slot 0)
    const uint32_t ldsA = lds_addr(&sA[0][0]) + 8 * wave * 128;
    const uint32_t ldsB = lds_addr(&sB[0][0]) + 64 * wave * 128;
    const uint32_t ldsM = lds_addr(&sMX[0][0]) + 64 * wave * 8;
    const uint32_t ldsE = lds_addr(&sE[0][0]) + 64 * wave * 16;

    // one load of activation slot d into ring slot R (instruction I); a slot past the last one
    // reloads the last one (into a free ring slot, never read)
    auto load_a = [&](int d, auto r_tag, auto i_tag) {
        constexpr int R = decltype(r_tag)::value, I = decltype(i_tag)::value;
        lds_dma16_at(act + (size_t)aoff[I] * 16 + (size_t)min(d, nd - 1) * kAK,
                     ldsA + R * kM * 128 + 32 * I * 128);
    };
    // one load of weight slot s into ring slot R (I < 8: codes, 8..9: E8M0 scales); a slot past
    // the last one reloads the last one (into a free ring slot, never read)
    auto load_b = [&](int s, auto r_tag, auto i_tag) {
        constexpr int R = decltype(r_tag)::value, I = decltype(i_tag)::value;
        const int sl = min(s, nslots - 1);
        const bool part = half_last && sl == nslots - 1;
        if constexpr (I < 8) {
            const uint32_t off = part ? boff_part[I & 1] : boff[I & 1];
            lds_dma16_at(wbase + ((size_t)(8 * I) * row_bytes + (size_t)sl * 128) + off,
                         ldsB + R * kN * 128 + 8 * I * 128);
        } else {
            const uint32_t off = part ? moff_part : moff;
            lds_dma4_at(mbase + ((size_t)(32 * (I - 8)) * (size_t)(K / 32) + (size_t)sl * 8) + off,
                        ldsM + R * kN * 8 + 32 * (I - 8) * 8);
        }
    };
    auto load_e = [&](int p) {
        lds_dma16_at((const uint8_t*)a.aexp + ((size_t)eoff + p) * 16, ldsE + (p & 1) * kM * 16);
    };

    // per-lane parts of the fragment addresses (the subtile and ring parts are constants); the
    // swizzle (row >> 1) & 7 of a fragment row is (fr >> 1) & 7, its subtile starting at a
    // multiple of 32 rows
    uint32_t xa[kSPA][2], xb[kSPS], xm, xe;
#pragma unroll
    for (int h = 0; h < kSPA; ++h)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            xa[h][j] = lds_addr(&sA[0][0]) + (wm * 32 + fr) * 128 +
                       (((4 * h + 2 * j + half) ^ ((fr >> 1) & 7)) << 4);
    const int bbase = kPhase == 1 ? 64 * wn : 128 * wn;
#pragma unroll
    for (int hs = 0; hs < kSPS; ++hs)
        xb[hs] = lds_addr(&sB[0][0]) + (bbase + fr) * 128 + (((2 * hs + half) ^ ((fr >> 1) & 7)) << 4);
    xm = lds_addr(&sMX[0][0]) + (bbase + fr) * 8 + half;
    xe = lds_addr(&sE[0][0]) + (wm * 32 + fr) * 16;
    // slot row of n-subtile ni relative to bbase
    auto nrow = [](int ni) { return kPhase == 1 ? (ni < 2 ? 32 * ni : 128 + 32 * (ni - 2)) : 32 * ni; };

    f32x16 acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int x = 0; x < 16; ++x) acc[mi][ni][x] = 0.0f;

    // two fragment sets: stage q's MFMAs read set q % 2 while set (q + 1) % 2 is filled
    i32x8 fa[2][4], fb[2][4];
    // activation exponents: one 4-byte word per m-subtile row holds the exponents e of four
    // 128-long blocks (eight stages), read once per eight stages; sc8 holds them as E8M0 bytes
    // (127 + e), the MFMA picking the block's byte by op_sel.  E8M0 weight scales: a byte a stage.
    uint32_t se[4], sc8[4];
    int sb[2][4];

    // fragment reads of stage q (ST = q mod kPeriod) into set ST % 2: n-subtile ni, m-subtile mi
    auto read_b = [&](auto st_tag, auto ni_tag) {
        constexpr int ST = decltype(st_tag)::value, NI = decltype(ni_tag)::value;
        constexpr int S = ST & 1, HS = ST % kSPS, R = (ST / kSPS) % kRing;
        fb[S][NI] = widen(lds_read16(xb[HS] + R * kN * 128 + nrow(NI) * 128));
        sb[S][NI] = lds_read_u8(xm + R * kN * 8 + nrow(NI) * 8 + 2 * HS);
    };
    auto read_a = [&](int q, auto st_tag, auto mi_tag) {
        constexpr int ST = decltype(st_tag)::value, MI = decltype(mi_tag)::value;
        constexpr int S = ST & 1, H = ST % kSPA, R = (ST / kSPA) % kRing;
        const uint32_t off = R * kM * 128 + 2 * MI * 32 * 128;
        fa[S][MI] = join2(lds_read16(xa[H][0] + off), lds_read16(xa[H][1] + off));
        if constexpr (ST % 8 == 0) {  // first stage of four blocks: their exponents
            const int kb = q >> 1;      // a multiple of 4
            se[MI] = lds_read_u32(xe + ((kb / kEPart) & 1) * kM * 16 + (kb & (kEPart - 1)) +
                                  2 * MI * 32 * 16);
        }
    };
    auto mfma = [&](auto st_tag, auto j_tag) {
        constexpr int S = decltype(st_tag)::value & 1, J = decltype(j_tag)::value;
        constexpr int MI = J / 4, NI = J % 4;
        constexpr int ST = decltype(st_tag)::value;
        acc[MI][NI] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            fa[S][MI], fb[S][NI], acc[MI][NI], kFmtFP8, kFmtFP4, (ST / 2) % 4, (int)sc8[MI], 0,
            sb[S][NI]);
    };

    // Stage q (ST = q mod kPeriod): its first two MFMAs; the wait for this wave's loads of stage
    // q + 1 and the barrier; exponent part q / 32 + 2 when q % 32 == 31 (if it exists); then the
    // other MFMAs with the rest of the stage's work between them, in order: a part of a weight
    // slot (q % 4 == 3 or 0), activation slot (q + 3) / 2 (q odd), the reads of stage q + 1's
    // fragments.  Past the end of K the loads reload the last slots into ring slots just freed
    // and the reads fetch fragments no MFMA uses, so that part of the stage has no branches.
    // The newest load that stage q + 1 needs is activation slot D = (q + 1) / 2, issued last in
    // stage 2 D - 3 (or in the prologue, D < 2); its weight slot and exponent part went out before
    // it.  The loads issued after it are: for q == 0, activation slot 1 (prologue); for q odd,
    // those of stage q - 1 (even): a weight part when q - 1 == 0 mod 4; for q even, those of
    // stages q - 2 (even: a weight part when q - 2 == 0 mod 4) and q - 1 (odd: an exponent part if
    // one was issued, a weight part when q - 1 == 3 mod 4, 2 nA activation loads).  Together:
    // q == 0: 2 nA; q even: 2 nA + 5 (+ 1); q == 1 mod 4: 5; q == 3 mod 4: 0.
    auto stage = [&](int q, auto st_tag, auto na_tag, auto ns_tag) {
        constexpr int ST = decltype(st_tag)::value, NA = decltype(na_tag)::value;
        constexpr int NS = decltype(ns_tag)::value;
        constexpr int ST1 = (ST + 1) % kPeriod;
        // weight part issued here: part 0 of slot q / 4 + 2 (ST % 4 == 3) or part 1 of slot
        // q / 4 + 1 (ST % 4 == 0), ring slot = slot % 2
        constexpr int JB = ST % kSPS == kSPS - 1 ? 0 : (ST % kSPS == 0 ? 1 : -1);
        constexpr int RB = JB == 0 ? (ST / kSPS) % kRing : ((ST / kSPS) + 1) % kRing;
        constexpr int NB = JB >= 0 ? kBPart : 0;
        constexpr int NAL = ST % 2 == 1 ? 2 * NA : 0;        // activation loads issued here
        constexpr int RA = ((ST + 3) / kSPA) % kRing;        // their ring slot
        constexpr int NM = 4 * NS;  // MFMAs
        constexpr int NT = NB + NAL + 4 + NS;  // work items between MFMAs
        constexpr int GAPS = NM > 2 ? NM - 2 : 1;
        constexpr int PER = (NT + GAPS - 1) / GAPS;  // items before each of MFMAs 2..
        if constexpr (ST % 8 == 0) {
            // int8 e -> E8M0 127 + e in every byte: e ^ 0x80 is e + 128 in [1, 255] (e >= -127),
            // so subtracting 1 from each byte borrows nothing across bytes
#pragma unroll
            for (int mi = 0; mi < NS; ++mi) sc8[mi] = (se[mi] ^ 0x80808080u) - 0x01010101u;
        }
        if constexpr (NM > 0) mfma(st_tag, std::integral_constant<int, 0>{});
        if constexpr (NM > 1) mfma(st_tag, std::integral_constant<int, 1>{});
        __builtin_amdgcn_sched_barrier(0);
        if (q + 1 < nq) {
            if constexpr (ST % 2 == 1)
                wait_loads(ST % kSPS == 1 ? kBPart : 0);
            else
                wait_loads(q == 0 ? 2 * NA
                                  : 2 * NA + kBPart +
                                        ((q & 31) == 0 && q / 32 + 1 < nparts ? 1 : 0));
            __syncthreads();
        }
        if ((q & 31) == 31 && q / 32 + 2 < nparts) load_e(q / 32 + 2);
        __builtin_amdgcn_sched_barrier(0);
        const int sb_ = q / kSPS + (JB == 0 ? 2 : 1);
        const int da = (q + 3) / kSPA;
        // reads in the order the next stage's first MFMAs use them: n-subtile 0, m-subtile 0,
        // n-subtiles 1..3, m-subtiles 1..
        auto item = [&](auto t_tag) {
            constexpr int T = decltype(t_tag)::value, U = T - NB - NAL;
            constexpr int BI = U == 0 ? 0 : (NS > 0 && U <= 4 ? U - 1 : U);  // n-subtile of read U
            constexpr int AI = U == 1 ? 0 : U - 4;                            // m-subtile of read U
            constexpr bool kIsB = U == 0 || (NS > 0 ? (U >= 2 && U <= 4) : U < 4);
            if constexpr (T < NB) {
                load_b(sb_, std::integral_constant<int, RB>{},
                       std::integral_constant<int, (JB == 1 ? kBPart : 0) + T>{});
            } else if constexpr (T < NB + NAL) {
                load_a(da, std::integral_constant<int, RA>{}, std::integral_constant<int, T - NB>{});
            } else if constexpr (T < NT && kIsB) {
                read_b(std::integral_constant<int, ST1>{}, std::integral_constant<int, BI>{});
            } else if constexpr (T < NT) {
                read_a(q + 1, std::integral_constant<int, ST1>{}, std::integral_constant<int, AI>{});
            }
        };
        static_for<GAPS + 1>([&](auto g) {
            constexpr int G = decltype(g)::value;
            static_for<PER>([&](auto u) {
                item(std::integral_constant<int, G * PER + decltype(u)::value>{});
            });
            if constexpr (G + 2 < NM) {
                __builtin_amdgcn_sched_barrier(0);
                mfma(st_tag, std::integral_constant<int, G + 2>{});
                __builtin_amdgcn_sched_barrier(0);
            }
        });
    };
    auto run = [&](auto na_tag, auto ns_tag) {
        constexpr int NA = decltype(na_tag)::value;
        using R0 = std::integral_constant<int, 0>;
        using R1 = std::integral_constant<int, 1>;
        load_e(0);
        if (nparts > 1) load_e(1);
        static_for<kBL>([&](auto i) { load_b(0, R0{}, i); });
        static_for<kBPart>([&](auto i) { load_b(1, R1{}, i); });  // part 0 of slot 1
        static_for<2 * NA>([&](auto i) { load_a(0, R0{}, i); });
        static_for<2 * NA>([&](auto i) { load_a(1, R1{}, i); });
        wait_loads(2 * NA);
        __syncthreads();
        static_for<4>([&](auto ni) { read_b(R0{}, ni); });
        static_for<decltype(ns_tag)::value>([&](auto mi) { read_a(0, R0{}, mi); });
        for (int q = 0; q < nq; q += kPeriod) {
            stage(q, std::integral_constant<int, 0>{}, na_tag, ns_tag);
            if (q + 1 < nq) stage(q + 1, std::integral_constant<int, 1>{}, na_tag, ns_tag);
            if (q + 2 < nq) stage(q + 2, std::integral_constant<int, 2>{}, na_tag, ns_tag);
            if (q + 3 < nq) stage(q + 3, std::integral_constant<int, 3>{}, na_tag, ns_tag);
            if (q + 4 < nq) stage(q + 4, std::integral_constant<int, 4>{}, na_tag, ns_tag);
            if (q + 5 < nq) stage(q + 5, std::integral_constant<int, 5>{}, na_tag, ns_tag);
            if (q + 6 < nq) stage(q + 6, std::integral_constant<int, 6>{}, na_tag, ns_tag);
            if (q + 7 < nq) stage(q + 7, std::integral_constant<int, 7>{}, na_tag, ns_tag);
        }
    };
    // nA: 64-row blocks holding tile rows; this wave's filled m-subtiles: wm + 2 mi < nvalid
    const int na = (nvalid + 1) >> 1;
    const bool full = wm == 0 || (nvalid & 1) == 0;  // this wave has na subtiles, else na - 1
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using I4 = std::integral_constant<int, 4>;
    if (na == 4) full ? run(I4{}, I4{}) : run(I4{}, I3{});
    else if (na == 3) full ? run(I3{}, I3{}) : run(I3{}, I2{});
    else if (na == 2) full ? run(I2{}, I2{}) : run(I2{}, I1{});
    else full ? run(I1{}, I1{}) : run(I1{}, I0{});
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

    // D layout of the 32x32 MFMA: value x of a lane is row 8 (x / 4) + 4 (lane / 32) + x % 4 of
    // the subtile, column lane % 32
    const int mine = (nvalid > wm) + (nvalid > wm + 2) + (nvalid > wm + 4) + (nvalid > wm + 6);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        if (mi >= mine) break;
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            const int p = tile.row0 + (wm + 2 * mi) * 32 + 8 * (x >> 2) + 4 * half + (x & 3);
            if (p >= tile.row1) continue;
            uint16_t* o = a.out + (size_t)p * a.N + c0 + fr;
            if (kPhase == 1) {
                const uint32_t b = f32x2_to_bf16x2(silu_mul(acc[mi][0][x], acc[mi][2][x]),
                                                   silu_mul(acc[mi][1][x], acc[mi][3][x]));
                o[64 * wn] = (uint16_t)b;
                o[64 * wn + 32] = (uint16_t)(b >> 16);
            } else {
#pragma unroll
                for (int ni = 0; ni < 4; ni += 2) {
                    const uint32_t b = f32x2_to_bf16x2(acc[mi][ni][x], acc[mi][ni + 1][x]);
                    o[128 * wn + 32 * ni] = (uint16_t)b;
                    o[128 * wn + 32 * ni + 32] = (uint16_t)(b >> 16);
                }
            }
        }
    }
}

bool w4a8_gemm_fits(int phase, const GemmArgs& a) {
    return a.fp4 && a8_gemm_fits(phase, a);
}

moe_status launch_gemm_w4a8(int phase, const GemmArgs& a, hipStream_t st) {
    if (!w4a8_gemm_fits(phase, a)) return MOE_ERR_UNSUPPORTED;
    const int cols = phase == 1 ? kN / 2 : kN;
    const int groups = a.offsets ? a.n_groups : 1;
    const int64_t mt = ((int64_t)a.rows + kM - 1) / kM + std::min<int64_t>(groups, a.rows);
    const int64_t wgs = mt * (a.N / cols);
    if (wgs > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)((wgs + 7) & ~int64_t(7))), block(256);
    const bool g = a.offsets != nullptr;
    if (phase == 1)
        g ? gemm_w4a8_kernel<1, true><<<grid, block, 0, st>>>(a)
          : gemm_w4a8_kernel<1, false><<<grid, block, 0, st>>>(a);
    else
        g ? gemm_w4a8_kernel<2, true><<<grid, block, 0, st>>>(a)
          : gemm_w4a8_kernel<2, false><<<grid, block, 0, st>>>(a);
    return launch_status();
}

}  // namespace moe

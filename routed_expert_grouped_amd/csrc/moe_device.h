// moe_device.h -- device-side helpers shared by the libmoe HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

constexpr int kWave = 64;

// ------------------------------------------------------------------ number formats

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even, by gfx950's conversion instruction (v_cvt_pk_bf16_f32); a
// NaN stays a NaN.  The bit-level form (add 0x7fff + lsb, keep the high half) rounds every finite
// value the same way, but its NaN test costs a branch per value.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// two floats -> two bf16 (one conversion instruction), a in the low half
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// SiLU(g) * u: g / (1 + e^-g) with the hardware reciprocal (about 1 ulp) in place of the IEEE
// division; the result is rounded to bf16 next
__device__ __forceinline__ float silu_mul(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Eight OCP E4M3FN codes (two little-endian words) -> eight bf16 values, exactly: every E4M3FN
// value, subnormals included, is a bf16 value.  gfx950's conversion instruction decodes the OCP
// encoding; the scale operand is 1.0, so nothing is rescaled here (block scales are applied to
// fp32 partial sums instead).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, false);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, true);
    bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, false);
    bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, true);
    bf16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    return r;
}

// Eight OCP MX FP4 (E2M1) codes (one word, element 2j in the low nibble of byte j) times the
// scale `s` (a power of two) -> eight bf16 values, exactly.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t w, float s) {
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((int)w, s, 0);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((int)w, s, 1);
    bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((int)w, s, 2);
    bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((int)w, s, 3);
    bf16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    return r;
}

// The E8M0 scale byte s as a float: 2^(s - 127); s = 0 is the subnormal 2^-127, s = 255 is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
    return __uint_as_float(s == 0 ? 0x00400000u : s == 255 ? 0x7fc00000u : s << 23);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// ------------------------------------------------------------------ wave primitives

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
    return v;
}

// Mask of the lanes whose `key` equals this lane's key, among lanes with `valid` set (0 for an
// invalid lane): one ballot per key bit.  Must be called by the whole wave.
__device__ __forceinline__ uint64_t match_peers(int key, bool valid, int nbits) {
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t bb = __ballot(valid && bit);
        m &= bit ? bb : ~bb;
    }
    return valid ? m : 0ull;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Maximum of v over each row of 16 lanes (every lane of the row gets it), by DPP:
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.  No LDS traffic.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
    return v;
}

// ------------------------------------------------------------------ grouped tile schedule
//
// Rows are grouped by expert: group g owns rows [offsets[g], offsets[g+1]).  Each group is cut
// into m-tiles of BM rows (the last one ragged) and each m-tile into n_tiles column tiles.  The
// host sizes the grid from an upper bound of the tile count (it never reads the counts), so the
// schedule is derived on the device from `offsets`, by every wave of a workgroup independently.
//
// XCD-aware order: MI355X dispatches consecutive workgroups round-robin to its 8 XCDs, each with
// a private L2.  Workgroup i gets logical tile (i % 8) * (R8 / 8) + i / 8 (R8 = real tile count
// rounded up to 8), so each XCD walks one contiguous range of logical tiles, and tiles that are
// close in that range run at about the same time on the same L2.
//
// An optional extra group (extra_rows > 0, group index n_groups) has extra_rows rows starting
// at extra_base.  extra_base is passed in rather than read from offsets[n_groups], so that a
// slice of the grouping (one expert range, whose offsets[n_groups] ends before the last grouped
// row) still puts the extra rows after all grouped rows.  Its tiles take the first workgroups
// (rounded up to a multiple of 8), in plain dispatch order: they spread over all XCDs and run
// at the start, where at the end of one XCD's range they would lengthen that XCD's work alone.
// The grouped tiles follow on the workgroups after them, in the XCD-aware order.
//
// Within a group, logical tiles go in supertiles of up to kSuperM m-tiles: the m-tiles of one
// supertile are the fastest index, its n-tiles the next.  Workgroups that read the same weight
// tile (same expert and n-tile, different rows) are therefore neighbours and walk K together,
// so the weight bytes come from HBM once per supertile instead of once per m-tile; the few
// activation row blocks of a supertile stay in L2 across the n-tiles that run alongside.
constexpr int kSuperM = 8;

struct Tile {
    int group;  // expert
    int row0;   // first row of the m-tile
    int row1;   // one past the last row (ragged)
    int nt;     // column tile
};

__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offsets, int n_groups,
                                          int identity_rows, int BM, int n_tiles, Tile& t,
                                          int extra_rows = 0, int extra_base = 0) {
    const int lane = lane_id();
    int wg = (int)blockIdx.x;
    if (extra_rows > 0) {
        const int xm = (extra_rows + BM - 1) / BM, X = xm * n_tiles, X8 = (X + 7) & ~7;
        if (wg < X8) {
            if (wg >= X) return false;
            t.group = n_groups;
            t.nt = wg % n_tiles;
            t.row0 = extra_base + (wg / n_tiles) * BM;
            t.row1 = min(t.row0 + BM, extra_base + extra_rows);
            return true;
        }
        wg -= X8;  // the grouped tiles from here
    }
    int total_m, incl = 0, local = 0;
    const int groups = n_groups;
    const int G = (groups + kWave - 1) / kWave;  // groups per lane, contiguous
    auto count = [&](int g) { return offsets[g + 1] - offsets[g]; };
    if (offsets == nullptr) {
        total_m = (identity_rows + BM - 1) / BM;
    } else {
        for (int i = 0; i < G; ++i) {
            const int g = lane * G + i;
            if (g < groups) {
                const int n = count(g);
                local += (n + BM - 1) / BM;
            }
        }
        incl = wave_inclusive_scan(local);
        total_m = __shfl(incl, kWave - 1, kWave);
    }
    total_m = uniform(total_m);
    const int R = total_m * n_tiles;
    const int R8 = (R + 7) & ~7;
    if (wg >= R8) return false;
    const int L = (wg & 7) * (R8 >> 3) + (wg >> 3);
    if (L >= R) return false;
    // the group that owns L: group g owns logical tiles [m0 * n_tiles, (m0 + m_g) * n_tiles),
    // m0 = m-tiles of the groups before it; then L's place inside the group's supertiles
    struct Place { int m, nt; };  // m-tile inside the group, n-tile
    auto place = [L, n_tiles](int m0, int m_g) -> Place {
        const int r = L - m0 * n_tiles;
        const int b = r / (kSuperM * n_tiles);
        const int rb = r - b * (kSuperM * n_tiles);
        const int gm = min(kSuperM, m_g - b * kSuperM);  // m-tiles in this supertile
        const int nt = rb / gm;
        return Place{b * kSuperM + (rb - nt * gm), nt};
    };
    const int mt = L / n_tiles;
    if (offsets == nullptr) {
        const Place pl = place(0, total_m);
        t.nt = pl.nt;
        t.group = 0;
        t.row0 = pl.m * BM;
        t.row1 = min(t.row0 + BM, identity_rows);
        return true;
    }
    const bool mine = (mt >= incl - local) && (mt < incl);
    const uint64_t owner = __ballot(mine);
    const int src = __ffsll((unsigned long long)owner) - 1;
    // the owning lane finds the group; the placement inside it is computed on the broadcast
    // (wave-uniform) values
    int group = 0, gm0 = 0, gtiles = 1, ga = 0, gn = 0;
    if (lane == src) {
        int m0 = incl - local;  // first m-tile of this lane's first group
        for (int i = 0; i < G; ++i) {
            const int g = lane * G + i;
            if (g >= groups) break;
            const int a = offsets[g], n = count(g);
            const int tiles = (n + BM - 1) / BM;
            if (mt < m0 + tiles) {
                group = g;
                gm0 = m0;
                gtiles = tiles;
                ga = a;
                gn = n;
                break;
            }
            m0 += tiles;
        }
    }
    group = uniform(__shfl(group, src, kWave));
    gm0 = uniform(__shfl(gm0, src, kWave));
    gtiles = uniform(__shfl(gtiles, src, kWave));
    ga = uniform(__shfl(ga, src, kWave));
    gn = uniform(__shfl(gn, src, kWave));
    const Place pl = place(gm0, gtiles);
    t.group = group;
    t.nt = pl.nt;
    t.row0 = ga + pl.m * BM;
    t.row1 = min(t.row0 + BM, ga + gn);
    return true;
}

}  // namespace moe

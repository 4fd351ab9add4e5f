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

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
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

// ------------------------------------------------------------------ grouped tile schedule
//
// Rows are grouped by expert: group g owns rows [offsets[g], offsets[g+1]).  Each group is cut
// into m-tiles of BM rows (the last one ragged) and each m-tile into n_tiles column tiles.  The
// host sizes the grid from an upper bound of the tile count (it never reads the counts), so the
// schedule is derived on the device from `offsets`, by every wave of a workgroup independently.
//
// XCD-aware order: MI355X dispatches consecutive workgroups round-robin to its 8 XCDs, each with
// a private L2.  Workgroup i gets logical tile (i % 8) * (R8 / 8) + i / 8 (R8 = real tile count
// rounded up to 8), so each XCD walks one contiguous range of logical tiles, whose n-tiles of the
// same m-tile (same activation rows) and m-tiles of the same expert stay in one L2.

struct Tile {
    int group;  // expert
    int row0;   // first row of the m-tile
    int row1;   // one past the last row (ragged)
    int nt;     // column tile
};

__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offsets, int n_groups,
                                          int identity_rows, int BM, int n_tiles, Tile& t) {
    const int lane = lane_id();
    const int wg = (int)blockIdx.x;
    int total_m, incl = 0, local = 0;
    const int G = (n_groups + kWave - 1) / kWave;  // groups per lane, contiguous
    if (offsets == nullptr) {
        total_m = (identity_rows + BM - 1) / BM;
    } else {
        for (int i = 0; i < G; ++i) {
            const int g = lane * G + i;
            if (g < n_groups) {
                const int n = offsets[g + 1] - offsets[g];
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
    const int mt = L / n_tiles;
    t.nt = L - mt * n_tiles;
    if (offsets == nullptr) {
        t.group = 0;
        t.row0 = mt * BM;
        t.row1 = min(t.row0 + BM, identity_rows);
        return true;
    }
    const bool mine = (mt >= incl - local) && (mt < incl);
    const uint64_t owner = __ballot(mine);
    const int src = __ffsll((unsigned long long)owner) - 1;
    int group = 0, row0 = 0, row1 = 0;
    if (lane == src) {
        int m = incl - local;  // first m-tile of this lane's first group
        for (int i = 0; i < G; ++i) {
            const int g = lane * G + i;
            if (g >= n_groups) break;
            const int a = offsets[g], n = offsets[g + 1] - a;
            const int tiles = (n + BM - 1) / BM;
            if (mt < m + tiles) {
                group = g;
                row0 = a + (mt - m) * BM;
                row1 = min(row0 + BM, a + n);
                break;
            }
            m += tiles;
        }
    }
    t.group = uniform(__shfl(group, src, kWave));
    t.row0 = uniform(__shfl(row0, src, kWave));
    t.row1 = uniform(__shfl(row1, src, kWave));
    return true;
}

}  // namespace moe

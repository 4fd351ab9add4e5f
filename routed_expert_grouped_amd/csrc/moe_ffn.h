// moe_ffn.h -- shared declarations of the grouped expert-projection kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "libmoe.h"

namespace moe {

// Arguments of one projection phase over grouped rows.
//   phase 1: act = x [T][H] gathered through perm, w0/w1 = gate/up [G][N=I][K=H], out = h
//   phase 2: act = h [rows][I] (grouped order),   w0 = down [G][N=H][K=I],        out = y
struct GemmArgs {
    const uint16_t* act;
    const int32_t* perm;     // phase 1 only; NULL = identity
    const int32_t* offsets;  // [n_groups+1]; NULL = one group of `rows` rows
    int k;                   // slots per token (perm[p] / k = token)
    int rows;                // grouped rows (T*k)
    int n_groups;
    int N, K;
    const void* w0;
    const void* w1;
    const float* s0;
    const float* s1;
    bool fp8;       // E4M3FN weights + fp32 128x128 block scales (s0/s1)
    bool fp4;       // MXFP4 weights: E2M1 codes two a byte + E8M0 bytes per 32 along K (s0/s1)
    uint16_t* out;  // [rows][N]
    // FP8 activation mode only: act holds E4M3FN codes [rows of act][K] (one byte each) and
    // aexp their block exponents e (scale 2^e), [rows of act][aexp_pitch]
    const int8_t* aexp;
    int aexp_pitch;
    // An extra group after the n_groups experts (the shared expert in the routed decode launch;
    // GEMV only): extra_rows rows starting at grouped row `rows` (after every grouped row, also
    // when offsets is a slice of one expert range), row
    // rows + t holding token t, with its own weights (one expert's matrices and scales).
    int extra_rows;
    const void* xw0;
    const void* xw1;
    const float* xs0;
    const float* xs1;
};

// gemv shape: m-tiles of 16 rows; kGemvWaves waves per workgroup, each wave owning 16 h-columns
// (phase 1: 16 gate + 16 up rows) or 32 y-columns (phase 2); FP8 gate/up splits each column
// group's K over 2 or 4 waves (moe_ffn.hip).
constexpr int kGemvBM = 16;
constexpr int kGemvWaves = 4;

// Few rows per expert (decode): stream the weights with 16-row m-tiles; many rows (prefill):
// 128-row LDS-staged GEMM tiles, which read each expert's weights once per 128 rows.
inline bool use_gemv(int rows, int n_groups) { return rows <= 32 * n_groups; }

moe_status launch_gemm(int phase, const GemmArgs& a, hipStream_t st);

// FP8 activation mode: the GEMM on FP8 codes of both operands, for the shapes a8_gemm_fits
// accepts (FP8 weights, many rows per expert, K <= kA8MaxK, N a multiple of the tile's columns,
// an exponent pitch that is a multiple of 16 and at most kA8MaxPitch).
constexpr int kA8MaxK = 8192;
constexpr int kA8MaxPitch = kA8MaxK / 128;
bool a8_gemm_fits(int phase, const GemmArgs& a);
moe_status launch_gemm_a8(int phase, const GemmArgs& a, hipStream_t st);

// MXFP4 weights with FP8 activations (W4A8): the one-wave-per-SIMD GEMM (moe_gemm_w4a8.hip),
// for the shapes a8_gemm_fits accepts
bool w4a8_gemm_fits(int phase, const GemmArgs& a);
// FP8 activations and FP8 weights, down projection with 160 x 512 tiles (moe_gemm_a8_wide.hip)
bool a8_wide_gemm_fits(int phase, const GemmArgs& a);
moe_status launch_gemm_a8_wide(int phase, const GemmArgs& a, hipStream_t st);
moe_status launch_gemm_w4a8(int phase, const GemmArgs& a, hipStream_t st);

// FP8 weights, bf16 activations: the 160 x 512 tile GEMM (moe_gemm_wide.hip)
bool wide_gemm_fits(int phase, const GemmArgs& a);
moe_status launch_gemm_wide(int phase, const GemmArgs& a, hipStream_t st);

// MXFP4 weights with bf16 activations, many rows per expert: the 4-bit GEMM (moe_gemm_w4.hip)
// for the shapes w4_gemm_fits accepts; the decode kernel runs the rest
bool w4_gemm_fits(int phase, const GemmArgs& a);
moe_status launch_gemm_w4(int phase, const GemmArgs& a, hipStream_t st);

}  // namespace moe

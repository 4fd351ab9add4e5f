/*
 * libmoe.h -- C ABI of the routed sparse-MoE expert FFN for AMD Instinct MI355X (gfx950).
 *
 * One MoE layer of a DeepSeek-V3-class model: each token is routed to k of E experts, the
 * (token, expert) assignments are grouped by expert so that every expert runs one GEMM over
 * all of its tokens instead of one GEMV per token, every expert computes
 * down( SiLU(gate x) * up x ), and the expert outputs are summed back per token with the gate
 * weights, together with the always-active shared expert.
 *
 * Sources (web pages; titles and sections):
 *   [A2]  CMU 11-868 appendix A2 lecture notes, "LLM serving on heterogeneous hardware"
 *         (semidirectx.com): 4.1 (sparse MoE FFN: a few of hundreds of small experts per
 *         token), 4.2 (per-expert reuse B*k/E tokens; DeepSeek-V3 expert = three 7168x2048
 *         matrices), exercises 6-7 and their worked answers.
 *   [OSDI] Xingyun / Tsinghua OSDI'26 CPU-GPU hybrid MoE inference article (xingyun.xin):
 *         DSLP / expert-parallel section (gating and sorting, expert compute, weighted
 *         reduction), "native FP8 GEMV" section with Figures 9-10 (E4M3FN weights, bf16
 *         activations, fp32 accumulation, one scale per 128-element block applied after the
 *         block's partial sum), "CPU fine-grained parallelism" section (gate and up before
 *         down within each expert; two global synchronisations per layer).
 *   [KT]  KTransformers article (chenxutan.com): 1.2 (256 routed experts, 8 per token, plus
 *         one shared expert), 2.2 (tokens that hit the same expert are batched so that GEMV
 *         becomes GEMM).
 *
 * Conventions for every call
 *   - Pointers are DEVICE pointers unless marked (host); all device buffers are owned by the
 *     caller, must not alias each other, and must be 16-byte aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Calls only
 *     enqueue work on that stream and return; they never allocate, free or synchronise.
 *   - Arguments are validated on the host before anything is enqueued; a failed validation
 *     returns an error and enqueues nothing.  T == 0 is valid and enqueues nothing (after the
 *     scalar arguments are checked, pointers are not looked at and may be NULL).
 *   - MOE_ERR_DEVICE is returned when the HIP runtime reports a launch error; faults that
 *     happen while kernels run surface at the caller's next stream synchronisation.
 *   - bf16 values are passed as their 16-bit patterns (uint16_t).
 *   - The library keeps no state between calls and is safe to call from several threads.
 */
#ifndef LIBMOE_H
#define LIBMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* null pointer, negative size, k outside [1, E], ... */
    MOE_ERR_UNSUPPORTED = 2, /* valid but outside this build's kernel limits (see each call) */
    MOE_ERR_WORKSPACE = 3,   /* workspace smaller than the size query returned */
    MOE_ERR_DEVICE = 4       /* the HIP runtime rejected a launch */
} moe_status;

typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score_fn;

typedef enum {
    MOE_W_FP8_E4M3_B128 = 0, /* OCP E4M3FN codes + one fp32 scale per 128x128 block: w = code * s */
    MOE_W_BF16 = 1,          /* plain bf16 weights, no scales */
    MOE_W_MXFP4_G32 = 2      /* OCP MX FP4: E2M1 codes + one E8M0 scale per 32 inputs: w = code * 2^(s-127) */
} moe_wdtype;

/* Kernel limits of this build. */
#define MOE_MAX_EXPERTS 1024 /* E (and n_groups) */
#define MOE_MAX_TOPK 32      /* k */
#define MOE_MAX_DIM 16384    /* H and I */

/* Weights of n_groups experts of one layer, in nn.Linear layout (rows = outputs, the input
 * dimension contiguous) [OSDI "native FP8 GEMV"; A2 4.2 for the 7168 x 2048 shape]:
 *   w_gate, w_up : [n_groups][I][H]     w_down : [n_groups][H][I]
 *   s_gate, s_up : [n_groups][I/128][H/128] fp32   s_down : [n_groups][H/128][I/128] fp32
 * For MOE_W_BF16 the s_* pointers are ignored (may be NULL).  H and I must be multiples of 128.
 * MOE_W_MXFP4_G32 (4-bit group-quantised weights, 4.25 bits a weight; the pages' quantised
 * comparison model is a 4-bit group-quantised one [OSDI quantised-model results]): w_gate and
 * w_up are bytes [n_groups][I][H/2], w_down [n_groups][H][I/2], each byte holding the codes of
 * two consecutive inputs (the first in the low nibble); s_gate and s_up point to E8M0 bytes
 * [n_groups][I][H/32], s_down to [n_groups][H][I/32] (one per 32 consecutive inputs of a row;
 * 16-byte aligned; the float pointer type is reused for these bytes).  With bf16 activations
 * the codes are expanded exactly to bf16 with their group's scale (few rows per expert: the
 * decode kernel; many: a 4-bit GEMM, for phase 1 with I a multiple of 128 and phase 2 with H a
 * multiple of 256, else the decode kernel).  The FP8-activation calls take them too (W4A8: E2M1
 * weight codes and their E8M0 scales go straight into the scaled matrix instruction, beside the
 * E4M3FN activation codes).
 * The struct itself is read on the host during the call; the arrays it points to are device
 * memory and must stay valid until the enqueued work completes. */
typedef struct {
    int32_t dtype;    /* moe_wdtype */
    int32_t n_groups; /* number of experts in the arrays */
    int32_t H;        /* hidden size (input of gate/up, output of down) */
    int32_t I;        /* expert intermediate size */
    const void* w_gate;
    const void* w_up;
    const void* w_down;
    const float* s_gate;
    const float* s_up;
    const float* s_down;
} moe_expert_weights;

/* Top-k routing [A2 4.1; KT 1.2; OSDI DSLP section "gating"].
 *   scores   : fp32 [T][E] router logits, row-major, finite.
 *   topk_ids : int32 [T][k] out. The k experts with the largest score, in descending order of
 *              (score, then lower expert id); scores compare as floats (-0 == +0).
 *   topk_w   : fp32 [T][k] out. score_fn SOFTMAX: exp(s_j - s_max) / D with D the sum over the
 *              k selected (renorm != 0) or over all E experts (renorm == 0).  SIGMOID:
 *              g_j = 1/(1+exp(-s_j)), divided by the sum of the k selected g (renorm != 0) or
 *              used as is (renorm == 0).  Computed in double, rounded to fp32.
 * Limits: 1 <= k <= min(E, MOE_MAX_TOPK), E <= MOE_MAX_EXPERTS.  Errors: INVALID_ARG for null
 * pointers, T < 0, k outside [1, E], unknown score_fn; UNSUPPORTED beyond the limits. */
moe_status moe_route(const float* scores, int32_t T, int32_t E, int32_t k, int32_t score_fn,
                     int32_t renorm, int32_t* topk_ids, float* topk_w, void* stream);

/* Bytes of device workspace moe_permute needs for T*k assignments over E experts (host output):
 * 0 up to 2048 assignments (one workgroup groups them), else a count table of
 * ceil(T*k / 2048) x E int32 (one row per block of 2048 consecutive assignments).
 * Errors: INVALID_ARG for a null `bytes`, T < 0, k < 1, E < 1; UNSUPPORTED for E >
 * MOE_MAX_EXPERTS or T*k >= 2^31. */
moe_status moe_permute_workspace_size(int32_t T, int32_t k, int32_t E, size_t* bytes);

/* Grouping of the T*k assignments by expert [OSDI DSLP section "sorting"; KT 2.2].
 *   topk_ids : int32 [T][k], each row k distinct ids in [0, E) (as moe_route writes them).
 *   counts   : int32 [E] out, number of assignments per expert.
 *   offsets  : int32 [E+1] out, exclusive prefix sum of counts; offsets[E] = T*k.
 *   perm     : int32 [T*k] out, perm[p] = flat index t*k+j of the p-th assignment in expert
 *              order; stable: within one expert the flat indices ascend (so do the tokens).
 *   inv      : int32 [T*k] out, inv[perm[p]] = p.
 *   ws       : device workspace of ws_bytes >= moe_permute_workspace_size(T, k, E) bytes,
 *              16-byte aligned, owned by the caller (may be NULL when that size is 0).  Its
 *              contents on entry do not matter and are undefined after the call; it must not
 *              be used by other work until the enqueued launches complete.
 * The result is unique and deterministic (no atomics decide an order).  Above 2048 assignments
 * the call is four launches over blocks of 2048 assignments: per-block expert counts into the
 * workspace, one scan of them, per-block stable placement, the inverse.  Ids outside [0, E) are
 * a precondition violation: they are skipped (not counted), and the perm entries past
 * offsets[E] and the inv entries of the skipped assignments are unspecified.
 * Limits: E <= MOE_MAX_EXPERTS, T*k < 2^31.  Errors: INVALID_ARG for null pointers, T < 0,
 * k < 1, E < 1, an unaligned ws; WORKSPACE when ws is NULL or ws_bytes is below the queried
 * size. */
moe_status moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t* counts,
                       int32_t* offsets, int32_t* perm, int32_t* inv, void* ws, size_t ws_bytes,
                       void* stream);

/* moe_permute for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same call and results without
 * the workspace arguments.  The count table lives in a static device array of the library,
 * MOE_PERMUTE_NOALLOC_MAX_BYTES large, which each GPU the library runs on holds from the first
 * call there until the process ends (that first call on a device also looks up the array's
 * address, with the device current; it allocates nothing).  The current device must be the
 * device of `stream` (else INVALID_ARG) and of the buffers.  Every call on one GPU shares that GPU's array, so
 * calls whose launches can overlap on one GPU (other streams, other threads) race and must be
 * ordered by the caller; the array needs no clearing between calls.  Errors as for moe_permute,
 * plus UNSUPPORTED when the table, ceil(T*k / 2048) * E int32 above 2048 assignments, exceeds
 * the array (e.g. more than 2,097,152 assignments at E = 256), and DEVICE when the address
 * lookup fails. */
#define MOE_PERMUTE_NOALLOC_MAX_BYTES (1u << 20)
moe_status moe_permute_noalloc(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                               int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                               void* stream);

/* moe_route followed by moe_permute in one launch, for decode-sized batches (T*k <= 2048): the
 * same outputs, bit for bit, as the two calls [A2 4.1 and OSDI DSLP "gating + sorting"]; one
 * workgroup routes the tokens (a wave per token) and one of its waves then groups the
 * assignments, which saves a launch and a dependent kernel boundary on the decode critical path.
 * Arguments as for the two calls.  Errors as for the two calls, plus UNSUPPORTED for
 * T*k > 2048. */
moe_status moe_route_permute(const float* scores, int32_t T, int32_t E, int32_t k,
                             int32_t score_fn, int32_t renorm, int32_t* topk_ids, float* topk_w,
                             int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                             void* stream);

/* Expert phase 1: gate and up projections with the activated product
 * [OSDI "CPU fine-grained parallelism" (gate and up feed act*mul before down), "native FP8
 * GEMV" (E4M3FN, 128-blocks, post-scaling); KT 2.2 (grouped GEMM)].
 * For every grouped row p (p in [0, T*k)), with expert e such that offsets[e] <= p < offsets[e+1]
 * and token t = perm[p] / k:
 *     g = Wg[e] x_t,  u = Wu[e] x_t   (bf16 x, weights dequantised exactly, fp32 accumulation;
 *                                      FP8 block scales applied to each 128-long partial sum)
 *     h[p][n] = bf16_rne( SiLU(g_n) * u_n ),  SiLU(v) = v / (1 + exp(-v))
 *   x       : bf16 [T][H].
 *   perm    : int32 [T*k] from moe_permute; NULL selects the identity grouping used for the
 *             shared expert (then k must be 1, offsets NULL, w->n_groups 1, and row p = token p).
 *   offsets : int32 [n_groups+1] from moe_permute (n_groups = E); NULL with perm == NULL.
 *             One rank's share under expert parallelism [OSDI SmallEP section] passes the
 *             slice offsets + e0 with w holding experts e0 .. e0 + n_groups - 1 (the same arrays
 *             advanced by e0 experts): only grouped rows [offsets[e0], offsets[e0 + n_groups])
 *             are computed, and the other rows of h are not written.
 *   h       : bf16 [T*k][I] out, in grouped order.
 * Rows of experts with no assignment cost nothing: their weights are not read.
 * Errors: INVALID_ARG for null pointers, T < 0, k < 1, inconsistent identity grouping, unknown
 * dtype; UNSUPPORTED when H or I is not a multiple of 128, H or I > MOE_MAX_DIM, or
 * n_groups > MOE_MAX_EXPERTS. */
moe_status moe_expert_gate_up(const uint16_t* x, int32_t T, int32_t k, const int32_t* perm,
                              const int32_t* offsets, const moe_expert_weights* w, uint16_t* h,
                              void* stream);

/* Expert phase 2: down projection [OSDI "CPU fine-grained parallelism"; "native FP8 GEMV"].
 *     y[p] = Wd[e] h[p]   (fp32 accumulation, block scales after each 128-long partial sum)
 *   h       : bf16 [T*k][I] from moe_expert_gate_up (grouped order).
 *   offsets : as for moe_expert_gate_up (NULL = one group of T rows, k must be 1).
 *   y       : bf16 [T*k][H] out, grouped order (rounded to nearest even).
 * Errors as for moe_expert_gate_up. */
moe_status moe_expert_down(const uint16_t* h, int32_t T, int32_t k, const int32_t* offsets,
                           const moe_expert_weights* w, uint16_t* y, void* stream);

/* The routed experts and the shared expert together [KT 1.2: one shared expert beside the routed
 * ones, used by every token]: moe_expert_gate_up / moe_expert_down over the T*k grouped rows
 * followed by T more rows, row T*k + t being token t for the shared expert `ws` (one expert,
 * n_groups == 1, the same dtype, H and I as w).  At decode sizes (T*k <= 32 * n_groups) each
 * phase is one launch whose grid covers both, so the shared expert needs no stream of its own;
 * otherwise the routed and the shared GEMM run one after the other on `stream`.  The routed rows
 * are those of moe_expert_gate_up / moe_expert_down bit for bit; the shared rows are those of
 * the separate identity-grouped calls bit for bit when T <= 32 or outside decode sizes (the same
 * kernel runs), and otherwise equal up to the order of the fp32 sums (the grid's decode kernel
 * against the separate call's GEMM).
 *   h : bf16 [T*k + T][I] (gate_up out, down in);  y : bf16 [T*k + T][H] out; the shared
 *       expert's output is y + T*k*H (as moe_combine's shared_y).
 * perm and offsets are required (from moe_permute).  Errors as for the separate calls, plus
 * INVALID_ARG for a missing or mismatched ws and UNSUPPORTED when T*k + T >= 2^31. */
moe_status moe_expert_gate_up_shared(const uint16_t* x, int32_t T, int32_t k, const int32_t* perm,
                                     const int32_t* offsets, const moe_expert_weights* w,
                                     const moe_expert_weights* ws, uint16_t* h, void* stream);
moe_status moe_expert_down_shared(const uint16_t* h, int32_t T, int32_t k, const int32_t* offsets,
                                  const moe_expert_weights* w, const moe_expert_weights* ws,
                                  uint16_t* y, void* stream);

/* Bytes of workspace moe_expert_ffn needs (host output): the bf16 intermediate h [T*k][I]. */
moe_status moe_expert_ffn_workspace_size(int32_t T, int32_t k, const moe_expert_weights* w,
                                         size_t* bytes);

/* Both expert phases in one call: h goes to the first T*k*I*2 bytes of `ws` (where it can be
 * read after the stream synchronises), y as in moe_expert_down.  Arguments as for the two
 * phases; ws must hold at least moe_expert_ffn_workspace_size bytes (else ERR_WORKSPACE). */
moe_status moe_expert_ffn(const uint16_t* x, int32_t T, int32_t k, const int32_t* perm,
                          const int32_t* offsets, const moe_expert_weights* w, uint16_t* y,
                          void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- FP8 activation mode (A8W8)
 * [OSDI "native FP8 GEMV", Figures 9-10] quantises weights to E4M3FN with one scale per
 * 128-element block.  This opt-in mode quantises the activations the same way along the
 * contraction dimension, so that both operands of each expert GEMM are E4M3FN (the form the
 * gfx950 FP8 matrix instructions take):
 *   per row, per 128 consecutive values v: e = the smallest integer with max|v| <= 448 * 2^e,
 *   clamped to [-127, 127] (e = 0 for an all-zero block); code = E4M3FN(v * 2^-e), rounded to
 *   nearest even in fp32; the block then stands for code * 2^e exactly.
 * Scales are powers of two (E8M0 numbers), so the codes never overflow and dequantisation is
 * exact; only the rounding to a 3-bit mantissa differs from the bf16 path. */

/* Quantise a bf16 [rows][K] matrix row by row in 128-blocks (as above).
 *   codes     : uint8 [rows][K] out, E4M3FN bit patterns (same layout as x).
 *   exps      : int8 [rows][exp_pitch] out, the block exponents e (scale = 2^e) in the first
 *               K/128 bytes of each row (the rest of the row is not written).
 *   exp_pitch : bytes per exps row, >= K/128; a multiple of 16 for moe_expert_*_a8.
 * Errors: INVALID_ARG for rows < 0, K < 1, exp_pitch < K/128, null or unaligned pointers;
 * UNSUPPORTED when K is not a multiple of 128 or rows * K/128 > 2^27.  rows == 0 enqueues
 * nothing. */
moe_status moe_quantize_act(const uint16_t* x, int32_t rows, int32_t K, uint8_t* codes,
                            int8_t* exps, int32_t exp_pitch, void* stream);

/* Expert phase 1 on FP8 activations: moe_expert_gate_up with x given as moe_quantize_act writes
 * it (x_codes [T][H], x_exps [T][exp_pitch]), i.e. with activations x = code * 2^e.  Both
 * operands go to the scaled matrix instruction with fp32 accumulation; FP8 weights' block
 * scales multiply each 128-long partial sum, MXFP4 weights' E8M0 scales are applied by the
 * instruction with the codes (W4A8); h as in moe_expert_gate_up.
 * For the shapes of the FP8-code GEMM only: UNSUPPORTED when T*k <= 32*n_groups (few rows per
 * expert: moe_expert_ffn_a8 covers those), H > 8192, exp_pitch not a multiple of 16 or above 64,
 * or weights neither MOE_W_FP8_E4M3_B128 nor MOE_W_MXFP4_G32; INVALID_ARG for
 * exp_pitch < H/128; other errors as for moe_expert_gate_up. */
moe_status moe_expert_gate_up_a8(const uint8_t* x_codes, const int8_t* x_exps, int32_t exp_pitch,
                                 int32_t T, int32_t k, const int32_t* perm,
                                 const int32_t* offsets, const moe_expert_weights* w, uint16_t* h,
                                 void* stream);

/* Expert phase 2 on FP8 activations: moe_expert_down with h given quantised (h_codes [T*k][I],
 * h_exps [T*k][exp_pitch], grouped order).  Same limits as moe_expert_gate_up_a8, with I in
 * place of H, and H a multiple of 256. */
moe_status moe_expert_down_a8(const uint8_t* h_codes, const int8_t* h_exps, int32_t exp_pitch,
                              int32_t T, int32_t k, const int32_t* offsets,
                              const moe_expert_weights* w, uint16_t* y, void* stream);

/* Bytes of workspace moe_expert_ffn_a8 needs (host output). */
moe_status moe_expert_ffn_a8_workspace_size(int32_t T, int32_t k, const moe_expert_weights* w,
                                            size_t* bytes);

/* Both expert phases with FP8 activations: x is quantised per token before the gate/up
 * projection and h (after its bf16 rounding) per assignment before the down projection, as
 * above; everything else is as in moe_expert_ffn (same arguments, same y layout, same errors).
 * With many rows per expert both operands of each expert GEMM are FP8 codes and the activation
 * scales are applied by the matrix instruction; otherwise the activations are dequantised
 * exactly to bf16 first (same values up to the order of fp32 sums).  The workspace begins with
 * h (bf16 [T*k][I], before its quantisation); the rest holds the quantised activations.  FP8
 * (MOE_W_FP8_E4M3_B128) and MXFP4 (MOE_W_MXFP4_G32) weights are accepted; bf16 weights are
 * UNSUPPORTED, and so are T*H/128 or T*k*I/128 above 2^27 (the quantiser's limit). */
moe_status moe_expert_ffn_a8(const uint16_t* x, int32_t T, int32_t k, const int32_t* perm,
                             const int32_t* offsets, const moe_expert_weights* w, uint16_t* y,
                             void* ws, size_t ws_bytes, void* stream);

/* Weighted combine [OSDI DSLP section "weighted reduction"; KT 1.2 shared expert]:
 *     out[t][c] = bf16_rne( S[t][c] + sum_{j=0..k-1} w[t][j] * y[inv[t*k+j]][c] )
 * accumulated in fp32 in that order (S first, then j ascending).
 *   y        : bf16 [T*k][H] grouped order (moe_expert_down / moe_expert_ffn).
 *   inv      : int32 [T*k] from moe_permute.
 *   topk_w   : fp32 [T][k] from moe_route.
 *   shared_y : bf16 [T][H], the shared expert's output (weight 1), or NULL for none.
 *   out      : bf16 [T][H] out.
 * Limits: H a multiple of 8.  Errors: INVALID_ARG for null pointers, T < 0, k < 1, H < 1. */
moe_status moe_combine(const uint16_t* y, const int32_t* inv, const float* topk_w,
                       const uint16_t* shared_y, int32_t T, int32_t k, int32_t H, uint16_t* out,
                       void* stream);

/* One rank's local weighted partial reduction under expert parallelism [OSDI SmallEP section:
 * each rank reduces its local experts' outputs to a partial T x H before the partials are
 * exchanged and summed]:
 *     out[t][c] = bf16_rne( S[t][c] + sum_{j : e_begin <= ids[t][j] < e_end} w[t][j] * y[inv[t*k+j]][c] )
 * accumulated in fp32 in that order (S first, then j ascending, skipping other experts); rows
 * of y of skipped assignments are never read (the rank did not compute them).  A token none of
 * whose experts is local gets S (0 without shared_y).
 *   ids      : int32 [T][k] from moe_route; the other arguments as for moe_combine.
 * Errors as for moe_combine, plus INVALID_ARG for a null ids or e_begin > e_end. */
moe_status moe_combine_partial(const uint16_t* y, const int32_t* inv, const int32_t* ids,
                               const float* topk_w, int32_t e_begin, int32_t e_end,
                               const uint16_t* shared_y, int32_t T, int32_t k, int32_t H,
                               uint16_t* out, void* stream);

/* Static, human-readable name of a status code. */
const char* moe_status_string(moe_status s);

#ifdef __cplusplus
}
#endif

#endif /* LIBMOE_H */

// moe_host.h -- host-side helpers of libmoe: argument checks and launch-error mapping.
#pragma once

#include <hip/hip_runtime.h>

#include "libmoe.h"

namespace moe {

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Status of the launches just enqueued (clears the runtime's sticky launch error).
inline moe_status launch_status() {
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int ceil_log2(int v) {
    int b = 0;
    while ((1 << b) < v) ++b;
    return b;
}

// Validation shared by the expert calls.  `rows` is the number of grouped rows (T*k).
inline moe_status check_weights(const moe_expert_weights* w) {
    if (!w) return MOE_ERR_INVALID_ARG;
    if (w->dtype != MOE_W_FP8_E4M3_B128 && w->dtype != MOE_W_BF16 && w->dtype != MOE_W_MXFP4_G32)
        return MOE_ERR_INVALID_ARG;
    if (w->n_groups < 1 || w->H < 1 || w->I < 1) return MOE_ERR_INVALID_ARG;
    if (!w->w_gate || !w->w_up || !w->w_down) return MOE_ERR_INVALID_ARG;
    if (w->dtype != MOE_W_BF16 && (!w->s_gate || !w->s_up || !w->s_down))
        return MOE_ERR_INVALID_ARG;
    if (w->dtype == MOE_W_MXFP4_G32 &&
        (!aligned16(w->s_gate) || !aligned16(w->s_up) || !aligned16(w->s_down)))
        return MOE_ERR_INVALID_ARG;
    if (!aligned16(w->w_gate) || !aligned16(w->w_up) || !aligned16(w->w_down))
        return MOE_ERR_INVALID_ARG;
    if (w->H % 128 != 0 || w->I % 128 != 0) return MOE_ERR_UNSUPPORTED;
    if (w->H > MOE_MAX_DIM || w->I > MOE_MAX_DIM) return MOE_ERR_UNSUPPORTED;
    if (w->n_groups > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

inline moe_status check_grouping(int32_t T, int32_t k, const int32_t* perm, const int32_t* offsets,
                                 const moe_expert_weights* w, bool need_perm) {
    if (T < 0 || k < 1) return MOE_ERR_INVALID_ARG;
    if ((int64_t)T * k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (need_perm ? (perm == nullptr) != (offsets == nullptr) : false) return MOE_ERR_INVALID_ARG;
    if (offsets == nullptr && (k != 1 || w->n_groups != 1)) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

}  // namespace moe

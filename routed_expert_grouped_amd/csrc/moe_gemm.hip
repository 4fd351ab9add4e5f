// moe_gemm.hip -- grouped expert GEMM for many rows per expert (prefill shapes).
#include "libmoe.h"
#include "moe_device.h"
#include "moe_ffn.h"
#include "moe_host.h"

namespace moe {

moe_status launch_gemm(int phase, const GemmArgs& a, hipStream_t st) {
    (void)phase;
    (void)a;
    (void)st;
    return MOE_ERR_UNSUPPORTED;
}

}  // namespace moe

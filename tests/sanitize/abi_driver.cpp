// Drives the argument validation of every libmoe entry point (null pointers, bad sizes, limits,
// short workspaces, T == 0, size queries) in a host-only build with AddressSanitizer and
// UndefinedBehaviorSanitizer.  Every call here returns before anything is enqueued, so no GPU
// is needed and no pointer passed is ever dereferenced on the host or the device.
#include <cstdint>
#include <cstdio>

#include "libmoe.h"

static int failures = 0;

static void expect(moe_status got, moe_status want, const char* what) {
    if (got != want) {
        std::printf("FAIL %s: got %d want %d\n", what, (int)got, (int)want);
        ++failures;
    }
}

int main() {
    // a 16-byte aligned address that no call below may dereference
    void* F = reinterpret_cast<void*>(uintptr_t(0x1000));
    auto* Fi = static_cast<int32_t*>(F);
    auto* Ff = static_cast<float*>(F);
    auto* Fh = static_cast<uint16_t*>(F);
    auto* Fc = static_cast<uint8_t*>(F);
    auto* Fe = static_cast<int8_t*>(F);
    moe_expert_weights w{MOE_W_FP8_E4M3_B128, 4, 256, 128, F, F, F, Ff, Ff, Ff};
    moe_expert_weights ws1 = w;
    ws1.n_groups = 1;
    moe_expert_weights bad = w;
    bad.dtype = 7;
    moe_expert_weights odd = w;
    odd.H = 200;
    size_t n = 0;

    expect(moe_route(nullptr, 4, 8, 2, 0, 1, Fi, Ff, nullptr), MOE_ERR_INVALID_ARG, "route null");
    expect(moe_route(Ff, 4, 8, 9, 0, 1, Fi, Ff, nullptr), MOE_ERR_INVALID_ARG, "route k > E");
    expect(moe_route(Ff, 4, 2048, 2, 0, 1, Fi, Ff, nullptr), MOE_ERR_UNSUPPORTED, "route E");
    expect(moe_route(Ff, 0, 8, 2, 0, 1, Fi, Ff, nullptr), MOE_OK, "route T == 0");

    expect(moe_permute_workspace_size(4096, 8, 256, &n), MOE_OK, "permute ws size");
    expect(n == 16u * 256u * 4u ? MOE_OK : MOE_ERR_DEVICE, MOE_OK, "permute ws bytes");
    expect(moe_permute_workspace_size(4, 2, 8, nullptr), MOE_ERR_INVALID_ARG, "permute ws null");
    expect(moe_permute(Fi, 4096, 8, 256, Fi, Fi, Fi, Fi, nullptr, 0, nullptr), MOE_ERR_WORKSPACE,
           "permute no ws");
    expect(moe_permute(Fi, 4096, 8, 256, Fi, Fi, Fi, Fi, F, n - 1, nullptr), MOE_ERR_WORKSPACE,
           "permute short ws");
    expect(moe_permute(nullptr, 4, 2, 8, Fi, Fi, Fi, Fi, nullptr, 0, nullptr),
           MOE_ERR_INVALID_ARG, "permute null");
    expect(moe_permute(Fi, 0, 2, 8, Fi, Fi, Fi, Fi, nullptr, 0, nullptr), MOE_OK, "permute T 0");
    expect(moe_permute_noalloc(Fi, 300000, 8, 1024, Fi, Fi, Fi, Fi, nullptr), MOE_ERR_UNSUPPORTED,
           "noalloc beyond the array");
    expect(moe_permute_noalloc(nullptr, 4, 2, 8, Fi, Fi, Fi, Fi, nullptr), MOE_ERR_INVALID_ARG,
           "noalloc null");
    expect(moe_route_permute(Ff, 300, 256, 8, 1, 1, Fi, Ff, Fi, Fi, Fi, Fi, nullptr),
           MOE_ERR_UNSUPPORTED, "route_permute above 2048");

    expect(moe_expert_gate_up(Fh, 4, 2, Fi, Fi, &bad, Fh, nullptr), MOE_ERR_INVALID_ARG, "dtype");
    expect(moe_expert_gate_up(Fh, 4, 2, Fi, Fi, &odd, Fh, nullptr), MOE_ERR_UNSUPPORTED, "H % 128");
    expect(moe_expert_gate_up(Fh, 4, 2, nullptr, nullptr, &w, Fh, nullptr), MOE_ERR_INVALID_ARG,
           "identity grouping with k 2");
    expect(moe_expert_gate_up(Fh, 0, 2, Fi, Fi, &w, Fh, nullptr), MOE_OK, "gate_up T 0");
    expect(moe_expert_down(nullptr, 4, 2, Fi, &w, Fh, nullptr), MOE_ERR_INVALID_ARG, "down null");
    expect(moe_expert_gate_up_shared(Fh, 4, 2, Fi, Fi, &w, &w, Fh, nullptr), MOE_ERR_INVALID_ARG,
           "shared with 4 groups");
    expect(moe_expert_down_shared(Fh, 4, 2, nullptr, &w, &ws1, Fh, nullptr), MOE_ERR_INVALID_ARG,
           "shared down without offsets");

    expect(moe_expert_ffn_workspace_size(16, 2, &w, &n), MOE_OK, "ffn ws size");
    expect(moe_expert_ffn(Fh, 16, 2, Fi, Fi, &w, Fh, F, n - 1, nullptr), MOE_ERR_WORKSPACE,
           "ffn short ws");
    expect(moe_expert_ffn_a8_workspace_size(16, 2, &w, &n), MOE_OK, "ffn a8 ws size");
    expect(moe_expert_ffn_a8(Fh, 16, 2, Fi, Fi, &w, Fh, F, n - 1, nullptr), MOE_ERR_WORKSPACE,
           "ffn a8 short ws");
    expect(moe_quantize_act(Fh, 4, 200, Fc, Fe, 16, nullptr), MOE_ERR_UNSUPPORTED, "quant K");
    expect(moe_quantize_act(Fh, 4, 256, Fc, Fe, 1, nullptr), MOE_ERR_INVALID_ARG, "quant pitch");
    expect(moe_expert_gate_up_a8(Fc, Fe, 16, 4, 2, Fi, Fi, &w, Fh, nullptr), MOE_ERR_UNSUPPORTED,
           "a8 few rows");
    expect(moe_expert_down_a8(Fc, Fe, 16, 0, 2, Fi, &w, Fh, nullptr), MOE_OK, "a8 down T 0");
    expect(moe_combine(nullptr, Fi, Ff, nullptr, 4, 2, 256, Fh, nullptr), MOE_ERR_INVALID_ARG,
           "combine null");
    expect(moe_combine_partial(Fh, Fi, Fi, Ff, 5, 2, nullptr, 4, 2, 256, Fh, nullptr),
           MOE_ERR_INVALID_ARG, "partial range");
    for (int s = 0; s < 6; ++s)
        if (moe_status_string((moe_status)s) == nullptr) ++failures;
    std::printf("abi driver: %d failures\n", failures);
    return failures != 0;
}

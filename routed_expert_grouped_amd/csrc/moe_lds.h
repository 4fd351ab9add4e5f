// moe_lds.h -- direct global -> LDS loads (gfx950 global_load_lds_dword[x4]) and the wait
// encoding the kernels that use them count their own loads with.
//
// The loads are inline assembly (they set M0), so the compiler does not track them: a kernel
// waits for them explicitly with s_waitcnt vmcnt(n).  A wave's vector-memory loads complete in
// issue order, so vmcnt(n) means "all but the last n loads issued have landed".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// s_waitcnt immediate that waits until at most n vector-memory loads are outstanding (gfx9
// encoding: vmcnt in bits 3:0 and 15:14; expcnt 6:4 and lgkmcnt 11:8 left at "no wait").
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// One direct global -> LDS load of 16 bytes per lane: lane l's bytes land at lds + 16 * l.
__device__ __forceinline__ void lds_dma16(const void* src, const void* lds) {
    const uint32_t addr = (uint32_t)(size_t)(const __attribute__((address_space(3))) void*)lds;
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(__builtin_amdgcn_readfirstlane(addr))
                 : "memory", "m0");
}

// One direct global -> LDS load of 4 bytes per lane: lane l's dword lands at lds + 4 * l.
__device__ __forceinline__ void lds_dma4(const void* src, const void* lds) {
    const uint32_t addr = (uint32_t)(size_t)(const __attribute__((address_space(3))) void*)lds;
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(src), "s"(__builtin_amdgcn_readfirstlane(addr))
                 : "memory", "m0");
}

// The same two loads with the LDS byte address given directly (a wave-uniform value).
__device__ __forceinline__ void lds_dma16_at(const void* src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory", "m0");
}

__device__ __forceinline__ void lds_dma4_at(const void* src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory", "m0");
}

}  // namespace moe

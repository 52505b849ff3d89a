// lds_dma.hpp -- direct global-to-LDS loads for the batched matrix-core kernels.
//
// global_load_lds_dwordx4 (gfx950) moves 16 bytes per lane from global memory
// straight into LDS: lane i of the wave writes LDS bytes [M0 + 16 i, M0 + 16 i
// + 16), M0 being the wave-uniform LDS address loaded just before.  Nothing
// passes through VGPRs, and with the non-temporal hint a wave streaming 8 rows
// x 128 contiguous bytes per instruction reads HBM at the rate of a plain
// contiguous read (measured on MI355X: 6.9 TB/s against 7.0 TB/s; without the
// hint 6.1 TB/s).
//
// The load is written as inline assembly so that the compiler does not see an
// LDS write: when it does (the builtin), it waits for every outstanding load
// before each LDS read, which serialises a ring of loads in flight.  The asm
// has no register outputs (it writes LDS only), and the caller waits with
// wait_vmcnt<N>() -- vector memory operations complete in issue order, so
// waiting until at most N remain outstanding means every load issued before
// the last N has landed.  Any VMEM instruction the compiler issues in between
// only adds to the operations after a given load, so such a wait stays
// correct (just more conservative).  M0 is set inside the same asm statement;
// the kernels using this issue no other instruction that reads M0.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rt {

// 16 bytes per lane from sbase + voff (bytes) into LDS at lds + 16 * lane.
// (M0 is a reserved register, hence the clobber warning; no compiler-generated
// instruction of the kernels that use this reads M0.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_nt(const void *sbase, int voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
}
// 16 bytes per lane from the lane's own 64-bit address into LDS at lds + 16 * lane.
__device__ __forceinline__ void dma16_nt_addr(const void *addr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(addr), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(N), the other counters untouched (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Position (in 16-byte units) of unit u of row r within a chunk slot of 32 rows
// x 128 bytes is u ^ dma_swizzle(r): every 128-byte row stays whole (the 8
// lanes loading it still read 128 contiguous bytes), and 16 lanes reading one
// unit of 16 consecutive rows -- the MFMA-layout reads -- hit 16 distinct
// 16-byte bank groups (also 8 distinct among any 8 consecutive rows).
__device__ __forceinline__ int dma_swizzle(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// The 32-bit LDS address of a __shared__ / dynamic-LDS pointer, wave-uniform.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)(p));
}

}  // namespace rt

// lds_dma.h -- buffer loads that write LDS directly (gfx950 buffer_load ... lds).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace sscnn {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource of base (stride 0, num_records = bytes): loads at offsets
// outside [0, bytes) return zeros.  Wave-uniform, in scalar registers.
__device__ __forceinline__ i32x4 plane_rsrc(const float* base, int bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
    r.z = __builtin_amdgcn_readfirstlane(bytes);
    r.w = 0x00020000;
    return r;
}

// 16 bytes per lane from the buffer at byte offset voff straight into LDS at
// lds + 16 * lane (lds wave-uniform).  Issued as inline assembly so that the
// compiler does not treat every later LDS read as depending on it (it would
// wait for all outstanding loads first); the kernels wait for these loads
// themselves (s_waitcnt vmcnt) before the barrier that publishes the data.
// The load writes no register.  s_nop: one wait state between writing M0 and
// the load that reads it.
__device__ __forceinline__ void dma16(const i32x4& rs, const float* lds, int voff)
{
    const int l = __builtin_amdgcn_readfirstlane((int)(uint32_t)reinterpret_cast<uintptr_t>(lds));
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                 :: "v"(voff), "s"(l), "s"(rs) : "memory", "m0");
}

// The same load with the LDS destination given as an LDS (address space 3)
// pointer, whose value is the byte address itself; used where the compiler
// fails to select the generic-to-LDS conversion of the form above.
typedef __attribute__((address_space(3))) float lds_float;

__device__ __forceinline__ void dma16_lds(const i32x4& rs, lds_float* lds, int voff)
{
    const int l = __builtin_amdgcn_readfirstlane((int)(uint32_t)reinterpret_cast<uintptr_t>(lds));
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                 :: "v"(voff), "s"(l), "s"(rs) : "memory", "m0");
}

// Wait until at most N of this wave's vector memory operations are
// outstanding (gfx9 s_waitcnt: vmcnt in bits 3:0, expcnt 6:4 and lgkmcnt
// 11:8 left at their maxima, i.e. not waited for).
template <int N>
__device__ __forceinline__ void wait_vmem_le()
{
    static_assert(N >= 0 && N < 16, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(N | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void wait_vmem() { wait_vmem_le<0>(); }

}  // namespace sscnn

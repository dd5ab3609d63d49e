// internal.h -- declarations shared by the host layer (api.cpp) and the
// kernel translation units of libsscnn.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "sscnn.h"

namespace sscnn {

// Workgroup barrier for LDS hand-offs only.  The fences are scoped to the
// workgroup AND to the LDS address space, so they order LDS accesses around
// s_barrier (and wait for this wave's LDS operations) without the global
// memory part of __syncthreads()'s fences, which would also wait for every
// outstanding global load and store -- including prefetches meant to stay in
// flight across the barrier.  Use it only where the waves exchange data
// through LDS and not through global memory.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Read-only data that every lane of a wave reads at the same address (a
// plane's filter taps, a bias): viewed through the constant address space,
// such loads become scalar-cache loads (s_load), which complete on their own
// counter and never wait behind the wave's outstanding vector loads.  Only
// for buffers the kernel does not write.
// A wave-uniform value copied into a vector register (the compiler would
// otherwise keep it in a scalar register and feed it to VALU ops from there).
__device__ __forceinline__ float to_vgpr(float s)
{
    float v;
    asm("v_mov_b32 %0, %1" : "=v"(v) : "s"(s));
    return v;
}

template <typename T>
__device__ __forceinline__ const __attribute__((address_space(4))) T* as_const(const T* p)
{
    return (const __attribute__((address_space(4))) T*)(p);
}

// Workgroups are dealt to the 8 XCDs round-robin (workgroup b runs on XCD
// b % 8, each XCD with its own L2).  xcd_order maps them to logical indices so
// that XCD x takes one contiguous range, [x q + min(x, r), ...) of q or q + 1
// indices (q = G / 8, r = G % 8): workgroups next to each other in logical
// order -- ones that read the same operand tiles -- share an L2.  A bijection
// for any G.
__device__ __forceinline__ int xcd_order(int b, int G)
{
    const int x = b % 8, slot = b / 8;
    const int q = G / 8, r = G % 8;
    return x * q + (x < r ? x : r) + slot;
}

// Everything a kernel needs about one shard's layer, passed by value.
struct Geom {
    int n, ci, co, h, wl, k, stride, pad, groups;
    int ho, wol;         // output rows, output columns owned by the shard
    int hl, hr;          // input halo widths (left, right)
    int ghl, ghr;        // grad_output halo widths (left, right)
    int cig, cog;        // channels per group, in and out
};

// --- halo.hip ---------------------------------------------------------------
// halo[p, r, e] for p < planes, r < rows, e < hl + hr (see sscnn_halo_gather).
hipError_t launch_halo_gather(const float* left, const float* right, int64_t planes, int rows,
                              int width, int hl, int hr, float* halo, hipStream_t st);
// out[i] = sum over parts in order (see sscnn_partial_reduce).
constexpr int kMaxParts = 64;
hipError_t launch_partial_reduce(const float* const* parts, int nparts, int64_t count, float* out,
                                 hipStream_t st);
// out[i] = sum_{s < nsplit} ws[s * count + i], fixed order: the second pass of
// a split reduction.
hipError_t launch_split_reduce(const float* ws, int nsplit, int64_t count, float* out,
                               hipStream_t st);

// --- direct.hip: one thread per output element, any shape ----------------------
hipError_t launch_direct_fwd(const Geom& g, const float* x, const float* xh, const float* w,
                             const float* b, float* y, hipStream_t st);
hipError_t launch_direct_bwd_input(const Geom& g, const float* gy, const float* gyh,
                                   const float* w, float* gx, hipStream_t st);
hipError_t launch_direct_bwd_weight(const Geom& g, const float* x, const float* xh,
                                    const float* gy, float* gw, float* gb, hipStream_t st);

// Push form of the halo exchange for a slice t (planes, rows, width) written by a kernel that does not
// push from its epilogue (halo.hip): its edge columns into the neighbours' halos, zeros on the open sides.
hipError_t launch_push_edges(const float* t, int64_t planes, int rows, int width, int hl, int hr, float* to_left,
                             float* to_right, float* own, hipStream_t st);

// Streaming copy of count floats (stream.hip); src and dst 16-byte aligned.
hipError_t launch_stream_copy(const float* src, float* dst, int64_t count, hipStream_t st);

// No-allocation entry point (noalloc.hip): the device address, on the
// current device, of the library's file-scope scratch array of
// kNoAllocScratchBytes (looked up once per device).
constexpr size_t kNoAllocScratchBytes = SSCNN_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(void** out);

}  // namespace sscnn

// wavesum.h -- fixed-order cross-lane sums of a wave (gfx950 lane swaps and
// DPP), shared by the grad_weight kernels that reduce many per-lane values.
#pragma once

#include "internal.h"

namespace sscnn {
namespace {

// Sum of N per-lane values over the 64 lanes of a wave, leaving one total per
// lane (a reduce-scatter): stage k pairs lanes that differ in one lane bit
// (32, 16, 8, 4, 2, 1) and halves the list, the lower lane of a pair keeping
// the first half of the list and the upper lane the second half.  Bits 5 and
// 4 are exchanged with the gfx950 lane-swap instructions, bits 3..0 with DPP
// (row mirror, half-row mirror, quad permutations; the pairings they make
// split the lanes by the same bits).  wave_sum_index() names the value a lane
// ends with.  Cost ~2.6 VALU per value instead of a 64-step loop per value.
__device__ __forceinline__ float lane_swap_sum(float x, float y, bool bit16)
{
    const auto r = bit16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false)
                         : __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int CTRL>
__device__ __forceinline__ float dpp_pair_sum(float x, float y, bool upper)
{
    const float send = upper ? x : y;
    const float keep = upper ? y : x;
    return keep + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send), CTRL, 0xf, 0xf, false));
}

template <int N, int STAGE>
__device__ __forceinline__ float wave_sum_stage(const float (&v)[N], int lane)
{
    constexpr int H = (N + 1) / 2;
    float u[H];
#pragma unroll
    for (int i = 0; i < H; ++i) {
        const float x = v[i], y = (i + H < N) ? v[i + H] : 0.f;
        if constexpr (STAGE == 0) u[i] = lane_swap_sum(x, y, false);
        else if constexpr (STAGE == 1) u[i] = lane_swap_sum(x, y, true);
        else if constexpr (STAGE == 2) u[i] = dpp_pair_sum<0x140>(x, y, lane & 8);   // row mirror
        else if constexpr (STAGE == 3) u[i] = dpp_pair_sum<0x141>(x, y, lane & 4);   // half-row mirror
        else if constexpr (STAGE == 4) u[i] = dpp_pair_sum<0x4E>(x, y, lane & 2);    // quad [2,3,0,1]
        else u[i] = dpp_pair_sum<0xB1>(x, y, lane & 1);                               // quad [1,0,3,2]
    }
    if constexpr (STAGE == 5) {
        static_assert(H == 1, "64 lanes reduce at most 64 values");
        return u[0];
    } else {
        return wave_sum_stage<H, STAGE + 1>(u, lane);
    }
}

template <int N>
__device__ __forceinline__ float wave_sum_scatter(const float (&v)[N], int lane)
{
    static_assert(N >= 2 && N <= 64, "values per lane");
    return wave_sum_stage<N, 0>(v, lane);
}

// Index of the total that lane holds after wave_sum_scatter<N>, or -1.
template <int N>
__device__ __forceinline__ int wave_sum_index(int lane)
{
    int n[7];
    n[0] = N;
#pragma unroll
    for (int k = 0; k < 6; ++k) n[k + 1] = (n[k] + 1) / 2;
    const int bit[6] = {32, 16, 8, 4, 2, 1};
    int j = 0;
#pragma unroll
    for (int k = 5; k >= 0; --k) {
        if (lane & bit[k]) j += n[k + 1];
        if (j >= n[k]) return -1;
    }
    return j;
}

}  // namespace
}  // namespace sscnn

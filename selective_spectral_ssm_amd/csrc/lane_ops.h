// lane_ops.h -- sums across the lanes of a 64-lane gfx950 wave in VALU instructions only (DPP
// lane moves within rows of 16 lanes, v_permlane16/32_swap across rows), so that a reduction
// costs no LDS round trip.
#pragma once

#include <hip/hip_runtime.h>

namespace essh {

// DPP lane move within a row of 16 lanes (row_mask and bank_mask all on); lanes whose source
// lies outside the row read zero
template <int CTRL>
__device__ __forceinline__ float dpp_zero(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}
constexpr int DPP_SHR1 = 0x111, DPP_SHR2 = 0x112, DPP_SHR4 = 0x114, DPP_SHR8 = 0x118;   // row_shr:n
constexpr int DPP_XOR1 = 0xb1;          // quad_perm [1, 0, 3, 2]
constexpr int DPP_XOR2 = 0x4e;          // quad_perm [2, 3, 0, 1]
constexpr int DPP_HALF_MIRROR = 0x141;  // lane l of each 8-lane half reads lane 7 - l
constexpr int DPP_MIRROR = 0x140;       // lane l of each row reads lane 15 - l

// sum over the 16 lanes of one row group (equal lane >> 4); every lane gets the total (every
// source lane lies inside the row, so the zero-fill form is exact and lets the move fold into
// the add)
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp_zero<DPP_XOR1>(x);
    x += dpp_zero<DPP_XOR2>(x);
    x += dpp_zero<DPP_HALF_MIRROR>(x);
    x += dpp_zero<DPP_MIRROR>(x);
    return x;
}
// sum over the four row groups (equal lane & 15): with the same value in both operands,
// v_permlane16_swap hands each row the row beside it (rows 0 and 1, rows 2 and 3) and
// v_permlane32_swap each half the other half
__device__ __forceinline__ float group_sum4(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// sum over all 64 lanes, in every lane
__device__ __forceinline__ float wave_sum64(float x) { return group_sum4(row_sum16(x)); }
// inclusive suffix sum within each row of 16 lanes (row_shl:n reads lane i + n of the row,
// zero past its end)
__device__ __forceinline__ float row_suffix16(float x) {
    x += dpp_zero<0x101>(x);
    x += dpp_zero<0x102>(x);
    x += dpp_zero<0x104>(x);
    x += dpp_zero<0x108>(x);
    return x;
}

}  // namespace essh

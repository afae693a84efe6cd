// Sums across aligned groups of 8 or 16 lanes on DPP row moves (VALU only, no LDS round
// trip); every lane of a group ends with the same value, since each step adds two operands
// that commute.
#pragma once

namespace treeattn {
namespace lanes {

template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sum over each aligned group of N = 4, 8 or 16 lanes.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(N == 4 || N == 8 || N == 16, "DPP row groups");
    v += dpp_row<0xB1>(v);                             // quad_perm [1, 0, 3, 2]: lane ^ 1
    v += dpp_row<0x4E>(v);                             // quad_perm [2, 3, 0, 1]: lane ^ 2
    if constexpr (N >= 8) v += dpp_row<0x141>(v);      // row_half_mirror: the other quad of the 8
    if constexpr (N >= 16) v += dpp_row<0x140>(v);     // row_mirror: the other half of the 16
    return v;
}

}  // namespace lanes
}  // namespace treeattn

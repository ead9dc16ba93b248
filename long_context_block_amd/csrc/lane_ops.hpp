// lane_ops.hpp — cross-lane exchanges and reductions within a wavefront, without LDS (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace bsa {
namespace lanes {

// Lane exchanges without LDS: DPP within a row of 16 lanes, v_permlane16/32_swap across rows.
// XOR<m>(x) returns x of lane (lane ^ m) for m in {1, 2, 8, 16, 32}; HALF(x) returns x of the
// lane mirrored within its group of 8 (lane ^ 7), which pairs each quad with the other quad of
// the group.
template <int CTRL>
__device__ inline float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
template <int M>
__device__ inline float xor_lane(float x) {
    if constexpr (M == 1) return dpp<0xb1>(x);        // quad_perm [1, 0, 3, 2]
    else if constexpr (M == 2) return dpp<0x4e>(x);   // quad_perm [2, 3, 0, 1]
    else if constexpr (M == 8) return dpp<0x128>(x);  // row_ror:8
    else {
        const uint32_t u = __float_as_uint(x);
        const auto sw = M == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                                : __builtin_amdgcn_permlane32_swap(u, u, false, false);
        // even rows (halves) find the partner in the second result, odd ones in the first
        const bool lo = M == 16 ? ((threadIdx.x >> 4) & 1) == 0 : (threadIdx.x & 32) == 0;
        return __uint_as_float(lo ? sw[1] : sw[0]);
    }
}
__device__ inline float half_mirror(float x) { return dpp<0x141>(x); }  // row_half_mirror

// sum over the N consecutive lanes of an aligned group (N in {8, 16, 32}); every lane gets it
template <int N>
__device__ inline float group_sum(float x) {
    x += xor_lane<1>(x);
    x += xor_lane<2>(x);
    x += half_mirror(x);  // the two quads of a group of 8 are uniform: pair them
    if constexpr (N >= 16) x += xor_lane<8>(x);
    if constexpr (N >= 32) x += xor_lane<16>(x);
    return x;
}

}  // namespace lanes
}  // namespace bsa

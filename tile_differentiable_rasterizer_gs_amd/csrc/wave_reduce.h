// Wave64 reductions shared by the gradient kernels (deterministic association order).
#pragma once

#include "gs_internal.h"

namespace gsr {

template <int kCtrl>
__device__ __forceinline__ float dpp_shifted(float v) {
    // row_shr: lane i reads lane i - n of its 16-lane row, 0 where that leaves the row
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, true));
}

// Sum over the 64 lanes of a wave, returned uniformly (fixed association order).
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_shifted<0x111>(v);
    v += dpp_shifted<0x112>(v);
    v += dpp_shifted<0x114>(v);
    v += dpp_shifted<0x118>(v);   // lane 15 of each row now holds the row's sum
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 47));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
    return (r0 + r1) + (r2 + r3);
}

template <int kCtrl>
__device__ __forceinline__ float dpp_moved(float v) {
    // a lane permutation inside each 16-lane row (every source lane valid)
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, true));
}

// One butterfly level that reduces two values at once: lanes with `mask` clear keep
// a + partner's a, the others b + partner's b.
__device__ __forceinline__ float fold(float a, float b, int mask, bool upper) {
    const float send = upper ? a : b;
    return (upper ? b : a) + __shfl_xor(send, mask);
}

// Sums nine per-lane values over the wave.  On return lane l holds, in `packed`, the
// total of value ((l >> 3) & 1) * 4 + ((l >> 4) & 1) * 2 + ((l >> 5) & 1), and every
// lane holds the total of v[8] in `last`.
__device__ __forceinline__ void reduce9(const float v[9], int lane, float &packed, float &last) {
    const bool u32 = lane & 32, u16 = lane & 16, u8 = lane & 8;
    const float r0 = fold(v[0], v[1], 32, u32), r1 = fold(v[2], v[3], 32, u32);
    const float r2 = fold(v[4], v[5], 32, u32), r3 = fold(v[6], v[7], 32, u32);
    float e = v[8] + __shfl_xor(v[8], 32);
    const float s0 = fold(r0, r1, 16, u16), s1 = fold(r2, r3, 16, u16);
    e += __shfl_xor(e, 16);
    float t = fold(s0, s1, 8, u8);
    e += __shfl_xor(e, 8);
    // the last three levels stay inside groups of 8 lanes: row moves instead of permutes
    // (lane ^ 1, lane ^ 2, then lane i with 7 - i); every lane of a group ends with the same sum
    t += dpp_moved<0xB1>(t);
    e += dpp_moved<0xB1>(e);
    t += dpp_moved<0x4E>(t);
    e += dpp_moved<0x4E>(e);
    t += dpp_moved<0x141>(t);
    e += dpp_moved<0x141>(e);
    packed = t;
    last = e;
}

// The nine totals of reduce9 gathered into lanes 0-8 (lane j < 9 returns value j).
__device__ __forceinline__ float gather9(float packed, float last, int lane) {
    const int j = lane & 7;
    const float mine = __shfl(packed, 32 * (j & 1) + 16 * ((j >> 1) & 1) + 8 * ((j >> 2) & 1));
    return lane < 8 ? mine : last;
}

// Sum over a 16-lane row; the row's last lane (15) holds the result.
__device__ __forceinline__ float row_sum(float v) {
    v += dpp_shifted<0x111>(v);
    v += dpp_shifted<0x112>(v);
    v += dpp_shifted<0x114>(v);
    v += dpp_shifted<0x118>(v);
    return v;
}

}  // namespace gsr

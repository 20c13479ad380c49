// binary32 -> bfloat16 rounding used by every kernel that writes bf16.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace detred {

// binary32 -> bf16 bits, nearest even; NaN -> quiet NaN of the same sign.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace detred

// mfma_bf16.h -- operand types and loads for the bf16 matrix-core kernels of
// the feature path (v_mfma_f32_16x16x32_bf16 and v_mfma_f32_16x16x16_bf16).
//
// Lane layouts, checked with in-bounds probes:
//   16x16x32: A[l % 16][8 (l / 16) + e], B[8 (l / 16) + e][l % 16];
//   16x16x16: A[l % 16][4 (l / 16) + e], B[4 (l / 16) + e][l % 16];
//   both give D[4 (l / 16) + r][l % 16] in register r.
#pragma once

#include "common.h"

namespace sk {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// eight consecutive bf16 values (one 16-byte load; p 16-byte aligned)
__device__ __forceinline__ bf16x8 load8(const uint16_t *p)
{
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(p));
}

// four consecutive bf16 values (one 8-byte load; p 8-byte aligned)
__device__ __forceinline__ i16x4 load4(const uint16_t *p)
{
    return __builtin_bit_cast(i16x4, *reinterpret_cast<const uint2 *>(p));
}

// four fp32 values -> hi and lo bf16 pieces (round to nearest even, the
// hardware conversion), v ~ hi + lo to 16 bits
__device__ __forceinline__ void split2(const float (&v)[4], i16x4 &hi, i16x4 &lo)
{
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const __bf16 h = (__bf16)v[e];
        const __bf16 l = (__bf16)(v[e] - (float)h);
        hi[e] = __builtin_bit_cast(short, h);
        lo[e] = __builtin_bit_cast(short, l);
    }
}

}  // namespace sk

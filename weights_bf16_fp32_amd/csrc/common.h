// Internal definitions shared by the HIP sources of the spectral library
// (gfx950 only).  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef double f64x4_t __attribute__((ext_vector_type(4)));

#define SPEC_DEVICE __device__ __forceinline__

// Exact widening of a bf16 bit pattern (low 16 bits) to f32.
SPEC_DEVICE float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
SPEC_DEVICE float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }
SPEC_DEVICE float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Lower-triangle tile enumeration: linear index t -> (ti, tj) with ti >= tj,
// t = ti (ti + 1) / 2 + tj.
SPEC_DEVICE void tri_tile(int64_t t, int &ti, int &tj)
{
    int i = (int)((__builtin_sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
    while ((int64_t)(i + 1) * (i + 2) / 2 <= t) ++i;
    while ((int64_t)i * (i + 1) / 2 > t) --i;
    ti = i;
    tj = (int)(t - (int64_t)i * (i + 1) / 2);
}

// Remap a linear workgroup id so that consecutive logical tiles land on the
// same XCD (the hardware deals workgroups round-robin over the 8 XCDs, each
// with its own L2): logical = xcd * per_xcd + slot.
// Bijective on [0, nblocks): ids of the complete rounds of 8 are regrouped,
// the ids of a final partial round keep their value.
SPEC_DEVICE int64_t xcd_remap(int64_t bid, int64_t nblocks)
{
    const int64_t nx = 8;
    int64_t full = nblocks / nx;  // complete rounds
    int64_t xcd = bid % nx, slot = bid / nx;
    if (slot >= full) return bid;
    return xcd * full + slot;
}

// Launch error code -> library status (see abi.cpp).
#define SPEC_LAUNCH_CHECK()                                                  \
    do {                                                                     \
        hipError_t e__ = hipGetLastError();                                  \
        if (e__ != hipSuccess) return e__;                                   \
    } while (0)

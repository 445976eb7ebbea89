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

// Lower-triangle tile enumeration in 8 x 8 super-blocks: linear index t ->
// (ti, tj), ti >= tj, nt tiles per side.  The super-blocks (I, J), I >= J, come
// in row order and the tiles of one super-block are consecutive (row order,
// the triangle only on the diagonal), so a run of 64 consecutive indices
// covers a compact block that shares 8 + 8 operand panels.
SPEC_DEVICE void tri_tile_blocked(int64_t t, int nt, int &ti, int &tj)
{
    constexpr int SB = 8;
    const int ns = (nt + SB - 1) / SB;
    for (int I = 0; I < ns; ++I) {
        const int rows = min(SB, nt - SB * I);
        for (int J = 0; J <= I; ++J) {
            const int cols = min(SB, nt - SB * J);
            const int64_t cnt = I == J ? (int64_t)rows * (rows + 1) / 2 : (int64_t)rows * cols;
            if (t < cnt) {
                const int u = (int)t;
                if (I == J) {
                    int r = 0;
                    while ((r + 1) * (r + 2) / 2 <= u) ++r;
                    ti = SB * I + r;
                    tj = SB * J + (u - r * (r + 1) / 2);
                } else {
                    ti = SB * I + u / cols;
                    tj = SB * J + u % cols;
                }
                return;
            }
            t -= cnt;
        }
    }
    ti = tj = 0;
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

// Cross-lane moves without the LDS pipeline: DPP within rows of 16 lanes
// (quad permutes 0xB1 = lane^1 and 0x4E = lane^2, half-row mirror 0x141,
// row mirror 0x140) and the gfx950 row swaps (permlane16/32_swap), which
// exchange the odd rows (16 lanes) or the upper half (32 lanes) of the first
// operand with the even rows or the lower half of the second.
template <int CTRL>
SPEC_DEVICE float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
SPEC_DEVICE double dpp(double x)
{
    const int lo = __double2loint(x), hi = __double2hiint(x);
    return __hiloint2double(__builtin_amdgcn_update_dpp(0, hi, CTRL, 0xF, 0xF, false),
                            __builtin_amdgcn_update_dpp(0, lo, CTRL, 0xF, 0xF, false));
}
// (a, b) -> (a', b'): a' = a in even rows, b from the row below in odd rows;
// b' = a from the row above in even rows, b in odd rows
SPEC_DEVICE void rowswap16(float &a, float &b)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
SPEC_DEVICE void rowswap16(double &a, double &b)
{
    const auto l = __builtin_amdgcn_permlane16_swap((unsigned)__double2loint(a), (unsigned)__double2loint(b), false, false);
    const auto h = __builtin_amdgcn_permlane16_swap((unsigned)__double2hiint(a), (unsigned)__double2hiint(b), false, false);
    a = __hiloint2double((int)h[0], (int)l[0]);
    b = __hiloint2double((int)h[1], (int)l[1]);
}
SPEC_DEVICE void halfswap32(float &a, float &b)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
SPEC_DEVICE void halfswap32(double &a, double &b)
{
    const auto l = __builtin_amdgcn_permlane32_swap((unsigned)__double2loint(a), (unsigned)__double2loint(b), false, false);
    const auto h = __builtin_amdgcn_permlane32_swap((unsigned)__double2hiint(a), (unsigned)__double2hiint(b), false, false);
    a = __hiloint2double((int)h[0], (int)l[0]);
    b = __hiloint2double((int)h[1], (int)l[1]);
}
// x + x[lane ^ 32]
template <typename T>
SPEC_DEVICE T pair32_sum(T x)
{
    T a = x, b = x;
    halfswap32(a, b);
    return a + b;
}
// in lanes 32..63 the value of lane - 32; lanes 0..31 keep their own
template <typename T>
SPEC_DEVICE T from_lower_half(T x)
{
    T a = x, b = x;
    halfswap32(a, b);
    return a;
}
// sum over the 32 lanes of each half-wave
template <typename T>
SPEC_DEVICE T half_sum(T x)
{
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    x += dpp<0x140>(x);
    T a = x, b = x;
    rowswap16(a, b);
    return a + b;
}

SPEC_DEVICE float readlane_t(float x, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
SPEC_DEVICE double readlane_t(double x, int l)
{
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(x), l),
                            __builtin_amdgcn_readlane(__double2loint(x), l));
}
SPEC_DEVICE float readlane0(float x) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)); }
SPEC_DEVICE double readlane0(double x)
{
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(x), 0), __builtin_amdgcn_readlane(__double2loint(x), 0));
}

// Orders LDS traffic between the lanes of one wave (a wave's LDS operations
// complete in program order; this keeps the compiler from moving them).
SPEC_DEVICE void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Launch error code -> library status (see abi.cpp).
#define SPEC_LAUNCH_CHECK()                                                  \
    do {                                                                     \
        hipError_t e__ = hipGetLastError();                                  \
        if (e__ != hipSuccess) return e__;                                   \
    } while (0)

// Marchenko-Pastur distribution function with sigma^2 = 1 and ratio 0 < c <= 1
// in the angle phi of lambda = (1 + c) - 2 sqrt(c) cos(phi): the antiderivative
// of h^2 sin^2(phi) / (2 pi c lambda(phi)), h = 2 sqrt c, with
// kappa = (1 + sqrt c) / (1 - sqrt c) ("Random matrix theory spectral methods"
// page, section 2.1, the MP density).  F(0) = 0, F(pi) = 1.
__device__ inline double mp_cdf_phi(double phi, double c)
{
    const double sc = sqrt(c);
    double third = 0.0;
    if (c < 1.0) {
        const double kappa = (1.0 + sc) / (1.0 - sc);
        third = ((1.0 - c) / c) * atan2(kappa * sin(0.5 * phi), cos(0.5 * phi));
    }
    return (sin(phi) / sc + (1.0 + c) * phi / (2.0 * c) - third) / M_PI;
}

// Shared device helpers for the gfx950 Muon bank kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mb {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

#define MB_LDS __attribute__((address_space(3)))
// LDS pointer from a generic pointer into LDS: the low 32 bits of such a pointer are its LDS byte
// address.  (An address-space cast would add a null check, which some instantiations of the tile
// turned into an instruction the backend rejects.)
template <class T>
__device__ __forceinline__ MB_LDS T* lds_ptr(const void* p) {
    return (MB_LDS T*)(uint32_t)(uintptr_t)p;
}
typedef MB_LDS uint16_t lds_u16;

// bf16 bits -> float (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// float -> bf16 bits, round to nearest even (finite inputs; inf stays inf).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t b = __float_as_uint(f);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

// Two floats -> packed bf16 bits (first in the low half), round to nearest even, with the
// gfx950 conversion instruction (v_cvt_pk_bf16_f32).  Identical to f32_to_bf16_rne on every
// finite input, denormals included, in the default (denormal-preserving) float mode.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Knuth's TwoSum: the exact error of s = RN(a + b), so that a + b = s + err.
__device__ __forceinline__ double two_sum_err(double a, double b, double s) {
    double bb = s - a;
    return (a - (s - bb)) + (b - bb);
}

// Round-to-odd of the exact sum a + b to binary64: if the sum is not
// representable, the neighbour with an odd last bit.  A later single
// round-to-nearest to any format with at least two fewer significand bits
// then equals the correctly rounded exact sum (Boldo and Melquiond, "Emulation
// of FMA and correctly rounded sums: proved algorithms using rounding to odd").
__device__ __forceinline__ double sum_round_odd(double a, double b) {
    double s = a + b;
    double e = two_sum_err(a, b, s);
    if (e != 0.0) {
        unsigned long long bits = (unsigned long long)__double_as_longlong(s);
        if ((bits & 1ull) == 0ull) {
            // the exact value lies between s and its neighbour in the direction of e
            bits += ((e > 0.0) == (s > 0.0)) ? 1ull : ~0ull;
            s = __longlong_as_double((long long)bits);
        }
    }
    return s;
}

// Round a binary64 value that is already round-to-odd at 53 bits to float32,
// round-to-nearest-even (53 >= 24 + 2, so this is the correct rounding of the
// exact value).
__device__ __forceinline__ float odd53_to_f32(double s) { return (float)s; }

// RN_bf16 of the exact sum a + b of two binary64 values (correct rounding, ties to even), without
// a round-to-odd pass through binary64 and float32.  With s = RN53(a + b)
// and f = RN32(s): a bf16 rounding boundary strictly between the exact sum and s, or between s
// and f, would be a representable value closer than the one rounded to, so RN_bf16(f) is the
// answer unless f is a bf16 midpoint.  Then the side of f the exact sum lies on decides: the
// side of s if s != f (it is the same side), else the sign of the TwoSum error (zero: an
// exact tie, to even).  Only lanes at a midpoint reach the slower part.
__device__ __forceinline__ uint16_t sum_to_bf16(double a, double b) {
    const double s = a + b;
    const float f = (float)s;
    const uint32_t fb = __float_as_uint(f);
    const double fd = (double)f;
    const bool mid = (fb & 0xFFFFu) == 0x8000u;
    // selects, not branches, for the common cases: midpoints of f are frequent enough (a few in a
    // hundred sums) that a branch on them would be taken by almost every wavefront
    uint32_t h = f32_to_bf16_rne(f);
    const uint32_t side = (fb >> 16) + (fabs(s) > fabs(fd) ? 1u : 0u);
    h = (mid && fd != s) ? side : h;
    if (mid && fd == s) {
        // s itself is a midpoint (rare): the TwoSum error decides; zero is an exact tie
        const double e = two_sum_err(a, b, s);
        if (e != 0.0) h = (fb >> 16) + (((e > 0.0) == (s > 0.0)) ? 1u : 0u);
    }
    return (uint16_t)h;
}

// Per-slot live word of the Newton-Schulz kernels: 0 for an all-zero slot; bit 0 for a live slot; bit 1
// when the first round reads the pre-scaled copy X0 = u * 2^k (k in bits 8 and up, biased) instead of u.
constexpr int kLiveBit = 1;
constexpr int kPrescaledBit = 2;
constexpr int kPrescaleShift = 8;
constexpr int kPrescaleBias = 512;
__host__ __device__ __forceinline__ int prescale_exp(int word) { return (word >> kPrescaleShift) - kPrescaleBias; }

// Wavefront (64-lane) sum of doubles with a fixed reduction tree.
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Wavefront (64-lane) sum with a fixed reduction tree.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

}  // namespace mb

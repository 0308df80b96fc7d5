// codec.hpp -- bf16 / e4m3 conversions used by the HIP kernels (gfx950).
//
// The fp8 format is OCP E4M3 ("fn", max 448), the one gfx950's conversion
// instructions implement.  Narrowing to e4m3 is: clamp to [-448, 448] in fp32,
// then v_cvt_pk_fp8_f32, which rounds to nearest even, keeps the sign of zero
// and handles the subnormal range; narrowing to bf16 is v_cvt_pk_bf16_f32
// (round to nearest even).  Both instructions were checked against a software
// round-to-nearest-even encoder on every one of the 2^32 fp32 inputs.
//
// wire_quotient() is shared with a host build: its division is checked on the
// CPU against IEEE fp32 division for every (x, amax) pair of bf16 values the
// per-row quantizer can meet.
#pragma once
#include <stdint.h>

#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)
#define BS_HD __host__ __device__
#else
#define BS_HD
#endif

#include <math.h>

// The quotient x / s rounded to nearest fp32, for a per-row (or per-block)
// scale s > 0, computed as RN32( RN64( x * R ) ) with R = RN64(1 / s), the
// reciprocal taken once per row in fp64.  This equals the IEEE fp32 quotient:
// RN64 errors total below 2^-51 relative, while a quotient of two fp32 values
// that is not itself a representable midpoint stays at least 2^-49 (relative)
// away from every fp32 rounding midpoint, and a normal quotient is never
// exactly a midpoint (its odd significand would need 25 bits).  Quotients in
// the fp32 subnormal range are below every e4m3 code, so any rounding there
// yields code 0 with the right sign.  The plain fp32 reciprocal-and-correct
// form is NOT exact and is not used.
BS_HD inline float wire_quotient(float x, double R) { return (float)((double)x * R); }

#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)
#include <hip/hip_runtime.h>

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// two fp32 -> packed bf16 pair (a in the low half), round to nearest even
__device__ inline uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ inline float clamp448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

// four fp32 -> four e4m3 codes in one dword (a in the lowest byte)
__device__ inline uint32_t pack_e4m3x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), w, true);
    return (uint32_t)w;
}

#endif

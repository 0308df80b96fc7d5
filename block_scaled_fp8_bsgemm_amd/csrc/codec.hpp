// codec.hpp -- bf16 / e4m3 conversions used by the HIP kernels (gfx950).
//
// The fp8 format is OCP E4M3 ("fn", max 448), the one gfx950's conversion
// instructions implement.  Narrowing to e4m3 is v_cvt_pk_fp8_f32, which rounds
// to nearest even, keeps the sign of zero and handles the subnormal range (on
// inputs within +-(448 + 2^-15), see pack_e4m3x4); narrowing to bf16 is
// v_cvt_pk_bf16_f32 (round to nearest even).  Both instructions were checked
// against a software round-to-nearest-even encoder on every fp32 input in
// those ranges.
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

// four fp32 -> four e4m3 codes in one dword (a in the lowest byte), by
// v_cvt_pk_fp8_f32 (round to nearest even), for inputs of magnitude below 464
// (the midpoint between 448 and the next e4m3 step, past which the
// instruction gives NaN).  The quantizers of bf16 data meet only such
// quotients: with s = RN32(amax / 448) and |x| <= amax, x / s exceeds 448 only
// by s's rounding, at most one fp32 step while s is normal and at most
// 448.88 for the subnormal s that the smallest bf16 amax values give (checked
// for every bf16 amax on the CPU); the E8M0 path scales by an exact power of
// two chosen so that amax fits 448.  Those values round to the +-448 codes
// (device test with rows whose amax puts the quotient there).  Dropping the
// clamp took 1.8 us off the row quantizer's 11.3.
__device__ inline uint32_t pack_e4m3x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// The same after clamping to [-448, 448], for the fp32-input block quantizer:
// an fp32 amax below 448 * 2^-140 gives a subnormal s whose rounding can put
// x / s far past 464 (a saturating encode maps it to +-448).
__device__ inline float clamp448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }
__device__ inline uint32_t pack_e4m3x4_sat(float a, float b, float c, float d) {
    return pack_e4m3x4(clamp448(a), clamp448(b), clamp448(c), clamp448(d));
}

#endif

// stream.hip -- the HBM-bound kernels of the wo_b hot path (gfx950):
//
//   band_reduce  fp32 sum of P bf16 partial bands -> bf16 band
//                ("MORI GEMM + All-Reduce Benchmark", "Where the time goes",
//                row reduce; "The fp8 wire": fp32 accumulation, bf16 output;
//                "Negative results": a flat grid over 16-byte packs, each
//                pack streamed through all P source slices at once)
//   rowq_e4m3    per-row e4m3 quantize, one fp32 scale per row ("The fp8
//                wire"; "Negative results": the row amax forces a row-wide
//                reduction, so the quantizer is its own kernel)
//   rowdq_e4m3   per-row dequantize to bf16 ("Where the time goes",
//                dequantize; "Who moves the gather")
//   blockq_e4m3  fp32 operand -> e4m3 + fp32 scale per 1x128 or 128x128 block
//                (the blockscale operand format of "Running the benchmark")
//   mxq_e4m3     bf16 -> e4m3 + E8M0 scale per 1x32 block (the mxfp8 operand
//                format of sglang PR 43480, "Not in this PR")
//   actq_e4m3    bf16 activation -> e4m3 + fp32 scale per 1x128 block (sglang
//                PR 43480, "Numerics, measured where the path engages": a
//                plain bf16 layer input is quantised by the layer itself)
//
// All of them move 16-byte vectors with coalesced, unit-stride accesses and
// keep each lane's data in registers between the load and the store.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "codec.hpp"
#include "launch.hpp"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ band reduce --

struct PartPtrs {
    const u32x4 *p[16];
};

// Flat grid over 16-byte packs (8 bf16): each lane takes two packs 256
// apart and issues all 2P loads (non-temporal: every part is read once)
// before the fp32 adds, which run in part order from +0; the outputs are
// written non-temporally.
template <int P>
__device__ __forceinline__ u32x4 reduce_pack(const u32x4 (&w)[P]) {
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; e++) acc[e] = 0.0f;
#pragma unroll
    for (int p = 0; p < P; p++) {
#pragma unroll
        for (int e = 0; e < 4; e++) {
            acc[2 * e] += bf16_lo(w[p][e]);
            acc[2 * e + 1] += bf16_hi(w[p][e]);
        }
    }
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; e++) o[e] = pack_bf16x2(acc[2 * e], acc[2 * e + 1]);
    return o;
}

template <int P>
__global__ void __launch_bounds__(256)
band_reduce_kernel(PartPtrs parts, u32x4 *__restrict__ out, int64_t nvec) {
    const int64_t stride = (int64_t)gridDim.x * 512;
    for (int64_t v0 = (int64_t)blockIdx.x * 512 + threadIdx.x; v0 < nvec; v0 += stride) {
        const int64_t v1 = v0 + 256;
        const bool two = v1 < nvec;
        u32x4 w0[P], w1[P];
#pragma unroll
        for (int p = 0; p < P; p++) w0[p] = __builtin_nontemporal_load(parts.p[p] + v0);
        if (two) {
#pragma unroll
            for (int p = 0; p < P; p++) w1[p] = __builtin_nontemporal_load(parts.p[p] + v1);
        }
        __builtin_nontemporal_store(reduce_pack<P>(w0), out + v0);
        if (two) __builtin_nontemporal_store(reduce_pack<P>(w1), out + v1);
    }
}

template <int P>
int launch_reduce_p(const PartPtrs &pp, u32x4 *out, int64_t nvec, hipStream_t stream) {
    int64_t blocks = (nvec + 511) / 512;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    return bs_enqueue(band_reduce_kernel<P>, dim3((unsigned)blocks), dim3(256), stream, pp, out,
                      nvec);
}

// ----------------------------------------------------------- row quantize --

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// 8 bf16 (one 16-byte pack) -> 8 e4m3 codes with per-row reciprocal R
__device__ __forceinline__ u32x2 quant_pack(u32x4 w, double R) {
    u32x2 o;
    o[0] = pack_e4m3x4(wire_quotient(bf16_lo(w[0]), R), wire_quotient(bf16_hi(w[0]), R),
                      wire_quotient(bf16_lo(w[1]), R), wire_quotient(bf16_hi(w[1]), R));
    o[1] = pack_e4m3x4(wire_quotient(bf16_lo(w[2]), R), wire_quotient(bf16_hi(w[2]), R),
                      wire_quotient(bf16_lo(w[3]), R), wire_quotient(bf16_hi(w[3]), R));
    return o;
}

__device__ __forceinline__ float pack_absmax(u32x4 w) {
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; e++) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[e])), fabsf(bf16_hi(w[e]))));
    return m;
}

// One wavefront per row (four rows per workgroup): each lane loads its CPL
// packs of the row at once (non-temporal: the band is read once), the row
// amax is a shuffle reduction inside the wavefront (no LDS, no barrier), and
// the codes are written from registers.  Row length N <= 512 * CPL.  FULL
// says the row is exactly 64 * CPL packs: then no access needs a lane guard
// and the compiler may interleave the conversions with the stores, which is
// worth about 2 us on a [2048, 7168] band (the guarded form fences every pack
// into its own exec-masked block and runs load, convert and store as three
// phases one after the other).
template <int CPL, bool FULL>
__global__ void __launch_bounds__(256)
rowq_kernel(const u32x4 *__restrict__ x, u32x2 *__restrict__ q, float *__restrict__ scale,
            int64_t rows, int nch) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const u32x4 *xr = x + row * nch;
    u32x4 v[CPL];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; i++) {
        const int c = lane + 64 * i;
        if (FULL || c < nch) v[i] = __builtin_nontemporal_load(xr + c);
    }
#pragma unroll
    for (int i = 0; i < CPL; i++) {
        const int c = lane + 64 * i;
        if (FULL || c < nch) amax = fmaxf(amax, pack_absmax(v[i]));
    }
    // after the butterfly every lane holds the row amax; readfirstlane makes
    // the scale, and the zero-row branch below, visibly wave-uniform
    const float s = __builtin_bit_cast(
        float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, wave_max(amax) / 448.0f)));
    if (lane == 0) scale[row] = s;
    u32x2 *qr = q + row * nch;
    if (s != 0.0f) {
        const double R = 1.0 / (double)s;
#pragma unroll
        for (int i = 0; i < CPL; i++) {
            const int c = lane + 64 * i;
            if (FULL || c < nch) __builtin_nontemporal_store(quant_pack(v[i], R), qr + c);
        }
    } else {
        // an all-zero row has scale 0 and all-zero codes (+0, also for -0 inputs)
#pragma unroll
        for (int i = 0; i < CPL; i++) {
            const int c = lane + 64 * i;
            if (FULL || c < nch) __builtin_nontemporal_store((u32x2){0u, 0u}, qr + c);
        }
    }
}

// Fused reduce + row quantize (the pages' "Negative results" experiment): one
// 256-lane workgroup per row of the reduced band, lane t owning packs t,
// t + 256, t + 512, t + 768 of the row (N <= 8192).  The parts are read G at
// a time with every load of the group in flight before the adds (non-temporal:
// each part is read once), and each lane sums its packs over the P parts in
// part order from +0 in fp32; the sums are rounded to bf16 as band_reduce
// does, the row amax goes through one LDS exchange between the four
// wavefronts, and the bf16 values are quantized exactly as rowq_kernel does.
// The result equals rowq(band_reduce(parts)) bit for bit, without the bf16
// band in memory.
constexpr int BRQ_CPT = 4;   // packs per lane: rows of up to 4 * 256 packs
template <int G>
__global__ void __launch_bounds__(256)
band_rowq_kernel(PartPtrs parts, int P, u32x2 *__restrict__ q, float *__restrict__ scale, int nch) {
    __shared__ float red[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t row = blockIdx.x;
    const int64_t base = row * nch;
    float acc[BRQ_CPT][8];
#pragma unroll
    for (int i = 0; i < BRQ_CPT; i++)
#pragma unroll
        for (int e = 0; e < 8; e++) acc[i][e] = 0.0f;
    for (int p0 = 0; p0 < P; p0 += G) {
        u32x4 w[G][BRQ_CPT];
#pragma unroll
        for (int g = 0; g < G; g++)
#pragma unroll
            for (int i = 0; i < BRQ_CPT; i++) {
                const int c = tid + 256 * i;
                if (p0 + g < P && c < nch) w[g][i] = __builtin_nontemporal_load(parts.p[p0 + g] + base + c);
            }
#pragma unroll
        for (int g = 0; g < G; g++)
#pragma unroll
            for (int i = 0; i < BRQ_CPT; i++) {
                const int c = tid + 256 * i;
                if (p0 + g < P && c < nch) {
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        acc[i][2 * e] += bf16_lo(w[g][i][e]);
                        acc[i][2 * e + 1] += bf16_hi(w[g][i][e]);
                    }
                }
            }
    }
    u32x4 v[BRQ_CPT];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < BRQ_CPT; i++) {
        const int c = tid + 256 * i;
#pragma unroll
        for (int e = 0; e < 4; e++) v[i][e] = pack_bf16x2(acc[i][2 * e], acc[i][2 * e + 1]);
        if (c < nch) amax = fmaxf(amax, pack_absmax(v[i]));
    }
    amax = wave_max(amax);
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = amax / 448.0f;
    if (tid == 0) scale[row] = s;
    u32x2 *qr = q + base;
    const double R = s != 0.0f ? 1.0 / (double)s : 0.0;
#pragma unroll
    for (int i = 0; i < BRQ_CPT; i++) {
        const int c = tid + 256 * i;
        if (c < nch) {
            const u32x2 o = s != 0.0f ? quant_pack(v[i], R) : (u32x2){0u, 0u};
            __builtin_nontemporal_store(o, qr + c);
        }
    }
}

// Rows longer than the register-resident variant: amax pass, then a second
// pass that re-reads the row (from L2) and encodes it.
__global__ void __launch_bounds__(256)
rowq_long_kernel(const u32x4 *__restrict__ x, u32x2 *__restrict__ q, float *__restrict__ scale,
                 int64_t rows, int nch) {
    __shared__ float red[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const u32x4 *xr = x + row * nch;
        float amax = 0.0f;
        for (int c = tid; c < nch; c += 256) amax = fmaxf(amax, pack_absmax(xr[c]));
        amax = wave_max(amax);
        if (lane == 0) red[wave] = amax;
        __syncthreads();
        amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        __syncthreads();
        const float s = amax / 448.0f;
        if (tid == 0) scale[row] = s;
        u32x2 *qr = q + row * nch;
        if (s == 0.0f) {
            for (int c = tid; c < nch; c += 256) qr[c] = (u32x2){0u, 0u};
            continue;
        }
        const double R = 1.0 / (double)s;
        for (int c = tid; c < nch; c += 256) qr[c] = quant_pack(xr[c], R);
    }
}

// --------------------------------------------------------- row dequantize --

// 8 codes -> 8 bf16: exact decode, one fp32 multiply, round to nearest even
__device__ __forceinline__ u32x4 dequant_pack(u32x2 c, float s) {
    const v2f a = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[0], false);
    const v2f b = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[0], true);
    const v2f d = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[1], false);
    const v2f e = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[1], true);
    u32x4 o;
    o[0] = pack_bf16x2(a[0] * s, a[1] * s);
    o[1] = pack_bf16x2(b[0] * s, b[1] * s);
    o[2] = pack_bf16x2(d[0] * s, d[1] * s);
    o[3] = pack_bf16x2(e[0] * s, e[1] * s);
    return o;
}

// A flat grid over the packs of 8 codes (row = pack / nch), two packs per
// lane with both loads issued before the stores; non-temporal loads and
// stores (every byte is touched once).  IDX is the pack index type.
template <typename IDX>
__global__ void __launch_bounds__(256)
rowdq_kernel(const u32x2 *__restrict__ q, const float *__restrict__ scale, u32x4 *__restrict__ y,
             IDX npack, IDX nch) {
    const IDX stride = (IDX)gridDim.x * 256;
    for (IDX v0 = (IDX)blockIdx.x * 256 + threadIdx.x; v0 < npack; v0 += 2 * stride) {
        const IDX v1 = v0 + stride;
        const u32x2 c0 = __builtin_nontemporal_load(q + v0);
        const float s0 = scale[v0 / nch];
        u32x2 c1 = {0u, 0u};
        float s1 = 0.0f;
        if (v1 < npack) {
            c1 = __builtin_nontemporal_load(q + v1);
            s1 = scale[v1 / nch];
        }
        __builtin_nontemporal_store(dequant_pack(c0, s0), y + v0);
        if (v1 < npack) __builtin_nontemporal_store(dequant_pack(c1, s1), y + v1);
    }
}

// -------------------------------------------------------- block quantizer --

__device__ __forceinline__ float pack_absmax_f32(u32x4 w) {
    return fmaxf(fmaxf(fabsf(__uint_as_float(w[0])), fabsf(__uint_as_float(w[1]))),
                 fmaxf(fabsf(__uint_as_float(w[2])), fabsf(__uint_as_float(w[3]))));
}

__device__ __forceinline__ uint32_t quant4_f32(u32x4 w, double R) {
    return pack_e4m3x4_sat(wire_quotient(__uint_as_float(w[0]), R), wire_quotient(__uint_as_float(w[1]), R),
                       wire_quotient(__uint_as_float(w[2]), R), wire_quotient(__uint_as_float(w[3]), R));
}

// 1x128 blocks: 16 lanes per block, 8 consecutive fp32 per lane.  Blocks are
// contiguous in a row-major [rows, cols] matrix with cols % 128 == 0, so the
// flat block index is also the index into the [rows, cols/128] scale array.
__global__ void __launch_bounds__(256)
blockq_1x128_kernel(const u32x4 *__restrict__ x, u32x2 *__restrict__ q, float *__restrict__ scale,
                    int64_t nblocks) {
    const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t blk = gt >> 4;
    const bool live = blk < nblocks;
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (live) {
        a = x[gt * 2];
        b = x[gt * 2 + 1];
    }
    float amax = fmaxf(pack_absmax_f32(a), pack_absmax_f32(b));
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if (!live) return;
    const float s = amax / 448.0f;
    if ((threadIdx.x & 15) == 0) scale[blk] = s;
    u32x2 o = (u32x2){0u, 0u};
    if (s != 0.0f) {
        const double R = 1.0 / (double)s;
        o[0] = quant4_f32(a, R);
        o[1] = quant4_f32(b, R);
    }
    q[gt] = o;
}

// 128x128 blocks: one 256-lane workgroup per block; lane t covers row t/2 of
// the block and 64 consecutive columns.
__global__ void __launch_bounds__(256)
blockq_128x128_kernel(const float *__restrict__ x, uint8_t *__restrict__ q,
                      float *__restrict__ scale, int64_t rows, int64_t cols) {
    __shared__ float red[4];
    const int64_t nbc = cols / 128;
    const int64_t br = blockIdx.x / nbc, bc = blockIdx.x % nbc;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t r = br * 128 + (tid >> 1);
    const int64_t c0 = bc * 128 + (tid & 1) * 64;
    const bool live = r < rows;
    u32x4 v[16];
    float amax = 0.0f;
    const u32x4 *xr = (const u32x4 *)(x + r * cols + c0);
#pragma unroll
    for (int i = 0; i < 16; i++) {
        v[i] = live ? xr[i] : (u32x4){0u, 0u, 0u, 0u};
        amax = fmaxf(amax, pack_absmax_f32(v[i]));
    }
    amax = wave_max(amax);
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = amax / 448.0f;
    if (tid == 0) scale[blockIdx.x] = s;
    if (!live) return;
    u32x4 *qr = (u32x4 *)(q + r * cols + c0);
    const double R = s != 0.0f ? 1.0 / (double)s : 0.0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        u32x4 o = {0u, 0u, 0u, 0u};
        if (s != 0.0f) {
            o[0] = quant4_f32(v[4 * i + 0], R);
            o[1] = quant4_f32(v[4 * i + 1], R);
            o[2] = quant4_f32(v[4 * i + 2], R);
            o[3] = quant4_f32(v[4 * i + 3], R);
        }
        qr[i] = o;
    }
}

// ------------------------------------------------- activation quantizer --

// bf16 [rows, cols] in 1x128 blocks: each lane takes two adjacent 16-byte
// packs (16 values), 8 lanes per block, so a block's amax is an 8-lane
// shuffle reduction and each lane writes 16 bytes of codes.  Blocks are
// contiguous (cols % 128 == 0), so the flat block index is also the index
// into the [rows, cols/128] scale array.  Non-temporal loads and stores.
__global__ void __launch_bounds__(256)
actq_1x128_kernel(const u32x4 *__restrict__ x, u32x4 *__restrict__ q, float *__restrict__ scale,
                  uint64_t npair) {
    const uint64_t stride = (uint64_t)gridDim.x * 256;
    // every lane of an 8-lane block group has the same v < npair: npair and
    // the stride are multiples of 8
    for (uint64_t v = (uint64_t)blockIdx.x * 256 + threadIdx.x; v < npair; v += stride) {
        const u32x4 a = __builtin_nontemporal_load(x + 2 * v);
        const u32x4 b = __builtin_nontemporal_load(x + 2 * v + 1);
        float amax = fmaxf(pack_absmax(a), pack_absmax(b));
#pragma unroll
        for (int off = 4; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
        const float s = amax / 448.0f;
        if ((v & 7) == 0) scale[v >> 3] = s;
        const double R = s != 0.0f ? 1.0 / (double)s : 0.0;
        const u32x2 o0 = s != 0.0f ? quant_pack(a, R) : (u32x2){0u, 0u};
        const u32x2 o1 = s != 0.0f ? quant_pack(b, R) : (u32x2){0u, 0u};
        __builtin_nontemporal_store((u32x4){o0[0], o0[1], o1[0], o1[1]}, q + v);
    }
}

// ------------------------------------------------------ mxfp8 quantizer --

// bf16 [rows, cols] in 1x32 blocks: one 16-byte pack (8 values) per lane, 4
// lanes per block (amax by two shuffles).  The block scale is 2^k with k the
// smallest integer such that amax <= 448 * 2^k, read off amax's IEEE bits:
// amax = 1.f * 2^E fits under 1.75 * 2^(E+1) = 448 * 2^(E-7) exactly when
// 1.f <= 1.75, i.e. when the fraction bits are <= 0x600000, else k = E - 7.
// The codes are e4m3 RNE of x * 2^-k (an exact scaling; results below the
// fp32 normal range encode to zero either way).  A zero block gets scale
// byte 0 and codes 0x00.  Two packs per lane, non-temporal loads and stores.
__device__ __forceinline__ void mxq_pack(u32x4 w, u32x2 *q, uint8_t *e, uint64_t v, bool live) {
    float amax = live ? pack_absmax(w) : 0.0f;
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    if (!live) return;
    const uint32_t bits = __float_as_uint(amax);
    const int ef = (int)(bits >> 23);
    int k = ef == 0 ? -127 : (ef - 127) - ((bits & 0x7FFFFFu) > 0x600000u ? 7 : 8);
    if (k < -127) k = -127;
    const bool zero = amax == 0.0f;
    if ((v & 3) == 0) e[v >> 2] = zero ? (uint8_t)0 : (uint8_t)(k + 127);
    const float r = __uint_as_float((uint32_t)(127 - k) << 23);   // 2^-k, k in [-127, 120]
    u32x2 o = {0u, 0u};
    if (!zero) {
        o[0] = pack_e4m3x4(bf16_lo(w[0]) * r, bf16_hi(w[0]) * r, bf16_lo(w[1]) * r, bf16_hi(w[1]) * r);
        o[1] = pack_e4m3x4(bf16_lo(w[2]) * r, bf16_hi(w[2]) * r, bf16_lo(w[3]) * r, bf16_hi(w[3]) * r);
    }
    __builtin_nontemporal_store(o, q + v);
}

__global__ void __launch_bounds__(256)
mxq_1x32_kernel(const u32x4 *__restrict__ x, u32x2 *__restrict__ q, uint8_t *__restrict__ e,
                uint64_t npack) {
    const uint64_t stride = (uint64_t)gridDim.x * 256;
    // every lane of a 4-lane block group has the same v0 < npack and
    // v1 < npack: npack and the stride are multiples of 4
    for (uint64_t v0 = (uint64_t)blockIdx.x * 256 + threadIdx.x; v0 < npack; v0 += 2 * stride) {
        const uint64_t v1 = v0 + stride;
        const bool l1 = v1 < npack;
        const u32x4 w0 = __builtin_nontemporal_load(x + v0);
        u32x4 w1 = {0u, 0u, 0u, 0u};
        if (l1) w1 = __builtin_nontemporal_load(x + v1);
        mxq_pack(w0, q, e, v0, true);
        mxq_pack(w1, q, e, v1, l1);
    }
}

unsigned grid_rows(int64_t rows) { return (unsigned)(rows < 1048576 ? (rows > 0 ? rows : 1) : 1048576); }

}  // namespace

int bs_launch_band_reduce(const uint16_t *const *parts, int P, uint16_t *out, int64_t rows,
                          int64_t N, hipStream_t stream) {
    int rc = 0;
    PartPtrs pp;
    for (int p = 0; p < 16; p++) pp.p[p] = (const u32x4 *)parts[p < P ? p : 0];
    const int64_t nvec = rows * N / 8;
    u32x4 *o = (u32x4 *)out;
    switch (P) {
        case 1: rc = launch_reduce_p<1>(pp, o, nvec, stream); break;
        case 2: rc = launch_reduce_p<2>(pp, o, nvec, stream); break;
        case 3: rc = launch_reduce_p<3>(pp, o, nvec, stream); break;
        case 4: rc = launch_reduce_p<4>(pp, o, nvec, stream); break;
        case 5: rc = launch_reduce_p<5>(pp, o, nvec, stream); break;
        case 6: rc = launch_reduce_p<6>(pp, o, nvec, stream); break;
        case 7: rc = launch_reduce_p<7>(pp, o, nvec, stream); break;
        case 8: rc = launch_reduce_p<8>(pp, o, nvec, stream); break;
        case 9: rc = launch_reduce_p<9>(pp, o, nvec, stream); break;
        case 10: rc = launch_reduce_p<10>(pp, o, nvec, stream); break;
        case 11: rc = launch_reduce_p<11>(pp, o, nvec, stream); break;
        case 12: rc = launch_reduce_p<12>(pp, o, nvec, stream); break;
        case 13: rc = launch_reduce_p<13>(pp, o, nvec, stream); break;
        case 14: rc = launch_reduce_p<14>(pp, o, nvec, stream); break;
        case 15: rc = launch_reduce_p<15>(pp, o, nvec, stream); break;
        case 16: rc = launch_reduce_p<16>(pp, o, nvec, stream); break;
        default: return -1;
    }
    return rc;
}

template <int CPL>
static int launch_rowq(dim3 grid, dim3 block, hipStream_t stream, const u32x4 *xv, u32x2 *qv,
                       float *scale, int64_t rows, int nch) {
    if (nch == 64 * CPL)
        return bs_enqueue(rowq_kernel<CPL, true>, grid, block, stream, xv, qv, scale, rows, nch);
    return bs_enqueue(rowq_kernel<CPL, false>, grid, block, stream, xv, qv, scale, rows, nch);
}

int bs_launch_rowq(const uint16_t *x, uint8_t *q, float *scale, int64_t rows, int64_t N,
                   hipStream_t stream) {
    int rc = 0;
    const int nch = (int)(N / 8);
    const u32x4 *xv = (const u32x4 *)x;
    u32x2 *qv = (u32x2 *)q;
    if (nch > 2048) {
        const dim3 grid(grid_rows(rows)), block(256);
        return bs_enqueue(rowq_long_kernel, grid, block, stream, xv, qv, scale, rows, nch);
    }
    const int64_t wg = (rows + 3) / 4;
    if (wg > 0x7FFFFFFF) return -1;
    const dim3 grid((unsigned)wg), block(256);
    if (nch <= 256)
        rc |= launch_rowq<4>(grid, block, stream, xv, qv, scale, rows, nch);
    else if (nch <= 512)
        rc |= launch_rowq<8>(grid, block, stream, xv, qv, scale, rows, nch);
    else if (nch <= 896)
        rc |= launch_rowq<14>(grid, block, stream, xv, qv, scale, rows, nch);
    else if (nch <= 1024)
        rc |= launch_rowq<16>(grid, block, stream, xv, qv, scale, rows, nch);
    else
        rc |= launch_rowq<32>(grid, block, stream, xv, qv, scale, rows, nch);
    return rc;
}

int bs_launch_rowdq(const uint8_t *q, const float *scale, uint16_t *y, int64_t rows, int64_t N,
                    hipStream_t stream) {
    const int64_t nch = N / 8;
    const int64_t npack = rows * nch;
    int64_t blocks = (npack + 511) / 512;
    if (blocks > 1048576) blocks = 1048576;
    if (blocks < 1) blocks = 1;
    const u32x2 *qv = (const u32x2 *)q;
    u32x4 *yv = (u32x4 *)y;
    if (npack < 0x7FFFFFFF - 2 * 256 * blocks)
        return bs_enqueue(rowdq_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), stream, qv, scale,
                          yv, (uint32_t)npack, (uint32_t)nch);
    return bs_enqueue(rowdq_kernel<uint64_t>, dim3((unsigned)blocks), dim3(256), stream, qv, scale, yv,
                      (uint64_t)npack, (uint64_t)nch);
}

int bs_launch_blockq(const float *x, uint8_t *q, float *scale, int64_t rows, int64_t cols,
                     int block_rows, hipStream_t stream) {
    if (block_rows == 1) {
        const int64_t nblocks = rows * (cols / 128);
        const int64_t threads = nblocks * 16;
        const int64_t wg = (threads + 255) / 256;
        if (wg > 0x7FFFFFFF) return -1;
        return bs_enqueue(blockq_1x128_kernel, dim3((unsigned)(wg > 0 ? wg : 1)), dim3(256), stream,
                          (const u32x4 *)x, (u32x2 *)q, scale, nblocks);
    }
    const int64_t nb = ((rows + 127) / 128) * (cols / 128);
    if (nb > 0x7FFFFFFF) return -1;
    return bs_enqueue(blockq_128x128_kernel, dim3((unsigned)(nb > 0 ? nb : 1)), dim3(256), stream, x, q,
                      scale, rows, cols);
}

int bs_launch_actq(const uint16_t *x, uint8_t *q, float *scale, int64_t rows, int64_t cols,
                   hipStream_t stream) {
    const uint64_t npair = (uint64_t)rows * (uint64_t)(cols / 16);
    uint64_t blocks = (npair + 255) / 256;
    if (blocks > 1048576) blocks = 1048576;
    if (blocks < 1) blocks = 1;
    return bs_enqueue(actq_1x128_kernel, dim3((unsigned)blocks), dim3(256), stream, (const u32x4 *)x,
                      (u32x4 *)q, scale, npair);
}

int bs_launch_mxq(const uint16_t *x, uint8_t *q, uint8_t *e, int64_t rows, int64_t cols,
                  hipStream_t stream) {
    const uint64_t npack = (uint64_t)rows * (uint64_t)(cols / 8);
    uint64_t blocks = (npack + 511) / 512;
    if (blocks > 1048576) blocks = 1048576;
    if (blocks < 1) blocks = 1;
    return bs_enqueue(mxq_1x32_kernel, dim3((unsigned)blocks), dim3(256), stream, (const u32x4 *)x,
                      (u32x2 *)q, e, npack);
}

int bs_launch_band_rowq(const uint16_t *const *parts, int P, uint8_t *q, float *scale, int64_t rows,
                        int64_t N, hipStream_t stream) {
    PartPtrs pp;
    for (int p = 0; p < 16; p++) pp.p[p] = (const u32x4 *)parts[p < P ? p : 0];
    const int nch = (int)(N / 8);
    if (rows > 0x7FFFFFFF || nch > 256 * BRQ_CPT) return -1;
    // parts per load group: 4 measured fastest at P = 8, [2048, 7168]
    // (42.2 us against 43.7 for 2 and 43.1 for 8)
    constexpr int G = 4;
    return bs_enqueue(band_rowq_kernel<G>, dim3((unsigned)rows), dim3(256), stream, pp, P,
                      (u32x2 *)q, scale, nch);
}

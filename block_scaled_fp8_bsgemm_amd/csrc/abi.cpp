// abi.cpp -- the extern "C" entry points of libbsgemm (declared, with their
// contracts, in include/bsgemm.h).  Every argument is checked on the host
// before anything is enqueued; a rejected call launches nothing and writes
// nothing.  The kernels themselves live in gemm.hip and stream.hip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsgemm.h"
#include "launch.hpp"

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;   // rows / columns per matrix
constexpr int64_t kMaxK = (int64_t)1 << 22;     // keeps in-tile byte offsets in 32 bits

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

inline Range range_of(const void *p, int64_t bytes) {
    uintptr_t a = (uintptr_t)p;
    return Range{a, a + (uintptr_t)(bytes > 0 ? bytes : 0)};
}

inline bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

inline hipStream_t as_stream(void *s) { return (hipStream_t)s; }

}  // namespace

extern "C" {

const char *bs_status_str(bs_status status) {
    switch (status) {
        case BS_OK: return "ok";
        case BS_ERR_INVALID: return "invalid argument (null pointer, negative size, bad count or overlapping buffers)";
        case BS_ERR_UNSUPPORTED: return "unsupported shape, stride or alignment";
        case BS_ERR_LAUNCH: return "the HIP runtime rejected the kernel launch";
    }
    return "unknown status";
}

}  // extern "C"

namespace {

typedef int (*blockscale_launch)(const uint8_t *, const float *, const uint8_t *, const float *,
                                 uint16_t *, int64_t, int64_t, int64_t, int64_t, int64_t,
                                 hipStream_t);

// Validation shared by the two blockscale GEMM entry points: B is either the
// weight [N, K] row-major or its prepacked form, the same N * K bytes.
bs_status blockscale_gemm(blockscale_launch launch, const uint8_t *A, const float *a_scale,
                          const uint8_t *B, const float *b_scale, uint16_t *C, int64_t M,
                          int64_t N, int64_t K, int32_t bands, int64_t band_stride,
                          void *stream) {
    if (!A || !a_scale || !B || !b_scale || !C) return BS_ERR_INVALID;
    if (M < 0 || N <= 0 || K <= 0 || bands < 1 || band_stride < 0) return BS_ERR_INVALID;
    if (N % 128 || K % 128 || bands > 64) return BS_ERR_UNSUPPORTED;
    if (M >= kMaxDim || N >= kMaxDim || K > kMaxK) return BS_ERR_UNSUPPORTED;
    if (M % bands) return BS_ERR_UNSUPPORTED;
    const int64_t band_rows = M / bands;
    const int64_t stride = band_stride == 0 ? band_rows * N : band_stride;
    if (stride < band_rows * N || stride % 8) return BS_ERR_UNSUPPORTED;
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(a_scale, 4) ||
        !aligned(b_scale, 4))
        return BS_ERR_UNSUPPORTED;
    const int64_t KB = K / 128, NB = N / 128;
    const Range rc = range_of(C, ((bands - 1) * stride + band_rows * N) * 2);
    if (overlap(rc, range_of(A, M * K)) || overlap(rc, range_of(B, N * K)) ||
        overlap(rc, range_of(a_scale, M * KB * 4)) || overlap(rc, range_of(b_scale, NB * KB * 4)))
        return BS_ERR_INVALID;
    if (M == 0) return BS_OK;
    return launch(A, a_scale, B, b_scale, C, M, N, K, band_rows == 0 ? 1 : band_rows, stride,
                  as_stream(stream)) == 0
               ? BS_OK
               : BS_ERR_LAUNCH;
}

}  // namespace

extern "C" {

bs_status bsgemm_fp8(const uint8_t *A, const float *a_scale, const uint8_t *B, const float *b_scale,
                     uint16_t *C, int64_t M, int64_t N, int64_t K, int32_t bands,
                     int64_t band_stride, void *stream) {
    return blockscale_gemm(bs_launch_gemm, A, a_scale, B, b_scale, C, M, N, K, bands, band_stride,
                           stream);
}

bs_status bsgemm_fp8_pb(const uint8_t *A, const float *a_scale, const uint8_t *Bp,
                        const float *b_scale, uint16_t *C, int64_t M, int64_t N, int64_t K,
                        int32_t bands, int64_t band_stride, void *stream) {
    return blockscale_gemm(bs_launch_gemm_pb, A, a_scale, Bp, b_scale, C, M, N, K, bands,
                           band_stride, stream);
}

bs_status bprepack_e4m3(const uint8_t *B, uint8_t *Bp, int64_t N, int64_t K, void *stream) {
    if (!B || !Bp || N <= 0 || K <= 0) return BS_ERR_INVALID;
    if (N % 128 || K % 128 || N >= kMaxDim || K > kMaxK) return BS_ERR_UNSUPPORTED;
    if (!aligned(B, 16) || !aligned(Bp, 16)) return BS_ERR_UNSUPPORTED;
    if (overlap(range_of(B, N * K), range_of(Bp, N * K))) return BS_ERR_INVALID;
    return bs_launch_bprepack(B, Bp, N, K, as_stream(stream)) == 0 ? BS_OK : BS_ERR_LAUNCH;
}

bs_status mxgemm_fp8(const uint8_t *A, const uint8_t *a_scale, const uint8_t *B, const uint8_t *b_scale,
                     uint16_t *C, int64_t M, int64_t N, int64_t K, int32_t bands,
                     int64_t band_stride, void *stream) {
    if (!A || !a_scale || !B || !b_scale || !C) return BS_ERR_INVALID;
    if (M < 0 || N <= 0 || K <= 0 || bands < 1 || band_stride < 0) return BS_ERR_INVALID;
    if (N % 128 || K % 128 || bands > 64) return BS_ERR_UNSUPPORTED;
    if (M >= kMaxDim || N >= kMaxDim || K > kMaxK) return BS_ERR_UNSUPPORTED;
    if (M % bands) return BS_ERR_UNSUPPORTED;
    const int64_t band_rows = M / bands;
    const int64_t stride = band_stride == 0 ? band_rows * N : band_stride;
    if (stride < band_rows * N || stride % 8) return BS_ERR_UNSUPPORTED;
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(a_scale, 4) ||
        !aligned(b_scale, 4))
        return BS_ERR_UNSUPPORTED;
    const int64_t KQ = K / 32;
    const Range rc = range_of(C, ((bands - 1) * stride + band_rows * N) * 2);
    if (overlap(rc, range_of(A, M * K)) || overlap(rc, range_of(B, N * K)) ||
        overlap(rc, range_of(a_scale, M * KQ)) || overlap(rc, range_of(b_scale, N * KQ)))
        return BS_ERR_INVALID;
    if (M == 0) return BS_OK;
    return bs_launch_mxgemm(A, a_scale, B, b_scale, C, M, N, K, band_rows == 0 ? 1 : band_rows,
                            stride, as_stream(stream)) == 0
               ? BS_OK
               : BS_ERR_LAUNCH;
}

bs_status band_reduce(const uint16_t *const *parts, int32_t P, uint16_t *out, int64_t rows,
                      int64_t N, void *stream) {
    if (!parts || !out || P < 1 || P > 16 || rows < 0 || N <= 0) return BS_ERR_INVALID;
    for (int p = 0; p < P; p++)
        if (!parts[p]) return BS_ERR_INVALID;
    if (N % 8 || rows >= kMaxDim * 8 || N >= kMaxDim) return BS_ERR_UNSUPPORTED;
    if (!aligned(out, 16)) return BS_ERR_UNSUPPORTED;
    for (int p = 0; p < P; p++)
        if (!aligned(parts[p], 16)) return BS_ERR_UNSUPPORTED;
    const Range ro = range_of(out, rows * N * 2);
    for (int p = 0; p < P; p++)
        if (overlap(ro, range_of(parts[p], rows * N * 2))) return BS_ERR_INVALID;
    if (rows == 0) return BS_OK;
    return bs_launch_band_reduce(parts, P, out, rows, N, as_stream(stream)) == 0 ? BS_OK : BS_ERR_LAUNCH;
}

bs_status band_rowq_e4m3(const uint16_t *const *parts, int32_t P, uint8_t *q, float *scale,
                         int64_t rows, int64_t N, void *stream) {
    if (!parts || !q || !scale || P < 1 || P > 16 || rows < 0 || N <= 0) return BS_ERR_INVALID;
    for (int p = 0; p < P; p++)
        if (!parts[p]) return BS_ERR_INVALID;
    if (N % 8 || N > 8192 || rows >= kMaxDim) return BS_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(scale, 4)) return BS_ERR_UNSUPPORTED;
    for (int p = 0; p < P; p++)
        if (!aligned(parts[p], 16)) return BS_ERR_UNSUPPORTED;
    const Range rq = range_of(q, rows * N), rs = range_of(scale, rows * 4);
    if (overlap(rq, rs)) return BS_ERR_INVALID;
    for (int p = 0; p < P; p++) {
        const Range rp = range_of(parts[p], rows * N * 2);
        if (overlap(rq, rp) || overlap(rs, rp)) return BS_ERR_INVALID;
    }
    if (rows == 0) return BS_OK;
    return bs_launch_band_rowq(parts, P, q, scale, rows, N, as_stream(stream)) == 0 ? BS_OK
                                                                                     : BS_ERR_LAUNCH;
}

bs_status rowq_e4m3(const uint16_t *x, uint8_t *q, float *scale, int64_t rows, int64_t N,
                    void *stream) {
    if (!x || !q || !scale || rows < 0 || N <= 0) return BS_ERR_INVALID;
    if (N % 8 || N / 8 >= kMaxDim || rows >= kMaxDim * 8) return BS_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4)) return BS_ERR_UNSUPPORTED;
    const Range rx = range_of(x, rows * N * 2), rq = range_of(q, rows * N), rs = range_of(scale, rows * 4);
    if (overlap(rq, rx) || overlap(rs, rx) || overlap(rq, rs)) return BS_ERR_INVALID;
    if (rows == 0) return BS_OK;
    return bs_launch_rowq(x, q, scale, rows, N, as_stream(stream)) == 0 ? BS_OK : BS_ERR_LAUNCH;
}

bs_status rowdq_e4m3(const uint8_t *q, const float *scale, uint16_t *y, int64_t rows, int64_t N,
                     void *stream) {
    if (!q || !scale || !y || rows < 0 || N <= 0) return BS_ERR_INVALID;
    if (N % 8 || N / 8 >= kMaxDim || rows >= kMaxDim * 8) return BS_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(y, 16) || !aligned(scale, 4)) return BS_ERR_UNSUPPORTED;
    const Range ry = range_of(y, rows * N * 2);
    if (overlap(ry, range_of(q, rows * N)) || overlap(ry, range_of(scale, rows * 4))) return BS_ERR_INVALID;
    if (rows == 0) return BS_OK;
    return bs_launch_rowdq(q, scale, y, rows, N, as_stream(stream)) == 0 ? BS_OK : BS_ERR_LAUNCH;
}

bs_status blockq_e4m3(const float *x, uint8_t *q, float *scale, int64_t rows, int64_t cols,
                      int32_t block_rows, void *stream) {
    if (!x || !q || !scale || rows < 0 || cols <= 0) return BS_ERR_INVALID;
    if (block_rows != 1 && block_rows != 128) return BS_ERR_UNSUPPORTED;
    if (cols % 128 || cols >= kMaxDim || rows >= kMaxDim) return BS_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4)) return BS_ERR_UNSUPPORTED;
    const int64_t nscale = ((rows + block_rows - 1) / block_rows) * (cols / 128);
    const Range rx = range_of(x, rows * cols * 4), rq = range_of(q, rows * cols),
                rs = range_of(scale, nscale * 4);
    if (overlap(rq, rx) || overlap(rs, rx) || overlap(rq, rs)) return BS_ERR_INVALID;
    if (rows == 0) return BS_OK;
    return bs_launch_blockq(x, q, scale, rows, cols, block_rows, as_stream(stream)) == 0 ? BS_OK
                                                                                         : BS_ERR_LAUNCH;
}

bs_status actq_e4m3(const uint16_t *x, uint8_t *q, float *scale, int64_t rows, int64_t cols,
                    void *stream) {
    if (!x || !q || !scale || rows < 0 || cols <= 0) return BS_ERR_INVALID;
    if (cols % 128 || cols >= kMaxDim || rows >= kMaxDim) return BS_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4)) return BS_ERR_UNSUPPORTED;
    const Range rx = range_of(x, rows * cols * 2), rq = range_of(q, rows * cols),
                rs = range_of(scale, rows * (cols / 128) * 4);
    if (overlap(rq, rx) || overlap(rs, rx) || overlap(rq, rs)) return BS_ERR_INVALID;
    if (rows == 0) return BS_OK;
    return bs_launch_actq(x, q, scale, rows, cols, as_stream(stream)) == 0 ? BS_OK : BS_ERR_LAUNCH;
}

bs_status mxq_e4m3(const uint16_t *x, uint8_t *q, uint8_t *scale, int64_t rows, int64_t cols,
                   void *stream) {
    if (!x || !q || !scale || rows < 0 || cols <= 0) return BS_ERR_INVALID;
    if (cols % 32 || cols >= kMaxDim || rows >= kMaxDim) return BS_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(q, 16)) return BS_ERR_UNSUPPORTED;
    const Range rx = range_of(x, rows * cols * 2), rq = range_of(q, rows * cols),
                rs = range_of(scale, rows * (cols / 32));
    if (overlap(rq, rx) || overlap(rs, rx) || overlap(rq, rs)) return BS_ERR_INVALID;
    if (rows == 0) return BS_OK;
    return bs_launch_mxq(x, q, scale, rows, cols, as_stream(stream)) == 0 ? BS_OK : BS_ERR_LAUNCH;
}

}  // extern "C"

// launch.hpp -- internal launchers behind the C ABI (arguments already
// validated by abi.cpp).  Each returns 0 when the launch was accepted.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

int bs_launch_gemm(const uint8_t *A, const float *sa, const uint8_t *B, const float *sb,
                   uint16_t *C, int64_t M, int64_t N, int64_t K, int64_t band_rows,
                   int64_t band_stride, hipStream_t stream);

int bs_launch_gemm_pb(const uint8_t *A, const float *sa, const uint8_t *Bp, const float *sb,
                      uint16_t *C, int64_t M, int64_t N, int64_t K, int64_t band_rows,
                      int64_t band_stride, hipStream_t stream);
int bs_launch_bprepack(const uint8_t *B, uint8_t *Bp, int64_t N, int64_t K, hipStream_t stream);
int bs_launch_mxgemm(const uint8_t *A, const uint8_t *sa, const uint8_t *B, const uint8_t *sb,
                     uint16_t *C, int64_t M, int64_t N, int64_t K, int64_t band_rows,
                     int64_t band_stride, hipStream_t stream);
int bs_launch_band_reduce(const uint16_t *const *parts, int P, uint16_t *out, int64_t rows,
                          int64_t N, hipStream_t stream);

int bs_launch_rowq(const uint16_t *x, uint8_t *q, float *scale, int64_t rows, int64_t N,
                   hipStream_t stream);

int bs_launch_rowdq(const uint8_t *q, const float *scale, uint16_t *y, int64_t rows, int64_t N,
                    hipStream_t stream);

int bs_launch_blockq(const float *x, uint8_t *q, float *scale, int64_t rows, int64_t cols,
                     int block_rows, hipStream_t stream);
int bs_launch_band_rowq(const uint16_t *const *parts, int P, uint8_t *q, float *scale, int64_t rows,
                        int64_t N, hipStream_t stream);
int bs_launch_actq(const uint16_t *x, uint8_t *q, float *scale, int64_t rows, int64_t cols,
                   hipStream_t stream);
int bs_launch_mxq(const uint16_t *x, uint8_t *q, uint8_t *e, int64_t rows, int64_t cols,
                  hipStream_t stream);

#include <tuple>

// Enqueue `kernel` with hipLaunchKernel and report that launch's own status
// (not a sticky error left by an unrelated earlier call).
template <typename... KArgs, typename... Args>
int bs_enqueue(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream, Args... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
    std::tuple<KArgs...> a(args...);
    hipError_t rc = hipSuccess;
    std::apply(
        [&](auto &...e) {
            void *argv[] = {(void *)&e...};
            rc = hipLaunchKernel((const void *)kernel, grid, block, argv, 0, stream);
        },
        a);
    return rc == hipSuccess ? 0 : -1;
}

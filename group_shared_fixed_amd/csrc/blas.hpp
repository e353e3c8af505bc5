// rocBLAS helpers for the plain dense products of libhaste (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>
#include <stdint.h>

namespace haste {

// One rocBLAS handle per host thread and device, created on first use and
// kept for the process: its atomics are off (bitwise repeatable products)
// and each call sets the stream and the caller's workspace.
inline rocblas_handle blas_handle(hipStream_t stream, void* ws, size_t ws_bytes)
{
    thread_local rocblas_handle handles[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    rocblas_handle& h = handles[dev];
    if (!h) {
        if (rocblas_create_handle(&h) != rocblas_status_success) {
            h = nullptr;
            return nullptr;
        }
        (void)rocblas_set_atomics_mode(h, rocblas_atomics_not_allowed);
    }
    if (rocblas_set_stream(h, stream) != rocblas_status_success) return nullptr;
    if (rocblas_set_workspace(h, ws, ws_bytes) != rocblas_status_success) return nullptr;
    return h;
}

// Row-major C (M x N, fp32) = alpha op(A) op(B) + beta C with bf16 A and B,
// expressed as the column-major product C^T = op(B)^T op(A)^T.
inline rocblas_status gemm_rm(rocblas_handle h, bool ta, bool tb, int64_t M, int64_t N, int64_t Kd, const uint16_t* A,
                       int64_t lda, const uint16_t* Bm, int64_t ldb, float beta, float* C, int64_t ldc)
{
    const float alpha = 1.0f;
    return rocblas_gemm_ex(h, tb ? rocblas_operation_transpose : rocblas_operation_none,
                           ta ? rocblas_operation_transpose : rocblas_operation_none, (rocblas_int)N, (rocblas_int)M,
                           (rocblas_int)Kd, &alpha, Bm, rocblas_datatype_bf16_r, (rocblas_int)ldb, A,
                           rocblas_datatype_bf16_r, (rocblas_int)lda, &beta, C, rocblas_datatype_f32_r,
                           (rocblas_int)ldc, C, rocblas_datatype_f32_r, (rocblas_int)ldc, rocblas_datatype_f32_r,
                           rocblas_gemm_algo_standard, 0, 0);
}


}  // namespace haste

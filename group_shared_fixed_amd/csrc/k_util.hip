// Small support kernels: feature-major copy of h, fills, input validation.
#include "common.hpp"
#include "kernels.hpp"

namespace haste {

// hT[j, b] = h[b, j] for b < B, 0 for B <= b < Bp (64 x 64 tiles via LDS).
__global__ __launch_bounds__(256) void k_transpose_h(const uint16_t* __restrict__ h, uint16_t* __restrict__ hT,
                                                     int64_t B, int64_t H, int64_t Bp)
{
    __shared__ uint16_t t[64][66];
    const int64_t j0 = (int64_t)blockIdx.x * 64, b0 = (int64_t)blockIdx.y * 64;
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        const int r = i >> 6, c = i & 63;
        const int64_t b = b0 + r, j = j0 + c;
        t[r][c] = (b < B && j < H) ? h[b * H + j] : (uint16_t)0;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        const int r = i >> 6, c = i & 63;
        const int64_t j = j0 + r, b = b0 + c;
        if (j < H && b < Bp) hT[j * Bp + b] = t[c][r];
    }
}

template <typename T>
__global__ __launch_bounds__(256) void k_fill_zero(T* __restrict__ p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = T(0);
}

// One thread per row: entries in [0, H) and strictly increasing.
__global__ __launch_bounds__(256) void k_validate_idx(const int32_t* __restrict__ idx, int64_t rows, int64_t F,
                                                      int64_t H, int32_t* bad)
{
    const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (r >= rows) return;
    bool ok = true;
    int32_t prev = -1;
    for (int64_t f = 0; f < F; ++f) {
        const int32_t v = idx[r * F + f];
        ok = ok && v > prev && v < H;
        prev = v;
    }
    if (!ok) atomicAdd(bad, 1);
}

// One thread per sample: rowptr non-decreasing, ids in [0, L), strictly increasing.
__global__ __launch_bounds__(256) void k_validate_labels(const int32_t* __restrict__ rowptr,
                                                         const int32_t* __restrict__ col, int64_t B, int64_t L,
                                                         int32_t* bad)
{
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= B) return;
    const int32_t p0 = rowptr[b], p1 = rowptr[b + 1];
    bool ok = p0 >= 0 && p1 >= p0;
    if (ok) {
        int32_t prev = -1;
        for (int32_t p = p0; p < p1; ++p) {
            const int32_t v = col[p];
            ok = ok && v > prev && v < L;
            prev = v;
        }
    }
    if (!ok) atomicAdd(bad, 1);
}

static unsigned fill_grid(int64_t n)
{
    int64_t g = (n + 255) / 256;
    return (unsigned)(g < 1 ? 1 : (g > 4096 ? 4096 : g));
}

void launch_transpose_h(const uint16_t* h, uint16_t* hT, int64_t B, int64_t H, int64_t Bp, hipStream_t s)
{
    const dim3 grid((unsigned)((H + 63) / 64), (unsigned)((Bp + 63) / 64));
    hipLaunchKernelGGL(k_transpose_h, grid, dim3(256), 0, s, h, hT, B, H, Bp);
}

void launch_fill_f32(float* p, int64_t n, hipStream_t s)
{
    hipLaunchKernelGGL(k_fill_zero<float>, dim3(fill_grid(n)), dim3(256), 0, s, p, n);
}

void launch_fill_f64(double* p, int64_t n, hipStream_t s)
{
    hipLaunchKernelGGL(k_fill_zero<double>, dim3(fill_grid(n)), dim3(256), 0, s, p, n);
}

void launch_fill_i32(int32_t* p, int64_t n, hipStream_t s)
{
    hipLaunchKernelGGL(k_fill_zero<int32_t>, dim3(fill_grid(n)), dim3(256), 0, s, p, n);
}

void launch_validate_idx(const int32_t* idx, int64_t rows, int64_t F, int64_t H, int32_t* bad, hipStream_t s)
{
    hipLaunchKernelGGL(k_validate_idx, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, idx, rows, F, H,
                       bad);
}

void launch_validate_labels(const int32_t* rowptr, const int32_t* col, int64_t B, int64_t L, int32_t* bad,
                            hipStream_t s)
{
    hipLaunchKernelGGL(k_validate_labels, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, s, rowptr, col, B, L,
                       bad);
}

}  // namespace haste

// Small support kernels: feature-major copy of h, fills, input validation.
#include "common.hpp"
#include "kernels.hpp"

namespace haste {

// hT[j, b] = h[b, j] for b < B, 0 for B <= b < Bp (64 x 64 tiles via LDS).
// Also clears the optional outputs zf[0, nzf) and *zd that later kernels of
// the same call accumulate into, and the status word *zi (saves separate
// launches).
__global__ __launch_bounds__(256) void k_transpose_h(const uint16_t* __restrict__ h, uint16_t* __restrict__ hT,
                                                     int64_t B, int64_t H, int64_t Bp, float* __restrict__ zf,
                                                     int64_t nzf, double* __restrict__ zd, int32_t* __restrict__ zi)
{
    {
        const int64_t nthreads = (int64_t)gridDim.x * gridDim.y * 256;
        const int64_t tid = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * 256 + threadIdx.x;
        for (int64_t i = tid; i < nzf; i += nthreads)
            zf[i] = 0.f;
        if (zd && tid == 0) *zd = 0.0;
        if (zi && tid == 0) *zi = 0;
    }
    // tile of 32 batch rows x 64 features; each thread moves one 16-byte
    // piece in (row b, features j .. j+8) and one out (feature j, rows b .. b+8)
    __shared__ uint16_t t[64][32 + 2];
    const int64_t j0 = (int64_t)blockIdx.x * 64, b0 = (int64_t)blockIdx.y * 32;
    {
        const int r = threadIdx.x >> 3, c8 = (threadIdx.x & 7) * 8;
        const int64_t b = b0 + r, j = j0 + c8;
        uint16_t v[8];
        if (b < B && j + 8 <= H && (H & 7) == 0) {
            const uint4 x = *reinterpret_cast<const uint4*>(h + b * H + j);
            v[0] = x.x & 0xffff; v[1] = x.x >> 16; v[2] = x.y & 0xffff; v[3] = x.y >> 16;
            v[4] = x.z & 0xffff; v[5] = x.z >> 16; v[6] = x.w & 0xffff; v[7] = x.w >> 16;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = (b < B && j + e < H) ? h[b * H + j + e] : (uint16_t)0;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
            t[c8 + e][r] = v[e];
    }
    __syncthreads();
    {
        const int jl = threadIdx.x >> 2, bc = (threadIdx.x & 3) * 8;
        const int64_t j = j0 + jl, b = b0 + bc;
        if (j < H && b < Bp) {
            uint4 x;
            x.x = t[jl][bc + 0] | ((uint32_t)t[jl][bc + 1] << 16);
            x.y = t[jl][bc + 2] | ((uint32_t)t[jl][bc + 3] << 16);
            x.z = t[jl][bc + 4] | ((uint32_t)t[jl][bc + 5] << 16);
            x.w = t[jl][bc + 6] | ((uint32_t)t[jl][bc + 7] << 16);
            *reinterpret_cast<uint4*>(hT + j * Bp + b) = x;
        }
    }
}

template <typename T>
__global__ __launch_bounds__(256) void k_fill_zero(T* __restrict__ p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = T(0);
}

__global__ __launch_bounds__(256) void k_fill_zero_f32_i32(float* __restrict__ p, int64_t n, int32_t* __restrict__ zi)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = 0.f;
    if (zi && blockIdx.x == 0 && threadIdx.x == 0) *zi = 0;
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

// dst[0] = (float)src[0]: a loss accumulated in fp64, handed out as fp32.
__global__ void k_f64_to_f32(const double* __restrict__ src, float* __restrict__ dst)
{
    if (threadIdx.x == 0) dst[0] = (float)src[0];
}

void launch_f64_to_f32(const double* src, float* dst, hipStream_t s)
{
    hipLaunchKernelGGL(k_f64_to_f32, dim3(1), dim3(64), 0, s, src, dst);
}

static unsigned fill_grid(int64_t n)
{
    int64_t g = (n + 255) / 256;
    return (unsigned)(g < 1 ? 1 : (g > 4096 ? 4096 : g));
}

void launch_transpose_h(const uint16_t* h, uint16_t* hT, int64_t B, int64_t H, int64_t Bp, hipStream_t s,
                        float* zero_f, int64_t n_zero_f, double* zero_d, int32_t* zero_i)
{
    const dim3 grid((unsigned)((H + 63) / 64), (unsigned)(Bp / 32));   // Bp is a multiple of 32
    hipLaunchKernelGGL(k_transpose_h, grid, dim3(256), 0, s, h, hT, B, H, Bp, zero_f, zero_f ? n_zero_f : 0,
                       zero_d, zero_i);
}

void launch_fill_f32(float* p, int64_t n, hipStream_t s)
{
    hipLaunchKernelGGL(k_fill_zero<float>, dim3(fill_grid(n)), dim3(256), 0, s, p, n);
}

void launch_fill_f32_i32(float* p, int64_t n, int32_t* i, hipStream_t s)
{
    hipLaunchKernelGGL(k_fill_zero_f32_i32, dim3(fill_grid(n)), dim3(256), 0, s, p, n, i);
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

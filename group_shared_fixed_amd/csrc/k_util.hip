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

// One wave per row: entries in [0, H) and pairwise distinct.  The slots of a
// row may come in any order (a group is defined by its index set); each lane
// checks its own entries against every earlier entry of the row.
__global__ __launch_bounds__(256) void k_validate_idx(const int32_t* __restrict__ idx, int64_t rows, int64_t F,
                                                      int64_t H, int32_t* bad)
{
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (r >= rows) return;                   // whole wave
    const int32_t* row = idx + r * F;
    bool ok = true;
    for (int64_t f0 = 0; f0 < F; f0 += 64) {
        const int64_t f = f0 + lane;
        const int32_t v = f < F ? row[f] : 0;
        ok = ok && (f >= F || (v >= 0 && v < H));
        for (int64_t e = 0; e < f0 + 64 && e < F; ++e)
            ok = ok && !(e < f && f < F && row[e] == v);
    }
    if (__any(!ok) && lane == 0) atomicAdd(bad, 1);
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
    hipLaunchKernelGGL(k_validate_idx, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, idx, rows, F, H, bad);
}

void launch_validate_labels(const int32_t* rowptr, const int32_t* col, int64_t B, int64_t L, int32_t* bad,
                            hipStream_t s)
{
    hipLaunchKernelGGL(k_validate_labels, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, s, rowptr, col, B, L,
                       bad);
}


// Bank-balanced slot order of each group (the layer's results do not depend
// on the order of a group's slots as long as W_k's columns move with them).
// The feature-gradient accumulator keeps feature column j's rows in bank group
// (j >> 1) mod 8 and one read-add-write instruction covers a run of 8
// consecutive slots.  Per group: sort the F slots by that key, equal keys in
// slot order, and deal the sorted slots over the R = F / 8 runs in turn (the
// p-th one becomes slot 8 (p mod R) + p div R).
//
// One wave per group; lane owns slots lane + 64 i.  A slot's place p in the
// sorted list is the number of slots with a smaller key plus the number of
// earlier slots with its key, counted from one ballot per key value.  The
// wave reads its whole index row and each weight row before writing it, so
// the permutation runs in place.
template <int FPL>
__global__ __launch_bounds__(256) void k_order_slots(int32_t* idx, uint16_t* W, uint8_t* perm, int64_t K, int G,
                                                     int F)
{
    const int lane = threadIdx.x & 63;
    const int64_t k = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (k >= K) return;                      // whole wave
    const int R = F >> 3;
    int col[FPL], key[FPL], dst[FPL];
    uint64_t m[FPL][8];
#pragma unroll
    for (int i = 0; i < FPL; ++i) {
        const int f = lane + 64 * i;
        col[i] = f < F ? idx[k * F + f] : 0;
        key[i] = f < F ? (col[i] >> 1) & 7 : 8;      // 8: no slot
#pragma unroll
        for (int v = 0; v < 8; ++v)
            m[i][v] = __ballot(key[i] == v);
    }
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int i = 0; i < FPL; ++i) {
        int p = 0;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            int all = 0, before = 0;
#pragma unroll
            for (int j = 0; j < FPL; ++j) {
                all += __popcll(m[j][v]);
                before += j < i ? __popcll(m[j][v]) : (j == i ? __popcll(m[j][v] & below) : 0);
            }
            p += v < key[i] ? all : (v == key[i] ? before : 0);
        }
        dst[i] = 8 * (p % R) + p / R;
    }
#pragma unroll
    for (int i = 0; i < FPL; ++i) {
        if (lane + 64 * i < F) {
            idx[k * F + dst[i]] = col[i];
            if (perm) perm[k * F + dst[i]] = (uint8_t)(lane + 64 * i);
        }
    }
    if (!W) return;
    // weight rows, eight at a time: all loads of a row precede its stores
    uint16_t* Wk = W + k * G * F;
    for (int g0 = 0; g0 < G; g0 += 8) {
        uint16_t v[8][FPL];
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int i = 0; i < FPL; ++i) {
                const int f = lane + 64 * i;
                v[r][i] = (g0 + r < G && f < F) ? Wk[(int64_t)(g0 + r) * F + f] : (uint16_t)0;
            }
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int i = 0; i < FPL; ++i)
                if (g0 + r < G && lane + 64 * i < F) Wk[(int64_t)(g0 + r) * F + dst[i]] = v[r][i];
    }
}

void launch_order_slots(int32_t* idx, uint16_t* W, uint8_t* perm, int64_t K, int G, int F, hipStream_t s)
{
    const dim3 grid((unsigned)((K + 3) / 4));
    if (F <= 64) hipLaunchKernelGGL(k_order_slots<1>, grid, dim3(256), 0, s, idx, W, perm, K, G, F);
    else hipLaunchKernelGGL(k_order_slots<2>, grid, dim3(256), 0, s, idx, W, perm, K, G, F);
}

}  // namespace haste

// Label embeddings for the grouping ("group-shared fixed fan-in" section of
// the HASTE notes): a label's embedding is the normalized mean of the encoder
// features of the samples it is positive for.  Over batches of features h
// (B x H bf16) and labels (CSR), the library keeps per label an fp32 sum of
// those features and a count; the embedding is the sum's direction in bf16.
//
// Per batch, without atomics (so the sums repeat bit for bit): the batch's
// (label, CSR position) pairs are sorted with the grouping's bitonic sort,
// which orders each label's entries by position, i.e. by sample; then one
// wave per label segment adds its samples' feature rows in sample order and
// adds that batch total to the label's sum, once.
#include "common.hpp"
#include "kernels.hpp"

namespace haste {

// sample[p] = the b with rowptr[b] <= p < rowptr[b + 1], for p < nnz (binary
// search; every entry gets a sample id in [0, B) whatever the row pointers).
__global__ __launch_bounds__(256) void k_csr_rows(const int32_t* __restrict__ rowptr, int64_t B, int64_t nnz,
                                                  int32_t* __restrict__ sample)
{
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (p >= nnz) return;
    int64_t lo = 0, hi = B - 1;                     // largest b with rowptr[b] <= p
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        if ((int64_t)rowptr[mid] <= p) lo = mid; else hi = mid - 1;
    }
    sample[p] = (int32_t)lo;
}

// One wave per sorted key position; the first position of each label
// segment sums the segment's feature rows (16-byte pieces, NP per lane) in
// key order and adds the total to S[label]; counts[label] += segment length.
template <int NP>
__global__ __launch_bounds__(256) void k_emb_accumulate(const uint16_t* __restrict__ h,
                                                        const int32_t* __restrict__ sample,
                                                        const uint64_t* __restrict__ keys, int64_t n, int64_t H,
                                                        float* __restrict__ S, int32_t* __restrict__ counts)
{
    const int lane = threadIdx.x & 63;
    const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= n) return;
    const uint32_t lab = (uint32_t)(keys[i] >> 32);
    if (i > 0 && (uint32_t)(keys[i - 1] >> 32) == lab) return;
    float acc[NP][8];
#pragma unroll
    for (int u = 0; u < NP; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[u][e] = 0.f;
    int64_t j = i;
    for (; j < n && (uint32_t)(keys[j] >> 32) == lab; ++j) {
        const int64_t b = sample[(uint32_t)keys[j]];
#pragma unroll
        for (int u = 0; u < NP; ++u) {
            const int64_t c = 8 * (lane + 64 * u);
            if (c < H) {
                const u32x4_t v = ldg16(h + b * H + c);
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    acc[u][2 * d] += bf16lo_to_f32(v[d]);
                    acc[u][2 * d + 1] += bf16hi_to_f32(v[d]);
                }
            }
        }
    }
    float* row = S + (int64_t)lab * H;
#pragma unroll
    for (int u = 0; u < NP; ++u) {
        const int64_t c = 8 * (lane + 64 * u);
        if (c < H) {
            f32x4_t* p = reinterpret_cast<f32x4_t*>(row + c);
            const f32x4_t a0 = p[0], a1 = p[1];
            p[0] = a0 + f32x4_t{acc[u][0], acc[u][1], acc[u][2], acc[u][3]};
            p[1] = a1 + f32x4_t{acc[u][4], acc[u][5], acc[u][6], acc[u][7]};
        }
    }
    if (lane == 0) counts[lab] += (int32_t)(j - i);
}

// One wave per label: E = bf16(S / |S|), 0 without positives or a zero sum
// (the squared norm summed per lane, then across the wave in a fixed order).
template <int NP>
__global__ __launch_bounds__(256) void k_emb_finalize(const float* __restrict__ S, const int32_t* __restrict__ counts,
                                                      int64_t L, int64_t H, uint16_t* __restrict__ E)
{
    const int lane = threadIdx.x & 63;
    const int64_t l = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (l >= L) return;
    const float* row = S + l * H;
    f32x4_t v[NP][2];
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < NP; ++u) {
        const int64_t c = 8 * (lane + 64 * u);
        v[u][0] = v[u][1] = zero4();
        if (c < H) {
            v[u][0] = *reinterpret_cast<const f32x4_t*>(row + c);
            v[u][1] = *reinterpret_cast<const f32x4_t*>(row + c + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ss = fmaf(v[u][0][e], v[u][0][e], fmaf(v[u][1][e], v[u][1][e], ss));
        }
    }
    ss = wave_sum(ss);
    const float inv = (counts[l] > 0 && ss > 0.f) ? 1.0f / sqrtf(ss) : 0.f;
#pragma unroll
    for (int u = 0; u < NP; ++u) {
        const int64_t c = 8 * (lane + 64 * u);
        if (c < H) {
            const f32x4_t a = v[u][0] * inv, b = v[u][1] * inv;
            *reinterpret_cast<u32x4_t*>(E + l * H + c) =
                u32x4_t{pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]), pack_bf16(b[0], b[1]), pack_bf16(b[2], b[3])};
        }
    }
}

void run_label_emb_accumulate(const uint16_t* h, const int32_t* rowptr, const int32_t* col, int64_t nnz, int64_t B,
                              int64_t H, float* S, int32_t* counts, uint64_t* keys, int32_t* sample, hipStream_t s)
{
    if (nnz == 0) return;
    hipLaunchKernelGGL(k_csr_rows, dim3((unsigned)((nnz + 255) / 256)), dim3(256), 0, s, rowptr, B, nnz, sample);
    group_sort_keys(col, nnz, keys, s);
    const dim3 grid((unsigned)((nnz + 3) / 4));
    if (H <= 512) hipLaunchKernelGGL(k_emb_accumulate<1>, grid, dim3(256), 0, s, h, sample, keys, nnz, H, S, counts);
    else hipLaunchKernelGGL(k_emb_accumulate<2>, grid, dim3(256), 0, s, h, sample, keys, nnz, H, S, counts);
}

void run_label_emb_finalize(const float* S, const int32_t* counts, int64_t L, int64_t H, uint16_t* E, hipStream_t s)
{
    const dim3 grid((unsigned)((L + 3) / 4));
    if (H <= 512) hipLaunchKernelGGL(k_emb_finalize<1>, grid, dim3(256), 0, s, S, counts, L, H, E);
    else hipLaunchKernelGGL(k_emb_finalize<2>, grid, dim3(256), 0, s, S, counts, L, H, E);
}

}  // namespace haste

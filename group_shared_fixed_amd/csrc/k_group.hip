// Semantic label grouping: mini-batch spherical k-means and greedy groups.
//
// HASTE notes, "group-shared fixed fan-in": labels are grouped by embedding
// similarity in two stages, mini-batch spherical k-means into C ~ L/(beta G)
// coarse clusters, then, inside each cluster, greedy groups of a seed and
// its G - 1 nearest neighbours.  Similarity is the dot product of bf16
// embeddings (the cosine for unit vectors).
//   assignment: the largest dot product, the lowest centre on ties (the
//     fused matrix-core kernel of k_assign.hip);
//   update: Sculley's mini-batch step (a centre becomes the running mean of
//     everything assigned to it so far) and projection onto the unit sphere,
//     summing each centre's batch members in batch order;
//   groups: per cluster, members in increasing id, the lowest-id ungrouped
//     member seeds a group and takes the G - 1 most similar ungrouped
//     members (lower id on ties); leftovers (fewer than G per cluster) are
//     concatenated in (cluster, id) order and cut into groups of G.
// Every step is deterministic: sorts are by (segment, index) keys, sums run
// in a fixed order, and comparisons break ties by index.
#include "common.hpp"
#include "kernels.hpp"

namespace haste {

// keys[i] = seg[i] << 32 | i for i < n, all ones for n <= i < N.
__global__ __launch_bounds__(256) void k_make_keys(const int32_t* __restrict__ seg, int64_t n, int64_t N,
                                                   uint64_t* __restrict__ keys)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < N; i += (int64_t)gridDim.x * 256)
        keys[i] = i < n ? (((uint64_t)(uint32_t)seg[i] << 32) | (uint64_t)i) : ~0ull;
}

// Bitonic sort of N = 2^p >= 2048 keys, ascending.  Pairs of stage (k, j):
// (i, i + j) with i = 2 j (t / j) + t % j; ascending where (i & k) == 0.
__device__ __forceinline__ void bitonic_lds(uint64_t* s, int64_t base, int t, int k, int j)
{
    const int i = 2 * j * (t / j) + (t % j), l = i + j;
    const bool up = ((base + i) & k) == 0;
    const uint64_t x = s[i], y = s[l];
    if ((x > y) == up) {
        s[i] = y;
        s[l] = x;
    }
}

__global__ __launch_bounds__(1024) void k_sort_block(uint64_t* __restrict__ keys)
{
    __shared__ uint64_t s[2048];
    const int t = threadIdx.x;
    const int64_t base = (int64_t)blockIdx.x * 2048;
    s[t] = keys[base + t];
    s[t + 1024] = keys[base + t + 1024];
    __syncthreads();
    for (int k = 2; k <= 2048; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            bitonic_lds(s, base, t, k, j);
            __syncthreads();
        }
    }
    keys[base + t] = s[t];
    keys[base + t + 1024] = s[t + 1024];
}

__global__ __launch_bounds__(256) void k_sort_merge_global(uint64_t* __restrict__ keys, int64_t N, int64_t j,
                                                           int64_t k)
{
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= N / 2) return;
    const int64_t i = 2 * j * (t / j) + (t % j), l = i + j;
    const bool up = (i & k) == 0;
    const uint64_t x = keys[i], y = keys[l];
    if ((x > y) == up) {
        keys[i] = y;
        keys[l] = x;
    }
}

__global__ __launch_bounds__(1024) void k_sort_merge_block(uint64_t* __restrict__ keys, int64_t k)
{
    __shared__ uint64_t s[2048];
    const int t = threadIdx.x;
    const int64_t base = (int64_t)blockIdx.x * 2048;
    s[t] = keys[base + t];
    s[t + 1024] = keys[base + t + 1024];
    __syncthreads();
    for (int j = 1024; j > 0; j >>= 1) {
        // k > 2048 here: the direction bit lies above the block
        const int i = 2 * j * (t / j) + (t % j), l = i + j;
        const bool up = ((base + i) & k) == 0;
        const uint64_t x = s[i], y = s[l];
        if ((x > y) == up) {
            s[i] = y;
            s[l] = x;
        }
        __syncthreads();
    }
    keys[base + t] = s[t];
    keys[base + t + 1024] = s[t + 1024];
}

// First and one-past-last position of every segment id in sorted keys
// (segments without keys keep the pre-cleared 0, 0; ids >= C are skipped).
__global__ __launch_bounds__(256) void k_seg_bounds(const uint64_t* __restrict__ keys, int64_t n, int64_t C,
                                                    int32_t* __restrict__ start, int32_t* __restrict__ end)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const uint32_t c = (uint32_t)(keys[i] >> 32);
    if ((int64_t)c >= C) return;
    if (i == 0 || (uint32_t)(keys[i - 1] >> 32) != c) start[c] = (int32_t)i;
    if (i == n - 1 || (uint32_t)(keys[i + 1] >> 32) != c) end[c] = (int32_t)(i + 1);
}

// Centres from labels: Mc (fp32) and Mb (bf16) rows = E[init[c]], counts 0.
__global__ __launch_bounds__(256) void k_kmeans_init(const uint16_t* __restrict__ E, const int32_t* __restrict__ init,
                                                     int64_t H, float* __restrict__ Mc, uint16_t* __restrict__ Mb,
                                                     int32_t* __restrict__ v)
{
    const int64_t c = blockIdx.x;
    const uint16_t* e = E + (int64_t)init[c] * H;
    for (int64_t h = threadIdx.x; h < H; h += 256) {
        Mc[c * H + h] = __uint_as_float((uint32_t)e[h] << 16);
        Mb[c * H + h] = e[h];
    }
    if (threadIdx.x == 0) v[c] = 0;
}

// One block per centre c with members in the sorted batch keys: the sum of
// its members' embeddings in batch order, mu = (v Mc + sum) / (v + m),
// Mc = mu / |mu| (the squared norm summed per thread, then per wave, then
// over the four waves in order), Mb = bf16 of Mc, v += m.
__global__ __launch_bounds__(256) void k_kmeans_update(const uint16_t* __restrict__ E, const int32_t* __restrict__ batch,
                                                       const uint64_t* __restrict__ keys,
                                                       const int32_t* __restrict__ start,
                                                       const int32_t* __restrict__ end, int64_t H,
                                                       float* __restrict__ Mc, uint16_t* __restrict__ Mb,
                                                       int32_t* __restrict__ v)
{
    __shared__ float red[4];
    const int64_t c = blockIdx.x;
    const int s0 = start[c], s1 = end[c];
    const int m = s1 - s0;
    if (m <= 0) return;
    const int t = threadIdx.x;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int i = s0; i < s1; ++i) {
        const int64_t lab = batch[(uint32_t)keys[i]];
        const uint16_t* e = E + lab * H;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t h = t + 256 * u;
            if (h < H) acc[u] += __uint_as_float((uint32_t)e[h] << 16);
        }
    }
    const float vc = (float)v[c];
    const float den = (float)(v[c] + m);
    float mu[4], sq = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t h = t + 256 * u;
        mu[u] = h < H ? (vc * Mc[c * H + h] + acc[u]) / den : 0.f;
        sq += mu[u] * mu[u];
    }
    const float w = wave_sum(sq);
    if ((t & 63) == 0) red[t >> 6] = w;
    __syncthreads();
    const float inv = 1.0f / sqrtf(((red[0] + red[1]) + red[2]) + red[3]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t h = t + 256 * u;
        if (h < H) {
            const float x = mu[u] * inv;
            Mc[c * H + h] = x;
            Mb[c * H + h] = (uint16_t)(pack_bf16(x, 0.f) & 0xffffu);
        }
    }
    if (t == 0) v[c] = v[c] + m;
}

// Per cluster c: n_c = size / G greedy groups and r_c = size % G leftovers;
// gbase / obase = exclusive prefix sums over clusters, *ngroups = sum n_c.
// One block: each thread sums a contiguous run of clusters, the run sums are
// scanned in LDS, then each thread writes its run's prefixes.
__global__ __launch_bounds__(1024) void k_group_scan(const int32_t* __restrict__ start, const int32_t* __restrict__ end,
                                                     int64_t C, int G, int32_t* __restrict__ gbase,
                                                     int32_t* __restrict__ obase, int32_t* __restrict__ ngroups)
{
    __shared__ int64_t sg[1024], so[1024];
    const int t = threadIdx.x;
    const int64_t per = (C + 1023) / 1024;
    const int64_t c0 = t * per, c1 = (c0 + per < C) ? c0 + per : C;
    int64_t g = 0, o = 0;
    for (int64_t c = c0; c < c1; ++c) {
        const int64_t s = end[c] - start[c];
        g += s / G;
        o += s % G;
    }
    sg[t] = g;
    so[t] = o;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
        const int64_t xg = t >= d ? sg[t - d] : 0, xo = t >= d ? so[t - d] : 0;
        __syncthreads();
        sg[t] += xg;
        so[t] += xo;
        __syncthreads();
    }
    int64_t bg = sg[t] - g, bo = so[t] - o;       // exclusive
    for (int64_t c = c0; c < c1; ++c) {
        const int64_t s = end[c] - start[c];
        gbase[c] = (int32_t)bg;
        obase[c] = (int32_t)bo;
        bg += s / G;
        bo += s % G;
    }
    if (t == 1023) *ngroups = (int32_t)sg[1023];
}

// One wave per cluster.  Members are the sorted keys' positions start[c] ..
// end[c] (label ids increasing); member i belongs to lane i % 64, which alone
// reads and writes its similarity and taken flag (in LDS for clusters of up
// to kGreedyLds members, else in the workspace at the member's key
// position).  Per group: the seed is the lowest untaken member (wave minimum
// of the lanes' cursors); its embedding goes to LDS as fp32; each lane
// computes the dot products of its untaken members (four partial sums over
// interleaved 8-feature pieces, four loads in flight, added pairwise);
// G - 1 rounds of a wave arg-max (larger similarity, then lower index) pick
// the neighbours; the group's member indices are sorted and written out.
// Leftovers go out in index order after the cluster's groups.
constexpr int kGreedyLds = 1024;   // members per cluster kept in LDS
__global__ __launch_bounds__(256) void k_group_greedy(const uint16_t* __restrict__ E, const uint64_t* __restrict__ keys,
                                                      const int32_t* __restrict__ start,
                                                      const int32_t* __restrict__ end,
                                                      const int32_t* __restrict__ gbase,
                                                      const int32_t* __restrict__ obase,
                                                      const int32_t* __restrict__ ngroups, int64_t C, int64_t H,
                                                      int G, float* __restrict__ sim, uint8_t* __restrict__ taken,
                                                      int32_t* __restrict__ perm)
{
    __shared__ float seedv[4][1024];
    __shared__ int gidx[4][64];
    __shared__ float sSim[4][kGreedyLds];
    __shared__ uint8_t sTaken[4][kGreedyLds];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t c = (int64_t)blockIdx.x * 4 + w;
    if (c >= C) return;                            // whole wave; no block barrier below
    const int s0 = start[c], m = end[c] - s0;
    if (m <= 0) return;
    const int ng = m / G;
    auto label = [&](int i) { return (int32_t)(uint32_t)keys[s0 + i]; };
    // per-member state: LDS for small clusters (cleared here), else the
    // workspace (cleared by the launcher)
    const bool small = m <= kGreedyLds;
    float* const simp = small ? sSim[w] : sim + s0;
    uint8_t* const tk = small ? sTaken[w] : taken + s0;
    if (small)
        for (int i = lane; i < m; i += 64) tk[i] = 0;
    wave_sync();
    int cur = lane;                                // lane's lowest member not yet taken
    for (int gi = 0; gi < ng; ++gi) {
        while (cur < m && tk[cur]) cur += 64;
        int seed = cur < m ? cur : 0x7fffffff;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const int x = __shfl_xor(seed, o, 64);
            seed = x < seed ? x : seed;
        }
        if ((seed & 63) == lane) tk[seed] = 1;
        const uint16_t* es = E + (int64_t)label(seed) * H;
        for (int64_t h = lane; h < H; h += 64) seedv[w][h] = __uint_as_float((uint32_t)es[h] << 16);
        wave_sync();
        for (int i = lane; i < m; i += 64) {
            if (tk[i]) continue;
            const uint16_t* e = E + (int64_t)label(i) * H;
            float d[4] = {0.f, 0.f, 0.f, 0.f};      // partial sums over pieces h / 8 mod 4
            int64_t h = 0;
            for (; h + 32 <= H; h += 32) {
                u32x4_t p[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) p[u] = ldg16(e + h + 8 * u);
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        d[u] = fmaf(bf16lo_to_f32(p[u][q]), seedv[w][h + 8 * u + 2 * q], d[u]);
                        d[u] = fmaf(bf16hi_to_f32(p[u][q]), seedv[w][h + 8 * u + 2 * q + 1], d[u]);
                    }
            }
            for (int u = 0; h < H; h += 8, ++u) {       // H % 32 pieces (H % 8 == 0)
                const u32x4_t p = ldg16(e + h);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    d[u] = fmaf(bf16lo_to_f32(p[q]), seedv[w][h + 2 * q], d[u]);
                    d[u] = fmaf(bf16hi_to_f32(p[q]), seedv[w][h + 2 * q + 1], d[u]);
                }
            }
            simp[i] = (d[0] + d[1]) + (d[2] + d[3]);
        }
        if (lane == 0) gidx[w][0] = seed;
        for (int r = 1; r < G; ++r) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
            for (int i = lane; i < m; i += 64) {
                if (tk[i]) continue;
                const float d = simp[i];
                if (d > bv || bi == 0x7fffffff) {  // indices rise within a lane
                    bv = d;
                    bi = i;
                }
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const float ov = __shfl_xor(bv, o, 64);
                const int oi = __shfl_xor(bi, o, 64);
                if (oi != 0x7fffffff && (bi == 0x7fffffff || ov > bv || (ov == bv && oi < bi))) {
                    bv = ov;
                    bi = oi;
                }
            }
            if ((bi & 63) == lane) tk[bi] = 1;
            if (lane == 0) gidx[w][r] = bi;
        }
        wave_sync();
        // the group's members in increasing index (= increasing label id)
        if (lane < G) {
            const int mine = gidx[w][lane];
            int rank = 0;
            for (int u = 0; u < G; ++u) rank += gidx[w][u] < mine ? 1 : 0;
            perm[(int64_t)(gbase[c] + gi) * G + rank] = label(mine);
        }
        wave_sync();
    }
    // leftovers in index order, after every greedy group of every cluster
    const int64_t lbase = (int64_t)(*ngroups) * G + obase[c];
    int done = 0;
    for (int i0 = 0; i0 < m; i0 += 64) {
        const int i = i0 + lane;
        const bool left = i < m && !tk[i];
        const uint64_t mask = __ballot(left);
        const int before = __popcll(mask & ((1ull << lane) - 1ull));
        if (left) perm[lbase + done + before] = label(i);
        done += __popcll(mask);
    }
}

namespace {

inline unsigned grid_for(int64_t n, int per_block)
{
    const int64_t g = (n + per_block - 1) / per_block;
    return (unsigned)(g > 65536 ? 65536 : (g < 1 ? 1 : g));
}

// Smallest power of two >= max(n, 2048).
inline int64_t sort_size(int64_t n)
{
    int64_t N = 2048;
    while (N < n) N <<= 1;
    return N;
}

void sort_keys(const int32_t* seg, int64_t n, uint64_t* keys, hipStream_t s)
{
    const int64_t N = sort_size(n);
    hipLaunchKernelGGL(k_make_keys, dim3(grid_for(N, 256)), dim3(256), 0, s, seg, n, N, keys);
    hipLaunchKernelGGL(k_sort_block, dim3((unsigned)(N / 2048)), dim3(1024), 0, s, keys);
    for (int64_t k = 4096; k <= N; k <<= 1) {
        for (int64_t j = k >> 1; j >= 2048; j >>= 1)
            hipLaunchKernelGGL(k_sort_merge_global, dim3((unsigned)((N / 2 + 255) / 256)), dim3(256), 0, s, keys, N,
                               j, k);
        hipLaunchKernelGGL(k_sort_merge_block, dim3((unsigned)(N / 2048)), dim3(1024), 0, s, keys, k);
    }
}

}  // namespace

int64_t group_sort_size(int64_t n) { return sort_size(n); }

void group_sort_keys(const int32_t* seg, int64_t n, uint64_t* keys, hipStream_t s) { sort_keys(seg, n, keys, s); }

void run_kmeans_init(const uint16_t* E, const int32_t* init, int64_t C, int64_t H, float* Mc, uint16_t* Mb,
                     int32_t* v, hipStream_t s)
{
    hipLaunchKernelGGL(k_kmeans_init, dim3((unsigned)C), dim3(256), 0, s, E, init, H, Mc, Mb, v);
}

void run_kmeans_update(const uint16_t* E, const int32_t* batch, const int32_t* a_batch, int64_t n, int64_t C,
                       int64_t H, float* Mc, uint16_t* Mb, int32_t* v, uint64_t* keys, int32_t* start, int32_t* end,
                       hipStream_t s)
{
    launch_fill_i32(start, C, s);
    launch_fill_i32(end, C, s);
    sort_keys(a_batch, n, keys, s);
    hipLaunchKernelGGL(k_seg_bounds, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, keys, n, C, start, end);
    hipLaunchKernelGGL(k_kmeans_update, dim3((unsigned)C), dim3(256), 0, s, E, batch, keys, start, end, H, Mc, Mb, v);
}

void run_group_greedy(const uint16_t* E, const int32_t* a, int64_t L, int64_t C, int64_t H, int G, int32_t* perm,
                      uint64_t* keys, int32_t* start, int32_t* end, int32_t* gbase, int32_t* obase, int32_t* ngroups,
                      float* sim, uint8_t* taken, hipStream_t s)
{
    launch_fill_i32(start, C, s);
    launch_fill_i32(end, C, s);
    launch_fill_i32(reinterpret_cast<int32_t*>(taken), (L + 3) / 4, s);
    sort_keys(a, L, keys, s);
    hipLaunchKernelGGL(k_seg_bounds, dim3((unsigned)((L + 255) / 256)), dim3(256), 0, s, keys, L, C, start, end);
    hipLaunchKernelGGL(k_group_scan, dim3(1), dim3(1024), 0, s, start, end, C, G, gbase, obase, ngroups);
    hipLaunchKernelGGL(k_group_greedy, dim3((unsigned)((C + 3) / 4)), dim3(256), 0, s, E, keys, start, end, gbase,
                       obase, ngroups, C, H, G, sim, taken, perm);
}

}  // namespace haste

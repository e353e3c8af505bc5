// Group-level rewiring of the index sets (dynamic sparse training).
//
// HASTE, "loss / training strategy": training alternates a continuous phase
// (weights fitted, index sets frozen) with a discrete phase that reselects
// each group's fan-in set I_k the RigL way while |I_k| = F stays fixed; the
// algorithm itself is not printed.  Here RigL's steps are taken with the
// group as the unit:
//   grow[k, j]  = sum over the group's labels of |(dZ_k^T h)[g, j]|, the size
//                 of the dense loss gradient each feature column j would get;
//   prune[k, f] = sum over the group's labels of |W[l, f]|;
//   drop the n slots with the smallest prune score, grow the n columns with
//   the largest grow score among those not kept (a dropped column may come
//   back), ties to the lower column id; the new set is sorted, kept columns
//   carry their weights, grown columns start at zero.
//
// k_rewire_score computes grow, the dense L x H gradient dZ^T h reduced on
// chip (an MFMA contraction over the batch); k_rewire_select is the integer
// work, one wave per group.
#include "common.hpp"
#include "kernels.hpp"

namespace haste {

namespace {

constexpr int kRwCols = 64;     // feature columns per pass

// Lane moves within rows of 16 lanes (DPP), every lane reading a valid lane.
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __int_as_float(dpp_i32<CTRL>(__float_as_int(v)));
}
constexpr int kRwColTiles = kRwCols / 16;

__host__ __device__ constexpr int pow2_at_least(int x)
{
    int p = 1;
    while (p < x) p *= 2;
    return p;
}

}  // namespace

// grow[k, j] for every group and column.  KS: 32-row k-steps of the batch
// (Bp = 32 KS); RT: 16-label row tiles per wave (4: a wave's 64 labels
// hold whole groups).  A workgroup owns NW * 64 consecutive labels;
// each wave keeps the matrix-core operands of its labels' dZ (transposed
// through LDS once) in registers and sweeps the feature columns in passes of
// 64, with the hT blocks of the passes staged in two LDS buffers for all
// waves (one barrier per pass).  Per pass and wave: RT x 4 result tiles;
// their absolute values are summed over each tile's 16 labels, then over
// the row tiles of each group in increasing order, in registers.
template <int KS, int RT, int NW>
__global__ __launch_bounds__(64 * NW) void k_rewire_score(const uint16_t* __restrict__ hT, int64_t Bp, int64_t B,
                                                      int64_t H, const uint16_t* __restrict__ dZ, int64_t L, int G,
                                                      float* __restrict__ grow)
{
    constexpr int CH = pow2_at_least(4 * KS);     // 16-byte chunks per staged hT row (swizzle span)
    constexpr int LW = RT * 16;                    // labels per wave
    constexpr int ZROW = LW + 8;                   // staged dZ row (bf16), padded against bank conflicts
    static_assert(RT == 4, "a wave's 64 labels hold whole groups of G <= 64");
    __shared__ u32x4_t sH[2][kRwCols * CH];
    __shared__ uint16_t sZ[NW][32 * ZROW];

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int q = lane >> 4, i16 = lane & 15;
    const int64_t lab0 = (int64_t)blockIdx.x * (NW * LW);
    const int64_t wl0 = lab0 + (int64_t)w * LW;

    // 1. this wave's dZ operands: a[ks][r] holds labels wl0 + 16r + i16,
    //    batch rows 32ks + 8q .. +8
    u32x4_t a[KS][RT];
    {
        uint16_t* z = sZ[w];
        constexpr int CPR = LW / 8;                // 16-byte chunks per staged row
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int i = 0; i < CPR / 2; ++i) {   // 32 rows x CPR chunks = 64 x (CPR / 2)
                const int c = lane + 64 * i;
                const int row = c / CPR, ch = c % CPR;
                const int64_t b = 32 * ks + row, l = wl0 + 8 * ch;
                u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
                if (b < B && l < L) v = ldg16(dZ + b * L + l);
                *reinterpret_cast<u32x4_t*>(z + row * ZROW + 8 * ch) = v;
            }
            wave_sync();
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                const int rr = i16 >> 2, cc = i16 & 3;
                const u32x2_t lo = lds_tr16(z + (8 * q + rr) * ZROW + 16 * r + 4 * cc);
                const u32x2_t hi = lds_tr16(z + (8 * q + 4 + rr) * ZROW + 16 * r + 4 * cc);
                a[ks][r] = cat(lo, hi);
            }
            wave_sync();
        }
    }

    const int npass = (int)((H + kRwCols - 1) / kRwCols);
    const int ntid = NW * 64;
    constexpr int NCH = kRwCols * 4 * KS;          // staged 16-byte pieces per pass
    constexpr int PER = (NCH + NW * 64 - 1) / (NW * 64);     // per thread
    u32x4_t pre[PER];
    auto fetch = [&](int pass) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = threadIdx.x + ntid * i;
            const int jc = c / (4 * KS), ch = c % (4 * KS);
            const int64_t j = (int64_t)pass * kRwCols + jc;
            pre[i] = (c < NCH && j < H) ? ldg16(hT + j * Bp + 8 * ch) : u32x4_t{0u, 0u, 0u, 0u};
        }
    };
    auto stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = threadIdx.x + ntid * i;
            const int jc = c / (4 * KS), ch = c % (4 * KS);
            if (c < NCH) sH[buf][jc * CH + (ch ^ (jc & (CH - 1)))] = pre[i];
        }
    };
    fetch(0);
    const int gpw = G / 16;                        // row tiles per group
    const int64_t K = L / G;
    stage(0);
    if (npass > 1) fetch(1);
    for (int pass = 0; pass < npass; ++pass) {
        const int buf = pass & 1;
        // one barrier per pass: stage `buf` is complete, and every wave is
        // past the pass that read stage buf ^ 1, which is refilled here
        __syncthreads();
        if (pass + 1 < npass) {
            stage(buf ^ 1);
            if (pass + 2 < npass) fetch(pass + 2);
        }

        f32x4_t acc[RT][kRwColTiles];
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int t = 0; t < kRwColTiles; ++t) acc[r][t] = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int t = 0; t < kRwColTiles; ++t) {
                const int jc = 16 * t + i16, ch = 4 * ks + q;
                const u32x4_t bop = sH[buf][jc * CH + (ch ^ (jc & (CH - 1)))];
#pragma unroll
                for (int r = 0; r < RT; ++r) acc[r][t] = mfma16(a[ks][r], bop, acc[r][t]);
            }
        }
        // |gradient| summed over each row tile's 16 labels in lane, over the
        // row tiles of a group in increasing order (the wave's labels hold
        // whole groups), then across the four lane groups by an exchange in
        // two steps that leaves lane group q with column tile q: three lane
        // shuffles per group
        float xs[RT][kRwColTiles];
#pragma unroll
        for (int r = 0; r < RT; ++r) {
#pragma unroll
            for (int t = 0; t < kRwColTiles; ++t) {
                const f32x4_t v = acc[r][t];
                xs[r][t] = ((fabsf(v[0]) + fabsf(v[1])) + fabsf(v[2])) + fabsf(v[3]);
            }
        }
        static_assert(kRwColTiles == 4, "one column tile per lane group");
        const int hq = q >> 1, lq = q & 1;
#pragma unroll
        for (int r0 = 0; r0 < RT; ++r0) {
            if (r0 % gpw != 0) continue;
            float s[kRwColTiles];
#pragma unroll
            for (int t = 0; t < kRwColTiles; ++t) {
                s[t] = xs[r0][t];
#pragma unroll
                for (int u = 1; u < RT; ++u)
                    if (u < gpw && r0 + u < RT) s[t] += xs[r0 + u][t];
            }
            // step 1 (lane groups q, q ^ 2): keep tiles 2 hq, 2 hq + 1
            const float u0 = (hq ? s[2] : s[0]) + __shfl_xor(hq ? s[0] : s[2], 32, 64);
            const float u1 = (hq ? s[3] : s[1]) + __shfl_xor(hq ? s[1] : s[3], 32, 64);
            // step 2 (lane groups q, q ^ 1): keep tile q
            const float mine = (lq ? u1 : u0) + __shfl_xor(lq ? u0 : u1, 16, 64);
            const int64_t k = (wl0 + 16 * r0) / G;
            const int64_t j = (int64_t)pass * kRwCols + 16 * q + i16;
            if (k < K && j < H) grow[k * H + j] = mine;
        }
    }
}

// One wave per group: prune scores, the drop set, the grown columns, the new
// sorted index row and the permuted weights.  W_k is read into LDS and the
// index row into registers (every lane's columns are used by every lane's
// rank before anything is written), so idx_out / W_out may be idx / W.
template <int G, int F>
__global__ __launch_bounds__(256) void k_rewire_select(const int32_t* idx, const uint16_t* W,
                                                       const float* __restrict__ grow, int64_t K, int64_t H,
                                                       int n_swap, int32_t* idx_out, uint16_t* W_out,
                                                       float* __restrict__ prune_out)
{
    constexpr int NW = 4;
    constexpr int NCHUNK = G * F / 8;              // 16-byte pieces of W_k
    constexpr int FPL = (F + 63) / 64;             // slots per lane
    __shared__ uint16_t sW[NW][G * F];
    __shared__ uint32_t sKept[NW][32];
    __shared__ uint32_t sNew[NW][32];
    __shared__ int16_t sSlot[NW][1024];
    __shared__ int16_t sSrc[NW][F];

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t k = (int64_t)blockIdx.x * NW + w;
    if (k >= K) return;                            // whole wave; no workgroup barrier below

    const uint16_t* Wk = W + k * G * F;
    // the group's grow scores, lane owns columns lane + 64 t (H <= 1024);
    // requested first so their latency overlaps the slot ranking
    constexpr int NT = 16;
    float v[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int64_t j = lane + 64 * t;
        v[t] = j < H ? grow[k * H + j] : -1.0f;
    }
#pragma unroll
    for (int i = 0; i < (NCHUNK + 63) / 64; ++i) {
        const int c = lane + 64 * i;
        if (c < NCHUNK) *reinterpret_cast<u32x4_t*>(&sW[w][8 * c]) = ldg16(Wk + 8 * c);
    }
    int colr[FPL];                                 // the lane's slots' columns
#pragma unroll
    for (int i = 0; i < FPL; ++i) {
        const int f = lane + 64 * i;
        colr[i] = f < F ? idx[k * F + f] : 0;
        if (f < F) sSrc[w][f] = -1;
    }
    if (lane < 32) {
        sKept[w][lane] = 0u;
        sNew[w][lane] = 0u;
    }
    wave_sync();

    // prune score of each slot: sum over the group's labels of |W|, in label order
    float pr[FPL];
#pragma unroll
    for (int i = 0; i < FPL; ++i) {
        const int f = lane + 64 * i;
        float s = 0.f;
        if (f < F) {
            for (int g = 0; g < G; ++g) s += fabsf(__uint_as_float((uint32_t)sW[w][g * F + f] << 16));
            if (prune_out) prune_out[k * F + f] = s;
        }
        pr[i] = s;
    }
    wave_sync();
    // drop the n_swap smallest (prune score, column id); record the kept
    // columns.  A slot's rank counts the slots below it; the other slots'
    // scores and columns come from their lanes' registers (lane reads).
#pragma unroll
    for (int i = 0; i < FPL; ++i) {
        const int f = lane + 64 * i;
        int rank = 0;
#pragma unroll
        for (int i2 = 0; i2 < FPL; ++i2) {
            const int nu = F - 64 * i2 < 64 ? F - 64 * i2 : 64;
            for (int u = 0; u < nu; ++u) {
                const float pu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pr[i2]), u));
                const int cu = __builtin_amdgcn_readlane(colr[i2], u);
                rank += (pu < pr[i] || (pu == pr[i] && cu < colr[i])) ? 1 : 0;
            }
        }
        if (f < F && rank >= n_swap) {
            const int col = colr[i];
            atomicOr(&sKept[w][col >> 5], 1u << (col & 31));
            sSlot[w][col] = (int16_t)f;
        }
    }
    wave_sync();

    // grow: n_swap rounds of a wave arg-max over the columns not kept
    // (largest score, then lowest id)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int64_t j = lane + 64 * t;
        if (j < H && ((sKept[w][j >> 5] >> (j & 31)) & 1u)) v[t] = -1.0f;
    }
    // Each lane keeps its best two candidates (larger score, then lower id);
    // a round reduces the lanes' bests, the winning lane promotes its second,
    // and a lane that has won twice since its last scan rescans its values
    // (taken ones marked below every candidate).
    auto better = [](float a, int ja, float b, int jb) { return a > b || (a == b && ja < jb); };
    struct Top2 {
        float v1, v2;
        int j1, j2;
    };
    auto scan = [&]() -> Top2 {
        Top2 r{-2.0f, -2.0f, 0x7fffffff, 0x7fffffff};
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float x = v[t];
            const int jx = lane + 64 * t;
            const bool b1 = better(x, jx, r.v1, r.j1);
            const bool b2 = better(x, jx, r.v2, r.j2);
            r.v2 = b1 ? r.v1 : (b2 ? x : r.v2);
            r.j2 = b1 ? r.j1 : (b2 ? jx : r.j2);
            r.v1 = b1 ? x : r.v1;
            r.j1 = b1 ? jx : r.j1;
        }
        return r;
    };
    Top2 c = scan();
    int have = 2;
    for (int round = 0; round < n_swap; ++round) {
        float bv = c.v1;
        int bj = c.j1;
        // wave arg-max; the pick is a total order, so any pairing of lanes
        // works: within quads, 8-lane halves and 16-lane rows by DPP moves,
        // then across rows by lane shuffles
        auto take = [&](float ov, int oj) {
            if (better(ov, oj, bv, bj)) {
                bv = ov;
                bj = oj;
            }
        };
        take(dpp_f32<0xB1>(bv), dpp_i32<0xB1>(bj));    // quad_perm [1, 0, 3, 2]
        take(dpp_f32<0x4E>(bv), dpp_i32<0x4E>(bj));    // quad_perm [2, 3, 0, 1]
        take(dpp_f32<0x141>(bv), dpp_i32<0x141>(bj));  // row_half_mirror
        take(dpp_f32<0x140>(bv), dpp_i32<0x140>(bj));  // row_mirror
        take(__shfl_xor(bv, 16, 64), __shfl_xor(bj, 16, 64));
        take(__shfl_xor(bv, 32, 64), __shfl_xor(bj, 32, 64));
        if ((bj & 63) == lane) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
                if (t == (bj >> 6)) v[t] = -3.0f;
            atomicOr(&sNew[w][bj >> 5], 1u << (bj & 31));
            c.v1 = c.v2;
            c.j1 = c.j2;
            --have;
        }
        if (__any(have == 0)) {
            const Top2 r = scan();
            if (have == 0) {
                c = r;
                have = 2;
            }
        }
    }
    wave_sync();
    if (lane < 32) sNew[w][lane] |= sKept[w][lane];
    wave_sync();

    // new index row: the set bits in increasing order; lane owns columns
    // 16 lane .. 16 lane + 15
    const uint32_t m = (sNew[w][lane >> 1] >> (16 * (lane & 1))) & 0xffffu;
    const int cnt = __popc(m);
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int x = __shfl_up(incl, o, 64);
        if (lane >= o) incl += x;
    }
    int slot = incl - cnt;
    for (int bit = 0; bit < 16; ++bit) {
        if ((m >> bit) & 1u) {
            const int col = 16 * lane + bit;
            const bool kept = (sKept[w][col >> 5] >> (col & 31)) & 1u;
            idx_out[k * F + slot] = col;
            sSrc[w][slot] = kept ? sSlot[w][col] : (int16_t)-1;
            ++slot;
        }
    }
    wave_sync();

    // weights: kept columns move with their column, grown ones start at zero
    uint16_t* Wo = W_out + k * G * F;
#pragma unroll
    for (int i = 0; i < (NCHUNK + 63) / 64; ++i) {
        const int c = lane + 64 * i;
        if (c < NCHUNK) {
            const int g = c / (F / 8), f0 = (c % (F / 8)) * 8;
            uint32_t p[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s0 = sSrc[w][f0 + 2 * e], s1 = sSrc[w][f0 + 2 * e + 1];
                const uint32_t v0 = s0 >= 0 ? sW[w][g * F + s0] : 0u;
                const uint32_t v1 = s1 >= 0 ? sW[w][g * F + s1] : 0u;
                p[e] = v0 | (v1 << 16);
            }
            *reinterpret_cast<u32x4_t*>(Wo + 8 * c) = u32x4_t{p[0], p[1], p[2], p[3]};
        }
    }
}

// Waves per workgroup: eight (two per SIMD) in general; four at 128 rows,
// where two four-wave workgroups still fit on a CU and run their passes out
// of step, so one's lane reductions overlap the other's products (733
// against 769 us for eight waves); four for the longest batches, whose
// operands need more registers.
template <int KS>
static void score_launch(const uint16_t* hT, int64_t Bp, int64_t B, int64_t H, const uint16_t* dZ, int64_t L, int G,
                         float* grow, hipStream_t s)
{
    constexpr int RT = 4, NW = (KS == 4 || KS >= 7) ? 4 : 8;
    const int64_t per = NW * RT * 16;
    hipLaunchKernelGGL((k_rewire_score<KS, RT, NW>), dim3((unsigned)((L + per - 1) / per)), dim3(NW * 64), 0, s, hT,
                       Bp, B, H, dZ, L, G, grow);
}

bool launch_rewire_score(const uint16_t* hT, int64_t Bp, int64_t B, int64_t H, const uint16_t* dZ, int64_t L, int G,
                         float* grow, hipStream_t s)
{
    switch (Bp / 32) {
    case 1: score_launch<1>(hT, Bp, B, H, dZ, L, G, grow, s); return true;
    case 2: score_launch<2>(hT, Bp, B, H, dZ, L, G, grow, s); return true;
    case 3: score_launch<3>(hT, Bp, B, H, dZ, L, G, grow, s); return true;
    case 4: score_launch<4>(hT, Bp, B, H, dZ, L, G, grow, s); return true;
    case 5: score_launch<5>(hT, Bp, B, H, dZ, L, G, grow, s); return true;
    case 6: score_launch<6>(hT, Bp, B, H, dZ, L, G, grow, s); return true;
    case 7: score_launch<7>(hT, Bp, B, H, dZ, L, G, grow, s); return true;
    case 8: score_launch<8>(hT, Bp, B, H, dZ, L, G, grow, s); return true;
    }
    return false;
}

template <int G, int F>
static void select_launch(const int32_t* idx, const uint16_t* W, const float* grow, int64_t K, int64_t H, int n_swap,
                          int32_t* idx_out, uint16_t* W_out, float* prune_out, hipStream_t s)
{
    hipLaunchKernelGGL((k_rewire_select<G, F>), dim3((unsigned)((K + 3) / 4)), dim3(256), 0, s, idx, W, grow, K, H,
                       n_swap, idx_out, W_out, prune_out);
}

bool launch_rewire_select(int G, int F, const int32_t* idx, const uint16_t* W, const float* grow, int64_t K,
                          int64_t H, int n_swap, int32_t* idx_out, uint16_t* W_out, float* prune_out, hipStream_t s)
{
#define HASTE_RW_SEL(g, f)                                                                  \
    if (G == g && F == f) {                                                                 \
        select_launch<g, f>(idx, W, grow, K, H, n_swap, idx_out, W_out, prune_out, s);      \
        return true;                                                                        \
    }
    HASTE_RW_SEL(16, 32) HASTE_RW_SEL(16, 64) HASTE_RW_SEL(16, 128)
    HASTE_RW_SEL(32, 32) HASTE_RW_SEL(32, 64) HASTE_RW_SEL(32, 128)
    HASTE_RW_SEL(64, 32) HASTE_RW_SEL(64, 64) HASTE_RW_SEL(64, 128)
#undef HASTE_RW_SEL
    return false;
}

}  // namespace haste

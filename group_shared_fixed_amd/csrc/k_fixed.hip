// Standard (per-label) fixed fan-in: the baseline the HASTE notes measure
// against ("background" and "key findings" sections): every label has its own
// F-index set, so each label is a thin dot product with no shared feature
// tile and no matrix-core work.
//
// These kernels are a tuned gfx950 implementation of that baseline.  Grouping
// saves the per-label gather (each label here reads its own B x F feature
// values) and the per-label scatter of the feature gradient; everything else
// is done as well as for the grouped path:
//   * gathers read the feature-major copy hT with 16-byte loads, a lane taking
//     eight consecutive batch rows of one feature column, so four lanes read
//     64 contiguous bytes;
//   * a wave works on blocks of 16 consecutive labels, so Z rows leave and dZ
//     rows arrive as contiguous row segments, staged through LDS;
//   * products use v_dot2_f32_bf16 (two bf16 products and an fp32 add in one
//     instruction) instead of widening every value;
//   * the feature gradient keeps a 32-row fp32 accumulator in LDS per
//     workgroup; each wave owns four of its rows, walks the labels of the
//     workgroup's chunk in order and adds a label's F products with one
//     16-byte read-add-write per lane (no hand-off between waves), then the
//     same atomic or deterministic split-K reduction as the grouped path.
#include "common.hpp"
#include "kernels.hpp"

namespace haste {

// Labels per block: one block's Z row segment is 64 bytes, its dZ row
// segment 32 bytes.
constexpr int kFixBlk = 16;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

// Row-octet layout: a lane holds batch rows c0 + 8 ro .. + 8 (ro = lane % RO)
// of label lab0 + lane / RO; 64 / RO labels per wave instruction, 8 RO rows per
// batch chunk.
template <int RO>
struct Oct {
    static constexpr int NLG = 64 / RO;   // labels per wave instruction
    static constexpr int CH = 8 * RO;     // batch rows per chunk
};

// Z[b, l] = sum_f h[b, idx1[l, f]] W[l, f].
template <int F, int RO>
__global__ __launch_bounds__(256, 3) void k_fixed_fwd(FixedArgs a)
{
    constexpr int NLG = Oct<RO>::NLG, CH = Oct<RO>::CH;
    constexpr int ZS = CH + 4;                    // row stride (floats) of the [label][row] Z tile
    constexpr int NIP = NLG * F / 4, NWP = NLG * F / 8;   // 16-byte pieces of the labels' idx / W rows
    __shared__ __attribute__((aligned(16))) int sIdx[4][NLG * F];
    __shared__ __attribute__((aligned(16))) uint16_t sWt[4][NLG * F];
    __shared__ __attribute__((aligned(16))) float sZ[4][kFixBlk * ZS];

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane / RO, ro = lane % RO;
    int* ti = sIdx[wv];
    uint16_t* tw = sWt[wv];
    float* tz = sZ[wv];
    const int64_t L = a.L;
    const int64_t nblk = (L + kFixBlk - 1) / kFixBlk;
    const int64_t nw = (int64_t)gridDim.x * 4;
    const bool vec_z = (L & 3) == 0;

    for (int64_t blk = (int64_t)blockIdx.x * 4 + wv; blk < nblk; blk += nw) {
        const int64_t l0 = blk * kFixBlk;
        for (int64_t c0 = 0; c0 < a.Bp; c0 += CH) {
            const int rows = (int)((a.Bp - c0) < CH ? (a.Bp - c0) : CH);   // multiple of 8 (Bp % 32 == 0)
            for (int sub = 0; sub < kFixBlk / NLG; ++sub) {
                const int64_t lab0 = l0 + sub * NLG;
                // the NLG labels' index and weight rows into LDS (coalesced)
#pragma unroll
                for (int p = lane; p < NIP; p += 64) {
                    const int64_t l = lab0 + p / (F / 4);
                    const u32x4_t v = l < L ? ldg16(a.idx1 + l * F + 4 * (p % (F / 4))) : u32x4_t{0u, 0u, 0u, 0u};
                    *reinterpret_cast<u32x4_t*>(ti + 4 * p) = v;
                }
#pragma unroll
                for (int p = lane; p < NWP; p += 64) {
                    const int64_t l = lab0 + p / (F / 8);
                    const u32x4_t v = l < L ? ldg16(a.W + l * F + 8 * (p % (F / 8))) : u32x4_t{0u, 0u, 0u, 0u};
                    *reinterpret_cast<u32x4_t*>(tw + 8 * p) = v;
                }
                wave_sync();
                const int* li = ti + g * F;
                const uint16_t* lw = tw + g * F;
                const bool rows_ok = 8 * ro < rows;
                const uint16_t* hb = a.hT + (c0 + (rows_ok ? 8 * ro : 0));
                float acc[8];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    acc[i] = 0.f;
                // slots in octets, two register buffers: the next octet's rows are
                // requested while this one is used
                u32x4_t hA[8], hB[8];
                auto fetch = [&](int o, u32x4_t (&dst)[8]) {
                    const u32x4_t i0 = *reinterpret_cast<const u32x4_t*>(li + 8 * o);
                    const u32x4_t i1 = *reinterpret_cast<const u32x4_t*>(li + 8 * o + 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        dst[e] = ldg16(hb + (int64_t)i0[e] * a.Bp);
                        dst[4 + e] = ldg16(hb + (int64_t)i1[e] * a.Bp);
                    }
                };
                auto use = [&](int o, const u32x4_t (&v)[8]) {
                    const u32x4_t wq = *reinterpret_cast<const u32x4_t*>(lw + 8 * o);   // 8 weights
#pragma unroll
                    for (int pr = 0; pr < 4; ++pr) {
                        // slots 8o + 2pr (a) and 8o + 2pr + 1 (b); weight pair (W_a, W_b)
                        const u32x4_t& va = v[2 * pr];
                        const u32x4_t& vb = v[2 * pr + 1];
                        const uint32_t wp = wq[pr];
#pragma unroll
                        for (int d = 0; d < 4; ++d) {
                            // (h[r][a], h[r][b]) for the two rows of dword d
                            const uint32_t p0 = __builtin_amdgcn_perm(vb[d], va[d], 0x05040100u);
                            const uint32_t p1 = __builtin_amdgcn_perm(vb[d], va[d], 0x07060302u);
                            acc[2 * d] = dot2(p0, wp, acc[2 * d]);
                            acc[2 * d + 1] = dot2(p1, wp, acc[2 * d + 1]);
                        }
                    }
                };
                fetch(0, hA);
#pragma unroll 1
                for (int o = 0; o < F / 8; o += 2) {   // F / 8 is even
                    fetch(o + 1, hB);
                    use(o, hA);
                    if (o + 2 < F / 8) fetch(o + 2, hA);
                    use(o + 1, hB);
                }
                // this label's rows into the Z tile [label][row]
                if (rows_ok) {
                    float* dz = tz + (sub * NLG + g) * ZS + 8 * ro;
                    *reinterpret_cast<f32x4_t*>(dz) = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
                    *reinterpret_cast<f32x4_t*>(dz + 4) = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
                }
                wave_sync();
            }
            // the block's Z rows: a lane stores four labels of one row (16 bytes)
            for (int p = lane; p < rows * 4; p += 64) {
                const int r = p >> 2, q4 = p & 3;
                const int64_t b = c0 + r;
                if (b >= a.B) continue;
                const f32x4_t v = f32x4_t{tz[(4 * q4 + 0) * ZS + r], tz[(4 * q4 + 1) * ZS + r],
                                          tz[(4 * q4 + 2) * ZS + r], tz[(4 * q4 + 3) * ZS + r]};
                const int64_t l = l0 + 4 * q4;
                float* dst = a.Z + b * L + l;
                if (vec_z && l + 4 <= L) {
                    stg_stream(dst, v);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (l + e < L) dst[e] = v[e];
                }
            }
            wave_sync();
        }
    }
}

// dW[l, f] = sum_b dZ[b, l] h[b, idx1[l, f]]: a lane accumulates, for its
// label and eight batch rows, all F slots (dot products over row pairs), then
// the RO lanes of a label reduce-scatter the F sums so that each keeps F / RO
// consecutive slots and stores them.
template <int F, int RO>
__global__ __launch_bounds__(256, 3) void k_fixed_bwd_w(FixedArgs a)
{
    constexpr int NLG = Oct<RO>::NLG, CH = Oct<RO>::CH;
    constexpr int DS = CH + 8;                    // row stride (halves) of the [label][row] dZ tile
    constexpr int NIP = NLG * F / 4;
    constexpr int SPL = F / RO;                   // slots per lane after the reduction
    static_assert(SPL >= 2 && SPL % 2 == 0, "the reduction leaves pairs of slots per lane");
    __shared__ __attribute__((aligned(16))) int sIdx[4][NLG * F];
    __shared__ __attribute__((aligned(16))) uint16_t sD[4][NLG * DS];

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane / RO, ro = lane % RO;
    int* ti = sIdx[wv];
    uint16_t* td = sD[wv];
    const int64_t L = a.L;
    const int64_t ngrp = (L + NLG - 1) / NLG;
    const int64_t nw = (int64_t)gridDim.x * 4;
    // label groups in blocks of kFixBlk consecutive labels per wave, so the
    // waves in flight read neighbouring dZ row segments
    constexpr int GPB = kFixBlk / NLG;
    const int64_t nblk = (ngrp + GPB - 1) / GPB;

    for (int64_t blk = (int64_t)blockIdx.x * 4 + wv; blk < nblk; blk += nw) {
        for (int sub = 0; sub < GPB; ++sub) {
            const int64_t lab0 = (blk * GPB + sub) * NLG;
            if (lab0 >= L) break;
#pragma unroll
            for (int p = lane; p < NIP; p += 64) {
                const int64_t l = lab0 + p / (F / 4);
                const u32x4_t v = l < L ? ldg16(a.idx1 + l * F + 4 * (p % (F / 4))) : u32x4_t{0u, 0u, 0u, 0u};
                *reinterpret_cast<u32x4_t*>(ti + 4 * p) = v;
            }
            const int* li = ti + g * F;
            // whole rows of NLG labels in 8-byte pieces when L keeps them aligned
            const bool vec_d = (L & 3) == 0 && lab0 + NLG <= L;
            float acc[F];
#pragma unroll
            for (int f = 0; f < F; ++f)
                acc[f] = 0.f;
            for (int64_t c0 = 0; c0 < a.Bp; c0 += CH) {
                const int rows = (int)((a.Bp - c0) < CH ? (a.Bp - c0) : CH);
                // dZ[c0 .. c0 + rows][lab0 .. lab0 + NLG] transposed into [label][row]
                // (rows past B and labels past L are zero)
                wave_sync();
                for (int r = lane; r < rows; r += 64) {
                    const int64_t b = c0 + r;
                    if (vec_d && b < a.B) {
                        // four labels of the row per 8-byte load
#pragma unroll
                        for (int e4 = 0; e4 < NLG; e4 += 4) {
                            const u32x2_t v = ldg8(a.dZ + b * L + lab0 + e4);
                            td[(e4 + 0) * DS + r] = (uint16_t)(v[0] & 0xffffu);
                            td[(e4 + 1) * DS + r] = (uint16_t)(v[0] >> 16);
                            td[(e4 + 2) * DS + r] = (uint16_t)(v[1] & 0xffffu);
                            td[(e4 + 3) * DS + r] = (uint16_t)(v[1] >> 16);
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < NLG; ++e) {
                            const int64_t l = lab0 + e;
                            td[e * DS + r] = (b < a.B && l < L) ? a.dZ[b * L + l] : (uint16_t)0;
                        }
                    }
                }
                wave_sync();
                const bool rows_ok = 8 * ro < rows;
                const u32x4_t dz = *reinterpret_cast<const u32x4_t*>(td + g * DS + (rows_ok ? 8 * ro : 0));
                const uint16_t* hb = a.hT + (c0 + (rows_ok ? 8 * ro : 0));
                // the gathers of all F slots are requested before the first is
                // used (F / 8 loads of 16 bytes per lane at a time)
#pragma unroll
                for (int o = 0; o < F / 8; ++o) {
                    const u32x4_t i0 = *reinterpret_cast<const u32x4_t*>(li + 8 * o);
                    const u32x4_t i1 = *reinterpret_cast<const u32x4_t*>(li + 8 * o + 4);
                    u32x4_t v[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v[e] = ldg16(hb + (int64_t)i0[e] * a.Bp);
                        v[4 + e] = ldg16(hb + (int64_t)i1[e] * a.Bp);
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float s = acc[8 * o + e];
                        s = dot2(v[e][0], dz[0], s);
                        s = dot2(v[e][1], dz[1], s);
                        s = dot2(v[e][2], dz[2], s);
                        s = dot2(v[e][3], dz[3], s);
                        acc[8 * o + e] = rows_ok ? s : acc[8 * o + e];
                    }
                }
            }
            // reduce-scatter over the RO lanes of the label: each halving step
            // keeps half of the slots (the lower lane of a pair the lower half)
#pragma unroll
            for (int st = RO / 2, n = F; st >= 1; st >>= 1, n >>= 1) {
                const bool up = (ro & st) != 0;
#pragma unroll
                for (int i = 0; i < n / 2; ++i) {
                    const float keep = up ? acc[i + n / 2] : acc[i];
                    const float send = up ? acc[i] : acc[i + n / 2];
                    acc[i] = keep + __shfl_xor(send, st, 64);
                }
            }
            // lane ro now holds slots ro * SPL .. + SPL (the step on bit st
            // moved the upper lanes to the block st * SPL further on)
            const int64_t l = lab0 + g;
            if (l < L) {
                float* dst = a.dW + l * F + ro * SPL;
#pragma unroll
                for (int i = 0; i < SPL; i += 2)
                    *reinterpret_cast<f32x2_t*>(dst + i) = f32x2_t{acc[i], acc[i + 1]};
            }
        }
    }
}

// Offset (floats) of (batch row r < 32, column j) in the 32-row accumulator:
// 32 floats per column, 4-row quads XORed with (j / 2) % 8.
__device__ __forceinline__ int fix_acc_off(int j, int r)
{
    return j * 32 + ((((r >> 2) ^ (j >> 1)) & 7) << 2) + (r & 3);
}

// dh via a 32-row accumulator per workgroup; wave w owns rows RW w .. + RW and
// walks every label of the workgroup's chunk in order, so each accumulator
// cell is updated by one wave in label order (deterministic, no hand-off).
// Lane f handles slot f (and f + 64 for F = 128): one label's slots are
// distinct columns, so the lanes of one read-add-write never share a cell.
constexpr int kFixDhBlk = 64;   // labels per staged dZ block
constexpr int kMetaAhead = 8;   // labels whose index / weight loads are in flight
constexpr int kFixDhRowsPerWave = 4;   // rows of the 32-row tile each wave owns (8 waves: 12.0 -> 8.7 ms at 3M against 4 waves x 8 rows)
constexpr int kFixDhWaves = 32 / kFixDhRowsPerWave;
template <int F, bool DET>
__global__ __launch_bounds__(64 * kFixDhWaves, 1) void k_fixed_bwd_h(FixedArgs a)
{
    constexpr int R = 32;
    constexpr int RW = kFixDhRowsPerWave;
    constexpr int NTH = 64 * kFixDhWaves;
    constexpr int NU = (F + 63) / 64;
    constexpr int DS = R + 4;                  // row stride (halves) of the [label][row] dZ tile
    extern __shared__ __attribute__((aligned(16))) float acc[];   // H x 32, fix_acc_off
    __shared__ __attribute__((aligned(16))) uint16_t sD[kFixDhBlk * DS];

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int xcd = blockIdx.x & 7;
    const int slot = blockIdx.x >> 3;
    const int tile = slot % a.ntiles;
    const int chunk = (slot / a.ntiles) * 8 + xcd;
    const int64_t lc0 = (int64_t)chunk * a.L / a.nchunks, lc1 = (int64_t)(chunk + 1) * a.L / a.nchunks;
    const int64_t b0 = (int64_t)tile * R;
    const int64_t H = a.H;
    const int64_t L = a.L;
    for (int64_t i = threadIdx.x; i < R * H; i += NTH)
        acc[i] = 0.f;

    // metadata of one label: the lane's slot columns and weights
    struct Meta {
        int col[NU];
        float w[NU];
    };
    auto load_meta = [&](int64_t l, Meta& m) {
        const int64_t lc = l < lc1 ? l : lc1 - 1;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int f = lane + 64 * u;
            const bool ok = f < F;
            m.col[u] = ok ? a.idx1[lc * F + f] : 0;
            m.w[u] = ok ? bf16lo_to_f32(a.W[lc * F + f]) : 0.f;
        }
    };

    for (int64_t lb = lc0; lb < lc1; lb += kFixDhBlk) {
        const int nl = (int)((lc1 - lb) < kFixDhBlk ? (lc1 - lb) : kFixDhBlk);
        __syncthreads();   // the previous block's dZ tile is no longer read
        // dZ[b0 .. b0 + 32][lb .. lb + nl] transposed into [label][row]
        for (int p = threadIdx.x; p < R * kFixDhBlk; p += NTH) {
            const int r = p / kFixDhBlk, e = p % kFixDhBlk;
            const int64_t b = b0 + r;
            sD[e * DS + r] = (b < a.B && e < nl) ? a.dZ[b * L + lb + e] : (uint16_t)0;
        }
        __syncthreads();
        // label metadata kMetaAhead labels ahead in a register ring
        Meta m[kMetaAhead];
#pragma unroll
        for (int j = 0; j < kMetaAhead; ++j)
            load_meta(lb + j, m[j]);
        for (int e0 = 0; e0 < nl; e0 += kMetaAhead) {
#pragma unroll
            for (int j = 0; j < kMetaAhead; ++j) {
                const int e = e0 + j;
                if (e < nl) {
#pragma unroll
                    for (int q = 0; q < RW / 4; ++q) {
                        // four of this wave's rows of dZ[:, l]
                        const int r0 = RW * wv + 4 * q;
                        const u32x2_t dd = *reinterpret_cast<const u32x2_t*>(sD + e * DS + r0);
                        const float d0 = bf16lo_to_f32(dd[0]), d1 = bf16hi_to_f32(dd[0]);
                        const float d2 = bf16lo_to_f32(dd[1]), d3 = bf16hi_to_f32(dd[1]);
#pragma unroll
                        for (int u = 0; u < NU; ++u) {
                            if (lane + 64 * u < F) {
                                f32x4_t* p = reinterpret_cast<f32x4_t*>(acc + fix_acc_off(m[j].col[u], r0));
                                f32x4_t v = *p;
                                v[0] = fmaf(d0, m[j].w[u], v[0]);
                                v[1] = fmaf(d1, m[j].w[u], v[1]);
                                v[2] = fmaf(d2, m[j].w[u], v[2]);
                                v[3] = fmaf(d3, m[j].w[u], v[3]);
                                *p = v;
                            }
                        }
                    }
                }
                load_meta(lb + e + kMetaAhead, m[j]);
            }
        }
    }
    __syncthreads();
    if constexpr (DET) {
        float* dst = a.part + ((int64_t)chunk * a.ntiles * R + b0) * H;
        for_cells(R, (int)H, threadIdx.x, NTH, [&](int r, int j) { dst[(int64_t)r * H + j] = acc[fix_acc_off(j, r)]; });
    } else {
        for_cells(R, (int)H, threadIdx.x, NTH, [&](int r, int j) {
            if (b0 + r < a.B) unsafeAtomicAdd(&a.dh[(b0 + r) * H + j], acc[fix_acc_off(j, r)]);
        });
    }
}

// Row octets per lane group by padded batch: 16 (128-row chunks) from 128
// rows on, else 8 (64-row chunks) from 64, else 4.
static int fixed_ro(int64_t Bp) { return Bp >= 128 ? 16 : (Bp >= 64 ? 8 : 4); }

template <template <int, int> class K, int F>
static void go_fixed(int ro, const FixedArgs& a, int grid, hipStream_t s)
{
    switch (ro) {
    case 16: hipLaunchKernelGGL((K<F, 16>::fn), dim3(grid), dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL((K<F, 8>::fn), dim3(grid), dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((K<F, 4>::fn), dim3(grid), dim3(256), 0, s, a); break;
    }
}
template <int F, int RO>
struct FwdK {
    static constexpr auto fn = k_fixed_fwd<F, RO>;
};
template <int F, int RO>
struct BwK {
    static constexpr auto fn = k_fixed_bwd_w<F, RO>;
};

bool launch_fixed_fwd(int F, const FixedArgs& a, int grid, hipStream_t s)
{
    const int ro = fixed_ro(a.Bp);
    switch (F) {
    case 32: go_fixed<FwdK, 32>(ro, a, grid, s); return true;
    case 64: go_fixed<FwdK, 64>(ro, a, grid, s); return true;
    case 128: go_fixed<FwdK, 128>(ro, a, grid, s); return true;
    }
    return false;
}

bool launch_fixed_bwd_w(int F, const FixedArgs& a, int grid, hipStream_t s)
{
    const int ro = fixed_ro(a.Bp);
    switch (F) {
    case 32: go_fixed<BwK, 32>(ro, a, grid, s); return true;
    case 64: go_fixed<BwK, 64>(ro, a, grid, s); return true;
    case 128: go_fixed<BwK, 128>(ro, a, grid, s); return true;
    }
    return false;
}

bool launch_fixed_bwd_h(int F, bool det, const FixedArgs& a, hipStream_t s)
{
    const size_t lds = (size_t)32 * a.H * sizeof(float);
    const dim3 grid(a.nchunks * a.ntiles), blk(64 * kFixDhWaves);
#define HASTE_FIXED_DH(FF)                                                                           \
    if (det) {                                                                                       \
        raise_dyn_lds<k_fixed_bwd_h<FF, true>>(lds);                                                 \
        hipLaunchKernelGGL((k_fixed_bwd_h<FF, true>), grid, blk, lds, s, a);                         \
    } else {                                                                                         \
        raise_dyn_lds<k_fixed_bwd_h<FF, false>>(lds);                                                \
        hipLaunchKernelGGL((k_fixed_bwd_h<FF, false>), grid, blk, lds, s, a);                        \
    }                                                                                                \
    return true;
    switch (F) {
    case 32: HASTE_FIXED_DH(32)
    case 64: HASTE_FIXED_DH(64)
    case 128: HASTE_FIXED_DH(128)
    }
#undef HASTE_FIXED_DH
    return false;
}

}  // namespace haste

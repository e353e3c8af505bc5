// Forward family of the group-shared fixed fan-in layer.
//
// HASTE ("gather-once + dense MMA kernel" section of the paper notes): per
// group k the feature tile H_k = h[:, I_k] is gathered once and reused by all
// G labels of the group, and the logits of the group are the dense product
// Z_k = H_k W_k^T; the weight gradient is the dense product
// dW_k = dZ_k^T H_k.  The BCE gradient dZ = s (sigmoid(Z) - Y) of the
// objective in the "head-tail split" section is applied in registers.
//
// One wavefront owns one group at a time and walks a contiguous range of
// groups.  Per 32-row batch chunk it
//   1. gathers the chunk of H_k from the feature-major copy hT (row I_k[f] of
//      hT holds h[:, I_k[f]]): one 16-byte load per lane per 16 slots, rows
//      read whole, and keeps it in registers in the matrix-core B layout of
//      the weight-gradient product (slot f = lane % 16, eight consecutive
//      batch rows per lane);
//   2. writes the same values transposed into a wave-private LDS tile
//      [batch row][slot], which feeds the forward product's A operand;
//   3. runs Z_chunk = H_chunk W_k^T on 16x16x32 bf16 matrix cores;
//   4. applies the epilogue of the mode: store Z, or BCE -> store dZ, or
//      BCE -> dW_k += dZ_chunk^T H_chunk with dZ split into bf16 hi + lo.
// Batch rows of the forward product are permuted so that every lane ends up
// holding eight consecutive batch rows of one label, which is exactly the A
// layout of the weight-gradient product: no data moves between the two.
#include "common.hpp"
#include "kernels.hpp"

namespace haste {

// Wide variants (weight-gradient tiles of G x 128 or 64 x F) need more than
// 256 registers per lane; they run one workgroup per CU with up to 512.
constexpr int fwd_min_blocks(int G, int F, int mode)
{
    return ((mode == STEP_DW && (F == 128 || G == 64)) || (G == 64 && F == 128)) ? 1 : 2;
}

// Offset (16-bit elements) of (slot f, batch row b) in a wave's gathered tile
// [F slots][32 rows]: the 16-byte chunk index is XORed with (f/8) % 4 and the
// 8-byte half with (f/8) % 2, so the chunk writes and the transposing reads of
// one instruction spread over the banks.
__device__ __forceinline__ int tile_off(int f, int b)
{
    return f * 32 + ((((b >> 3) ^ (f >> 3)) & 3) << 3) + (((((b >> 2) ^ (f >> 3)) & 1)) << 2) + (b & 3);
}

template <int G, int F, int MODE, bool LOSS>
__global__ __launch_bounds__(256, fwd_min_blocks(G, F, MODE)) void k_group_fwd(FwdArgs a)
{
    constexpr int NT = F / 16;    // 16-slot tiles (gather units, dW columns)
    constexpr int KS = F / 32;    // contraction steps of the forward product
    constexpr int GT = G / 16;    // 16-label tiles
    constexpr bool LABELS = (MODE == FWD_BCE || MODE == STEP_DW);
    constexpr bool FWD = (MODE != BWD_W);          // runs the forward product
    constexpr bool DW = (MODE == STEP_DW || MODE == BWD_W);
    constexpr int DST = G + 2;                     // row stride of the dZ tile (BWD_W)
    // Prefetch the next group's weights only when they are small; wide tiles
    // would push the wave past 256 registers (two waves per SIMD).
    constexpr bool PF_W = FWD && (GT * KS <= 4);

    __shared__ __attribute__((aligned(16))) uint16_t sH[4][FWD ? 32 * F : 8];
    __shared__ uint64_t sM[4][LABELS ? kMaxLabelBatch : 1];
    __shared__ __attribute__((aligned(16))) uint16_t sD[4][MODE == BWD_W ? 32 * DST : 2];

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int r16 = lane & 15;
    const int q = lane >> 4;
    const int tr_r = r16 >> 2, tr_c = r16 & 3;   // transposing-read source position
    uint16_t* tile = sH[wv];

    const int64_t L = a.K * G;
    const int64_t nw = (int64_t)gridDim.x * 4;
    const int64_t gw = (int64_t)blockIdx.x * 4 + wv;
    const int64_t k0 = gw * a.K / nw;
    const int64_t k1 = (gw + 1) * a.K / nw;
    const int nchunk = (int)(a.Bp / 32);
    const float scale = a.scale;
    const float inv_s = 1.0f / a.scale;

    LabelCursor cur[4];
    if constexpr (LABELS) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            cur[s].init(a.y_rowptr, a.y_col, lane + 64 * s, a.B, k0 * G);
    }
    float lsum = 0.f;

    // Software pipeline: the index row and weights of the next group and the
    // gathered rows of the next batch chunk are requested one step ahead.
    auto load_col = [&](int64_t kk, int (&cl)[NT]) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            cl[t] = a.idx[kk * F + 16 * t + r16];
    };
    auto load_w = [&](int64_t kk, u32x4_t (&wr)[FWD ? GT : 1][FWD ? KS : 1]) {
        if constexpr (FWD) {
#pragma unroll
            for (int gt = 0; gt < GT; ++gt)
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    wr[gt][s] = ldg16(a.W + ((kk * G + 16 * gt + r16) * F + 32 * s + 8 * q));
        }
    };
    // gather: lane (slot 16t + r16, q) <- h[32c + 8q .. +8, I_k[slot]]
    auto gather = [&](const int (&cl)[NT], int c, u32x4_t (&hr)[NT]) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            hr[t] = ldg16(a.hT + (int64_t)cl[t] * a.Bp + 32 * c + 8 * q);
    };

    int col[NT], col_n[NT];
    u32x4_t wreg[FWD ? GT : 1][FWD ? KS : 1], wreg_n[PF_W ? GT : 1][PF_W ? KS : 1];
    u32x4_t hreg[NT], hnext[NT];
    if (k0 < k1) {
        load_col(k0, col);
        load_w(k0, wreg);
        gather(col, 0, hreg);
    }

    for (int64_t k = k0; k < k1; ++k) {
        const int64_t kn = k + 1 < k1 ? k + 1 : k;
        load_col(kn, col_n);
        if constexpr (PF_W) load_w(kn, wreg_n);
        else if (k != k0) load_w(k, wreg);

        bool anypos = false;
        if constexpr (LABELS) {
            uint64_t m[4];
            bool mine = false;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                m[s] = cur[s].take(k * G, G, a.y_col);
                mine |= (m[s] != 0);
            }
            anypos = __any(mine);
            if (anypos) {
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    sM[wv][lane + 64 * s] = m[s];
                wave_sync();
            }
        }

        f32x4_t dw[DW ? GT : 1][DW ? NT : 1];
        if constexpr (DW) {
#pragma unroll
            for (int gt = 0; gt < GT; ++gt)
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    dw[gt][t] = zero4();
        }

        for (int c = 0; c < nchunk; ++c) {
            // 1. rows of this chunk are in hreg; request the next chunk's rows
            if (c + 1 < nchunk) gather(col, c + 1, hnext);
            else gather(col_n, 0, hnext);
            if constexpr (MODE == BWD_W) {
                // dZ chunk rows 32c .. 32c+31 of the group's G columns into LDS
                uint16_t* dt = sD[wv];
#pragma unroll
                for (int it = 0; it < (32 * G / 8 + 63) / 64; ++it) {
                    const int ci = lane + 64 * it;
                    if (ci < 32 * G / 8) {
                        const int r = ci / (G / 8), gc = ci % (G / 8);
                        const int64_t b = 32 * c + r;
                        u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
                        if (b < a.B) v = ldg16(a.dZ + b * L + k * G + 8 * gc);
                        uint32_t* d32 = reinterpret_cast<uint32_t*>(dt + r * DST + 8 * gc);
                        d32[0] = v[0]; d32[1] = v[1]; d32[2] = v[2]; d32[3] = v[3];
                    }
                }
                wave_sync();
                // dW_k += dZ_chunk^T H_chunk; A lane (label r16, q): rows 8q + e
#pragma unroll
                for (int gt = 0; gt < GT; ++gt) {
                    const uint16_t* cp = dt + 8 * q * DST + 16 * gt + r16;
                    u32x4_t av;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        av[j] = (uint32_t)cp[(2 * j) * DST] | ((uint32_t)cp[(2 * j + 1) * DST] << 16);
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        dw[gt][t] = mfma16(av, hreg[t], dw[gt][t]);
                }
                wave_sync();
            } else {
                // 2. the same rows into the wave's LDS tile [slot][32 batch rows]
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const int f = 16 * t + r16;
                    u32x4_t v = hreg[t];
                    if ((f >> 3) & 1) v = u32x4_t{v[2], v[3], v[0], v[1]};
                    *reinterpret_cast<u32x4_t*>(tile + f * 32 + ((q ^ ((f >> 3) & 3)) << 3)) = v;
                }
                wave_sync();
                // 3. Z_chunk = H_chunk W_k^T with A = H read transposed from the
                //    tile.  A row m of tile mt is batch row 8*(m/4) + 4*mt + m%4, so
                //    result lane (label r16, q) holds batch rows 8q + 4*mt + i.
                f32x4_t z[2][GT];
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int gt = 0; gt < GT; ++gt)
                        z[mt][gt] = zero4();
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        const int f0 = 32 * s + 8 * q + tr_r;
                        const u32x4_t av = cat(lds_tr16(tile + tile_off(f0, 8 * tr_c + 4 * mt)),
                                               lds_tr16(tile + tile_off(f0 + 4, 8 * tr_c + 4 * mt)));
#pragma unroll
                        for (int gt = 0; gt < GT; ++gt)
                            z[mt][gt] = mfma16(av, wreg[gt][s], z[mt][gt]);
                    }
                }
                wave_sync();

                // 4. epilogue over batch rows b = 32c + 8q + 4mt + i, label g = 16gt + r16
                const int64_t bq = 32 * c + 8 * q;
                if constexpr (MODE == FWD_Z) {
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int64_t b = bq + 4 * mt + i;
                            if (b < a.B) {
#pragma unroll
                                for (int gt = 0; gt < GT; ++gt)
                                    a.Z[b * L + k * G + 16 * gt + r16] = z[mt][gt][i];
                            }
                        }
                } else {
                    float dz[2][GT][4];
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int64_t b = bq + 4 * mt + i;
                            const bool valid = b < a.B;
                            const uint64_t mrow = anypos ? sM[wv][b & (kMaxLabelBatch - 1)] : 0ull;
#pragma unroll
                            for (int gt = 0; gt < GT; ++gt) {
                                const float zz = z[mt][gt][i];
                                const bool y = (mrow >> (16 * gt + r16)) & 1ull;
                                float d;
                                if constexpr (LOSS) {
                                    // u = e^-|z|; sigmoid(|z|) = 1/(1+u); sigmoid(-|z|) = u/(1+u)
                                    const float u = __builtin_amdgcn_exp2f(-fabsf(zz) * kLog2e);
                                    const float r = __builtin_amdgcn_rcpf(1.0f + u);
                                    const float sg = zz >= 0.f ? r : u * r;
                                    d = scale * sg;
                                    const float le = fmaxf(zz, 0.f) + __builtin_amdgcn_logf(1.0f + u) * kLn2 -
                                                     (y ? zz : 0.f);
                                    lsum += valid ? le : 0.f;
                                } else {
                                    // s * sigmoid(z) = 1 / ((1 + e^-z) / s); e^-z = +inf gives 0
                                    const float t = __builtin_amdgcn_exp2f(-zz * kLog2e);
                                    d = __builtin_amdgcn_rcpf(fmaf(t, inv_s, inv_s));
                                }
                                if (y) d -= scale;
                                dz[mt][gt][i] = d;
                                if constexpr (MODE == FWD_BCE) {
                                    if (valid) {
                                        const int64_t o = b * L + k * G + 16 * gt + r16;
                                        a.dZ[o] = (uint16_t)(pack_bf16(d, 0.f) & 0xffffu);
                                        if (a.Z) a.Z[o] = zz;
                                    }
                                } else {
                                    if (valid && a.Z) a.Z[b * L + k * G + 16 * gt + r16] = zz;
                                }
                            }
                        }
                    if constexpr (MODE == STEP_DW) {
                        // dW_k += dZ_chunk^T H_chunk; A = dZ^T (label r16, rows 8q + e),
                        // contraction element e <-> batch row 32c + 8q + e on both sides.
#pragma unroll
                        for (int gt = 0; gt < GT; ++gt) {
                            u32x4_t ahi, alo;
                            { const u32x2_t _p = split_pair(dz[0][gt][0], dz[0][gt][1]); ahi[0] = _p[0]; alo[0] = _p[1]; }
                            { const u32x2_t _p = split_pair(dz[0][gt][2], dz[0][gt][3]); ahi[1] = _p[0]; alo[1] = _p[1]; }
                            { const u32x2_t _p = split_pair(dz[1][gt][0], dz[1][gt][1]); ahi[2] = _p[0]; alo[2] = _p[1]; }
                            { const u32x2_t _p = split_pair(dz[1][gt][2], dz[1][gt][3]); ahi[3] = _p[0]; alo[3] = _p[1]; }
#pragma unroll
                            for (int t = 0; t < NT; ++t) {
                                dw[gt][t] = mfma16(ahi, hreg[t], dw[gt][t]);
                                dw[gt][t] = mfma16(alo, hreg[t], dw[gt][t]);
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < NT; ++t)
                hreg[t] = hnext[t];
        }

        if constexpr (DW) {
            // result lane (slot 16t + r16, q) holds labels 16gt + 4q + i
#pragma unroll
            for (int gt = 0; gt < GT; ++gt)
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        a.dW[(k * G + 16 * gt + 4 * q + i) * F + 16 * t + r16] = dw[gt][t][i];
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
            col[t] = col_n[t];
        if constexpr (PF_W) {
#pragma unroll
            for (int gt = 0; gt < GT; ++gt)
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    wreg[gt][s] = wreg_n[gt][s];
        }
    }

    if constexpr (LOSS) {
        const float tot = wave_sum(lsum);
        if (lane == 0) atomicAdd(a.loss, (double)tot * (double)scale);
    }
}

template <int G, int F>
static bool launch_gf(int mode, bool loss, const FwdArgs& a, int grid, hipStream_t s)
{
    switch (mode) {
    case FWD_Z:
        hipLaunchKernelGGL((k_group_fwd<G, F, FWD_Z, false>), dim3(grid), dim3(256), 0, s, a);
        return true;
    case FWD_BCE:
        if (loss) hipLaunchKernelGGL((k_group_fwd<G, F, FWD_BCE, true>), dim3(grid), dim3(256), 0, s, a);
        else hipLaunchKernelGGL((k_group_fwd<G, F, FWD_BCE, false>), dim3(grid), dim3(256), 0, s, a);
        return true;
    case STEP_DW:
        if (loss) hipLaunchKernelGGL((k_group_fwd<G, F, STEP_DW, true>), dim3(grid), dim3(256), 0, s, a);
        else hipLaunchKernelGGL((k_group_fwd<G, F, STEP_DW, false>), dim3(grid), dim3(256), 0, s, a);
        return true;
    case BWD_W:
        hipLaunchKernelGGL((k_group_fwd<G, F, BWD_W, false>), dim3(grid), dim3(256), 0, s, a);
        return true;
    }
    return false;
}

template <int G>
static bool launch_g(int F, int mode, bool loss, const FwdArgs& a, int grid, hipStream_t s)
{
    switch (F) {
    case 32: return launch_gf<G, 32>(mode, loss, a, grid, s);
    case 64: return launch_gf<G, 64>(mode, loss, a, grid, s);
    case 128: return launch_gf<G, 128>(mode, loss, a, grid, s);
    }
    return false;
}

bool launch_fwd(int G, int F, int mode, bool loss, const FwdArgs& a, int grid, hipStream_t s)
{
    switch (G) {
    case 16: return launch_g<16>(F, mode, loss, a, grid, s);
    case 32: return launch_g<32>(F, mode, loss, a, grid, s);
    case 64: return launch_g<64>(F, mode, loss, a, grid, s);
    }
    return false;
}

}  // namespace haste

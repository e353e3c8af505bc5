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
//   1. has the chunk of H_k in registers, gathered from the feature-major
//      copy hT (row I_k[f] of hT holds h[:, I_k[f]]) with one 16-byte load
//      per lane per 16 slots; each quad of lanes reads 64 contiguous bytes of
//      one row, so an instruction asks for 16 cache lines, not 64; the next
//      chunk's rows are requested meanwhile;
//   2. writes them into a wave-private LDS tile [slot][row] and reads them
//      back K-contiguous with transposing LDS reads as the A operand of the
//      forward product, and row-wise as the B operand of the weight-gradient
//      product (slot f = lane % 16, eight consecutive batch rows per lane);
//   3. runs Z_chunk = H_chunk W_k^T on 16x16x32 bf16 matrix cores;
//   4. applies the epilogue of the mode: store Z, or BCE -> store dZ, or
//      BCE -> dW_k += dZ_chunk^T H_chunk with dZ split into bf16 hi + lo.
// Batch rows of the forward product are permuted so that every lane ends up
// holding eight consecutive batch rows of one label, which is exactly the A
// layout of the weight-gradient product: no data moves between the two.
//
// Vector-memory operations retire in issue order, so waiting for one load
// also waits for every older one, and loads share their counter with stores.
// Each chunk therefore first waits for its own rows, then issues the stores
// deferred from the previous chunk or group (staged in LDS), then the loads
// of the next chunk and, once per group, the next group's weights.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace haste {

// Wide variants (weight-gradient tiles of G x 128 or 64 x F) need more than
// 256 registers per lane; they run one workgroup per CU with up to 512.
// The fused G = 16, F = 128 step fits two waves per SIMD (256 registers,
// under 80 KB of LDS) without prefetching the next group's weights, and
// gains more from the second wave's latency hiding than it loses.
constexpr int fwd_min_blocks(int G, int F, int mode)
{
    return ((mode == STEP_DW && ((F == 128 && G > 16) || G == 64)) || (G == 64 && F == 128)) ? 1 : 2;
}

// Offset (16-bit elements) of (slot f, batch row b) in a wave's gathered tile
// [F slots][32 rows]: the 16-byte chunk index is XORed with (f/8) % 4 so the
// transposing reads of one instruction spread over more banks.
__device__ __forceinline__ int tile_off(int f, int b)
{
    return f * 32 + ((((b >> 3) ^ (f >> 3)) & 3) << 3) + (b & 7);
}

// WZ: also write the fp32 logits (optional output of the BCE modes).
// WQ: the weights come as FP8 E4M3 codes with one power-of-two scale per
// group (a.W8, a.wexp); they are widened to exact bf16 values on their way
// into LDS, so the arithmetic is that of the bf16 kernel on those values.
// DWB (fused step only): the weight gradient is stored as bf16 (a.dW16), each
// value the fp32 accumulator rounded to nearest even: half the dW bytes.
template <int G, int F, int MODE, bool LOSS, bool WZ, bool WQ = false, bool DWB = false>
__global__ __launch_bounds__(256, fwd_min_blocks(G, F, MODE)) void k_group_fwd(FwdArgs a)
{
    static_assert(!DWB || MODE == STEP_DW, "a bf16 weight gradient is an option of the fused step");
    constexpr int NT = F / 16;    // 16-slot tiles (gather units, dW columns)
    constexpr int KS = F / 32;    // contraction steps of the forward product
    constexpr int GT = G / 16;    // 16-label tiles
    constexpr bool LABELS = (MODE == FWD_BCE || MODE == STEP_DW);
    constexpr bool FWD = (MODE != BWD_W);          // runs the forward product
    constexpr bool DW = (MODE == STEP_DW || MODE == BWD_W);
    constexpr bool STORE_Z = (MODE == FWD_Z) || WZ;
    constexpr bool STORE_DZ = (MODE == FWD_BCE);
    constexpr int DST = G + 2;                     // row stride of the dZ input tile (BWD_W)
    constexpr int NDZ = (32 * G / 8 + 63) / 64;    // 16-byte dZ pieces per lane per chunk (BWD_W)
    // Prefetch the next group's weights only when they are small; wide tiles
    // would push the wave past 256 registers (two waves per SIMD).
    constexpr bool PF_W = FWD && (GT * KS <= 4) && !(MODE == STEP_DW && G == 16 && F == 128);
    // Four-chunk groups run as two chunk pairs where the registers for a
    // second set of inputs are there (see the chunk loop); with per-chunk
    // outputs the pair's two chunks are staged in two buffers.
    constexpr bool PAIRS_Z = (MODE == FWD_Z || (MODE == FWD_BCE && !LOSS && !WZ)) && F <= 64 && G <= 32;
    constexpr bool PAIRS = (((MODE == STEP_DW && !WZ && !LOSS && PF_W) || (MODE == BWD_W && G * F <= 2048)) &&
                            fwd_min_blocks(G, F, MODE) == 2) ||
                           PAIRS_Z;
    constexpr int ZB = PAIRS_Z ? 2 : 1;   // Z / dZ staging buffers
    // Output staging in LDS (row strides padded by 4 floats / 8 halves).  A
    // group's whole dW is staged and stored after the next group's first
    // wait when it fits; wide tiles go out per 16-label tile at once.
    constexpr int ZST = G + 4, DZST = G + 8, WST = F + 4;
    constexpr bool DEFER_DW = DW && (G * WST <= 2304);
    constexpr int DW_ROWS = DEFER_DW ? G : 16;
    // wide fused tiles with the optional Z output share one staging area
    // (Z is flushed before dW is staged)
    constexpr bool ALIAS_WZ = DW && !DEFER_DW && STORE_Z;
    constexpr int WO_SIZE = DW ? (ALIAS_WZ && 32 * ZST > DW_ROWS * WST ? 32 * ZST : DW_ROWS * WST) : 4;

    // W_k passes through LDS once per group, before the group's first chunk
    // is written to the gathered tile: for G <= 32 it fits in that tile.
    constexpr bool W_IN_H = (G <= 32);
    // label bits of one batch row: the group's G labels
    using MaskT = typename pick<(G <= 16), uint16_t, typename pick<(G <= 32), uint32_t, uint64_t>::type>::type;
    __shared__ __attribute__((aligned(16))) uint16_t sH[4][32 * F];
    __shared__ __attribute__((aligned(16))) uint16_t sWk[4][FWD && !W_IN_H ? G * F : 8];
    __shared__ MaskT sM[4][LABELS ? kMaxLabelBatch : 1];
    __shared__ __attribute__((aligned(16))) uint16_t sD[4][MODE == BWD_W ? 32 * DST : 2];
    __shared__ __attribute__((aligned(16))) float sWo[4][WO_SIZE];
    __shared__ __attribute__((aligned(16))) float sZo[4][ZB][STORE_Z && !ALIAS_WZ ? 32 * ZST : 4];
    __shared__ __attribute__((aligned(16))) uint16_t sDo[4][ZB][STORE_DZ ? 32 * DZST : 8];

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int r16 = lane & 15;
    const int q = lane >> 4;
    const int tr_r = r16 >> 2, tr_c = r16 & 3;   // transposing-read source position
    const int qr = lane >> 2, qc = lane & 3;     // quad-contiguous load position
    uint16_t* tile = sH[wv];

    const int64_t L = a.K * G;
    const int64_t nw = (int64_t)gridDim.x * 4;
    const int64_t gw = (int64_t)blockIdx.x * 4 + wv;
    // Group order.  The logits-only forward and the standalone dW take groups
    // gw, gw + nw, gw + 2 nw, ...: the waves in flight then write (Z) or read
    // (dZ) neighbouring column blocks of the same B x L rows, which measured
    // 2-12 % faster than one contiguous range per wave; so does the
    // standalone BCE forward at G = 16 (its plain dZ stores of neighbouring
    // groups then meet in L2: 339 -> 297 us at the 670K shape).  The other
    // label-driven cases keep contiguous ranges (strided, the fused step
    // measured 11-14 % slower and the BCE forward 8 % slower at 3M).
    constexpr bool STRIDED = (MODE == FWD_Z || MODE == BWD_W || (MODE == FWD_BCE && G < 32));
    const int64_t kstep = STRIDED ? nw : 1;
    const int64_t k0 = STRIDED ? gw : gw * a.K / nw;
    const int64_t k1 = STRIDED ? a.K : (gw + 1) * a.K / nw;
    const int nchunk = (int)(a.Bp / 32);
    const int wchunk = nchunk >= 2 ? 1 : 0;   // chunk that requests the next group's weights
    const float scale = a.scale;
    const float inv_s = 1.0f / a.scale;

    LabelCursor cur[4];
    if constexpr (LABELS) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            cur[s].init(a.y_rowptr, a.y_col, lane + 64 * s, a.B, k0 * G);
    }
    float lsum = 0.f;

    // index entries of the lane's gather slots 16t + qr
    auto load_col = [&](int64_t kk, int (&cl)[NT]) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            cl[t] = a.idx[kk * F + 16 * t + qr];
    };
    // W_k (G x F, contiguous) as pieces of eight weights, lane + 64 p in
    // order: 16 bytes of bf16, or 8 bytes of FP8 codes plus the group's exponent
    constexpr int NWP = FWD ? (G * F / 8 + 63) / 64 : 1;
    using WPiece = typename pick<WQ, u32x2_t, u32x4_t>::type;
    int wex = 0;
    // Non-temporal weight loads (read once; they leave L2 to the gathered
    // rows): measured faster in every mode and shape but the logits-only
    // forward at F = 128 (381 against 213 us at the 670K shape).
    constexpr bool W_STREAM = !(MODE == FWD_Z && F == 128);
    auto load_w = [&](int64_t kk, WPiece (&wr)[NWP]) {
        if constexpr (FWD) {
#pragma unroll
            for (int p = 0; p < NWP; ++p) {
                if constexpr (WQ) wr[p] = ldg8_stream(a.W8 + kk * G * F + 8 * (lane + 64 * p));
                else if constexpr (W_STREAM) wr[p] = ldg16_stream(a.W + kk * G * F + 8 * (lane + 64 * p));
                else wr[p] = ldg16(a.W + kk * G * F + 8 * (lane + 64 * p));
            }
            if constexpr (WQ) wex = a.wexp[kk];
        }
    };
    // gather: lane (slot 16t + qr, quad position qc) <- h[32c + 8qc .. +8, I_k[slot]];
    // the row pointers of a group are formed once and reused for its chunks
    // (as 32-bit byte offsets into hT, which holds H x Bp < 2^31 bytes)
    auto rows_of = [&](const int (&cl)[NT], uint32_t (&gp)[NT]) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            gp[t] = 2u * ((uint32_t)cl[t] * (uint32_t)a.Bp + 8u * (uint32_t)qc);
    };
    auto gather = [&](const uint32_t (&gp)[NT], int c, u32x4_t (&hr)[NT]) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            hr[t] = ldg16(reinterpret_cast<const char*>(a.hT) + (gp[t] + 64u * (uint32_t)c));
    };
    // BWD_W: lane's 16-byte pieces of the chunk's dZ rows (piece ci = lane + 64 it:
    // row ci / (G/8), labels 8 (ci % (G/8)) .. +8 of the group)
    auto load_dz = [&](int64_t kk, int c, u32x4_t (&dv)[NDZ]) {
#pragma unroll
        for (int it = 0; it < NDZ; ++it) {
            const int ci = lane + 64 * it;
            const int64_t b = 32 * c + ci / (G / 8);
            dv[it] = u32x4_t{0u, 0u, 0u, 0u};
            if (ci < 32 * G / 8 && b < a.B) dv[it] = ldg16(a.dZ + b * L + kk * G + 8 * (ci % (G / 8)));
        }
    };

    // Deferred stores.  Vector-memory loads and stores share one counter, and
    // a wait for a load while a store is outstanding drains everything, so
    // outputs are staged in LDS and stored right after the next wait for
    // input data, a whole chunk of work before the next wait.
    int64_t pend_dw = -1;                    // group whose dW sits in sWo
    int64_t pend_zk = -1;                    // group and chunk whose Z / dZ sit in sZo / sDo
    int pend_zc = 0;
    auto flush_dw = [&]() {
        if constexpr (DEFER_DW) {
            if (pend_dw >= 0) {
                const float* so = sWo[wv];
                constexpr int NP = (G * F / 4 + 63) / 64;
#pragma unroll
                for (int pp = 0; pp < NP; ++pp) {
                    const int u = lane + 64 * pp;
                    const int g = u / (F / 4), cc = u % (F / 4);
                    if (u < G * F / 4) {
                        const int64_t o = (pend_dw * G + g) * F + 4 * cc;
                        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(so + g * WST + 4 * cc);
                        // plain stores in the fused step (non-temporal ones
                        // measured 13 % slower there); the standalone call streams
                        if constexpr (DWB)
                            *reinterpret_cast<u32x2_t*>(a.dW16 + o) = u32x2_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
                        else if constexpr (MODE == STEP_DW) *reinterpret_cast<f32x4_t*>(a.dW + o) = v;
                        else stg_stream(a.dW + o, v);
                    }
                }
                pend_dw = -1;
            }
        }
    };
    // the staged Z / dZ rows of chunk cz of group pend_zk, from buffer zb
    auto store_zc = [&](int zb, int cz) {
        if constexpr (STORE_Z || STORE_DZ) {
            if constexpr (STORE_Z) {
                // piece u: chunk row u / (G/4), labels 4 (u % (G/4)) ..
                const float* so = ALIAS_WZ ? sWo[wv] : sZo[wv][zb];
                constexpr int NP = (8 * G + 63) / 64;
#pragma unroll
                for (int pp = 0; pp < NP; ++pp) {
                    const int u = lane + 64 * pp;
                    const int lr = u / (G / 4), cc = u % (G / 4);
                    const int64_t b = 32 * cz + lr;
                    if (u < 8 * G && b < a.B)
                        stg_stream(a.Z + b * L + pend_zk * G + 4 * cc,
                                   *reinterpret_cast<const f32x4_t*>(so + lr * ZST + 4 * cc));
                }
            }
            if constexpr (STORE_DZ) {
                // piece u: chunk row u / (G/8), labels 8 (u % (G/8)) ..
                const uint16_t* so = sDo[wv][zb];
                constexpr int NP = (4 * G + 63) / 64;
#pragma unroll
                for (int pp = 0; pp < NP; ++pp) {
                    const int u = lane + 64 * pp;
                    const int lr = u / (G / 8), cc = u % (G / 8);
                    const int64_t b = 32 * cz + lr;
                    // a group's row segment is 2G bytes: at G = 16 half a
                    // 64-byte run, so plain stores that L2 can merge with the
                    // neighbouring group's (546 -> 340 us at the 670K shape);
                    // streaming ones for G >= 32 (5-6 % faster there)
                    if (u < 4 * G && b < a.B) {
                        uint16_t* dst = a.dZ + b * L + pend_zk * G + 8 * cc;
                        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(so + lr * DZST + 8 * cc);
                        if constexpr (G < 32) *reinterpret_cast<u32x4_t*>(dst) = v;
                        else stg_stream(dst, v);
                    }
                }
            }
        }
    };
    // (with pairs: both chunks of the pending pair, from their two buffers)
    auto flush_z = [&]() {
        if constexpr (STORE_Z || STORE_DZ) {
            if (pend_zk >= 0) {
#pragma unroll
                for (int zb = 0; zb < ZB; ++zb)
                    store_zc(zb, pend_zc + zb);
                pend_zk = -1;
            }
        }
    };

    int col[NT], col_n[NT];
    uint32_t gp[NT];
    WPiece wraw[NWP];                       // weights as loaded
    u32x4_t wreg[FWD ? GT : 1][FWD ? KS : 1];
    // Modes without per-chunk outputs (and registers to spare) run four-chunk
    // groups as two chunk pairs: a pair's inputs
    // are requested a whole pair ahead (sets A2 / B2 hold the second chunk),
    // the next group's weights at the group's first pair, and a group's dW
    // goes out after the wait of the next group's last pair.  Each load so
    // gets two chunks (the weights a group) before the wait that needs it:
    // vector memory operations retire in issue order, so a wait for a
    // chunk's rows also waits for every older load.
    constexpr int NT2 = NT, NDZ2 = MODE == BWD_W ? NDZ : 1;   // second-chunk sets (unused without pairs)
    u32x4_t hA[NT], hB[NT], hA2[NT2], hB2[NT2];
    u32x4_t dA[MODE == BWD_W ? NDZ : 1], dB[MODE == BWD_W ? NDZ : 1], dA2[NDZ2], dB2[NDZ2];
    if (k0 < k1) {
        load_col(k0, col);
        if constexpr (!PAIRS) load_w(k0, wraw);
        rows_of(col, gp);
        gather(gp, 0, hA);
        if constexpr (MODE == BWD_W) load_dz(k0, 0, dA);
        if (PAIRS && nchunk == 4) {
            gather(gp, 1, hA2);
            if constexpr (MODE == BWD_W) load_dz(k0, 1, dA2);
        }
        if constexpr (PAIRS) load_w(k0, wraw);
    }

    for (int64_t k = k0; k < k1; k += kstep) {
        const int64_t kn = k + kstep < k1 ? k + kstep : k;
        // the next group's index entries: needed by the last chunk's request,
        // so they are loaded before any chunk of this group
        load_col(kn, col_n);
        if constexpr (FWD) {
            // this group's weights: through LDS into the matrix-core B layout
            // of the forward product (lane (label 16gt + r16, q): slots 32s + 8q ..)
            uint16_t* wk = W_IN_H ? tile : sWk[wv];
            if constexpr (!PF_W) {
                if (k != k0) load_w(k, wraw);
            }
            // 16-byte piece j of label row g sits at piece j ^ (g % (F/8)) of the row
            constexpr int PR = F / 8;
            const float wsc = WQ ? __builtin_amdgcn_ldexpf(1.0f, wex) : 1.0f;
#pragma unroll
            for (int p = 0; p < NWP; ++p) {
                const int u = lane + 64 * p;
                if (u < G * PR)
                    *reinterpret_cast<u32x4_t*>(wk + (u / PR) * F + 8 * ((u ^ (u / PR)) & (PR - 1))) =
                        widen_w8(wraw[p], wsc);
            }
            wave_sync();
#pragma unroll
            for (int gt = 0; gt < GT; ++gt)
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const int g = 16 * gt + r16;
                    wreg[gt][s] = *reinterpret_cast<const u32x4_t*>(wk + g * F + 8 * (((4 * s + q) ^ g) & (PR - 1)));
                }
        }

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
                    sM[wv][lane + 64 * s] = (MaskT)m[s];
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

        // one 32-row chunk: rows in hc (and dZ pieces in dc for BWD_W).  Kind
        // 0 / 1: single-chunk schedule (0 issues the deferred dW stores), the
        // next chunk's inputs go to hn / dn.  Kind 3: second chunk of a pair.
        // Kinds 5 and 6: first chunk of the first / last pair of a four-chunk
        // group; the pair's second chunk sits in hc2 and the next pair's
        // inputs go to (hn, hn2): chunks 2, 3 of this group and the next
        // group's weights (5), or chunks 0, 1 of the next group after the
        // deferred dW stores (6).
        auto chunk = [&](auto kind, int c, u32x4_t (&hc)[NT], u32x4_t (&hn)[NT],
                         u32x4_t (&dc)[MODE == BWD_W ? NDZ : 1], u32x4_t (&dn)[MODE == BWD_W ? NDZ : 1],
                         u32x4_t (&hc2)[NT2], u32x4_t (&hn2)[NT2], u32x4_t (&dc2)[NDZ2], u32x4_t (&dn2)[NDZ2]) {
            constexpr int KIND = decltype(kind)::value;
            // 1. this chunk's rows into the wave's LDS tile [slot][32 batch rows]
            //    (the wait for the chunk's loads)
#pragma unroll
            for (int t = 0; t < NT; ++t)
                *reinterpret_cast<u32x4_t*>(tile + tile_off(16 * t + qr, 8 * qc)) = hc[t];
            if constexpr (MODE == BWD_W) {
                // dZ chunk into LDS [row][label]
                uint16_t* dt = sD[wv];
#pragma unroll
                for (int it = 0; it < NDZ; ++it) {
                    const int ci = lane + 64 * it;
                    if (ci < 32 * G / 8) {
                        const int r = ci / (G / 8), gc = ci % (G / 8);
                        uint32_t* d32 = reinterpret_cast<uint32_t*>(dt + r * DST + 8 * gc);
                        d32[0] = dc[it][0]; d32[1] = dc[it][1]; d32[2] = dc[it][2]; d32[3] = dc[it][3];
                    }
                }
            }
            if constexpr (KIND >= 5) {
                // the pair's second chunk counts as arrived here, before any
                // store is issued (see settle)
#pragma unroll
                for (int t = 0; t < NT2; ++t) settle(hc2[t]);
                if constexpr (MODE == BWD_W) {
#pragma unroll
                    for (int it = 0; it < NDZ2; ++it) settle(dc2[it]);
                }
            }
            // 2. stores deferred from the previous chunk (pair) / group
            if constexpr (KIND != 3) flush_z();
            if constexpr (KIND == 0 || KIND == 6) flush_dw();
            // 3. requests: the next chunk or pair (or the next group's first),
            //    and once per group the next group's weights
            if constexpr (KIND < 2) {
                if (c + 1 < nchunk) {
                    gather(gp, c + 1, hn);
                    if constexpr (MODE == BWD_W) load_dz(k, c + 1, dn);
                } else {
                    uint32_t gpn[NT];
                    rows_of(col_n, gpn);
                    gather(gpn, 0, hn);
                    if constexpr (MODE == BWD_W) load_dz(kn, 0, dn);
                }
                if constexpr (PF_W) {
                    if (c == wchunk) load_w(kn, wraw);
                }
            } else if constexpr (KIND == 5) {
                gather(gp, 2, hn);
                gather(gp, 3, hn2);
                if constexpr (MODE == BWD_W) {
                    load_dz(k, 2, dn);
                    load_dz(k, 3, dn2);
                }
                if constexpr (PF_W) load_w(kn, wraw);
            } else if constexpr (KIND == 6) {
                uint32_t gpn[NT];
                rows_of(col_n, gpn);
                gather(gpn, 0, hn);
                gather(gpn, 1, hn2);
                if constexpr (MODE == BWD_W) {
                    load_dz(kn, 0, dn);
                    load_dz(kn, 1, dn2);
                }
            }
            wave_sync();
            // B operand of the weight-gradient product: lane (slot 16t + r16, q)
            // holds batch rows 32c + 8q .. +8
            auto hrow = [&](int t) {
                return *reinterpret_cast<const u32x4_t*>(tile + tile_off(16 * t + r16, 8 * q));
            };
            if constexpr (MODE == BWD_W) {
                // dW_k += dZ_chunk^T H_chunk; A lane (label r16, q): rows 8q + e
                const uint16_t* dt = sD[wv];
#pragma unroll
                for (int gt = 0; gt < GT; ++gt) {
                    const uint16_t* cp = dt + 8 * q * DST + 16 * gt + r16;
                    u32x4_t av;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        av[j] = (uint32_t)cp[(2 * j) * DST] | ((uint32_t)cp[(2 * j + 1) * DST] << 16);
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        dw[gt][t] = mfma16(av, hrow(t), dw[gt][t]);
                }
                wave_sync();
                return;
            } else {
                // 4. Z_chunk = H_chunk W_k^T with A = H read transposed from the
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

                // 5. epilogue over batch rows b = 32c + 8q + 4mt + i, label g = 16gt + r16;
                //    chunk outputs are staged for the deferred store (chunk row 8q + 4mt + i)
                const int64_t bq = 32 * c + 8 * q;
                if constexpr (STORE_Z) {
                    float* so = ALIAS_WZ ? sWo[wv] : sZo[wv][ZB > 1 ? (c & 1) : 0];
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int gt = 0; gt < GT; ++gt)
                                so[(8 * q + 4 * mt + i) * ZST + 16 * gt + r16] = z[mt][gt][i];
                }
                if constexpr (MODE != FWD_Z) {
                    float dz[2][GT][4];
                    if constexpr (!LOSS) {
                        // s * sigmoid(z) = 1 / ((1 + e^-z) / s), and e^-z = +inf gives 0
#pragma unroll
                        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                            for (int gt = 0; gt < GT; ++gt)
#pragma unroll
                                for (int i = 0; i < 4; ++i) {
                                    const float t = __builtin_amdgcn_exp2f(-z[mt][gt][i] * kLog2e);
                                    dz[mt][gt][i] = __builtin_amdgcn_rcpf(fmaf(t, inv_s, inv_s));
                                }
                        if (anypos) {   // rare: positive labels in this group
#pragma unroll
                            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                                for (int i = 0; i < 4; ++i) {
                                    const uint64_t mrow = sM[wv][(bq + 4 * mt + i) & (kMaxLabelBatch - 1)];
#pragma unroll
                                    for (int gt = 0; gt < GT; ++gt)
                                        if ((mrow >> (16 * gt + r16)) & 1ull) dz[mt][gt][i] -= scale;
                                }
                        }
                    } else {
                        // with the loss l = max(z, 0) + ln(1 + e^-|z|) - y z per
                        // valid row: the logarithms of the lane's 8 GT terms are
                        // taken once, as the log of their product (each factor
                        // 1 + e^-|z| lies in [1, 2], so the product stays below 2^32)
                        float prod = 1.f, lin = 0.f;
#pragma unroll
                        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const bool valid = bq + 4 * mt + i < a.B;
#pragma unroll
                                for (int gt = 0; gt < GT; ++gt) {
                                    const float zz = z[mt][gt][i];
                                    // u = e^-|z|; sigmoid(|z|) = 1/(1+u); sigmoid(-|z|) = u/(1+u)
                                    const float u = __builtin_amdgcn_exp2f(-fabsf(zz) * kLog2e);
                                    const float w1 = 1.0f + u;
                                    const float r = __builtin_amdgcn_rcpf(w1);
                                    dz[mt][gt][i] = scale * (zz >= 0.f ? r : u * r);
                                    prod *= valid ? w1 : 1.0f;
                                    lin += valid ? fmaxf(zz, 0.f) : 0.f;
                                }
                            }
                        if (anypos) {   // rare: positive labels in this group
#pragma unroll
                            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                                for (int i = 0; i < 4; ++i) {
                                    const int64_t b = bq + 4 * mt + i;
                                    const uint64_t mrow = sM[wv][b & (kMaxLabelBatch - 1)];
#pragma unroll
                                    for (int gt = 0; gt < GT; ++gt)
                                        if ((mrow >> (16 * gt + r16)) & 1ull) {
                                            dz[mt][gt][i] -= scale;
                                            if (b < a.B) lin -= z[mt][gt][i];
                                        }
                                }
                        }
                        lsum += lin + __builtin_amdgcn_logf(prod) * kLn2;
                    }
                    if constexpr (STORE_DZ) {
                        uint16_t* so = sDo[wv][ZB > 1 ? (c & 1) : 0];
#pragma unroll
                        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
#pragma unroll
                                for (int gt = 0; gt < GT; ++gt)
                                    so[(8 * q + 4 * mt + i) * DZST + 16 * gt + r16] =
                                        (uint16_t)(pack_bf16(dz[mt][gt][i], 0.f) & 0xffffu);
                    }
                    if constexpr (MODE == STEP_DW) {
                        // dW_k += dZ_chunk^T H_chunk; A = dZ^T (label r16, rows 8q + e),
                        // contraction element e <-> batch row 32c + 8q + e on both sides.
                        // Padding rows carry zero features, so they add nothing.
#pragma unroll
                        for (int gt = 0; gt < GT; ++gt) {
                            u32x4_t ahi, alo;
                            { const u32x2_t p = split_pair(dz[0][gt][0], dz[0][gt][1]); ahi[0] = p[0]; alo[0] = p[1]; }
                            { const u32x2_t p = split_pair(dz[0][gt][2], dz[0][gt][3]); ahi[1] = p[0]; alo[1] = p[1]; }
                            { const u32x2_t p = split_pair(dz[1][gt][0], dz[1][gt][1]); ahi[2] = p[0]; alo[2] = p[1]; }
                            { const u32x2_t p = split_pair(dz[1][gt][2], dz[1][gt][3]); ahi[3] = p[0]; alo[3] = p[1]; }
#pragma unroll
                            for (int t = 0; t < NT; ++t) {
                                const u32x4_t hb = hrow(t);
                                dw[gt][t] = mfma16(ahi, hb, dw[gt][t]);
                                dw[gt][t] = mfma16(alo, hb, dw[gt][t]);
                            }
                        }
                    }
                }
                if constexpr (STORE_Z || STORE_DZ) {
                    pend_zk = k;
                    pend_zc = ZB > 1 ? (c & ~1) : c;
                }
                wave_sync();
            }
        };

        if (PAIRS && nchunk == 4) {
            // four chunks in two pairs: (0, 1) from the A sets requests (2, 3)
            // into the B sets, (2, 3) requests the next group's (0, 1) into A
            const std::integral_constant<int, 5> pfirst;
            const std::integral_constant<int, 6> plast;
            const std::integral_constant<int, 3> psecond;
            chunk(pfirst, 0, hA, hB, dA, dB, hA2, hB2, dA2, dB2);
            chunk(psecond, 1, hA2, hB, dA2, dB, hA2, hB2, dA2, dB2);
            chunk(plast, 2, hB, hA, dB, dA, hB2, hA2, dB2, dA2);
            chunk(psecond, 3, hB2, hA, dB2, dA, hB2, hA2, dB2, dA2);
        } else {
            // Chunk 0 (which issues the deferred dW stores) is peeled off, so
            // the chunk loop holds no stores and its waits stay exact; the rest
            // run in pairs so the register buffers alternate without copies.
            const std::integral_constant<int, 0> first;
            const std::integral_constant<int, 1> later;
            chunk(first, 0, hA, hB, dA, dB, hA2, hB2, dA2, dB2);
            int c = 1;
            for (; c + 1 < nchunk; c += 2) {
                chunk(later, c, hB, hA, dB, dA, hA2, hB2, dA2, dB2);
                chunk(later, c + 1, hA, hB, dA, dB, hA2, hB2, dA2, dB2);
            }
            if (c < nchunk) {
                chunk(later, c, hB, hA, dB, dA, hA2, hB2, dA2, dB2);
            } else {
                // odd chunk count: the next group's first rows landed in the B set
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    hA[t] = hB[t];
                if constexpr (MODE == BWD_W) {
#pragma unroll
                    for (int it = 0; it < NDZ; ++it)
                        dA[it] = dB[it];
                }
            }
        }

        if constexpr (DW) {
            // result lane (slot 16t + r16, q) holds labels 16gt + 4q + i; staged in
            // LDS so the stores are contiguous 16-byte pieces
            float* so = sWo[wv];
            if constexpr (DEFER_DW) {
#pragma unroll
                for (int gt = 0; gt < GT; ++gt)
#pragma unroll
                    for (int t = 0; t < NT; ++t)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            so[(16 * gt + 4 * q + i) * WST + 16 * t + r16] = dw[gt][t][i];
                pend_dw = k;
            } else {
                if constexpr (ALIAS_WZ) {
                    wave_sync();
                    flush_z();
                }
                constexpr int NP = (4 * F + 63) / 64;
#pragma unroll
                for (int gt = 0; gt < GT; ++gt) {
#pragma unroll
                    for (int t = 0; t < NT; ++t)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            so[(4 * q + i) * WST + 16 * t + r16] = dw[gt][t][i];
                    wave_sync();
#pragma unroll
                    for (int pp = 0; pp < NP; ++pp) {
                        const int u = lane + 64 * pp;
                        const int g = u / (F / 4), cc = u % (F / 4);
                        if (u < 4 * F) {
                            const int64_t o = (k * G + 16 * gt + g) * F + 4 * cc;
                            const f32x4_t v = *reinterpret_cast<const f32x4_t*>(so + g * WST + 4 * cc);
                            if constexpr (DWB)
                                *reinterpret_cast<u32x2_t*>(a.dW16 + o) =
                                    u32x2_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
                            else if constexpr (MODE == STEP_DW) *reinterpret_cast<f32x4_t*>(a.dW + o) = v;
                            else stg_stream(a.dW + o, v);
                        }
                    }
                    wave_sync();
                }
            }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
            col[t] = col_n[t];
        rows_of(col, gp);
    }
    wave_sync();
    flush_z();
    flush_dw();

    if constexpr (LOSS) {
        const float tot = wave_sum(lsum);
        if (lane == 0) atomicAdd(a.loss, (double)tot * (double)scale);
    }
}

template <int G, int F, int MODE, bool LOSS, bool WZ, bool WQ, bool DWB = false>
static void go(const FwdArgs& a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((k_group_fwd<G, F, MODE, LOSS, WZ, WQ, DWB>), dim3(grid), dim3(256), 0, s, a);
}

template <int G, int F, int MODE, bool WQ>
static void go_bce(bool loss, bool wz, const FwdArgs& a, int grid, hipStream_t s)
{
    if (loss) {
        if (wz) go<G, F, MODE, true, true, WQ>(a, grid, s);
        else go<G, F, MODE, true, false, WQ>(a, grid, s);
    } else {
        if (wz) go<G, F, MODE, false, true, WQ>(a, grid, s);
        else go<G, F, MODE, false, false, WQ>(a, grid, s);
    }
}

template <int G, int F>
static bool launch_gf(int mode, bool loss, const FwdArgs& a, int grid, hipStream_t s, bool w8)
{
    const bool wz = a.Z != nullptr;
    if (w8 && a.dW16) return false;   // the bf16 weight gradient comes with bf16 weights only
    if (w8) {
        switch (mode) {
        case FWD_Z: go<G, F, FWD_Z, false, false, true>(a, grid, s); return true;
        case STEP_DW: go_bce<G, F, STEP_DW, true>(loss, wz, a, grid, s); return true;
        }
        return false;
    }
    if (a.dW16) {
        // the fused step with a bf16 weight gradient (no logits output)
        if (mode != STEP_DW || wz) return false;
        if (loss) go<G, F, STEP_DW, true, false, false, true>(a, grid, s);
        else go<G, F, STEP_DW, false, false, false, true>(a, grid, s);
        return true;
    }
    switch (mode) {
    case FWD_Z: go<G, F, FWD_Z, false, false, false>(a, grid, s); return true;
    case FWD_BCE: go_bce<G, F, FWD_BCE, false>(loss, wz, a, grid, s); return true;
    case STEP_DW: go_bce<G, F, STEP_DW, false>(loss, wz, a, grid, s); return true;
    case BWD_W: go<G, F, BWD_W, false, false, false>(a, grid, s); return true;
    }
    return false;
}

template <int G>
static bool launch_g(int F, int mode, bool loss, const FwdArgs& a, int grid, hipStream_t s, bool w8)
{
    switch (F) {
    case 32: return launch_gf<G, 32>(mode, loss, a, grid, s, w8);
    case 64: return launch_gf<G, 64>(mode, loss, a, grid, s, w8);
    case 128: return launch_gf<G, 128>(mode, loss, a, grid, s, w8);
    }
    return false;
}

bool launch_fwd(int G, int F, int mode, bool loss, const FwdArgs& a, int grid, hipStream_t s, bool w8)
{
    switch (G) {
    case 16: return launch_g<16>(F, mode, loss, a, grid, s, w8);
    case 32: return launch_g<32>(F, mode, loss, a, grid, s, w8);
    case 64: return launch_g<64>(F, mode, loss, a, grid, s, w8);
    }
    return false;
}

}  // namespace haste

// Feature gradient of the group-shared fixed fan-in layer.
//
// HASTE ("gather-once + dense MMA kernel" section of the paper notes): the
// feature gradient is the sum over groups of dZ_k W_k added into the columns
// I_k; index sets of different groups overlap, so partial results from
// subsets of groups are computed in parallel and then reduced ("split-K"
// along the label dimension).
//
// Work split: a workgroup owns one chunk of consecutive groups and one tile
// of batch rows (16, or 32 in k_group_dh32), and accumulates
// P_k = dZ_k[tile] W_k for its groups into an LDS accumulator acc[rows][H]
// (scatter-add into columns I_k).
// The workgroups of one chunk sit on one XCD (workgroup ids are dealt to the
// XCDs round-robin), so the W_k they all read is fetched from HBM once and
// served to the other batch tiles from that XCD's L2.  With NW waves per
// workgroup, each wave takes every NW-th group of the chunk.
//
// dZ comes either from the caller (bf16) or is recomputed from the logits
// of the tile (Z_k^T = W_k H_k^T on matrix cores) and the labels, as
// s (sigmoid(Z) - Y), split into bf16 hi + lo.
//
// Reduction of the per-workgroup accumulators:
//   atomic:        fp32 atomic adds into dh (order of the adds varies);
//   deterministic: the waves of a workgroup add their P_k into acc in a
//                  fixed order (turns handed on through counters in LDS:
//                  one in k_group_dh; in k_group_dh32 one per 16-row half
//                  of the accumulator, or per 8-row quarter at F = 128),
//                  each workgroup writes its accumulator to its own slice of
//                  a partials buffer, and a second kernel sums the slices in
//                  chunk order: bitwise reproducible for a fixed shape.
// The turn waits are bounded; a wave whose wait gives up skips its update and
// the workgroup reports it (DhArgs::status / DhArgs::flags), so a broken
// hand-off is an error the caller sees, never a silent wrong result.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace haste {

// W_k tile in LDS, [label g][slot f] as in W: the 16-byte chunk index of a
// row is XORed with (g / 2) so the row writes and the transposing operand
// reads of one instruction spread over the banks.
template <int F>
__device__ __forceinline__ int wt_off(int g, int f)
{
    constexpr int NCH = F / 8;
    return g * F + ((((f >> 3) ^ (g >> 1)) & (NCH - 1)) << 3) + (f & 7);
}

// Gathered H tile in LDS, [slot f][16 batch rows] (32-byte rows, the layout
// of hT); rows f with bit 3 set are stored 4 rows further so the four
// lane groups of a transposing read cover all banks.
__device__ __forceinline__ int ht_off(int f, int b)
{
    return ((f ^ (((f >> 3) & 1) << 2)) << 4) + b;
}

// Offset (floats) of (batch row r, column j) in the column-major accumulator:
// 16 floats per column, 4-row quads XORed with (j / 4) % 4 so the 16-byte
// read-add-writes of one instruction (random columns) use all bank quads.
__device__ __forceinline__ int acc_off(int j, int r)
{
    return j * 16 + ((((r >> 2) ^ (j >> 2)) & 3) << 2) + (r & 3);
}

// Offset (16-bit elements) of (batch row r, 16-byte label chunk c) in the
// dZ tile [16 rows][G]: the chunk index is XORed with (r G / 128) so the
// matrix-core operand reads (16 rows, one chunk each) spread over the banks.
template <int G>
__device__ __forceinline__ int dz_off(int r, int c)
{
    return r * G + ((((c ^ ((r * G) >> 7))) & (G / 8 - 1)) << 3);
}

// Rounds per batch of the 16-row kernel and whether the batch shares one
// accumulator turn (else one turn per round): as many groups per turn as
// the registers for their P tiles allow.
constexpr int dh16_rpt(int G, int F, int src)
{
    return (src == DH_FROM_DZ && F <= 64) ? 4 : 2;
}
constexpr bool dh16_turn_per_round(int G, int F, int src)
{
    return src == DH_FROM_DZ ? G * F > 4096 : (G * F > 2048 && F > 64);
}

template <int G, int F, int SRC, bool DET, int RPT, bool WQ = false>
__global__ __launch_bounds__(256, 2) void k_group_dh(DhArgs a)
{
    constexpr int NT = F / 16;          // output slot tiles of P
    constexpr int KSF = F / 32;         // contraction steps of Z^T = W H^T
    constexpr int GT = G / 16;          // label tiles
    constexpr int KSG = (G + 31) / 32;  // contraction steps of P = dZ W
    constexpr int R = kDhRows;
    constexpr bool LAB = (SRC == DH_FROM_LABELS);
    constexpr int NWP = (G * F / 8 + 63) / 64;   // 16-byte pieces of W_k per lane
    constexpr int NHP = F / 32;                  // 16-byte pieces of the gathered tile per lane
    constexpr int DCH = G / 8;                   // 16-byte chunks of a dZ row
    constexpr int NDP = (16 * DCH + 63) / 64;    // 16-byte pieces of the dZ tile per lane
    static_assert(R == 16, "one 16-row matrix-core tile per workgroup");

    extern __shared__ __attribute__((aligned(16))) float acc[];   // column-major: acc[j * 16 + row]
    __shared__ __attribute__((aligned(16))) uint16_t sW[4][G * F];
    __shared__ __attribute__((aligned(16))) uint16_t sT[4][LAB ? F * 16 : 16 * G];
    __shared__ int sTurn;                     // accumulator hand-off counter
    __shared__ int sLost;                     // a turn wait gave up

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int r16 = lane & 15;
    const int q = lane >> 4;
    const int tr_r = r16 >> 2, tr_c = r16 & 3;   // transposing-read source position

    const int xcd = blockIdx.x & 7;
    const int slot = blockIdx.x >> 3;
    const int tile = slot % a.ntiles;
    const int chunk = (slot / a.ntiles) * 8 + xcd;
    const int64_t kc0 = (int64_t)chunk * a.K / a.nchunks;
    const int64_t kc1 = (int64_t)(chunk + 1) * a.K / a.nchunks;
    const int64_t b0 = (int64_t)tile * R;
    const int64_t L = a.K * G;
    const int64_t H = a.H;

    for (int64_t i = threadIdx.x; i < R * H; i += 256)
        acc[i] = 0.f;
    if (threadIdx.x == 0) {
        sTurn = 0;
        sLost = 0;
    }

    LabelCursor cur;
    if constexpr (LAB)
        cur.init(a.y_rowptr, a.y_col, b0 + r16, a.B, kc0 * G);
    const float scale = a.scale;
    const float inv_s = 1.0f / a.scale;
    const int64_t brow = b0 + r16;            // batch row of this lane's A rows
    const bool brow_ok = brow < a.B;
    const bool tile_full = b0 + R <= a.B;

    uint16_t* wt = sW[wv];
    uint16_t* tt = sT[wv];

    // Inputs of one round of a wave.
    struct Stage {
        typename pick<WQ, u32x2_t, u32x4_t>::type w[NWP];   // W_k (G x F, contiguous), pieces lane + 64 p
        int wex;                    // group exponent (FP8 weights)
        u32x4_t h[LAB ? NHP : 1];   // gathered tile pieces
        u32x4_t d[LAB ? 1 : NDP];   // dZ tile pieces
        int col[NT];                // accumulator columns I_k[16t + r16]
    };
    // W_k as contiguous 16-byte pieces (four consecutive lanes read 64
    // consecutive bytes, which keeps the address units' per-line work low)
    auto load_w = [&](int64_t kk, auto& st) {
#pragma unroll
        for (int p = 0; p < NWP; ++p) {
            if (lane + 64 * p < G * F / 8) {
                if constexpr (WQ) st.w[p] = ldg8(a.W8 + kk * G * F + 8 * (lane + 64 * p));
                else st.w[p] = ldg16(a.W + kk * G * F + 8 * (lane + 64 * p));
            }
        }
        st.wex = WQ ? a.wexp[kk] : 0;
    };
    auto load_col = [&](int64_t kk, int (&cl)[NT]) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            cl[t] = a.idx[kk * F + 16 * t + r16];
    };
    // gathered tile: piece lane + 64 u is slot lane/2 + 32 u, batch rows
    // b0 + 8 (lane % 2) .. +8, so four consecutive lanes read two 32-byte runs
    auto load_gcol = [&](int64_t kk, int (&gc)[NHP]) {
#pragma unroll
        for (int u = 0; u < NHP; ++u)
            gc[u] = a.idx[kk * F + (lane >> 1) + 32 * u];
    };
    auto gather = [&](const int (&gc)[NHP], u32x4_t (&hv)[NHP]) {
#pragma unroll
        for (int u = 0; u < NHP; ++u)
            hv[u] = ldg16(a.hT + ((uint32_t)gc[u] * (uint32_t)a.Bp + (uint32_t)(b0 + 8 * (lane & 1))));
    };
    // dZ tile.  Up to G = 32, lane (row r16, q) loads labels 8q .. +8 of batch
    // row b0 + r16 straight into the A layout of P = dZ W_k; at G = 64 piece
    // pc = lane + 64 u is batch row b0 + pc / DCH, labels 8 (pc % DCH) .. +8,
    // staged through the tile (as in the 32-row kernel).
    constexpr bool DZ_DIRECT = (G <= 32);
    static_assert(LAB || !DZ_DIRECT || (NDP == 1 && KSG == 1), "one dZ piece per lane");
    auto load_dz = [&](int64_t kk, u32x4_t (&dv)[NDP]) {
#pragma unroll
        for (int u = 0; u < NDP; ++u) {
            dv[u] = u32x4_t{0u, 0u, 0u, 0u};
            if constexpr (DZ_DIRECT) {
                const int64_t b = b0 + r16;
                if (q < DCH && b < a.B) dv[u] = ldg16(a.dZ + b * L + kk * G + 8 * q);
            } else {
                const int pc = lane + 64 * u;
                const int64_t b = b0 + pc / DCH;
                if (pc < 16 * DCH && b < a.B) dv[u] = ldg16(a.dZ + b * L + kk * G + 8 * (pc % DCH));
            }
        }
    };

    const int64_t ng = kc1 - kc0;
    const int64_t nrounds = (ng + 3) / 4;
    auto group_of = [&](int64_t rd) {
        const int64_t kk = kc0 + 4 * rd + wv;
        return kk < kc1 ? kk : kc1 - 1;       // idle waves reload a valid group
    };

    // Software pipeline (vector-memory operations retire in issue order, so
    // every load is issued a round before it is needed and after the loads
    // that must arrive first): round rd consumes the gathered tile / dZ tile,
    // W_k and columns of its group, all issued in round rd - 1, and issues
    // the gather for round rd + 1 (its index entries arrived during round
    // rd - 1), the gather indices for round rd + 2, and the columns and
    // weights for round rd + 1.
    Stage sa, sb;
    int gcn[LAB ? NHP : 1];
    if (ng > 0) {
        const int64_t kk = group_of(0);
        if constexpr (LAB) {
            load_gcol(kk, gcn);
            gather(gcn, sa.h);
            load_gcol(group_of(1), gcn);
        } else {
            load_dz(kk, sa.d);
        }
        load_col(kk, sa.col);
        load_w(kk, sa);
    }

    __syncthreads();

    // One round: this wave's group k = kc0 + 4 rd + wv, up to P.
    auto round = [&](int64_t rd, const Stage& c, Stage& n, f32x4_t (&p)[NT]) {
        const int64_t k = kc0 + 4 * rd + wv;
        const bool active = k < kc1;
        const int64_t kn = group_of(rd + 1);
        if constexpr (LAB) {
            gather(gcn, n.h);
            load_gcol(group_of(rd + 2), gcn);
        } else {
            load_dz(kn, n.d);
        }
        load_col(kn, n.col);
        load_w(kn, n);

        if (active) {
            // W_k rows into LDS (the contraction over labels reads them transposed)
#pragma unroll
            for (int pp = 0; pp < NWP; ++pp) {
                const int u = lane + 64 * pp;
                if (u < G * F / 8)
                    *reinterpret_cast<u32x4_t*>(wt + wt_off<F>(u / (F / 8), 8 * (u % (F / 8)))) =
                        widen_w8(c.w[pp], WQ ? __builtin_amdgcn_ldexpf(1.0f, c.wex) : 1.0f);
            }

#pragma unroll
            for (int t = 0; t < NT; ++t)
                p[t] = zero4();
            u32x4_t ahi[KSG], alo[KSG];
            if constexpr (!LAB && DZ_DIRECT) {
                ahi[0] = c.d[0];
                alo[0] = u32x4_t{0u, 0u, 0u, 0u};
            } else if constexpr (!LAB) {
#pragma unroll
                for (int u = 0; u < NDP; ++u) {
                    const int pc = lane + 64 * u;
                    if (pc < 16 * DCH)
                        *reinterpret_cast<u32x4_t*>(tt + dz_off<G>(pc / DCH, pc % DCH)) = c.d[u];
                }
                wave_sync();
                // A = dZ rows of the tile: lane (row r16, q) holds labels 32s + 8q .. +8
#pragma unroll
                for (int s = 0; s < KSG; ++s) {
                    const int c = 4 * s + q;
                    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(tt + dz_off<G>(r16, c < DCH ? c : 0));
                    ahi[s] = c < DCH ? v : u32x4_t{0u, 0u, 0u, 0u};
                    alo[s] = u32x4_t{0u, 0u, 0u, 0u};
                }
            } else {
#pragma unroll
                for (int u = 0; u < NHP; ++u)
                    *reinterpret_cast<u32x4_t*>(tt + ht_off((lane >> 1) + 32 * u, 8 * (lane & 1))) = c.h[u];
                wave_sync();
                // Z^T = W_k H^T; A = W_k rows (lane (label 16gt + r16, q): slots
                // 32s + 8q ..), B = H^T read transposed: lane (row r16, q) gets
                // slots 32s + 8q + e.  Result lane (row r16, q) holds labels 16gt + 4q + i.
                f32x4_t zt[GT];
#pragma unroll
                for (int gt = 0; gt < GT; ++gt)
                    zt[gt] = zero4();
#pragma unroll
                for (int s = 0; s < KSF; ++s) {
                    const int f0 = 32 * s + 8 * q + tr_r;
                    const u32x4_t bv = cat(lds_tr16(tt + ht_off(f0, 4 * tr_c)), lds_tr16(tt + ht_off(f0 + 4, 4 * tr_c)));
#pragma unroll
                    for (int gt = 0; gt < GT; ++gt) {
                        const u32x4_t wa =
                            *reinterpret_cast<const u32x4_t*>(wt + wt_off<F>(16 * gt + r16, 32 * s + 8 * q));
                        zt[gt] = mfma16(wa, bv, zt[gt]);
                    }
                }
                // labels of this row for this group
                const uint64_t mrow = cur.take(k * G, G, a.y_col);
                float dz[GT][4];
                // s * sigmoid(z) = 1 / ((1 + e^-z) / s); e^-z = +inf gives 0
#pragma unroll
                for (int gt = 0; gt < GT; ++gt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float t = __builtin_amdgcn_exp2f(-zt[gt][i] * kLog2e);
                        dz[gt][i] = __builtin_amdgcn_rcpf(fmaf(t, inv_s, inv_s));
                    }
                if (__any(mrow != 0) || !tile_full) {   // rare: positives or padding rows
#pragma unroll
                    for (int gt = 0; gt < GT; ++gt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            float d = dz[gt][i];
                            if ((mrow >> (16 * gt + 4 * q + i)) & 1ull) d -= scale;
                            dz[gt][i] = brow_ok ? d : 0.f;
                        }
                }
                // contraction element e of step s <-> label 32s + 16*(e/4) + 4q + e%4
#pragma unroll
                for (int s = 0; s < KSG; ++s) {
                    const int g0 = 2 * s, g1 = 2 * s + 1;
                    const float x0 = dz[g0][0], x1 = dz[g0][1], x2 = dz[g0][2], x3 = dz[g0][3];
                    const float y0 = g1 < GT ? dz[g1 < GT ? g1 : 0][0] : 0.f;
                    const float y1 = g1 < GT ? dz[g1 < GT ? g1 : 0][1] : 0.f;
                    const float y2 = g1 < GT ? dz[g1 < GT ? g1 : 0][2] : 0.f;
                    const float y3 = g1 < GT ? dz[g1 < GT ? g1 : 0][3] : 0.f;
                    { const u32x2_t _p = split_pair(x0, x1); ahi[s][0] = _p[0]; alo[s][0] = _p[1]; }
                    { const u32x2_t _p = split_pair(x2, x3); ahi[s][1] = _p[0]; alo[s][1] = _p[1]; }
                    { const u32x2_t _p = split_pair(y0, y1); ahi[s][2] = _p[0]; alo[s][2] = _p[1]; }
                    { const u32x2_t _p = split_pair(y2, y3); ahi[s][3] = _p[0]; alo[s][3] = _p[1]; }
                }
            }
            wave_sync();
            // P = dZ_tile W_k with B = W_k read transposed: lane (slot 16t + r16, q)
            // gets the labels of contraction elements e.  Result lane
            // (slot 16t + r16, q) holds batch rows 4q + i.
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int fc = 16 * t + 4 * tr_c;
#pragma unroll
                for (int s = 0; s < KSG; ++s) {
                    // Transposing reads run with the whole wave active (under a
                    // partial EXEC mask they overwrite the inactive lanes'
                    // registers); rows past G read a valid row and are zeroed.
                    u32x2_t lo2, hi2;
                    const u32x2_t z2 = u32x2_t{0u, 0u};
                    if constexpr (!LAB) {
                        const int g = 32 * s + 8 * q;          // elements e <-> g + e
                        const bool ok = g < G;
                        const int gr = ok ? g : 0;
                        lo2 = lds_tr16(wt + wt_off<F>(gr + tr_r, fc));
                        hi2 = lds_tr16(wt + wt_off<F>(gr + 4 + tr_r, fc));
                        lo2 = ok ? lo2 : z2;
                        hi2 = ok ? hi2 : z2;
                    } else {
                        const int ga = 32 * s + 4 * q;         // e < 4 <-> ga + e
                        const int gb = ga + 16;                // e >= 4 <-> gb + e - 4
                        lo2 = lds_tr16(wt + wt_off<F>(ga + tr_r, fc));
                        if constexpr (G > 16) hi2 = lds_tr16(wt + wt_off<F>(gb + tr_r, fc));
                        else hi2 = z2;
                    }
                    const u32x4_t bv = cat(lo2, hi2);
                    p[t] = mfma16(ahi[s], bv, p[t]);
                    if constexpr (LAB)
                        p[t] = mfma16(alo[s], bv, p[t]);
                }
            }
        } else {
            // the inputs of an idle round still count as consumed (see settle)
#pragma unroll
            for (int pp = 0; pp < NWP; ++pp) settle(c.w[pp]);
#pragma unroll
            for (int u = 0; u < (LAB ? NHP : 1); ++u) settle(c.h[u]);
#pragma unroll
            for (int u = 0; u < (LAB ? 1 : NDP); ++u) settle(c.d[u]);
        }

    };

    // Scatter-add P into the accumulator columns I_k with 16-byte
    // read-add-write (rows 4q .. 4q+3 of column col[t] are adjacent).  Inside
    // one wave the index set is duplicate-free, so no two lanes touch the same
    // cell, and a later read-add-write of the wave sees its earlier writes.
    auto rmw = [&](const f32x4_t (&p)[NT], const int (&off)[NT]) {
        f32x4_t v[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t)
            v[t] = *reinterpret_cast<const f32x4_t*>(acc + off[t]);
#pragma unroll
        for (int t = 0; t < NT; ++t)
            *reinterpret_cast<f32x4_t*>(acc + off[t]) = v[t] + p[t];
    };
    // The accumulator offsets are formed before the turn wait and consumed
    // there by an empty asm statement: otherwise the compiler sinks their
    // arithmetic into the held turn, where every instruction delays the
    // waves queued behind.
    auto offs = [&](const int (&col)[NT], int (&off)[NT]) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            off[t] = acc_off(col[t], 4 * q);
            asm volatile("" ::"v"(off[t]));
        }
    };

    // Rounds in batches of RPT: the wave computes P for its groups of the
    // batch, then takes its turn on the accumulator.  Turns go in the fixed
    // order (batch, wave), handed on through an LDS counter, so every cell is
    // updated by one wave at a time and in a fixed group order.  Every round
    // of a batch runs (past the last round it only issues clamped loads), so
    // every path reaches the hand-off with the same loads in flight; a
    // round's accumulator offsets are formed before the round after it
    // overwrites its input set.
    static_assert(RPT % 2 == 0, "rounds alternate between the two input sets");
    const int64_t nbatch = (nrounds + RPT - 1) / RPT;
    for (int64_t i = 0; i < nbatch; ++i) {
        const int64_t rd = RPT * i;
        if constexpr (dh16_turn_per_round(G, F, SRC)) {
            // wide tiles: each round's P goes into the accumulator at once
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                Stage& c = (r % 2 == 0) ? sa : sb;
                Stage& n = (r % 2 == 0) ? sb : sa;
                f32x4_t p[NT];
                round(rd + r, c, n, p);
                int off[NT];
                offs(c.col, off);
                const int turn = (int)(4 * (rd + r)) + wv;
                const bool got = wait_turn(&sTurn, turn, a.spins);
                if (got && kc0 + 4 * (rd + r) + wv < kc1) rmw(p, off);
                if (!got) sLost = 1;
                pass_turn(&sTurn, turn);
            }
        } else {
            f32x4_t p[RPT][NT];
            int cl[RPT][NT];
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                Stage& c = (r % 2 == 0) ? sa : sb;
                Stage& n = (r % 2 == 0) ? sb : sa;
                round(rd + r, c, n, p[r]);
                offs(c.col, cl[r]);
            }
            const int turn = (int)(4 * i) + wv;
            const bool got = wait_turn(&sTurn, turn, a.spins);
            if (got) {
#pragma unroll
                for (int r = 0; r < RPT; ++r)
                    if (kc0 + 4 * (rd + r) + wv < kc1) rmw(p[r], cl[r]);
            } else {
                sLost = 1;
            }
            pass_turn(&sTurn, turn);
        }
    }
    __syncthreads();

    if constexpr (DET) {
        float* dst = a.part + ((int64_t)chunk * a.ntiles * R + b0) * H;
        for_cells(R, (int)H, threadIdx.x, 256, [&](int r, int j) { dst[(int64_t)r * H + j] = acc[acc_off(j, r)]; });
        if (threadIdx.x == 0) a.flags[blockIdx.x] = sLost;
    } else {
        for_cells(R, (int)H, threadIdx.x, 256, [&](int r, int j) {
            if (b0 + r < a.B) unsafeAtomicAdd(&a.dh[(b0 + r) * H + j], acc[acc_off(j, r)]);
        });
        if (threadIdx.x == 0 && sLost) *a.status = 1;
    }
}

// Offset (floats) of (batch row r < 32, column j) in the 32-row accumulator:
// 32 floats per column, 4-row quads XORed with (j / 2) % 8 so the 16-byte
// read-add-writes of one instruction (random columns) use all bank groups.
__device__ __forceinline__ int acc32_off(int j, int r)
{
    return j * 32 + ((((r >> 2) ^ (j >> 1)) & 7) << 2) + (r & 3);
}

// Variant with 32 batch rows per workgroup and NWV waves: each wave runs a
// group for both 16-row matrix-core tiles, so the W_k staging, its
// transposed operand reads, the index loads and the accumulator addressing
// serve twice the rows.  One workgroup per CU (accumulator 32 x H fp32 plus
// per-wave tiles); used when G*F <= 2048 (or G = 64 with F = 64) and
// H <= 768.  With F <= 64 a wave takes its turn on the accumulator once per
// RPT rounds (RPT groups per turn): four when dZ is given (the turn
// hand-offs bound that kernel, and its per-group registers are few), two
// when the logits are recomputed; with F = 128 once per round.
template <int G, int F, int SRC, bool DET, int NWV, int RPT, bool WQ = false>
__global__ __launch_bounds__(64 * NWV, 1) void k_group_dh32(DhArgs a)
{
    constexpr int NT = F / 16;          // output slot tiles of P
    constexpr int KSF = F / 32;         // contraction steps of Z^T = W H^T
    constexpr int GT = G / 16;          // label tiles
    constexpr int KSG = (G + 31) / 32;  // contraction steps of P = dZ W
    constexpr int R = 32;
    constexpr int NT_ = 64 * NWV;       // threads per workgroup
    constexpr bool LAB = (SRC == DH_FROM_LABELS);
    constexpr int NWP = (G * F / 8 + 63) / 64;   // 16-byte pieces of W_k per lane
    constexpr int NHH = F / 32;                  // gathered 16-byte pieces per lane per 16-row half
    constexpr int DCH = G / 8;                   // 16-byte chunks of a dZ row
    constexpr int NDH = (16 * DCH + 63) / 64;    // dZ pieces per lane per 16-row half
    static_assert(G * F <= 4096 && F <= 128, "per-wave tiles sized for the 32-row workgroup");
    static_assert(NWV * (G * F + (LAB ? F * 16 : 16 * G)) * 2 + 32 * 768 * 4 + 160 <= 160 * 1024,
                  "per-wave tiles and a 32 x 768 accumulator fit in LDS");

    extern __shared__ __attribute__((aligned(128))) float acc[];  // acc[j * 32 + row], quads swizzled;
                                                                  // 128-byte aligned for the address flips below
    __shared__ __attribute__((aligned(16))) uint16_t sW[NWV][G * F];
    __shared__ __attribute__((aligned(16))) uint16_t sT[NWV][LAB ? F * 16 : 16 * G];   // one 16-row half
    __shared__ int sTurn[4];                  // accumulator hand-off counters: per 16-row half, or per 8-row quarter (F > 64)
    __shared__ int sLost;                     // a turn wait gave up

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int r16 = lane & 15;
    const int q = lane >> 4;
    const int tr_r = r16 >> 2, tr_c = r16 & 3;   // transposing-read source position

    const int xcd = blockIdx.x & 7;
    const int slot = blockIdx.x >> 3;
    const int tile = slot % a.ntiles;
    const int chunk = (slot / a.ntiles) * 8 + xcd;
    const int64_t kc0 = (int64_t)chunk * a.K / a.nchunks;
    const int64_t kc1 = (int64_t)(chunk + 1) * a.K / a.nchunks;
    const int64_t b0 = (int64_t)tile * R;
    const int64_t L = a.K * G;
    const int64_t H = a.H;

    for (int64_t i = threadIdx.x; i < R * H; i += NT_)
        acc[i] = 0.f;
    if (threadIdx.x < 4) sTurn[threadIdx.x] = 0;
    if (threadIdx.x == 0) sLost = 0;

    // each lane's A rows: b0 + r16 (tile 0) and b0 + 16 + r16 (tile 1)
    LabelCursor cur[2];
    if constexpr (LAB) {
        cur[0].init(a.y_rowptr, a.y_col, b0 + r16, a.B, kc0 * G);
        cur[1].init(a.y_rowptr, a.y_col, b0 + 16 + r16, a.B, kc0 * G);
    }
    const float scale = a.scale;
    const float inv_s = 1.0f / a.scale;
    const bool tile_full = b0 + R <= a.B;

    uint16_t* wt = sW[wv];
    uint16_t* tt = sT[wv];

    // Inputs of one round as loaded from global memory.
    struct In {
        typename pick<WQ, u32x2_t, u32x4_t>::type w[NWP];   // W_k (G x F, contiguous), pieces lane + 64 p
        int wex;                         // group exponent (FP8 weights)
        u32x4_t h[LAB ? 2 : 1][NHH];     // gathered pieces, per 16-row half
        u32x4_t d[LAB ? 1 : 2][NDH];     // dZ tile pieces, per 16-row half
        int col[NT];                     // accumulator columns I_k[16t + r16]
    };
    // W_k as contiguous 16-byte pieces (four consecutive lanes read 64 bytes)
    auto load_w = [&](int64_t kk, auto& st) {
#pragma unroll
        for (int p = 0; p < NWP; ++p) {
            if (lane + 64 * p < G * F / 8) {
                if constexpr (WQ) st.w[p] = ldg8(a.W8 + kk * G * F + 8 * (lane + 64 * p));
                else st.w[p] = ldg16(a.W + kk * G * F + 8 * (lane + 64 * p));
            }
        }
        st.wex = WQ ? a.wexp[kk] : 0;
    };
    auto load_col = [&](int64_t kk, int (&cl)[NT]) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            cl[t] = a.idx[kk * F + 16 * t + r16];
    };
    // gathered half tile: piece lane + 64 u is slot lane/2 + 32 u, batch rows
    // b0 + 16 hf + 8 (lane % 2) .. +8
    auto load_gcol = [&](int64_t kk, int (&gc)[NHH]) {
#pragma unroll
        for (int u = 0; u < NHH; ++u)
            gc[u] = a.idx[kk * F + (lane >> 1) + 32 * u];
    };
    auto gather = [&](const int (&gc)[NHH], u32x4_t (&hv)[2][NHH]) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int u = 0; u < NHH; ++u)
                hv[hf][u] = ldg16(a.hT + ((uint32_t)gc[u] * (uint32_t)a.Bp +
                                          (uint32_t)(b0 + 16 * hf + 8 * (lane & 1))));
    };
    // dZ half tile.  Up to G = 32 a row's labels fit one contraction step,
    // and lane (row r16, q) loads labels 8q .. +8 of batch row b0 + 16 hf +
    // r16 straight into the A layout of P = dZ W_k (no pass through LDS;
    // 345 -> 328 us for the given-dZ call at 3M).  At G = 64 (two steps)
    // piece pc = lane + 64 u is batch row b0 + 16 hf + pc / DCH, labels
    // 8 (pc % DCH) .., staged through the tile: each row's 128 bytes then
    // come from 8 neighbouring lanes (the direct form measured 1 % slower).
    constexpr bool DZ_DIRECT = (G <= 32);
    static_assert(LAB || !DZ_DIRECT || (NDH == 1 && KSG == 1), "one dZ piece per half");
    auto load_dz = [&](int64_t kk, u32x4_t (&dv)[2][NDH]) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int u = 0; u < NDH; ++u) {
                dv[hf][u] = u32x4_t{0u, 0u, 0u, 0u};
                if constexpr (DZ_DIRECT) {
                    const int64_t b = b0 + 16 * hf + r16;
                    if (q < DCH && b < a.B) dv[hf][u] = ldg16(a.dZ + b * L + kk * G + 8 * q);
                } else {
                    const int pc = lane + 64 * u;
                    const int64_t b = b0 + 16 * hf + pc / DCH;
                    if (pc < 16 * DCH && b < a.B) dv[hf][u] = ldg16(a.dZ + b * L + kk * G + 8 * (pc % DCH));
                }
            }
    };

    const int64_t ng = kc1 - kc0;
    const int64_t nrounds = (ng + NWV - 1) / NWV;
    auto group_of = [&](int64_t rd) {
        const int64_t kk = kc0 + NWV * rd + wv;
        return kk < kc1 ? kk : kc1 - 1;       // idle waves reload a valid group
    };

    // Software pipeline as in the 16-row kernel: round rd consumes inputs
    // issued in round rd - 1 and issues the gather for round rd + 1 (its
    // index entries arrived during round rd - 1), the gather indices for
    // round rd + 2 and the columns and weights for round rd + 1.
    In sa, sb;
    int gcn[LAB ? NHH : 1];
    if (ng > 0) {
        const int64_t kk = group_of(0);
        if constexpr (LAB) {
            load_gcol(kk, gcn);
            gather(gcn, sa.h);
            load_gcol(group_of(1), gcn);
        } else {
            load_dz(kk, sa.d);
        }
        load_col(kk, sa.col);
        load_w(kk, sa);
    }

    __syncthreads();

    // One round: this wave's group k = kc0 + 8 rd + wv, up to P for both tiles.
    auto round = [&](int64_t rd, const In& c, In& n, f32x4_t (&p)[2][NT]) {
        const int64_t k = kc0 + NWV * rd + wv;
        const bool active = k < kc1;
        const int64_t kn = group_of(rd + 1);
        if constexpr (LAB) {
            gather(gcn, n.h);
            load_gcol(group_of(rd + 2), gcn);
        } else {
            load_dz(kn, n.d);
        }
        load_col(kn, n.col);
        load_w(kn, n);
        if (!active) {
            // the inputs of an idle round still count as consumed (see settle)
#pragma unroll
            for (int pp = 0; pp < NWP; ++pp) settle(c.w[pp]);
#pragma unroll
            for (int hf = 0; hf < (LAB ? 2 : 1); ++hf)
#pragma unroll
                for (int u = 0; u < NHH; ++u) settle(c.h[hf][u]);
#pragma unroll
            for (int hf = 0; hf < (LAB ? 1 : 2); ++hf)
#pragma unroll
                for (int u = 0; u < NDH; ++u) settle(c.d[hf][u]);
            return;
        }

        // W_k rows into LDS (the contraction over labels reads them transposed)
#pragma unroll
        for (int pp = 0; pp < NWP; ++pp) {
            const int u = lane + 64 * pp;
            if (u < G * F / 8)
                *reinterpret_cast<u32x4_t*>(wt + wt_off<F>(u / (F / 8), 8 * (u % (F / 8)))) =
                    widen_w8(c.w[pp], WQ ? __builtin_amdgcn_ldexpf(1.0f, c.wex) : 1.0f);
        }
        u32x4_t ahi[2][KSG], alo[2][KSG];
        if constexpr (!LAB) {
            // A of P = given dZ rows: as loaded, or one 16-row half at a time
            // through the tile
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                if constexpr (DZ_DIRECT) {
                    ahi[hf][0] = c.d[hf][0];
                    alo[hf][0] = u32x4_t{0u, 0u, 0u, 0u};
                    continue;
                }
#pragma unroll
                for (int u = 0; u < NDH; ++u) {
                    const int pc = lane + 64 * u;
                    if (pc < 16 * DCH)
                        *reinterpret_cast<u32x4_t*>(tt + dz_off<G>(pc / DCH, pc % DCH)) = c.d[hf][u];
                }
                wave_sync();
#pragma unroll
                for (int s = 0; s < KSG; ++s) {
                    const int cc = 4 * s + q;
                    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(tt + dz_off<G>(r16, cc < DCH ? cc : 0));
                    ahi[hf][s] = cc < DCH ? v : u32x4_t{0u, 0u, 0u, 0u};
                    alo[hf][s] = u32x4_t{0u, 0u, 0u, 0u};
                }
                wave_sync();
            }
        } else {
            // labels of this lane's two rows for this group, taken first: the
            // cursor walk is a loop and the label correction a rare branch,
            // and each ends a scheduling region
            uint64_t mrow[2];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
                mrow[hf] = cur[hf].take(k * G, G, a.y_col);
            // B of Z^T = H^T read transposed, per 16-row half: lane (row r16, q)
            // gets slots 32s + 8q + e
            u32x4_t bz[2][KSF];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
                for (int u = 0; u < NHH; ++u)
                    *reinterpret_cast<u32x4_t*>(tt + ht_off((lane >> 1) + 32 * u, 8 * (lane & 1))) = c.h[hf][u];
                wave_sync();
#pragma unroll
                for (int s = 0; s < KSF; ++s) {
                    const int f0 = 32 * s + 8 * q + tr_r;
                    bz[hf][s] = cat(lds_tr16(tt + ht_off(f0, 4 * tr_c)), lds_tr16(tt + ht_off(f0 + 4, 4 * tr_c)));
                }
                wave_sync();
            }
            // Z^T = W_k H^T for both tiles; A = W_k rows (lane (label 16gt + r16, q):
            // slots 32s + 8q ..).  Result lane (row r16, q) holds labels 16gt + 4q + i.
            f32x4_t zt[2][GT];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int gt = 0; gt < GT; ++gt)
                    zt[hf][gt] = zero4();
#pragma unroll
            for (int s = 0; s < KSF; ++s)
#pragma unroll
                for (int gt = 0; gt < GT; ++gt) {
                    const u32x4_t wa =
                        *reinterpret_cast<const u32x4_t*>(wt + wt_off<F>(16 * gt + r16, 32 * s + 8 * q));
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf)
                        zt[hf][gt] = mfma16(wa, bz[hf][s], zt[hf][gt]);
                }
            // With up to two label tiles both halves' epilogues run side by
            // side (one sigmoid region, one correction branch, both splits):
            // 670K dh 570 -> 552 us.  At G = 64 (four label tiles, 252
            // registers) that measured slower (490 -> 499 us at 8.6M), so the
            // halves there run one after the other.
            constexpr bool JOINT = (GT <= 2);
            constexpr int NH = JOINT ? 2 : 1;   // halves per pass
#pragma unroll
            for (int h0 = 0; h0 < 2; h0 += NH) {
                // s * sigmoid(z) = 1 / ((1 + e^-z) / s); e^-z = +inf gives 0
                float dz[NH][GT][4];
#pragma unroll
                for (int u = 0; u < NH; ++u)
#pragma unroll
                    for (int gt = 0; gt < GT; ++gt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float t = __builtin_amdgcn_exp2f(-zt[h0 + u][gt][i] * kLog2e);
                            dz[u][gt][i] = __builtin_amdgcn_rcpf(fmaf(t, inv_s, inv_s));
                        }
                const uint64_t many = JOINT ? (mrow[0] | mrow[1]) : mrow[h0];
                if (__any(many != 0) || !tile_full) {   // rare: positives or padding rows
#pragma unroll
                    for (int u = 0; u < NH; ++u) {
                        const int hf = h0 + u;
                        const bool brow_ok = b0 + 16 * hf + r16 < a.B;
#pragma unroll
                        for (int gt = 0; gt < GT; ++gt)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                float d = dz[u][gt][i];
                                if ((mrow[hf] >> (16 * gt + 4 * q + i)) & 1ull) d -= scale;
                                dz[u][gt][i] = brow_ok ? d : 0.f;
                            }
                    }
                }
                // contraction element e of step s <-> label 32s + 16*(e/4) + 4q + e%4
#pragma unroll
                for (int u = 0; u < NH; ++u)
#pragma unroll
                    for (int s = 0; s < KSG; ++s) {
                        const int hf = h0 + u;
                        const int g0 = 2 * s, g1 = 2 * s + 1;
                        const float x0 = dz[u][g0][0], x1 = dz[u][g0][1], x2 = dz[u][g0][2], x3 = dz[u][g0][3];
                        const float y0 = g1 < GT ? dz[u][g1 < GT ? g1 : 0][0] : 0.f;
                        const float y1 = g1 < GT ? dz[u][g1 < GT ? g1 : 0][1] : 0.f;
                        const float y2 = g1 < GT ? dz[u][g1 < GT ? g1 : 0][2] : 0.f;
                        const float y3 = g1 < GT ? dz[u][g1 < GT ? g1 : 0][3] : 0.f;
                        { const u32x2_t _p = split_pair(x0, x1); ahi[hf][s][0] = _p[0]; alo[hf][s][0] = _p[1]; }
                        { const u32x2_t _p = split_pair(x2, x3); ahi[hf][s][1] = _p[0]; alo[hf][s][1] = _p[1]; }
                        { const u32x2_t _p = split_pair(y0, y1); ahi[hf][s][2] = _p[0]; alo[hf][s][2] = _p[1]; }
                        { const u32x2_t _p = split_pair(y2, y3); ahi[hf][s][3] = _p[0]; alo[hf][s][3] = _p[1]; }
                    }
            }
        }
        // P = dZ_tile W_k with B = W_k read transposed (shared by both tiles):
        // lane (slot 16t + r16, q) gets the labels of contraction elements e.
        // Result lane (slot 16t + r16, q) holds batch rows 16 hf + 4q + i.
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int fc = 16 * t + 4 * tr_c;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
                p[hf][t] = zero4();
#pragma unroll
            for (int s = 0; s < KSG; ++s) {
                // Transposing reads run with the whole wave active (under a
                // partial EXEC mask they overwrite the inactive lanes'
                // registers); rows past G read a valid row and are zeroed.
                u32x2_t lo2, hi2;
                const u32x2_t z2 = u32x2_t{0u, 0u};
                if constexpr (!LAB) {
                    const int g = 32 * s + 8 * q;          // elements e <-> g + e
                    const bool ok = g < G;
                    const int gr = ok ? g : 0;
                    lo2 = lds_tr16(wt + wt_off<F>(gr + tr_r, fc));
                    hi2 = lds_tr16(wt + wt_off<F>(gr + 4 + tr_r, fc));
                    lo2 = ok ? lo2 : z2;
                    hi2 = ok ? hi2 : z2;
                } else {
                    const int ga = 32 * s + 4 * q;         // e < 4 <-> ga + e
                    const int gb = ga + 16;                // e >= 4 <-> gb + e - 4
                    lo2 = lds_tr16(wt + wt_off<F>(ga + tr_r, fc));
                    if constexpr (G > 16) hi2 = lds_tr16(wt + wt_off<F>(gb + tr_r, fc));
                    else hi2 = z2;
                }
                const u32x4_t bv = cat(lo2, hi2);
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    p[hf][t] = mfma16(ahi[hf][s], bv, p[hf][t]);
                    if constexpr (LAB)
                        p[hf][t] = mfma16(alo[hf][s], bv, p[hf][t]);
                }
            }
        }
    };

    // Scatter-add P into the accumulator columns I_k with 16-byte
    // read-add-writes (rows 16 hf + 4q .. +3 of column col[t] are adjacent).
    // Inside one wave the index set is duplicate-free, so no two lanes touch
    // the same cell.  Each 16-row half of the accumulator has its own turn
    // counter; waves take turns on a half in the fixed order (batch of RPT
    // rounds, wave), RPT groups per turn in round order, so one wave can
    // update one half while the next updates the other.  The offsets are
    // the LDS byte addresses of half 0, formed before the turn wait: rows
    // 16 + 4q of a column sit at its rows 4q with quad index bit 2 flipped,
    // i.e. at float offset XOR 16, byte address XOR 64 (the accumulator
    // starts on a 128-byte boundary, so the flip never carries into the
    // base).  The addresses are consumed there by an empty asm statement:
    // otherwise the compiler sinks their arithmetic into the held turns,
    // where every instruction delays the waves queued behind; as finished
    // byte addresses the turn of half 0 starts with its LDS reads.
    using lds_f4 = __attribute__((address_space(3))) f32x4_t;
    const uint32_t accb = (uint32_t)(size_t)(__attribute__((address_space(3))) float*)acc;
    auto cell = [](uint32_t ad) { return (lds_f4*)(size_t)ad; };
    auto rmw = [&](int hf, const f32x4_t (&p)[2][NT], const uint32_t (&off)[NT]) {
        f32x4_t v[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t)
            v[t] = *cell(off[t] ^ (64u * hf));
#pragma unroll
        for (int t = 0; t < NT; ++t)
            *cell(off[t] ^ (64u * hf)) = v[t] + p[hf][t];
    };
    auto offs = [&](const int (&col)[NT], uint32_t (&off)[NT]) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            off[t] = accb + 4u * (uint32_t)acc32_off(col[t], 4 * q);
            asm volatile("" ::"v"(off[t]));
        }
    };
    // Wide tiles (F = 128: eight result tiles per half and round) hold a half
    // twice as long per turn, and there the turns are split once more: four
    // 8-row quarters, each with its own counter, so up to four waves update
    // the accumulator at once.  quarters() pairs result tiles 2u and 2u + 1
    // and swaps the upper 32 lanes of the first with the lower 32 of the
    // second (v_permlane32_swap): tile 2u then holds rows 0 .. 7 and tile
    // 2u + 1 rows 8 .. 15 of the pair's 32 columns, lane (r16, q) covering
    // column slot 16 (2u + q / 2) + r16 and rows 8 qa + 4 (q % 2) .. +3, so
    // every read-add-write instruction of a quarter has all 64 lanes.  The
    // rows of quarter qt sit at those of quarter 0 with offset XOR 8 qt.
    auto quarters = [&](f32x4_t (&p)[2][NT]) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int u = 0; u < NT / 2; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // The elements go in by value: __builtin_bit_cast of an
                    // indexed vector element reads element 0 in this clang.
                    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[hf][2 * u][e]),
                                                                     __float_as_uint(p[hf][2 * u + 1][e]), false, false);
                    p[hf][2 * u][e] = __uint_as_float((uint32_t)sw[0]);
                    p[hf][2 * u + 1][e] = __uint_as_float((uint32_t)sw[1]);
                }
    };
    auto rmw_q = [&](auto QT, const f32x4_t (&p)[2][NT], const int (&off)[NT / 2]) {
        constexpr int qt = decltype(QT)::value, hf = qt >> 1, qa = qt & 1;
        f32x4_t v[NT / 2];
#pragma unroll
        for (int u = 0; u < NT / 2; ++u)
            v[u] = *reinterpret_cast<const f32x4_t*>(acc + (off[u] ^ (8 * qt)));
#pragma unroll
        for (int u = 0; u < NT / 2; ++u)
            *reinterpret_cast<f32x4_t*>(acc + (off[u] ^ (8 * qt))) = v[u] + p[hf][2 * u + qa];
    };
    auto offs_q = [&](const int (&col)[NT], int (&off)[NT / 2]) {
        // (the lane's column is blended from both values: a select between
        // the two array elements would take their address and move the whole
        // input set out of registers)
        const int lo = -(int)(q < 2);
#pragma unroll
        for (int u = 0; u < NT / 2; ++u) {
            const int c0 = col[2 * u], c1 = col[2 * u + 1];
            off[u] = acc32_off((c0 & lo) | (c1 & ~lo), 4 * (q & 1));
            asm volatile("" ::"v"(off[u]));
        }
    };
    static_assert(RPT % 2 == 0, "rounds alternate between the two input sets");
    // Let the prologue's loads land here (vmcnt(0); the other counters are
    // left alone): the compiler's wait insertion otherwise carries some of
    // them as possibly outstanding into the loop and waits for them inside
    // the held turns, whose scratch registers they were loaded into.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    const int64_t nbatch = (nrounds + RPT - 1) / RPT;
    for (int64_t i = 0; i < nbatch; ++i) {
        const int64_t rd = RPT * i;
        if constexpr (F > 64) {
            // wide tiles (P of both halves is 2 F / 16 result tiles): each
            // round's P goes into the accumulator at once, a turn per round
            // and quarter
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                In& c = (r % 2 == 0) ? sa : sb;
                In& n = (r % 2 == 0) ? sb : sa;
                f32x4_t p[2][NT];
                round(rd + r, c, n, p);
                quarters(p);
                int off[NT / 2];
                offs_q(c.col, off);
                const int turn = (int)(NWV * (rd + r)) + wv;
                int nxt = turn + 1;
                asm volatile("" : "+v"(nxt));
                const bool live = kc0 + NWV * (rd + r) + wv < kc1;
                auto chain = [&](auto QT) {
                    constexpr int qt = decltype(QT)::value;
                    const bool got = wait_turn(&sTurn[qt], turn, a.spins);
                    if (got && live) rmw_q(QT, p, off);
                    if (!got) sLost = 1;
                    pass_turn_to(&sTurn[qt], nxt);
                };
                chain(std::integral_constant<int, 0>{});
                chain(std::integral_constant<int, 1>{});
                chain(std::integral_constant<int, 2>{});
                chain(std::integral_constant<int, 3>{});
            }
            continue;
        }
        f32x4_t p[RPT][2][NT];
        uint32_t cl[RPT][NT];
        // every round of the batch runs (past the last round it only issues
        // clamped loads), so every path reaches the hand-off with the same
        // loads outstanding; a round's accumulator offsets are formed before
        // the round after it overwrites its input set
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            In& c = (r % 2 == 0) ? sa : sb;
            In& n = (r % 2 == 0) ? sb : sa;
            round(rd + r, c, n, p[r]);
            offs(c.col, cl[r]);
        }
        const int turn = (int)(NWV * i) + wv;
        int nxt = turn + 1;   // the counters' next value, in a vector register before the turns
        asm volatile("" : "+v"(nxt));
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const bool got = wait_turn(&sTurn[hf], turn, a.spins);
            if (got) {
#pragma unroll
                for (int r = 0; r < RPT; ++r)
                    if (kc0 + NWV * (rd + r) + wv < kc1) rmw(hf, p[r], cl[r]);
            } else {
                sLost = 1;
            }
            pass_turn_to(&sTurn[hf], nxt);
        }
    }
    __syncthreads();

    if constexpr (DET) {
        float* dst = a.part + ((int64_t)chunk * a.ntiles * R + b0) * H;
        for_cells(R, (int)H, threadIdx.x, NT_, [&](int r, int j) { dst[(int64_t)r * H + j] = acc[acc32_off(j, r)]; });
        if (threadIdx.x == 0) a.flags[blockIdx.x] = sLost;
    } else {
        for_cells(R, (int)H, threadIdx.x, NT_, [&](int r, int j) {
            if (b0 + r < a.B) unsafeAtomicAdd(&a.dh[(b0 + r) * H + j], acc[acc32_off(j, r)]);
        });
        if (threadIdx.x == 0 && sLost) *a.status = 1;
    }
}

// dh[b, j] = sum over chunks c of part[c, b, j], in a fixed order: four lanes
// per 4 consecutive outputs each add every fourth chunk (c = lane % 4 + 4i,
// in i order), then the four partial sums are combined as (s0 + s1) + (s2 + s3).
__global__ __launch_bounds__(256) void k_dh_reduce(const float* __restrict__ part, float* __restrict__ dh,
                                                   int64_t B, int64_t H, int nchunks, int rows_per_chunk,
                                                   const int32_t* __restrict__ flags, int nflags,
                                                   int32_t* __restrict__ status)
{
    // the first workgroup folds the feature-gradient workgroups' hand-off
    // reports into the call's status word (written every call)
    if (status && blockIdx.x == 0) {
        int bad = 0;
        for (int i = threadIdx.x; i < nflags; i += 256)
            bad |= flags[i];
        bad = __syncthreads_or(bad);
        if (threadIdx.x == 0) *status = bad ? 1 : 0;
    }
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t o4 = t >> 2;               // index of 4 consecutive outputs
    const int sub = (int)(t & 3);
    const int64_t n = B * H;
    const int64_t i0 = 4 * o4;
    const bool ok = i0 < n;
    const int64_t b = ok ? i0 / H : 0, j = ok ? i0 % H : 0;
    const int64_t stride = (int64_t)rows_per_chunk * H;
    f32x4_t s = zero4();
    if (ok) {
        const float* p = part + b * H + j;
#pragma unroll 4
        for (int c = sub; c < nchunks; c += 4)
            s += *reinterpret_cast<const f32x4_t*>(p + c * stride);
    }
    // combine the four lanes of this output quad in a fixed pattern
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float x1 = __shfl_xor(s[e], 1, 64);
        const float y = (sub & 1) ? x1 + s[e] : s[e] + x1;   // s0+s1 / s2+s3 in lane order
        const float y2 = __shfl_xor(y, 2, 64);
        s[e] = (sub & 2) ? y2 + y : y + y2;
    }
    if (ok && sub == 0) {
        if (i0 + 4 <= n) {
            *reinterpret_cast<f32x4_t*>(dh + i0) = s;
        } else {
            for (int e = 0; e < 4; ++e)
                if (i0 + e < n) dh[i0 + e] = s[e];
        }
    }
}

// Launch with the kernel's dynamic-LDS limit raised to what this launch needs.
template <void (*Kern)(DhArgs)>
static void launch_kern(dim3 grid, dim3 blk, size_t lds, hipStream_t s, const DhArgs& a)
{
    raise_dyn_lds<Kern>(lds);
    hipLaunchKernelGGL(Kern, grid, blk, lds, s, a);
}

// Waves of the 32-row kernel: eight, or fewer where eight sets of per-wave
// tiles and the 32 x H accumulator would not fit in LDS (seven at G F = 2048
// with the gathered tile of F = 128, six at G = 64, F = 64).  160 bytes cover
// the hand-off counters (20) and the accumulator's 128-byte alignment (up to
// 124 bytes of padding after the static arrays).
constexpr int dh32_waves(int G, int F, int src)
{
    const int n = (160 * 1024 - 32 * 768 * 4 - 160) / ((G * F + (src == DH_FROM_LABELS ? F * 16 : 16 * G)) * 2);
    return n < 8 ? n : 8;
}

template <int G, int F>
static bool launch_dh_gf(int src, bool det, const DhArgs& a, hipStream_t s, bool w8)
{
    const int rows = dh_tile_rows((int)G, (int)F, a.H, src == DH_FROM_LABELS);
    const size_t lds = (size_t)rows * a.H * sizeof(float);
    constexpr int NWL = dh32_waves(G, F, DH_FROM_LABELS), NWZ = dh32_waves(G, F, DH_FROM_DZ);
    const dim3 grid(a.nchunks * a.ntiles);
    const dim3 blk(rows == 32 ? 64 * (src == DH_FROM_DZ ? NWZ : NWL) : 256);
#define go(...) launch_kern<__VA_ARGS__>(grid, blk, lds, s, a)
    if (w8) {
        // FP8 weights: the fused step's kernels (logits recomputed from labels)
        if (src != DH_FROM_LABELS) return false;
        if constexpr (dh32_fits(G, F, true)) {
            if (rows == 32) {
                if (det) go(k_group_dh32<G, F, DH_FROM_LABELS, true, NWL, 2, true>);
                else go(k_group_dh32<G, F, DH_FROM_LABELS, false, NWL, 2, true>);
                return true;
            }
        }
        if (rows != kDhRows) return false;
        constexpr int RP = dh16_rpt(G, F, DH_FROM_LABELS);
        if (det) go(k_group_dh<G, F, DH_FROM_LABELS, true, RP, true>);
        else go(k_group_dh<G, F, DH_FROM_LABELS, false, RP, true>);
        return true;
    }
    if constexpr (dh32_fits(G, F, false)) {
        if (rows == 32 && src == DH_FROM_DZ) {
            // four groups per accumulator turn where their P tiles fit in registers
            constexpr int RZ = G * F <= 2048 ? 4 : 2;
            if (det) go(k_group_dh32<G, F, DH_FROM_DZ, true, NWZ, RZ>);
            else go(k_group_dh32<G, F, DH_FROM_DZ, false, NWZ, RZ>);
            return true;
        }
    }
    if constexpr (dh32_fits(G, F, true)) {
        if (rows == 32 && src == DH_FROM_LABELS) {
            if (det) go(k_group_dh32<G, F, DH_FROM_LABELS, true, NWL, 2>);
            else go(k_group_dh32<G, F, DH_FROM_LABELS, false, NWL, 2>);
            return true;
        }
    }
    if (rows != kDhRows) return false;   // tile height and kernel disagree
    if (src == DH_FROM_DZ) {
        constexpr int RP = dh16_rpt(G, F, DH_FROM_DZ);
        if (det) go(k_group_dh<G, F, DH_FROM_DZ, true, RP>); else go(k_group_dh<G, F, DH_FROM_DZ, false, RP>);
    } else {
        constexpr int RP = dh16_rpt(G, F, DH_FROM_LABELS);
        if (det) go(k_group_dh<G, F, DH_FROM_LABELS, true, RP>);
        else go(k_group_dh<G, F, DH_FROM_LABELS, false, RP>);
    }
    return true;
#undef go
}

template <int G>
static bool launch_dh_g(int F, int src, bool det, const DhArgs& a, hipStream_t s, bool w8)
{
    switch (F) {
    case 32: return launch_dh_gf<G, 32>(src, det, a, s, w8);
    case 64: return launch_dh_gf<G, 64>(src, det, a, s, w8);
    case 128: return launch_dh_gf<G, 128>(src, det, a, s, w8);
    }
    return false;
}

bool launch_dh(int G, int F, int src, bool det, const DhArgs& a, hipStream_t s, bool w8)
{
    switch (G) {
    case 16: return launch_dh_g<16>(F, src, det, a, s, w8);
    case 32: return launch_dh_g<32>(F, src, det, a, s, w8);
    case 64: return launch_dh_g<64>(F, src, det, a, s, w8);
    }
    return false;
}

void launch_dh_reduce(const float* part, float* dh, int64_t B, int64_t H, int nchunks, int rows_per_chunk,
                      hipStream_t s, const int32_t* flags, int nflags, int32_t* status)
{
    // four threads per four consecutive outputs (the partials of a chunk hold
    // at least B rows, so a last partial quad stays inside them)
    const int64_t nthreads = (B * H + 3) / 4 * 4;
    hipLaunchKernelGGL(k_dh_reduce, dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0, s, part, dh, B, H,
                       nchunks, rows_per_chunk, flags, nflags, status);
}

}  // namespace haste

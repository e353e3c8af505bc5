// Dense head of the head-tail split.
//
// HASTE "head-tail split" section: the most frequent labels go to a dense
// head (every label sees all H features) and the rest to the group-shared
// sparse tail; one BCE objective covers both.  The head's three products are
// plain dense GEMMs (Z = h W^T, dW = dZ^T h, dh = dZ W), bf16 in, fp32
// accumulate and out.  For B <= 128, H % 64 == 0 and L % 8 == 0 they run on
// the kernels below (logits and BCE gradient fused in k_head_zbce); other
// shapes use rocBLAS for the products and k_head_bce between them.  dZ goes
// to the weight-side products as two bf16 matrices, hi and the rounding
// residual lo, so they carry about 16 significant bits of dZ, as the tail's
// fused kernels do.  The two parts are stacked (hi rows 0..B-1, lo rows
// B..2B-1) so that each weight-side product reads W or writes dW once:
// dW = [hi; lo]^T [h; h] (a 2B-deep contraction) and dh = [hi; lo] W (2B
// rows, whose halves are then added).
#include "blas.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace haste {

// dZ[b, l] = s (sigmoid(Z[b, l]) - Y[b, l]) as bf16 hi + lo, and optionally
// loss += s sum [max(z, 0) + log(1 + e^-|z|) - y z].  One thread per eight
// consecutive labels of one sample; Y comes from the sample's sorted CSR row.
__global__ __launch_bounds__(256) void k_head_bce(const float* __restrict__ Z, const int32_t* __restrict__ rowptr,
                                                  const int32_t* __restrict__ col, float scale,
                                                  uint16_t* __restrict__ dz_hi, uint16_t* __restrict__ dz_lo,
                                                  double* __restrict__ loss, int64_t B, int64_t L)
{
    const int64_t per_row = (L + 7) / 8;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    float lsum = 0.f;
    if (t < B * per_row) {
        const int64_t b = t / per_row;
        const int64_t l0 = (t % per_row) * 8;
        // positives of sample b among labels l0 .. l0 + 7
        int lo = rowptr[b];
        const int end = rowptr[b + 1];
        int hi = end;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if ((int64_t)col[mid] < l0) lo = mid + 1; else hi = mid;
        }
        uint32_t ymask = 0;
        for (int p = lo; p < end && (int64_t)col[p] < l0 + 8; ++p)
            ymask |= 1u << (int)((int64_t)col[p] - l0);

        const float* zr = Z + b * L + l0;
        float z[8];
        const bool full = (l0 + 8 <= L) && (L % 4 == 0);
        if (full) {
            const f32x4_t a = *reinterpret_cast<const f32x4_t*>(zr);
            const f32x4_t c = *reinterpret_cast<const f32x4_t*>(zr + 4);
            z[0] = a[0]; z[1] = a[1]; z[2] = a[2]; z[3] = a[3];
            z[4] = c[0]; z[5] = c[1]; z[6] = c[2]; z[7] = c[3];
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) z[e] = (l0 + e < L) ? zr[e] : 0.f;
        }
        float dz[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const bool y = (ymask >> e) & 1u;
            // u = e^-|z|: sigmoid(|z|) = 1 / (1 + u), sigmoid(-|z|) = u / (1 + u)
            const float u = __builtin_amdgcn_exp2f(-fabsf(z[e]) * kLog2e);
            const float r = __builtin_amdgcn_rcpf(1.0f + u);
            const float sg = z[e] >= 0.f ? r : u * r;         // sigmoid(z)
            const float om = z[e] >= 0.f ? u * r : r;         // 1 - sigmoid(z)
            dz[e] = y ? -scale * om : scale * sg;
            if (loss && l0 + e < L)
                lsum += fmaxf(z[e], 0.f) + __builtin_amdgcn_logf(1.0f + u) * kLn2 - (y ? z[e] : 0.f);
        }
        uint32_t ph[4], pl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x2_t p = split_pair(dz[2 * i], dz[2 * i + 1]);
            ph[i] = p[0];
            pl[i] = p[1];
        }
        uint16_t* oh = dz_hi + b * L + l0;
        uint16_t* ol = dz_lo + b * L + l0;
        if (l0 + 8 <= L && L % 8 == 0) {
            *reinterpret_cast<u32x4_t*>(oh) = u32x4_t{ph[0], ph[1], ph[2], ph[3]};
            *reinterpret_cast<u32x4_t*>(ol) = u32x4_t{pl[0], pl[1], pl[2], pl[3]};
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (l0 + e < L) {
                    oh[e] = (uint16_t)(ph[e / 2] >> (16 * (e % 2)));
                    ol[e] = (uint16_t)(pl[e / 2] >> (16 * (e % 2)));
                }
            }
        }
    }
    if (loss) {
        // block sum, then one double atomic per block
        __shared__ float red[4];
        const float w = wave_sum(lsum);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = w;
        __syncthreads();
        if (threadIdx.x == 0) atomicAdd(loss, (double)((red[0] + red[1]) + (red[2] + red[3])) * (double)scale);
    }
}


// Logits and BCE gradient of the dense head in one pass: Z = h W^T on matrix
// cores with the epilogue of k_head_bce applied to the accumulators, so Z
// never goes through HBM unless asked for.  A workgroup owns 128 labels
// (wave wv: labels 32 wv .. +31, two 16-label tiles) and all rows (B <= 128,
// up to eight 16-row tiles); the contraction over H runs in stages of 64:
// h[:, stage] is staged in LDS for the four waves (rows' 16-byte chunks
// XOR-swizzled with (row / 2) % 8 so the operand reads of 16 rows spread over
// the banks), the weights go from global memory straight into the B operand
// (a label's four lanes read 64 contiguous bytes) with plain loads, so the dh
// product that reads W next can find it in the last-level cache.  The
// epilogue stages each 16-row tile's hi / lo parts in LDS and stores 64
// contiguous bytes per row; Z (optional) is stored directly.
constexpr int kHzLabels = 128;   // labels per workgroup
constexpr int kHzStage = 64;     // contraction width per LDS stage
__global__ __launch_bounds__(256) void k_head_zbce(const uint16_t* __restrict__ h, const uint16_t* __restrict__ W,
                                                   const int32_t* __restrict__ rowptr,
                                                   const int32_t* __restrict__ col, float scale,
                                                   float* __restrict__ Z, uint16_t* __restrict__ dz_hi,
                                                   uint16_t* __restrict__ dz_lo, double* __restrict__ loss,
                                                   int64_t B, int64_t H, int64_t L)
{
    constexpr int NRT = 8;                      // row tiles (B <= 128)
    constexpr int CH = kHzStage / 8;            // 16-byte chunks per staged row
    __shared__ __attribute__((aligned(16))) uint16_t sh[2][128 * kHzStage];
    __shared__ uint32_t sY[128][4];             // label bits per row: word wv <-> the wave's 32 labels
    __shared__ __attribute__((aligned(16))) uint16_t sD[4][2][16 * 32];   // per wave: hi / lo, 16 rows x 32 labels
    __shared__ float red[4];

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, q = lane >> 4;
    const int64_t L0 = (int64_t)blockIdx.x * kHzLabels;
    const int64_t lw = L0 + 32 * wv;            // the wave's first label
    const int nrt = (int)((B + 15) / 16);
    const int nst = (int)(H / kHzStage);

    // label bits of the block's 128 labels, one row per thread, found before
    // the first loads are issued (issuing the loads first and searching under
    // them measured 10 % slower per head pass)
    auto label_bits = [&]() {
        if (threadIdx.x < 128) {
            uint32_t m[4] = {0u, 0u, 0u, 0u};
            const int64_t b = threadIdx.x;
            if (b < B) {
                int lo = rowptr[b], hi = rowptr[b + 1];
                const int end = hi;
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if ((int64_t)col[mid] < L0) lo = mid + 1; else hi = mid;
                }
                for (int p = lo; p < end && (int64_t)col[p] < L0 + kHzLabels; ++p) {
                    const int c = (int)((int64_t)col[p] - L0);
                    if (c >= 0) m[c >> 5] |= 1u << (c & 31);   // rows are sorted; guards a malformed one
                }
            }
#pragma unroll
            for (int w = 0; w < 4; ++w) sY[threadIdx.x][w] = m[w];
        }
    };

    // h stage loads: piece u = threadIdx.x + 256 j is row u / CH, chunk u % CH
    auto load_h = [&](int st, u32x4_t (&hv)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int u = threadIdx.x + 256 * j;
            const int64_t b = u / CH;
            hv[j] = b < B ? ldg16(h + b * H + (int64_t)st * kHzStage + 8 * (u % CH)) : u32x4_t{0u, 0u, 0u, 0u};
        }
    };
    auto store_h = [&](int buf, const u32x4_t (&hv)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int u = threadIdx.x + 256 * j;
            const int r = u / CH, c = u % CH;
            *reinterpret_cast<u32x4_t*>(&sh[buf][r * kHzStage + 8 * (c ^ ((r >> 1) & 7))]) = hv[j];
        }
    };
    // B operand: label lw + 16 lt + r16 (clamped into range), k = stage + 32 s + 8 q ..
    auto load_w = [&](int st, u32x4_t (&wv4)[2][2]) {
#pragma unroll
        for (int lt = 0; lt < 2; ++lt) {
            int64_t l = lw + 16 * lt + r16;
            l = l < L ? l : L - 1;
#pragma unroll
            for (int s = 0; s < 2; ++s)
                wv4[lt][s] = ldg16(W + l * H + (int64_t)st * kHzStage + 32 * s + 8 * q);
        }
    };

    f32x4_t acc[NRT][2];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        acc[rt][0] = zero4();
        acc[rt][1] = zero4();
    }
    // the weights of stage st + 2 are requested while stage st runs (a ring of
    // three register sets; every wait for the current stage's weights leaves
    // the next two stages' loads in flight)
    u32x4_t hv[4], w0[2][2], w1[2][2], w2[2][2];
    label_bits();
    load_w(0, w0);
    if (nst > 1) load_w(1, w1);
    load_h(0, hv);
    store_h(0, hv);
    __syncthreads();
    auto stage = [&](int st, const u32x4_t (&cur)[2][2], u32x4_t (&far)[2][2]) {
        if (st >= nst) return;                 // uniform over the workgroup
        const bool more = st + 1 < nst;
        if (more) load_h(st + 1, hv);
        if (st + 2 < nst) load_w(st + 2, far);
        const uint16_t* tile = sh[st & 1];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                if (rt < nrt) {
                    const int r = 16 * rt + r16, c = 4 * s + q;
                    const u32x4_t av = *reinterpret_cast<const u32x4_t*>(&tile[r * kHzStage + 8 * (c ^ ((r >> 1) & 7))]);
                    acc[rt][0] = mfma16(av, cur[0][s], acc[rt][0]);
                    acc[rt][1] = mfma16(av, cur[1][s], acc[rt][1]);
                }
            }
        }
        if (more) store_h((st + 1) & 1, hv);
        __syncthreads();
    };
    for (int st = 0; st < nst; st += 3) {
        stage(st, w0, w2);
        stage(st + 1, w1, w0);
        stage(st + 2, w2, w1);
    }

    // epilogue: lane holds label lw + 16 lt + r16, rows 16 rt + 4 q + i
    float lsum = 0.f;
    uint16_t* th = sD[wv][0];
    uint16_t* tl = sD[wv][1];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        if (rt >= nrt) break;
        float prod = 1.f, lin = 0.f;
#pragma unroll
        for (int lt = 0; lt < 2; ++lt) {
            const int64_t l = lw + 16 * lt + r16;
            const bool lok = l < L;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * rt + 4 * q + i;
                const bool ok = lok && r < B;
                const float z = acc[rt][lt][i];
                const bool y = (sY[r][wv] >> (16 * lt + r16)) & 1u;
                // u = e^-|z|: sigmoid(|z|) = 1 / (1 + u), sigmoid(-|z|) = u / (1 + u)
                const float u = __builtin_amdgcn_exp2f(-fabsf(z) * kLog2e);
                const float w1 = 1.0f + u;
                const float rc = __builtin_amdgcn_rcpf(w1);
                const float sg = z >= 0.f ? rc : u * rc;          // sigmoid(z)
                const float om = z >= 0.f ? u * rc : rc;          // 1 - sigmoid(z)
                const float d = y ? -scale * om : scale * sg;
                const uint32_t hb = pack_bf16(d, 0.f) & 0xffffu;
                const uint32_t lb = pack_bf16(d - __uint_as_float(hb << 16), 0.f) & 0xffffu;
                th[(4 * q + i) * 32 + 16 * lt + r16] = (uint16_t)hb;
                tl[(4 * q + i) * 32 + 16 * lt + r16] = (uint16_t)lb;
                if (Z && ok) Z[(int64_t)r * L + l] = z;
                if (loss) {
                    prod *= ok ? w1 : 1.0f;
                    lin += ok ? fmaxf(z, 0.f) - (y ? z : 0.f) : 0.f;
                }
            }
        }
        if (loss) lsum += lin + __builtin_amdgcn_logf(prod) * kLn2;
        wave_sync();
        // 16 rows x 32 labels: lane -> row lane / 4, labels 8 (lane % 4) ..
        const int64_t b = 16 * rt + (lane >> 2);
        const int64_t l0 = lw + 8 * (lane & 3);
        const u32x4_t vh = *reinterpret_cast<const u32x4_t*>(&th[(lane >> 2) * 32 + 8 * (lane & 3)]);
        const u32x4_t vl = *reinterpret_cast<const u32x4_t*>(&tl[(lane >> 2) * 32 + 8 * (lane & 3)]);
        if (b < B && l0 < L) {
            *reinterpret_cast<u32x4_t*>(dz_hi + b * L + l0) = vh;
            *reinterpret_cast<u32x4_t*>(dz_lo + b * L + l0) = vl;
        }
        wave_sync();
    }
    if (loss) {
        const float w = wave_sum(lsum);
        if (lane == 0) red[wv] = w;
        __syncthreads();
        if (threadIdx.x == 0) atomicAdd(loss, (double)((red[0] + red[1]) + (red[2] + red[3])) * (double)scale);
    }
}

// dh = base + the sum over the S label chunks of their partial products, in
// chunk order (base = dh when accumulating, else 0).  halves = 2: each
// chunk's partial is the stacked 2B x H product, whose two B x H halves
// (hi, lo) are added first; halves = 1: a B x H partial.
__global__ __launch_bounds__(256) void k_head_dh_sum(const float* __restrict__ part, float* __restrict__ dh, int64_t n,
                                                     int S, int halves, bool accumulate)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float r = 0.f;
    if (halves == 2) {
#pragma unroll 4
        for (int s = 0; s < S; ++s) r += part[(int64_t)s * 2 * n + i] + part[(int64_t)s * 2 * n + n + i];
    } else {
#pragma unroll 4
        for (int s = 0; s < S; ++s) r += part[(int64_t)s * n + i];
    }
    dh[i] = accumulate ? dh[i] + r : r;
}

// The feature-gradient product of one label chunk (Lc labels, a multiple of
// 32 chosen so that the grid is at most one workgroup per CU) on the matrix
// cores: part[c][b, j] = sum over the chunk's labels l of (hi + lo)[b, l]
// W[l, j], for a block of 128 batch rows and 256 feature columns; wave w
// owns columns 32 w .. 32 w + 31 of the block for all 128 rows, so every
// staged operand is read by one wave only.  The chunk is walked in steps
// of 32 labels; each step's W tile (32 labels x 256 columns) and dZ tile
// (hi and lo, 128 rows x 32 labels) go through two LDS buffers (the next
// step's pieces are loaded into registers a step ahead).  W is read with
// ds_read_b64_tr_b16 as the label-contiguous operand, dZ rows with plain
// 16-byte reads; hi and lo accumulate into the same registers.  Needs
// L % 8 == 0 and H % 8 == 0 (16-byte pieces).
__global__ __launch_bounds__(512) void k_head_dh(const uint16_t* __restrict__ dzcat, const uint16_t* __restrict__ W,
                                                 float* __restrict__ part, int64_t B, int64_t H, int64_t L,
                                                 int64_t Lc)
{
    constexpr int CB = 256, WROW = CB + 16, ZROW = 32 + 8;
    __shared__ __attribute__((aligned(16))) uint16_t sW[2][32 * WROW];
    __shared__ __attribute__((aligned(16))) uint16_t sZ[2][2 * 128 * ZROW];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int q = lane >> 4, i16 = lane & 15, rr = i16 >> 2, cc = i16 & 3;
    const int64_t c = blockIdx.x;
    const int64_t j0 = (int64_t)blockIdx.y * CB, b0 = (int64_t)blockIdx.z * 128;
    const int64_t l0 = c * Lc, l1 = (l0 + Lc < L) ? l0 + Lc : L;

    // two register sets of pieces: set st % 2 holds step st, loaded two steps
    // before it is staged
    u32x4_t pw2[2][2], pz2[2][2];
    auto fetch = [&](int64_t l, u32x4_t (&pw)[2], u32x4_t (&pz)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int p = tid + 512 * i;
            {   // W: row r (label l + r), 16-byte piece pc (columns j0 + 8 pc ..)
                const int r = p >> 5, pc = p & 31;
                const int64_t ll = l + r, jj = j0 + 8 * pc;
                pw[i] = (ll < l1 && jj < H) ? ldg16(W + ll * H + jj) : u32x4_t{0u, 0u, 0u, 0u};
            }
            {   // dZ: part hl (hi / lo), batch row b0 + row, labels l + 8 pc ..
                const int hl = p >> 9, row = (p >> 2) & 127, pc = p & 3;
                const int64_t b = b0 + row, ll = l + 8 * pc;
                pz[i] = (b < B && ll < l1) ? ldg16(dzcat + (hl * B + b) * L + ll) : u32x4_t{0u, 0u, 0u, 0u};
            }
        }
    };
    auto stage = [&](int buf, const u32x4_t (&pw)[2], const u32x4_t (&pz)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int p = tid + 512 * i;
            *reinterpret_cast<u32x4_t*>(&sW[buf][(p >> 5) * WROW + 8 * (p & 31)]) = pw[i];
            *reinterpret_cast<u32x4_t*>(&sZ[buf][((p >> 9) * 128 + ((p >> 2) & 127)) * ZROW + 8 * (p & 3)]) = pz[i];
        }
    };

    f32x4_t acc[8][2];
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) {
        acc[rt][0] = zero4();
        acc[rt][1] = zero4();
    }
    const int nsteps = (int)((l1 - l0 + 31) / 32);
    fetch(l0, pw2[0], pz2[0]);
    fetch(l0 + 32, pw2[1], pz2[1]);
    stage(0, pw2[0], pz2[0]);
    fetch(l0 + 64, pw2[0], pz2[0]);           // fetches past the chunk load zeros
    for (int s0 = 0; s0 < nsteps; s0 += 2)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int s = s0 + u;
        if (s >= nsteps) break;
        const int buf = u;        // s & 1
        __syncthreads();          // stage buf is complete; nobody still reads buf ^ 1
        if (s + 1 < nsteps) {
            stage(buf ^ 1, pw2[u ^ 1], pz2[u ^ 1]);
            fetch(l0 + 32 * (s + 3), pw2[u ^ 1], pz2[u ^ 1]);
        }
        // B: the wave's two column tiles, labels 8q .. 8q + 7
        u32x4_t bo[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint16_t* base = &sW[buf][(8 * q + rr) * WROW + 32 * w + 16 * t + 4 * cc];
            bo[t] = cat(lds_tr16(base), lds_tr16(base + 4 * WROW));
        }
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) {
            const int row = 16 * rt + i16;
            const u32x4_t ah = *reinterpret_cast<const u32x4_t*>(&sZ[buf][row * ZROW + 8 * q]);
            const u32x4_t al = *reinterpret_cast<const u32x4_t*>(&sZ[buf][(128 + row) * ZROW + 8 * q]);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                acc[rt][t] = mfma16(ah, bo[t], acc[rt][t]);
                acc[rt][t] = mfma16(al, bo[t], acc[rt][t]);
            }
        }
    }
    // lane: column j0 + 32 w + 16 t + i16, batch rows b0 + 16 rt + 4 q + i
    float* out = part + c * B * H;
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int64_t j = j0 + 32 * w + 16 * t + i16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t b = b0 + 16 * rt + 4 * q + i;
                if (b < B && j < H) out[b * H + j] = acc[rt][t][i];
            }
        }
}

// dW = [hi; lo]^T [h; h] on the matrix cores, without the stacked copies:
// a workgroup owns 64 labels and 768 feature columns; the labels' dZ (hi
// and lo, Bp <= 128 batch rows x 64 labels) is staged in LDS once and read
// transposed (ds_read_b64_tr_b16) as the label-row operand; the batch-
// contiguous operand comes from the feature-major copy hT (H x Bp, zero
// rows past B) in L2; wave w owns 96 columns for the 64 labels (24 result
// tiles), hi and lo accumulating into the same registers.  dW rows are
// written once, through LDS as 16-byte pieces.  Needs L % 8 == 0,
// H % 4 == 0 and Bp <= 128.
__global__ __launch_bounds__(512) void k_head_dw(const uint16_t* __restrict__ dzcat, const uint16_t* __restrict__ hT,
                                                 int64_t Bp, float* __restrict__ dW, int64_t B, int64_t H, int64_t L)
{
    constexpr int LB = 64, ZROW = LB + 8, CW = 96, CT = CW / 16, OROW = CW + 4;
    __shared__ __attribute__((aligned(16))) uint16_t sZ[2][128 * ZROW];
    __shared__ __attribute__((aligned(16))) float sO[8][16 * OROW];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int q = lane >> 4, i16 = lane & 15, rr = i16 >> 2, cc = i16 & 3;
    const int64_t l0 = (int64_t)blockIdx.x * LB;
    const int64_t jw = (int64_t)blockIdx.y * (8 * CW) + CW * w;   // the wave's first column
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = tid + 512 * i;                // 2 x 128 rows x 8 pieces
        const int hl = p >> 10, row = (p >> 3) & 127, pc = p & 7;
        const int64_t ll = l0 + 8 * pc;
        const u32x4_t v = (row < B && ll < L) ? ldg16(dzcat + ((int64_t)hl * B + row) * L + ll)
                                              : u32x4_t{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4_t*>(&sZ[hl][row * ZROW + 8 * pc]) = v;
    }
    __syncthreads();
    f32x4_t acc[4][CT];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int t = 0; t < CT; ++t) acc[rt][t] = zero4();
    const int nks = (int)(Bp / 32);
    // batch-contiguous operands of step ks, requested a step ahead
    auto load_b = [&](int ks, u32x4_t (&bo)[CT]) {
#pragma unroll
        for (int t = 0; t < CT; ++t) {
            const int64_t j = jw + 16 * t + i16;
            bo[t] = (j < H && ks < nks) ? ldg16(hT + j * Bp + 32 * ks + 8 * q) : u32x4_t{0u, 0u, 0u, 0u};
        }
    };
    u32x4_t bo[CT], bn[CT];
    load_b(0, bn);
    for (int ks = 0; ks < nks; ++ks) {
#pragma unroll
        for (int t = 0; t < CT; ++t) bo[t] = bn[t];
        load_b(ks + 1, bn);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
            for (int hl = 0; hl < 2; ++hl) {
                const uint16_t* base = &sZ[hl][(32 * ks + 8 * q + rr) * ZROW + 16 * rt + 4 * cc];
                const u32x4_t a = cat(lds_tr16(base), lds_tr16(base + 4 * ZROW));
#pragma unroll
                for (int t = 0; t < CT; ++t) acc[rt][t] = mfma16(a, bo[t], acc[rt][t]);
            }
        }
    }
    // out through LDS, one 16-label tile at a time, so dW rows go out as
    // 16-byte pieces of 384-byte runs (lane: column jw + 16 t + i16, labels
    // l0 + 16 rt + 4 q + i)
    float* so = sO[w];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
        for (int t = 0; t < CT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) so[(4 * q + i) * OROW + 16 * t + i16] = acc[rt][t][i];
        wave_sync();
#pragma unroll
        for (int u = 0; u < 6; ++u) {                // 16 rows x 24 pieces
            const int pc = lane + 64 * u, row = pc / 24, c4 = pc % 24;
            const int64_t l = l0 + 16 * rt + row, j = jw + 4 * c4;
            if (l < L && j < H) stg_stream(dW + l * H + j, *reinterpret_cast<const f32x4_t*>(&so[row * OROW + 4 * c4]));
        }
        wave_sync();
    }
}

// The head pass on `stream`: Z (B x L fp32, in zbuf), the BCE gradient as a
// stacked bf16 hi / lo matrix dzcat (2B x L), hcat = [h; h] (2B x H bf16),
// dW = dzcat^T hcat (L x H fp32), the stacked dh products of the
// head_dh_chunks(L) label chunks in dhcat (that many 2B x H fp32 blocks) and
// dh (B x H fp32, added to when accumulate_dh).  The feature-gradient
// product has a B x H output and an L-deep contraction; splitting the
// contraction into label chunks (a strided batch of GEMMs) is what spreads
// it over the chip.  Returns false if a rocBLAS call or a copy fails.
bool run_head(const uint16_t* h, const uint16_t* W, const int32_t* rowptr, const int32_t* col, float scale,
              float* dW, float* dh, float* zbuf, bool want_z, double* loss, int64_t B, int64_t H, int64_t L,
              bool accumulate_dh, uint16_t* dzcat, uint16_t* hcat, float* dhcat, uint16_t* hT, void* blas_ws,
              size_t blas_ws_bytes, hipStream_t stream)
{
    const int64_t Bp = (B + 31) / 32 * 32;
    const bool own_z = B <= 128 && H % kHzStage == 0 && L % 8 == 0;
    const bool own_dw = L % 8 == 0 && H % 4 == 0 && Bp <= 128;
    const bool own_dh = L % 8 == 0 && H % 8 == 0;
    // the rocBLAS handle (per thread and device, kept for the process) is
    // created only when some product is not one of libhaste's own kernels
    rocblas_handle bh = nullptr;
    if (!(own_z && own_dw && own_dh)) {
        bh = blas_handle(stream, blas_ws, blas_ws_bytes);
        if (!bh) return false;
    }
    if (own_dw) {
        launch_transpose_h(h, hT, B, H, Bp, stream);
    } else {
        const size_t hbytes = (size_t)B * (size_t)H * 2;
        if (hipMemcpyAsync(hcat, h, hbytes, hipMemcpyDeviceToDevice, stream) != hipSuccess) return false;
        if (hipMemcpyAsync(hcat + B * H, h, hbytes, hipMemcpyDeviceToDevice, stream) != hipSuccess) return false;
    }
    if (own_z) {
        // Z and the BCE gradient in one kernel (Z stored only when asked for)
        hipLaunchKernelGGL(k_head_zbce, dim3((unsigned)((L + kHzLabels - 1) / kHzLabels)), dim3(256), 0, stream, h,
                           W, rowptr, col, scale, want_z ? zbuf : nullptr, dzcat, dzcat + B * L, loss, B, H, L);
    } else {
        // Z = h W^T (B x L) on rocBLAS, then the BCE gradient
        if (gemm_rm(bh, false, true, B, L, H, h, H, W, H, 0.f, zbuf, L) != rocblas_status_success) return false;
        const int64_t n = B * ((L + 7) / 8);
        hipLaunchKernelGGL(k_head_bce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, zbuf, rowptr, col,
                           scale, dzcat, dzcat + B * L, loss, B, L);
    }
    // dW = [hi; lo]^T [h; h] (L x H)
    if (own_dw) {
        hipLaunchKernelGGL(k_head_dw, dim3((unsigned)((L + 63) / 64), (unsigned)((H + 767) / 768)), dim3(512), 0,
                           stream, dzcat, hT, Bp, dW, B, H, L);
    } else if (gemm_rm(bh, true, false, L, H, 2 * B, dzcat, L, hcat, H, 0.f, dW, H) != rocblas_status_success) {
        return false;
    }
    const int64_t m = B * H;
    if (own_dh) {
        // per label chunk c: (hi + lo)[:, chunk c] W[chunk c, :] (B x H) on libhaste's kernel
        const int64_t S = head_dh_mfma_chunks(B, H, L), Lc = head_dh_mfma_chunk_len(B, H, L);
        const dim3 grid((unsigned)S, (unsigned)((H + 255) / 256), (unsigned)((B + 127) / 128));
        hipLaunchKernelGGL(k_head_dh, grid, dim3(512), 0, stream, dzcat, W, dhcat, B, H, L, Lc);
        hipLaunchKernelGGL(k_head_dh_sum, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, stream, dhcat, dh, m,
                           (int)S, 1, accumulate_dh);
        return true;
    }
    // otherwise on rocBLAS: per label chunk c, [dh_hi; dh_lo]_c = [hi; lo][:, chunk c] W[chunk c, :] (2B x H)
    const int64_t Lc = kHeadDhChunk, full = L / Lc, rem = L % Lc;
    const float one = 1.0f, zero = 0.0f;
    if (full > 0 &&
        rocblas_gemm_strided_batched_ex(bh, rocblas_operation_none, rocblas_operation_none, (rocblas_int)H,
                                        (rocblas_int)(2 * B), (rocblas_int)Lc, &one, W, rocblas_datatype_bf16_r,
                                        (rocblas_int)H, Lc * H, dzcat, rocblas_datatype_bf16_r, (rocblas_int)L, Lc,
                                        &zero, dhcat, rocblas_datatype_f32_r, (rocblas_int)H, 2 * B * H, dhcat,
                                        rocblas_datatype_f32_r, (rocblas_int)H, 2 * B * H, (rocblas_int)full,
                                        rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0,
                                        0) != rocblas_status_success)
        return false;
    if (rem > 0 && gemm_rm(bh, false, false, 2 * B, H, rem, dzcat + full * Lc, L, W + full * Lc * H, H, 0.f,
                           dhcat + full * 2 * B * H, H) != rocblas_status_success)
        return false;
    hipLaunchKernelGGL(k_head_dh_sum, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, stream, dhcat, dh, m,
                       (int)head_dh_chunks(L), 2, accumulate_dh);
    return true;
}

}  // namespace haste

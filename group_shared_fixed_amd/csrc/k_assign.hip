// k-means assignment on the matrix cores, scores and arg-max fused: for each
// label row its nearest centre (the largest dot product, the lowest centre
// on ties) and that score, without the label x centre score matrix ever
// reaching memory.
//
// HASTE notes, "group-shared fixed fan-in": the coarse stage clusters label
// embeddings by spherical k-means; a label belongs to the centre whose
// embedding has the largest dot product with its own (bf16 inputs, fp32
// accumulation here).
//
// Layout: the label rows X (n x H bf16) and the centres M (C x H bf16) are
// both contiguous along the contraction, so a 16-byte piece of a row is
// directly one lane's operand of a 32x32x16 matrix-core product.  A
// workgroup of four waves scores one tile of 256 labels x 256 centres; each
// wave owns a 128 x 128 quarter, held as 16 accumulator tiles of 32 x 32
// (256 fp32 per lane, in the accumulation registers).
//
// The contraction runs in LDS stages of 32 through a ring of four stage
// buffers (32 KB each: both operands' 256 rows x 64 bytes).  The operands
// move from global memory straight into LDS (global_load_lds_dwordx4: each
// lane's 16 bytes land at the wave's LDS base + 16 x lane, no registers),
// three stages ahead of the products, so about 96 KB per CU is in flight.
// Per stage: wait for this wave's moves of the stage, one barrier (everyone's
// moves are done, and the buffer read one stage ago is free), issue the moves
// of the stage three ahead into that buffer, then the products.  The loop
// is unrolled over the ring so each buffer is a distinct LDS object and has
// no branches (past the end it repeats the last stage's moves into buffers
// nobody reads): the compiler then adds no waits of its own beyond these.
// Staged rows are 64 bytes; their 16-byte pieces are XOR-swizzled with
// (row / 4) % 4, so the 16 rows that 16 consecutive lanes read in one
// operand fetch fall in distinct banks.  H must be a multiple of 128 (four stages per loop
// turn); other widths are zero-padded into a copy first.
//
// Tiles are dealt so that the workgroups resident on one XCD (workgroup ids
// go round-robin over the 8 XCDs) work on neighbouring tiles, eight label
// tiles by a run of centre tiles, and share their operand rows in that
// XCD's L2.
//
// Epilogue: the workgroup reduces its tile to one (score, centre) per label
// row (through LDS) and folds it into a 64-bit key per label with an atomic
// maximum, one per row.  The key orders by score, then by the lower centre,
// so the maximum over all centre tiles is the assignment with its tie rule
// whatever the order in which the tiles arrive: the result is bitwise
// repeatable.
#include "common.hpp"
#include "kernels.hpp"

namespace haste {
namespace {

constexpr int kAsTile = 256;       // labels and centres per workgroup tile
constexpr int kAsStage = 32;       // contraction per LDS stage
constexpr int kAsWidth = 128;      // the kernel's H granularity (four stages)
constexpr int kAsGroupRows = 8;    // label tiles per dealing group
// Order-preserving image of an fp32 score in 32 unsigned bits (-0 and +0
// map to the same value, so equal scores compare equal).
__device__ __forceinline__ uint32_t score_order(float s)
{
    const uint32_t u = __float_as_uint(s == 0.f ? 0.f : s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_score(uint32_t o)
{
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
// Key of (score, centre): larger score first, then the lower centre.
__device__ __forceinline__ unsigned long long assign_key(float s, int c)
{
    return ((unsigned long long)score_order(s) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)c);
}

// s_waitcnt vmcnt(N) alone (expcnt and lgkmcnt at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Workgroup barrier without a memory fence (a fence would wait for every
// move in flight); the empty asm statements keep the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void bare_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// 32x32x16 bf16 matrix-core product, fp32 accumulate.  Lane l supplies A
// row (l % 32) and B column (l % 32), contraction elements 8 (l / 32) .. + 8;
// the result lands as: lane l holds column (l % 32), element e at row
// 8 (e / 4) + 4 (l / 32) + e % 4.
__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

// keys[i] (pre-zeroed) = max over centres c of assign_key(<X_i, M_c>, c), X:
// n x H bf16, M: C x H bf16, H % 128 == 0.  Grid: one workgroup per (label
// tile, centre tile), nrt x nct workgroups of 256 threads.
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_assign(
    const uint16_t* __restrict__ X, int64_t n, const uint16_t* __restrict__ M, int64_t C, int64_t H, uint32_t nrt,
    uint32_t nct, unsigned long long* __restrict__ keys)
{
    // the stage ring: [A: 256 rows x 32][B: 256 rows x 32] bf16 per buffer
    constexpr int kHalf = kAsTile * kAsStage;
    __shared__ __attribute__((aligned(1024))) uint16_t ring0[2 * kHalf];
    __shared__ __attribute__((aligned(1024))) uint16_t ring1[2 * kHalf];
    __shared__ __attribute__((aligned(1024))) uint16_t ring2[2 * kHalf];
    __shared__ __attribute__((aligned(1024))) uint16_t ring3[2 * kHalf];

    // tile of this workgroup: ids dealt XCD by XCD (the last nb % 8 in
    // order), then eight label tiles by the centre tiles in turn
    const uint32_t nb = gridDim.x, b = blockIdx.x, per = nb / 8;
    const uint32_t t = b < per * 8 ? (b & 7) * per + (b >> 3) : b;
    const uint32_t span = (uint32_t)kAsGroupRows * nct;
    const uint32_t grp = t / span, first = grp * kAsGroupRows;
    const uint32_t gr = nrt - first < (uint32_t)kAsGroupRows ? nrt - first : (uint32_t)kAsGroupRows;
    const uint32_t loc = t - grp * span;
    const int64_t row0 = (int64_t)(first + loc % gr) * kAsTile;
    const int64_t col0 = (int64_t)(loc / gr) * kAsTile;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = w >> 1, wc = w & 1, r16 = lane & 15, q = lane >> 4;

    // moves: wave w stages rows 64 w + 16 i + lane / 4 (i = 0..3) of both
    // operands; the lane's LDS slot is piece lane % 4 of that row, which holds
    // the row's piece (lane % 4) ^ (row / 4) % 4 = (lane % 4) ^ (lane / 16).
    // Rows past the end repeat the last row.  Offsets are 32-bit bytes from
    // the tile's first row (a tile spans at most 256 rows x 2 KB).
    const char* const Xt = reinterpret_cast<const char*>(X + row0 * H);
    const char* const Mt = reinterpret_cast<const char*>(M + col0 * H);
    const int rlast = (int)(n - 1 - row0 < kAsTile ? n - 1 - row0 : kAsTile - 1);
    const int clast = (int)(C - 1 - col0 < kAsTile ? C - 1 - col0 : kAsTile - 1);
    const uint32_t rowb = 2 * (uint32_t)H, pl = 16 * (uint32_t)((lane & 3) ^ (lane >> 4));
    uint32_t ao[4], bo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 64 * w + 16 * i + (lane >> 2);
        ao[i] = (uint32_t)(r < rlast ? r : rlast) * rowb + pl;
        bo[i] = (uint32_t)(r < clast ? r : clast) * rowb + pl;
    }
    const int nst = (int)(H / kAsStage);          // a multiple of 4
    auto move = [&](int st, uint16_t* buf) {
        const int64_t k = 2 * (int64_t)(st < nst ? st : nst - 1) * kAsStage;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            __builtin_amdgcn_global_load_lds(Xt + k + ao[i], (lds_ptr)(buf + (64 * w + 16 * i) * kAsStage), 16, 0,
                                             0);
            __builtin_amdgcn_global_load_lds(Mt + k + bo[i], (lds_ptr)(buf + kHalf + (64 * w + 16 * i) * kAsStage),
                                             16, 0, 0);
        }
    };

    // 32x32x16 products: per wave 4 x 4 result tiles of 32 x 32, 16 fp32 per
    // lane each.  (With 8 x 8 tiles of the 16x16x32 product the compiler
    // renamed most accumulator chains inside the loop and copied them back
    // at its end, ~700 accumulator moves per four stages, 25 % of the
    // kernel's time; these 16 chains stay in place.)
    f32x16_t acc[4][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[rt][ct] = f32x16_t{};

    // operand fetch: lane (h, r32) reads tile row 32 x + r32, logical piece
    // 2 s + h of the stage (s = the 16-deep step), stored as piece
    // (2 s + h) ^ (row / 4) % 4 = (2 s + h) ^ (r32 / 4) % 4
    const int r32 = lane & 31, h = lane >> 5, rsw = (r32 >> 2) & 3;
    auto products = [&](const uint16_t* buf) {
        const uint16_t* tA = buf + (128 * wr + r32) * kAsStage;
        const uint16_t* tB = buf + kHalf + (128 * wc + r32) * kAsStage;
        u32x4_t af[2][4], bf[2][4];
        auto rd = [&](int st16) {
            const int pc = 8 * ((2 * st16 + h) ^ rsw);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
                bf[st16][ct] = *reinterpret_cast<const u32x4_t*>(tB + 32 * ct * kAsStage + pc);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
                af[st16][rt] = *reinterpret_cast<const u32x4_t*>(tA + 32 * rt * kAsStage + pc);
        };
        // the second step's fragments are read while the first step's
        // products run (the scheduling barriers keep that interleave)
        rd(0);
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        rd(1);
#pragma unroll
        for (int st16 = 0; st16 < 2; ++st16)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) acc[rt][ct] = mfma32(af[st16][rt], bf[st16][ct], acc[rt][ct]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    };
    // stage st: this wave's moves of st done (those of st + 1 and st + 2,
    // 16 instructions, may be in flight), barrier, moves of st + 3 into the
    // buffer stage st - 1 used, products of st
    auto stage = [&](int st, const uint16_t* cur, uint16_t* nxt) {
        wait_vm<16>();
        bare_barrier();
        move(st + 3, nxt);
        __builtin_amdgcn_sched_group_barrier(0x020, 8, 0);   // the moves first
        products(cur);
    };

    move(0, ring0);
    move(1, ring1);
    move(2, ring2);
    for (int st = 0; st < nst; st += 4) {
        stage(st, ring0, ring3);
        stage(st + 1, ring1, ring0);
        stage(st + 2, ring2, ring1);
        stage(st + 3, ring3, ring2);
    }
    wait_vm<0>();              // the repeated moves past the end, into buffers reused below
    bare_barrier();

    // Lane (h, r32) holds, for result tile (rt, ct), element e: row
    // 32 rt + 8 (e / 4) + 4 h + e % 4, centre 32 ct + r32 of the wave's
    // quarter.  Each lane keeps, per row, its best over ct (centres rise with
    // ct, so a strict comparison keeps the lowest; centres past C only occur
    // in the last centre tile) and writes it to slot 32 wc + r32 of the row;
    // then thread t reduces row t over its 64 slots: the largest score, then
    // the lowest centre holding it.  Row r's slots sit in buffer r / 64 (the
    // whole ring), 512 bytes per row, pair s at s ^ 2 (r % 16), so that 16
    // consecutive threads' 16-byte reads fall in distinct banks.
    auto part_rows = [&](int quarter) {
        uint16_t* p = quarter == 0 ? ring0 : quarter == 1 ? ring1 : quarter == 2 ? ring2 : ring3;
        return reinterpret_cast<f32x2_t*>(p);
    };
    const int cw = (int)col0 + 128 * wc + r32;      // C < 2^30
    const int slot = 32 * wc + r32;
    auto lane_best = [&](bool ragged) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            f32x2_t* const part = part_rows(2 * wr + (rt >> 1));
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float bv = acc[rt][0][e];
                int bc = 0;
                if (ragged && cw >= C) bv = -INFINITY;
#pragma unroll
                for (int ct = 1; ct < 4; ++ct) {
                    float v = acc[rt][ct][e];
                    if (ragged && cw + 32 * ct >= C) v = -INFINITY;
                    if (v > bv) {
                        bv = v;
                        bc = ct;
                    }
                }
                const int lr = 32 * (rt & 1) + 8 * (e >> 2) + 4 * h + (e & 3);   // row within its buffer
                part[lr * 64 + (slot ^ (2 * (lr & 15)))] = f32x2_t{bv, __int_as_float(cw + 32 * bc)};
            }
        }
    };
    if (col0 + kAsTile > C)          // uniform: only the last centre tile has centres past C
        lane_best(true);
    else
        lane_best(false);
    __syncthreads();
    const int64_t r = row0 + tid;
    if (r < n) {
        const int lr = tid & 63;
        const f32x2_t* pr = part_rows(w) + lr * 64;
        // a running best over the 64 (score, centre) slots: the larger score,
        // the lower centre on equal scores
        float m = -INFINITY;
        int bc = 0x7fffffff;
#pragma unroll
        for (int u = 0; u < 32; ++u) {
            const f32x4_t v = *reinterpret_cast<const f32x4_t*>(pr + 2 * (u ^ (lr & 15)));
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
                const float sv = v[e];
                const int cv = __float_as_int(v[e + 1]);
                const bool better = sv > m || (sv == m && cv < bc);
                m = better ? sv : m;
                bc = better ? cv : bc;
            }
        }
        atomicMax(keys + r, assign_key(m, bc));
    }
}

// out[i] (row stride Hp, zero beyond H) = E[rows ? rows[i] : i] (H bf16,
// H % 8 == 0), 16-byte pieces.
__global__ __launch_bounds__(256) void k_pack_rows(const uint16_t* __restrict__ E, const int32_t* __restrict__ rows,
                                                   int64_t n, int64_t H, int64_t Hp, uint16_t* __restrict__ out)
{
    const int64_t pieces = Hp / 8;
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < n * pieces; t += (int64_t)gridDim.x * 256) {
        const int64_t i = t / pieces, p = t % pieces;
        const int64_t src = rows ? (int64_t)rows[i] : i;
        *reinterpret_cast<u32x4_t*>(out + i * Hp + 8 * p) =
            8 * p < H ? ldg16(E + src * H + 8 * p) : u32x4_t{0u, 0u, 0u, 0u};
    }
}

// a[i], smax[i] (nullable) from the keys.
__global__ __launch_bounds__(256) void k_assign_finish(const unsigned long long* __restrict__ keys, int64_t n,
                                                       int32_t* __restrict__ a, float* __restrict__ smax)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const unsigned long long k = keys[i];
        a[i] = (int32_t)(0xffffffffu - (uint32_t)k);
        if (smax) smax[i] = order_score((uint32_t)(k >> 32));
    }
}

unsigned blocks_for(int64_t n, int64_t cap)
{
    const int64_t g = (n + 255) / 256;
    return (unsigned)(g < 1 ? 1 : (g > cap ? cap : g));
}

}  // namespace

int64_t kmeans_assign_tiles(int64_t n_rows, int64_t C)
{
    return ((n_rows + kAsTile - 1) / kAsTile) * ((C + kAsTile - 1) / kAsTile);
}

int64_t kmeans_assign_width(int64_t H) { return (H + kAsWidth - 1) / kAsWidth * kAsWidth; }

void run_kmeans_assign(const uint16_t* E, const int32_t* rows, int64_t n_rows, const uint16_t* M, int64_t C,
                       int64_t H, int32_t* a, float* smax, uint64_t* keys, uint16_t* xpack, uint16_t* mpack,
                       hipStream_t s)
{
    const uint32_t nrt = (uint32_t)((n_rows + kAsTile - 1) / kAsTile);
    const uint32_t nct = (uint32_t)((C + kAsTile - 1) / kAsTile);
    const int64_t Hp = kmeans_assign_width(H);
    const uint16_t* X = E;
    if (rows || Hp != H) {
        hipLaunchKernelGGL(k_pack_rows, dim3(blocks_for(n_rows * (Hp / 8), 65536)), dim3(256), 0, s, E, rows, n_rows,
                           H, Hp, xpack);
        X = xpack;
    }
    if (Hp != H) {
        hipLaunchKernelGGL(k_pack_rows, dim3(blocks_for(C * (Hp / 8), 65536)), dim3(256), 0, s, M,
                           (const int32_t*)nullptr, C, H, Hp, mpack);
        M = mpack;
    }
    launch_fill_f64(reinterpret_cast<double*>(keys), n_rows, s);   // all-zero bits: below every key
    hipLaunchKernelGGL(k_assign, dim3(nrt * nct), dim3(256), 0, s, X, n_rows, M, C, Hp, nrt, nct,
                       reinterpret_cast<unsigned long long*>(keys));
    hipLaunchKernelGGL(k_assign_finish, dim3(blocks_for(n_rows, 4096)), dim3(256), 0, s,
                       reinterpret_cast<const unsigned long long*>(keys), n_rows, a, smax);
}

}  // namespace haste

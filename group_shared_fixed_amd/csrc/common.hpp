// Device helpers shared by the HIP kernels of libhaste (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

namespace haste {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16x16x32 bf16 matrix-core product, fp32 accumulate.
// Lane l supplies A row (l % 16) and B column (l % 16); the 32-deep
// contraction is split over the four lane groups q = l / 16, eight values
// per lane.  Any assignment of contraction indices to (q, element) works as
// long as A and B use the same one.  The 16x16 result lands as: lane l holds
// column (l % 16), rows 4*(l/16) + i for i = 0..3.
__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float bf16lo_to_f32(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

// Split fp32 pairs into bf16 hi parts and bf16 residual (lo) parts so that
// hi + lo carries about 16 significant bits of x.
// Returns {hi, lo} packed pairs.
__device__ __forceinline__ u32x2_t split_pair(float x0, float x1)
{
    const uint32_t hi = pack_bf16(x0, x1);
    const uint32_t lo = pack_bf16(x0 - bf16lo_to_f32(hi), x1 - bf16hi_to_f32(hi));
    return u32x2_t{hi, lo};
}

// Orders LDS accesses of one wavefront (LDS executes a wave's accesses in
// issue order; this keeps the compiler from moving them across).
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// gfx950 LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane 4r + c supplies the address of 4 consecutive 16-bit values;
// lane 4c + e receives value e of the lanes c, 4 + c, 8 + c, 12 + c (in that
// order).  So if lane 4r + c points at row k0 + r, column n0 + 4c of a tile
// stored row-major with rows along the contraction index, lane i receives
// column n0 + i, rows k0 .. k0 + 3: the K-contiguous matrix-core operand.
__device__ __forceinline__ u32x2_t lds_tr16(const uint16_t* p)
{
    typedef short s16x4_t __attribute__((ext_vector_type(4)));
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(p));
    return __builtin_bit_cast(u32x2_t, v);
}

__device__ __forceinline__ u32x4_t cat(u32x2_t a, u32x2_t b) { return u32x4_t{a[0], a[1], b[0], b[1]}; }

// An empty use of registers filled by loads: every path through this point
// has waited for those loads, so code further on that reuses the registers
// needs no wait (without it, a path that skipped the use leaves the loads
// pending and the compiler drains all outstanding loads before the reuse).
__device__ __forceinline__ void settle(const u32x4_t& v) { asm volatile("" ::"v"(v)); }
__device__ __forceinline__ void settle(int v) { asm volatile("" ::"v"(v)); }

__device__ __forceinline__ void settle(const u32x2_t& v) { asm volatile("" ::"v"(v)); }

// Type selection without <type_traits>.
template <bool C, class A, class B>
struct pick {
    using type = A;
};
template <class A, class B>
struct pick<false, A, B> {
    using type = B;
};

// Eight FP8 E4M3 weights (one 8-byte piece, weight i in byte i) times the
// power-of-two scale sc, as eight bf16 values in one 16-byte piece (value i
// in half i).  Exact: a code has four significant bits.
__device__ __forceinline__ u32x4_t widen_w8(u32x2_t v, float sc)
{
    return u32x4_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], sc, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], sc, true)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], sc, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], sc, true))};
}
// Identity for bf16 weight pieces (the same call site serves both formats).
__device__ __forceinline__ u32x4_t widen_w8(u32x4_t v, float) { return v; }

__device__ __forceinline__ u32x2_t ldg8(const void* p) { return *reinterpret_cast<const u32x2_t*>(p); }
__device__ __forceinline__ u32x2_t ldg8_stream(const void* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
}

__device__ __forceinline__ u32x4_t ldg16(const void* p)
{
    return *reinterpret_cast<const u32x4_t*>(p);
}

// 16-byte load of a streamed input (read once): non-temporal, so it does
// not displace the gathered feature rows cached in L2.  (Measured per use:
// a win for the weights in the forward family, a loss for its dZ input.)
__device__ __forceinline__ u32x4_t ldg16_stream(const void* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

// 16-byte store of a streamed output (written once, not read again soon):
// non-temporal, so it does not displace cached inputs.
__device__ __forceinline__ void stg_stream(float* p, f32x4_t v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(p));
}
__device__ __forceinline__ void stg_stream(uint16_t* p, u32x4_t v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v += __shfl_xor(v, o, 64);
    return v;
}

// Ordered hand-off between the waves of a workgroup through a counter in LDS:
// wait_turn blocks the wave until the counter reads v, pass_turn sets it to
// v + 1.  LDS executes the DS instructions of one wave in issue order, so the
// LDS writes a wave made before pass_turn are visible to the wave that next
// sees the counter move; only the compiler has to be kept from reordering
// them.  The wait is bounded (`spins` polls, by default kTurnSpins, far
// beyond any legitimate wait): wait_turn returns false when the bound is
// reached, and the caller then skips its update and reports the failure, so
// a broken turn sequence cannot hang the GPU or pass unnoticed.  While it
// holds the turn the wave runs at a raised issue priority, so the waves
// queued behind it (and spinning on the counter) do not slow it down.
constexpr int kTurnSpins = 1 << 24;
__device__ __forceinline__ bool wait_turn(const int* t, int v, int spins)
{
    bool got = false;
#pragma unroll 1
    for (int spin = 0; spin < spins; ++spin) {
        const int cur = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(t, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
        if (cur == v) {
            got = true;
            break;
        }
    }
    __builtin_amdgcn_s_setprio(2);
    return got;
}

// pass_turn_to stores a successor value the caller formed ahead of the turn
// (in a vector register), so the held turn ends with the store itself.
__device__ __forceinline__ void pass_turn_to(int* t, int next)
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __hip_atomic_store(t, next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __builtin_amdgcn_s_setprio(0);
}

__device__ __forceinline__ void pass_turn(int* t, int v) { pass_turn_to(t, v + 1); }

// XOR swizzle of 16-byte chunks inside a row of an LDS tile so that the
// transposing 2-byte writes and the 16-byte matrix-operand reads of one
// instruction spread over distinct banks.
__device__ __forceinline__ int swz(int r, int nchunks)
{
    int s = ((r & 3) | ((r >> 1) & 4)) ^ (((r >> 4) & 1) << 1);
    return s & (nchunks - 1);
}

// Visits the cells i = start, start + step, ... < rows * width of a row-major
// rows x width tile as (row, column) pairs, with one division for the start
// and additions after it (a per-element division by a run-time width costs
// a long instruction sequence, and 64-bit ones far more).
template <typename Fn>
__device__ __forceinline__ void for_cells(int rows, int width, int start, int step, Fn&& fn)
{
    int r = start / width, j = start - r * width;
    const int sr = step / width, sj = step - sr * width;
    while (r < rows) {
        fn(r, j);
        r += sr;
        j += sj;
        if (j >= width) {
            j -= width;
            ++r;
        }
    }
}

// Walks one sample's sorted positive-label list (a CSR row of the 0/1 label
// matrix) alongside groups visited in increasing order.  take(lo, G) returns
// the G-bit mask of positives with ids in [lo, lo + G) and skips ids below lo.
struct LabelCursor {
    int pos, end, next;

    __device__ __forceinline__ void init(const int32_t* rowptr, const int32_t* col, int64_t b, int64_t B,
                                         int64_t first)
    {
        pos = end = 0;
        next = 0x7fffffff;
        if (b < B) {
            int lo = rowptr[b], hi = rowptr[b + 1];
            end = hi;
            while (lo < hi) {
                int mid = (lo + hi) >> 1;
                if ((int64_t)col[mid] < first) lo = mid + 1; else hi = mid;
            }
            pos = lo;
            next = pos < end ? col[pos] : 0x7fffffff;
        }
    }

    __device__ __forceinline__ uint64_t take(int64_t lo, int G, const int32_t* col)
    {
        uint64_t m = 0;
        while ((int64_t)next < lo + G) {
            if ((int64_t)next >= lo) m |= 1ull << (int)((int64_t)next - lo);
            ++pos;
            next = pos < end ? col[pos] : 0x7fffffff;
        }
        return m;
    }
};

// Raises the dynamic-LDS limit of kernel Kern on the current device to
// `bytes` when a launch needs more than the default 64 KB (the attribute is
// per device, and it is only ever raised).  A refused raise is cleared from
// the thread's last error, so the launch that follows reports its own
// failure.  Safe to call from several host threads.
constexpr int kMaxDevices = 64;
template <auto Kern>
inline void raise_dyn_lds(size_t bytes)
{
    if (bytes <= 64 * 1024) return;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return;
    }
    static std::atomic<size_t> raised[kMaxDevices];
    size_t cur = raised[dev].load(std::memory_order_relaxed);
    if (bytes <= cur) return;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(Kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)bytes) != hipSuccess) {
        (void)hipGetLastError();
        return;
    }
    while (cur < bytes && !raised[dev].compare_exchange_weak(cur, bytes, std::memory_order_relaxed)) {
    }
}

}  // namespace haste

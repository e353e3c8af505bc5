// FP8 (E4M3) weights with one power-of-two scale per label group.
//
// HASTE notes, "limitations": pairing the layer with FP8 quantisation is the
// named next step.  Storage: W8[l, f] is the OCP E4M3 code (1 sign bit, 4
// exponent bits with bias 7, 3 mantissa bits, largest finite value 448) of
// W[l, f] * 2^-e_k, with e_k the smallest integer that keeps the group's
// largest |W| within 448.  A weight is decode(code) * 2^e_k, an exact bf16
// value, so the FP8 variants of the kernels run the bf16 arithmetic on it.
#include "common.hpp"
#include "kernels.hpp"

namespace haste {

namespace {

// Smallest e with m * 2^-e <= 448 for the magnitude m given by bf16 bits
// mb (non-negative, finite), clamped to [-120, 120]; 0 for m = 0.  With
// m = f * 2^p, f in [1, 2): e = p - 8 + (f > 1.75), since 448 = 1.75 * 2^8.
__device__ __forceinline__ int group_exponent(uint32_t mb)
{
    if (mb == 0) return 0;
    const int E = (int)(mb >> 7), m = (int)(mb & 0x7f);
    int e;
    if (E > 0) {
        e = (E - 127) - 8 + (m > 96 ? 1 : 0);          // f = 1 + m / 128
    } else {
        const int k = 31 - __clz(m);                    // subnormal: m * 2^-133 = (m / 2^k) 2^(k-133)
        e = (k - 133) - 8 + (4 * m > (7 << k) ? 1 : 0);
    }
    return e < -120 ? -120 : (e > 120 ? 120 : e);
}

// E4M3 code of an fp32 value with |x| <= 448, rounded to nearest, ties to
// the even code, from the bits of x: at or above 2^-6 the code is
// 8 (E + 6) + q with q the 4-bit significand (a carry to 16 moves into the
// next binade by itself); below it the code is |x| in units of 2^-9.
__device__ __forceinline__ uint32_t e4m3_code(float x)
{
    const uint32_t u = __float_as_uint(x);
    const uint32_t sgn = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    const int E32 = (int)(a >> 23);
    const uint32_t M = a & 0x7fffffu;
    uint32_t code;
    if (E32 >= 121) {
        uint32_t q = 8u | (M >> 20);
        const uint32_t rem = M & 0xfffffu;
        q += (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ? 1u : 0u;
        code = (uint32_t)((E32 - 121) * 8) + q;
    } else if (E32 == 0) {
        code = 0u;                                      // zero or below 2^-126
    } else {
        const int s = 141 - E32;                        // units of 2^-9: fm >> s, fm = 1.M 2^23
        const uint32_t fm = (1u << 23) | M;
        if (s >= 25) {
            code = 0u;                                  // below a quarter of a unit
        } else {
            uint32_t n = fm >> s;
            const uint32_t rem = fm & ((1u << s) - 1u), half = 1u << (s - 1);
            n += (rem > half || (rem == half && (n & 1u))) ? 1u : 0u;
            code = n;
        }
    }
    return code | sgn;
}

}  // namespace

// One wave per group: the largest |W| of the group (on the bf16 bits), its
// exponent, then the codes of W * 2^-e, eight weights per lane and piece.
template <int G, int F>
__global__ __launch_bounds__(256) void k_quantize_w8(const uint16_t* __restrict__ W, uint8_t* __restrict__ W8,
                                                     int32_t* __restrict__ wexp, int64_t K)
{
    constexpr int NP = G * F / 8;                  // 16-byte pieces of W_k
    constexpr int PPL = (NP + 63) / 64;            // per lane
    const int lane = threadIdx.x & 63;
    const int64_t k = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (k >= K) return;                            // whole wave
    const uint16_t* Wk = W + k * G * F;
    u32x4_t v[PPL];
    uint32_t mb = 0;
#pragma unroll
    for (int i = 0; i < PPL; ++i) {
        const int u = lane + 64 * i;
        v[i] = u < NP ? ldg16(Wk + 8 * u) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t lo = v[i][j] & 0x7fffu, hi = (v[i][j] >> 16) & 0x7fffu;
            mb = mb > lo ? mb : lo;
            mb = mb > hi ? mb : hi;
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const uint32_t x = (uint32_t)__shfl_xor((int)mb, o, 64);
        mb = mb > x ? mb : x;
    }
    const int e = group_exponent(mb);
    const float inv = __builtin_amdgcn_ldexpf(1.0f, -e);
    if (lane == 0) wexp[k] = e;
#pragma unroll
    for (int i = 0; i < PPL; ++i) {
        const int u = lane + 64 * i;
        if (u >= NP) continue;
        uint32_t c[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            c[2 * j] = e4m3_code(__uint_as_float(v[i][j] << 16) * inv);
            c[2 * j + 1] = e4m3_code(__uint_as_float(v[i][j] & 0xffff0000u) * inv);
        }
        const u32x2_t out = u32x2_t{c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                                    c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
        *reinterpret_cast<u32x2_t*>(W8 + (k * G * F + 8 * u)) = out;
    }
}

bool launch_quantize_w8(int G, int F, const uint16_t* W, uint8_t* W8, int32_t* wexp, int64_t K, hipStream_t s)
{
    const dim3 grid((unsigned)((K + 3) / 4)), blk(256);
#define HASTE_Q8(g, f)                                                               \
    if (G == g && F == f) {                                                          \
        hipLaunchKernelGGL((k_quantize_w8<g, f>), grid, blk, 0, s, W, W8, wexp, K); \
        return true;                                                                 \
    }
    HASTE_Q8(16, 32) HASTE_Q8(16, 64) HASTE_Q8(16, 128)
    HASTE_Q8(32, 32) HASTE_Q8(32, 64) HASTE_Q8(32, 128)
    HASTE_Q8(64, 32) HASTE_Q8(64, 64) HASTE_Q8(64, 128)
#undef HASTE_Q8
    return false;
}

}  // namespace haste

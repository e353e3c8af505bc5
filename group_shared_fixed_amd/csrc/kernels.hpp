// Internal launch interface between the C ABI (haste_api.hip) and the HIP
// kernels.  Nothing here is exported from libhaste.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace haste {

// Batch rows per dh accumulator tile (one LDS accumulator of kDhRows x H fp32
// per workgroup).
constexpr int kDhRows = 16;
// Row stride (floats) of an LDS dh accumulator: H rounded up to 16, plus 4,
// so the four row groups a matrix-core result tile spans start 16 banks apart.
__host__ __device__ inline int64_t dh_stride(int64_t H) { return (H + 15) / 16 * 16 + 4; }
// Largest batch the label cursors of the BCE paths cover (4 per lane).
constexpr int kMaxLabelBatch = 256;

enum FwdMode { FWD_Z = 0, FWD_BCE = 1, STEP_DW = 2, BWD_W = 3 };
enum DhSrc { DH_FROM_DZ = 0, DH_FROM_LABELS = 1 };

struct FwdArgs {
    const uint16_t* hT;   // H x Bp bf16, Bp = B rounded up to 32, zero padded
    int64_t Bp, B;
    const int32_t* idx;   // K x F
    const uint16_t* W;    // L x F bf16
    int64_t K;
    const int32_t* y_rowptr;
    const int32_t* y_col;
    float scale;
    float* Z;             // B x L fp32 (FWD_Z; optional otherwise)
    uint16_t* dZ;         // B x L bf16 (FWD_BCE output, BWD_W input)
    float* dW;            // L x F fp32 (STEP_DW)
    uint16_t* dW16;       // L x F bf16 (STEP_DW with a bf16 weight gradient, dW then unused)
    double* loss;         // 1 double, accumulated (optional)
    const uint8_t* W8;    // L x F FP8 E4M3 codes (FP8-weight variants, in place of W)
    const int32_t* wexp;  // K group exponents: weight = decode(code) * 2^wexp[k]
};

struct DhArgs {
    const uint16_t* hT;   // H x Bp bf16 (DH_FROM_LABELS)
    int64_t Bp, B, H;
    const int32_t* idx;
    const uint16_t* W;
    int64_t K;
    const uint16_t* dZ;   // B x L bf16 (DH_FROM_DZ)
    const int32_t* y_rowptr;
    const int32_t* y_col;
    float scale;
    int nchunks, ntiles;
    float* dh;            // B x H fp32, pre-zeroed (atomic flush)
    float* part;          // nchunks x (ntiles*kDhRows) x H fp32 (deterministic flush)
    const uint8_t* W8;    // FP8-weight variants: L x F E4M3 codes in place of W
    const int32_t* wexp;  // K group exponents
    // Report of the bounded accumulator hand-off (a wait that gave up):
    // atomic flush: *status (cleared by an earlier kernel of the call) is set
    // to 1; deterministic flush: every workgroup writes flags[blockIdx.x]
    // (0 or 1) and the reduce kernel folds them into *status.
    int32_t* status;
    int32_t* flags;
    int spins;            // bound of each turn wait (polls)
};
// Bound of the feature-gradient turn waits for the next launches (the
// default, or a test's setting through haste_test_set_turn_spins).
int turn_spins();

struct FixedArgs {
    const uint16_t* hT;
    int64_t Bp, B, H;
    const int32_t* idx1;  // L x F
    const uint16_t* W;    // L x F
    int64_t L;
    const uint16_t* dZ;   // B x L bf16
    float* Z;
    float* dW;
    int nchunks, ntiles;
    float* dh;
    float* part;
};

// Each launcher returns false when no kernel exists for (G, F).
// w8: weights as FP8 codes + group exponents (modes FWD_Z and STEP_DW only).
bool launch_fwd(int G, int F, int mode, bool loss, const FwdArgs& a, int grid, hipStream_t s, bool w8 = false);
// Whether the 32-row feature-gradient kernel exists for (G, F) and the dZ
// source: its per-wave tiles, for at least six waves, and a 32 x 768
// accumulator fit in LDS without spilling registers (G F <= 2048, or G = 64
// with F = 64), for either dZ source.
constexpr bool dh32_fits(int G, int F, bool /*from_labels*/)
{
    return (G * F <= 2048 || (G * F == 4096 && F == 64));
}
// Batch rows per feature-gradient workgroup: 32 (six to eight waves, one
// workgroup per CU) where that kernel exists and H <= 768, else 16.
inline int dh_tile_rows(int G, int F, int64_t H, bool from_labels)
{
    return (H <= 768 && dh32_fits(G, F, from_labels)) ? 32 : kDhRows;
}
// w8: weights as FP8 codes + group exponents (DH_FROM_LABELS only).
bool launch_dh(int G, int F, int src, bool det, const DhArgs& a, hipStream_t s, bool w8 = false);
// Also sets *status to the OR of flags[0, nflags) when status is non-null.
void launch_dh_reduce(const float* part, float* dh, int64_t B, int64_t H, int nchunks, int rows_per_chunk,
                      hipStream_t s, const int32_t* flags = nullptr, int nflags = 0, int32_t* status = nullptr);
bool launch_fixed_fwd(int F, const FixedArgs& a, int grid, hipStream_t s);
bool launch_fixed_bwd_w(int F, const FixedArgs& a, int grid, hipStream_t s);
bool launch_fixed_bwd_h(int F, bool det, const FixedArgs& a, hipStream_t s);
// h (B x H) -> hT (H x Bp, zero padded); optionally clears zero_f[0, n), *zero_d and *zero_i
void launch_transpose_h(const uint16_t* h, uint16_t* hT, int64_t B, int64_t H, int64_t Bp, hipStream_t s,
                        float* zero_f = nullptr, int64_t n_zero_f = 0, double* zero_d = nullptr,
                        int32_t* zero_i = nullptr);
void launch_fill_f32(float* p, int64_t n, hipStream_t s);
// clears p[0, n) and, when non-null, *i
void launch_fill_f32_i32(float* p, int64_t n, int32_t* i, hipStream_t s);
void launch_fill_f64(double* p, int64_t n, hipStream_t s);
// *dst = (float)*src
void launch_f64_to_f32(const double* src, float* dst, hipStream_t s);
void launch_fill_i32(int32_t* p, int64_t n, hipStream_t s);
void launch_validate_idx(const int32_t* idx, int64_t rows, int64_t F, int64_t H, int32_t* bad, hipStream_t s);
// Bank-balanced slot order of each group's index row and W_k's columns, in place (F <= 128).
void launch_order_slots(int32_t* idx, uint16_t* W, uint8_t* perm, int64_t K, int G, int F, hipStream_t s);
void launch_validate_labels(const int32_t* rowptr, const int32_t* col, int64_t B, int64_t L, int32_t* bad,
                            hipStream_t s);
// Dense head pass (head-tail split): Z = h W^T (into zbuf when want_z; the
// rocBLAS path always fills it), the BCE gradient as bf16 hi / lo,
// dW = dZ^T h, dh (+)= dZ W; false if rocBLAS fails.
bool run_head(const uint16_t* h, const uint16_t* W, const int32_t* rowptr, const int32_t* col, float scale,
              float* dW, float* dh, float* zbuf, bool want_z, double* loss, int64_t B, int64_t H, int64_t L,
              bool accumulate_dh, uint16_t* dzcat, uint16_t* hcat, float* dhcat, uint16_t* hT, void* blas_ws,
              size_t blas_ws_bytes, hipStream_t stream);
// Bytes of caller workspace the head pass hands to rocBLAS.
constexpr size_t kHeadBlasWorkspace = 64ull << 20;
// Labels per chunk of the head's split feature-gradient product, and the
// number of chunks (each leaves a 2B x H fp32 partial in the workspace).
constexpr int64_t kHeadDhChunk = 1024;
constexpr int64_t head_dh_chunks(int64_t L) { return (L + kHeadDhChunk - 1) / kHeadDhChunk; }
// The matrix-core feature-gradient kernel of the head splits the labels into
// chunks (a multiple of 32 labels each) so that chunks x column blocks x row
// blocks stays within one workgroup per CU (256): a second round of
// workgroups would double the kernel's time.
constexpr int64_t head_dh_mfma_chunk_len(int64_t B, int64_t H, int64_t L)
{
    const int64_t blocks = ((H + 255) / 256) * ((B + 127) / 128);
    int64_t s = 256 / blocks;
    if (s < 1) s = 1;
    const int64_t len = (L + s - 1) / s;
    return (len + 31) / 32 * 32;
}
constexpr int64_t head_dh_mfma_chunks(int64_t B, int64_t H, int64_t L)
{
    const int64_t len = head_dh_mfma_chunk_len(B, H, L);
    return (L + len - 1) / len;
}

// FP8 weights: W (L x F bf16) -> E4M3 codes W8 (L x F) and group exponents
// wexp (K int32); false if (G, F) has no kernel.
bool launch_quantize_w8(int G, int F, const uint16_t* W, uint8_t* W8, int32_t* wexp, int64_t K, hipStream_t s);

// Rewiring (dynamic sparse training): grow[k, j] = sum over group k's labels
// of |(dZ^T h)[l, j]| from hT (H x Bp, Bp = 32 * (1..8)) and bf16 dZ; then
// the per-group selection (idx_out / W_out may alias idx / W).
bool launch_rewire_score(const uint16_t* hT, int64_t Bp, int64_t B, int64_t H, const uint16_t* dZ, int64_t L, int G,
                         float* grow, hipStream_t s);
bool launch_rewire_select(int G, int F, const int32_t* idx, const uint16_t* W, const float* grow, int64_t K,
                          int64_t H, int n_swap, int32_t* idx_out, uint16_t* W_out, float* prune_out, hipStream_t s);

// Label grouping (mini-batch spherical k-means and greedy groups).
// Keys sorted for a segment list of n entries take group_sort_size(n) x 8 bytes.
int64_t group_sort_size(int64_t n);
// keys[i] = seg[i] << 32 | i for i < n, sorted ascending (padding keys, all
// ones, to group_sort_size(n) at the end).
void group_sort_keys(const int32_t* seg, int64_t n, uint64_t* keys, hipStream_t s);
// Label embeddings: one batch added into the fp32 per-label sums and counts
// (keys: group_sort_size(nnz) entries, sample: nnz entries), and the bf16
// directions of the sums.
void run_label_emb_accumulate(const uint16_t* h, const int32_t* rowptr, const int32_t* col, int64_t nnz, int64_t B,
                              int64_t H, float* S, int32_t* counts, uint64_t* keys, int32_t* sample, hipStream_t s);
void run_label_emb_finalize(const float* S, const int32_t* counts, int64_t L, int64_t H, uint16_t* E, hipStream_t s);
// k-means assignment (k_assign.hip): a[i] = the centre with the largest dot
// product with E[rows ? rows[i] : i] (the lowest on ties), smax[i]
// (nullable) that product.  Scratch: keys, n_rows 64-bit words; xpack,
// n_rows x kmeans_assign_width(H) bf16, used when rows is given or the width
// differs from H; mpack, C x that width, used when it differs.  One
// workgroup per (256-label, 256-centre) tile: kmeans_assign_tiles of them.
int64_t kmeans_assign_tiles(int64_t n_rows, int64_t C);
int64_t kmeans_assign_width(int64_t H);
void run_kmeans_assign(const uint16_t* E, const int32_t* rows, int64_t n_rows, const uint16_t* M, int64_t C,
                       int64_t H, int32_t* a, float* smax, uint64_t* keys, uint16_t* xpack, uint16_t* mpack,
                       hipStream_t s);
void run_kmeans_init(const uint16_t* E, const int32_t* init, int64_t C, int64_t H, float* Mc, uint16_t* Mb,
                     int32_t* v, hipStream_t s);
void run_kmeans_update(const uint16_t* E, const int32_t* batch, const int32_t* a_batch, int64_t n, int64_t C,
                       int64_t H, float* Mc, uint16_t* Mb, int32_t* v, uint64_t* keys, int32_t* start, int32_t* end,
                       hipStream_t s);
void run_group_greedy(const uint16_t* E, const int32_t* a, int64_t L, int64_t C, int64_t H, int G, int32_t* perm,
                      uint64_t* keys, int32_t* start, int32_t* end, int32_t* gbase, int32_t* obase, int32_t* ngroups,
                      float* sim, uint8_t* taken, hipStream_t s);

}  // namespace haste

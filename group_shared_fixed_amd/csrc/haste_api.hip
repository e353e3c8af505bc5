// C ABI of libhaste: host-side validation, workspace layout and launches.
// Every check runs before the first HIP call, so error paths behave the same
// on a machine without a GPU.
#include "haste.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

using namespace haste;

namespace {

constexpr int64_t kMaxLabels = 2147483647LL - 64;

// Bound of the feature-gradient turn waits; only haste_test_set_turn_spins
// changes it (to force the give-up path in tests).
std::atomic<int> g_turn_spins{kTurnSpins};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Layout {
    int64_t Bp;          // batch padded to 32 (feature-major copy of h)
    size_t status;       // offset of the status word (grouped feature gradient), or npos
    size_t flags;        // offset of the per-workgroup hand-off reports (deterministic), or npos
    size_t hT;           // offset of hT, H x Bp bf16
    size_t hT_bytes;
    size_t part;         // offset of the deterministic dh partials
    size_t part_bytes;
    int nchunks, ntiles; // dh split: label chunks x batch tiles
    int rows;            // batch rows per dh tile
    size_t total;
};

constexpr size_t kNone = ~(size_t)0;

bool op_needs_hT(int op)
{
    return op == HASTE_OP_FWD || op == HASTE_OP_BWD_W || op == HASTE_OP_FWD_BCE || op == HASTE_OP_STEP ||
           op == HASTE_OP_FIXED_FWD || op == HASTE_OP_FIXED_BWD_W;
}

bool op_has_dh(int op) { return op == HASTE_OP_BWD_H || op == HASTE_OP_STEP || op == HASTE_OP_FIXED_BWD_H; }

// The grouped feature-gradient kernels report a broken accumulator hand-off.
bool op_has_status(int op) { return op == HASTE_OP_BWD_H || op == HASTE_OP_STEP; }

// Workspace: [status word, 256 B][hand-off flags][hT][dh partials], each
// part present only where the op needs it, each 256-byte aligned.
Layout layout(int op, int64_t B, int64_t H, int64_t G, int64_t F, int dh_mode)
{
    Layout l{};
    l.Bp = round_up(B, 32);
    // grouped dh kernels pick their tile height by shape; the G = 1 baseline uses 32 rows.
    // About two workgroups per CU for 16-row tiles, one for 32-row tiles; the
    // chunk count is a multiple of the 8 XCDs.
    l.rows = (op == HASTE_OP_BWD_H || op == HASTE_OP_STEP) ? dh_tile_rows((int)G, (int)F, H, op == HASTE_OP_STEP)
             : (op == HASTE_OP_FIXED_BWD_H ? 32 : kDhRows);
    l.ntiles = (int)((B + l.rows - 1) / l.rows);
    const int target = l.rows == 32 ? 256 : 512;
    int nc = (target / l.ntiles) / 8 * 8;
    l.nchunks = nc < 8 ? 8 : nc;
    const bool det = dh_mode == HASTE_DH_DETERMINISTIC;
    size_t at = 0;
    l.status = l.flags = l.hT = l.part = kNone;
    if (op_has_status(op)) {
        l.status = at;
        at += 256;
        if (det) {
            l.flags = at;
            at += align256((size_t)l.nchunks * l.ntiles * 4);
        }
    }
    l.hT_bytes = op_needs_hT(op) ? align256((size_t)H * (size_t)l.Bp * 2) : 0;
    if (l.hT_bytes) {
        l.hT = at;
        at += l.hT_bytes;
    }
    l.part_bytes = (op_has_dh(op) && det) ? align256((size_t)l.nchunks * l.ntiles * l.rows * (size_t)H * 4) : 0;
    if (l.part_bytes) {
        l.part = at;
        at += l.part_bytes;
    }
    l.total = at;
    return l;
}

template <class T>
T* at_off(void* ws, size_t off)
{
    return off == kNone ? nullptr : (T*)((char*)ws + off);
}

int check_shape(int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, bool fixed)
{
    if (B < 1 || H < 1 || K < 1 || G < 1 || F < 1) return HASTE_ERR_DIM;
    if (F > H) return HASTE_ERR_DIM;
    if (fixed ? (G != 1) : (G != 16 && G != 32 && G != 64)) return HASTE_ERR_UNSUPPORTED;
    if (F != 32 && F != 64 && F != 128) return HASTE_ERR_UNSUPPORTED;
    if (H > 1024) return HASTE_ERR_UNSUPPORTED;
    if (K > kMaxLabels / G) return HASTE_ERR_UNSUPPORTED;
    if (B > (1 << 24)) return HASTE_ERR_UNSUPPORTED;
    // the gathers address the feature-major copy hT (H x Bp bf16) with 32-bit
    // byte offsets, and its transpose kernel runs Bp / 32 workgroups along y
    const int64_t Bp = round_up(B, 32);
    if (2 * H * Bp >= (1LL << 31) || Bp / 32 > 65535) return HASTE_ERR_UNSUPPORTED;
    return HASTE_OK;
}

int check_ws(void* ws, size_t ws_bytes, size_t need)
{
    if (need == 0) return HASTE_OK;
    if (ws == nullptr || ws_bytes < need || ((uintptr_t)ws & 255u) != 0) return HASTE_ERR_WORKSPACE;
    return HASTE_OK;
}

int hip_status()
{
    return hipGetLastError() == hipSuccess ? HASTE_OK : HASTE_ERR_HIP;
}

int fwd_grid(int64_t K)
{
    int64_t g = (K + 3) / 4;
    return (int)(g > 512 ? 512 : (g < 1 ? 1 : g));
}

}  // namespace

int haste::turn_spins() { return g_turn_spins.load(std::memory_order_relaxed); }

namespace {

#define HASTE_TRY(x)                 \
    do {                             \
        int _st = (x);               \
        if (_st != HASTE_OK) return _st; \
    } while (0)

}  // namespace

extern "C" {

size_t haste_workspace_size(int op, int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, int dh_mode)
{
    (void)K;
    if (op < HASTE_OP_FWD || op > HASTE_OP_FWD_BCE_BWD || B < 1 || H < 1) return 0;
    // the fused pass with an fp32 loss: the step's workspace plus its fp64 accumulator
    if (op == HASTE_OP_FWD_BCE_BWD) return layout(HASTE_OP_STEP, B, H, G, F, dh_mode).total + 256;
    return layout(op, B, H, G, F, dh_mode).total;
}

size_t haste_bwd_h_workspace_size(int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, int mode)
{
    return haste_workspace_size(HASTE_OP_BWD_H, B, H, K, G, F, mode);
}

namespace {

// Forward logits from bf16 weights (W) or FP8 codes and group exponents (W8, wexp).
int fwd_impl(const haste_bf16* h, const int32_t* idx, const haste_bf16* W, const uint8_t* W8, const int32_t* wexp,
             float* Z, int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, void* workspace,
             size_t workspace_bytes, hipStream_t stream)
{
    const bool w8 = W8 != nullptr;
    if (!h || !idx || !Z || (w8 ? !wexp : !W)) return HASTE_ERR_NULL;
    HASTE_TRY(check_shape(B, H, K, G, F, false));
    if (!aligned16(h) || !aligned16(idx) || !aligned16(Z) || (w8 ? (!aligned16(W8) || !aligned16(wexp)) : !aligned16(W)))
        return HASTE_ERR_ALIGN;
    const Layout l = layout(HASTE_OP_FWD, B, H, G, F, 0);
    HASTE_TRY(check_ws(workspace, workspace_bytes, l.total));
    uint16_t* hT = at_off<uint16_t>(workspace, l.hT);
    launch_transpose_h(h, hT, B, H, l.Bp, stream);
    FwdArgs a{};
    a.hT = hT; a.Bp = l.Bp; a.B = B; a.idx = idx; a.W = W; a.W8 = W8; a.wexp = wexp; a.K = K; a.scale = 1.f;
    a.Z = Z;
    if (!launch_fwd((int)G, (int)F, FWD_Z, false, a, fwd_grid(K), stream, w8)) return HASTE_ERR_UNSUPPORTED;
    return hip_status();
}

}  // namespace

int haste_fwd(const haste_bf16* h, const int32_t* idx, const haste_bf16* W, float* Z, int64_t B, int64_t H,
              int64_t K, int64_t G, int64_t F, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    return fwd_impl(h, idx, W, nullptr, nullptr, Z, B, H, K, G, F, workspace, workspace_bytes, stream);
}

int haste_fwd_w8(const haste_bf16* h, const int32_t* idx, const uint8_t* W8, const int32_t* wexp, float* Z,
                 int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, void* workspace, size_t workspace_bytes,
                 hipStream_t stream)
{
    if (!W8) return HASTE_ERR_NULL;
    return fwd_impl(h, idx, nullptr, W8, wexp, Z, B, H, K, G, F, workspace, workspace_bytes, stream);
}

int haste_quantize_w8(const haste_bf16* W, uint8_t* W8, int32_t* wexp, int64_t K, int64_t G, int64_t F,
                      hipStream_t stream)
{
    if (!W || !W8 || !wexp) return HASTE_ERR_NULL;
    if (K < 1) return HASTE_ERR_DIM;
    HASTE_TRY(check_shape(1, F, K, G, F, false));
    if (!aligned16(W) || !aligned16(W8) || !aligned16(wexp)) return HASTE_ERR_ALIGN;
    if (!launch_quantize_w8((int)G, (int)F, W, W8, wexp, K, stream)) return HASTE_ERR_UNSUPPORTED;
    return hip_status();
}

int haste_bwd_w(const haste_bf16* h, const int32_t* idx, const haste_bf16* dZ, float* dW, int64_t B, int64_t H,
                int64_t K, int64_t G, int64_t F, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!h || !idx || !dZ || !dW) return HASTE_ERR_NULL;
    HASTE_TRY(check_shape(B, H, K, G, F, false));
    if (!aligned16(h) || !aligned16(idx) || !aligned16(dZ) || !aligned16(dW)) return HASTE_ERR_ALIGN;
    const Layout l = layout(HASTE_OP_BWD_W, B, H, G, F, 0);
    HASTE_TRY(check_ws(workspace, workspace_bytes, l.total));
    uint16_t* hT = at_off<uint16_t>(workspace, l.hT);
    launch_transpose_h(h, hT, B, H, l.Bp, stream);
    FwdArgs a{};
    a.hT = hT; a.Bp = l.Bp; a.B = B; a.idx = idx; a.K = K; a.scale = 1.f;
    a.dZ = const_cast<uint16_t*>(dZ); a.dW = dW;
    if (!launch_fwd((int)G, (int)F, BWD_W, false, a, fwd_grid(K), stream)) return HASTE_ERR_UNSUPPORTED;
    return hip_status();
}

int haste_bwd_h(const haste_bf16* dZ, const int32_t* idx, const haste_bf16* W, float* dh, int64_t B, int64_t H,
                int64_t K, int64_t G, int64_t F, int dh_mode, void* workspace, size_t workspace_bytes,
                hipStream_t stream)
{
    if (!dZ || !idx || !W || !dh) return HASTE_ERR_NULL;
    HASTE_TRY(check_shape(B, H, K, G, F, false));
    if (dh_mode != HASTE_DH_ATOMIC && dh_mode != HASTE_DH_DETERMINISTIC) return HASTE_ERR_UNSUPPORTED;
    if (!aligned16(dZ) || !aligned16(idx) || !aligned16(W) || !aligned16(dh)) return HASTE_ERR_ALIGN;
    const Layout l = layout(HASTE_OP_BWD_H, B, H, G, F, dh_mode);
    HASTE_TRY(check_ws(workspace, workspace_bytes, l.total));
    const bool det = dh_mode == HASTE_DH_DETERMINISTIC;
    DhArgs a{};
    a.Bp = l.Bp; a.B = B; a.H = H; a.idx = idx; a.W = W; a.K = K; a.dZ = dZ; a.scale = 1.f;
    a.nchunks = l.nchunks; a.ntiles = l.ntiles; a.dh = dh; a.part = at_off<float>(workspace, l.part);
    a.status = at_off<int32_t>(workspace, l.status); a.flags = at_off<int32_t>(workspace, l.flags);
    a.spins = turn_spins();
    if (!det) launch_fill_f32_i32(dh, B * H, a.status, stream);
    if (!launch_dh((int)G, (int)F, DH_FROM_DZ, det, a, stream)) return HASTE_ERR_UNSUPPORTED;
    if (det)
        launch_dh_reduce(a.part, dh, B, H, l.nchunks, l.ntiles * l.rows, stream, a.flags, l.nchunks * l.ntiles,
                         a.status);
    return hip_status();
}

int haste_fwd_bce(const haste_bf16* h, const int32_t* idx, const haste_bf16* W, const int32_t* y_rowptr,
                  const int32_t* y_col, float scale, haste_bf16* dZ, float* Z, double* loss, int64_t B, int64_t H,
                  int64_t K, int64_t G, int64_t F, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!h || !idx || !W || !y_rowptr || !y_col || !dZ) return HASTE_ERR_NULL;
    HASTE_TRY(check_shape(B, H, K, G, F, false));
    if (B > kMaxLabelBatch) return HASTE_ERR_UNSUPPORTED;
    if (!(scale > 0.f)) return HASTE_ERR_DIM;
    if (!aligned16(h) || !aligned16(idx) || !aligned16(W) || !aligned16(y_rowptr) || !aligned16(y_col) ||
        !aligned16(dZ) || (Z && !aligned16(Z)) || (loss && !aligned16(loss)))
        return HASTE_ERR_ALIGN;
    const Layout l = layout(HASTE_OP_FWD_BCE, B, H, G, F, 0);
    HASTE_TRY(check_ws(workspace, workspace_bytes, l.total));
    uint16_t* hT = at_off<uint16_t>(workspace, l.hT);
    launch_transpose_h(h, hT, B, H, l.Bp, stream, nullptr, 0, loss);
    FwdArgs a{};
    a.hT = hT; a.Bp = l.Bp; a.B = B; a.idx = idx; a.W = W; a.K = K;
    a.y_rowptr = y_rowptr; a.y_col = y_col; a.scale = scale; a.Z = Z; a.dZ = dZ; a.loss = loss;
    if (!launch_fwd((int)G, (int)F, FWD_BCE, loss != nullptr, a, fwd_grid(K), stream))
        return HASTE_ERR_UNSUPPORTED;
    return hip_status();
}

namespace {

// Host-side checks of the fused step (everything but the workspace).
int step_check(const haste_bf16* h, const int32_t* idx, const haste_bf16* W, const uint8_t* W8, const int32_t* wexp,
               const int32_t* y_rowptr, const int32_t* y_col, float scale, const float* dW, const float* dh,
               const float* Z, const double* loss, int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, int dh_mode,
               const uint16_t* dW16 = nullptr)
{
    const bool w8 = W8 != nullptr;
    if (dW16) {
        // bf16 weight gradient: bf16 weights, no logits output
        if (w8 || Z) return HASTE_ERR_UNSUPPORTED;
        if (!aligned16(dW16)) return HASTE_ERR_ALIGN;
        dW = reinterpret_cast<const float*>(dW16);   // present; checked with the others below
    }
    if (!h || !idx || !y_rowptr || !y_col || !dW || !dh || (w8 ? !wexp : !W)) return HASTE_ERR_NULL;
    if (w8 ? (!aligned16(W8) || !aligned16(wexp)) : !aligned16(W)) return HASTE_ERR_ALIGN;
    HASTE_TRY(check_shape(B, H, K, G, F, false));
    if (B > kMaxLabelBatch) return HASTE_ERR_UNSUPPORTED;
    if (dh_mode != HASTE_DH_ATOMIC && dh_mode != HASTE_DH_DETERMINISTIC) return HASTE_ERR_UNSUPPORTED;
    if (!(scale > 0.f)) return HASTE_ERR_DIM;
    if (!aligned16(h) || !aligned16(idx) || !aligned16(y_rowptr) || !aligned16(y_col) || !aligned16(dW) ||
        !aligned16(dh) || (Z && !aligned16(Z)) || (loss && !aligned16(loss)))
        return HASTE_ERR_ALIGN;
    return HASTE_OK;
}

// The fused step from bf16 weights (W) or FP8 codes and group exponents (W8, wexp).
int step_impl(const haste_bf16* h, const int32_t* idx, const haste_bf16* W, const uint8_t* W8, const int32_t* wexp,
              const int32_t* y_rowptr, const int32_t* y_col, float scale, float* dW, float* dh, float* Z,
              double* loss, int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, int dh_mode, void* workspace,
              size_t workspace_bytes, hipStream_t stream, hipEvent_t* events, uint16_t* dW16 = nullptr)
{
    const bool w8 = W8 != nullptr;
    HASTE_TRY(step_check(h, idx, W, W8, wexp, y_rowptr, y_col, scale, dW, dh, Z, loss, B, H, K, G, F, dh_mode,
                         dW16));
    const Layout l = layout(HASTE_OP_STEP, B, H, G, F, dh_mode);
    HASTE_TRY(check_ws(workspace, workspace_bytes, l.total));
    const bool det = dh_mode == HASTE_DH_DETERMINISTIC;
    uint16_t* hT = at_off<uint16_t>(workspace, l.hT);
    float* part = at_off<float>(workspace, l.part);
    int32_t* status = at_off<int32_t>(workspace, l.status);
    int32_t* flags = at_off<int32_t>(workspace, l.flags);
    auto mark = [&](int i) {
        if (events) (void)hipEventRecord(events[i], stream);
    };
    mark(0);
    launch_transpose_h(h, hT, B, H, l.Bp, stream, det ? nullptr : dh, B * H, loss, det ? nullptr : status);
    mark(1);
    FwdArgs a{};
    a.hT = hT; a.Bp = l.Bp; a.B = B; a.idx = idx; a.W = W; a.W8 = W8; a.wexp = wexp; a.K = K;
    a.y_rowptr = y_rowptr; a.y_col = y_col; a.scale = scale; a.Z = Z; a.dW = dW16 ? nullptr : dW; a.loss = loss;
    a.dW16 = dW16;
    if (!launch_fwd((int)G, (int)F, STEP_DW, loss != nullptr, a, fwd_grid(K), stream, w8))
        return HASTE_ERR_UNSUPPORTED;
    mark(2);
    DhArgs d{};
    d.hT = hT; d.Bp = l.Bp; d.B = B; d.H = H; d.idx = idx; d.W = W; d.W8 = W8; d.wexp = wexp; d.K = K;
    d.y_rowptr = y_rowptr; d.y_col = y_col; d.scale = scale;
    d.nchunks = l.nchunks; d.ntiles = l.ntiles; d.dh = dh; d.part = part; d.status = status; d.flags = flags;
    d.spins = turn_spins();
    if (!launch_dh((int)G, (int)F, DH_FROM_LABELS, det, d, stream, w8)) return HASTE_ERR_UNSUPPORTED;
    mark(3);
    if (det) launch_dh_reduce(part, dh, B, H, l.nchunks, l.ntiles * l.rows, stream, flags, l.nchunks * l.ntiles, status);
    mark(4);
    return hip_status();
}

}  // namespace

int haste_step_timed(const haste_bf16* h, const int32_t* idx, const haste_bf16* W, const int32_t* y_rowptr,
                     const int32_t* y_col, float scale, float* dW, float* dh, float* Z, double* loss, int64_t B,
                     int64_t H, int64_t K, int64_t G, int64_t F, int dh_mode, void* workspace,
                     size_t workspace_bytes, hipStream_t stream, hipEvent_t* events)
{
    if (!W) return HASTE_ERR_NULL;
    return step_impl(h, idx, W, nullptr, nullptr, y_rowptr, y_col, scale, dW, dh, Z, loss, B, H, K, G, F, dh_mode,
                     workspace, workspace_bytes, stream, events);
}

int haste_step_bf16dw(const haste_bf16* h, const int32_t* idx, const haste_bf16* W, const int32_t* y_rowptr,
                      const int32_t* y_col, float scale, haste_bf16* dW, float* dh, double* loss, int64_t B,
                      int64_t H, int64_t K, int64_t G, int64_t F, int dh_mode, void* workspace,
                      size_t workspace_bytes, hipStream_t stream, hipEvent_t* events)
{
    if (!W || !dW) return HASTE_ERR_NULL;
    return step_impl(h, idx, W, nullptr, nullptr, y_rowptr, y_col, scale, nullptr, dh, nullptr, loss, B, H, K, G, F,
                     dh_mode, workspace, workspace_bytes, stream, events, reinterpret_cast<uint16_t*>(dW));
}

int haste_step_w8_timed(const haste_bf16* h, const int32_t* idx, const uint8_t* W8, const int32_t* wexp,
                        const int32_t* y_rowptr, const int32_t* y_col, float scale, float* dW, float* dh, float* Z,
                        double* loss, int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, int dh_mode,
                        void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* events)
{
    if (!W8) return HASTE_ERR_NULL;
    return step_impl(h, idx, nullptr, W8, wexp, y_rowptr, y_col, scale, dW, dh, Z, loss, B, H, K, G, F, dh_mode,
                     workspace, workspace_bytes, stream, events);
}

int haste_step_w8(const haste_bf16* h, const int32_t* idx, const uint8_t* W8, const int32_t* wexp,
                  const int32_t* y_rowptr, const int32_t* y_col, float scale, float* dW, float* dh, float* Z,
                  double* loss, int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, int dh_mode, void* workspace,
                  size_t workspace_bytes, hipStream_t stream)
{
    return haste_step_w8_timed(h, idx, W8, wexp, y_rowptr, y_col, scale, dW, dh, Z, loss, B, H, K, G, F, dh_mode,
                               workspace, workspace_bytes, stream, nullptr);
}

namespace {

// Device scratch of haste_step_noalloc: hT, the status word, the hand-off
// flags and the deterministic dh partials of one fused pass (the loss
// accumulator, dW, dh and Z are the caller's).  32 MiB covers every supported
// shape with B <= 256 and H <= 768 in both dh modes (the Amazon-3M-shaped
// pass in deterministic mode takes 25.4 MB); larger needs are refused.  Each
// GPU the library runs on holds its own copy until the process ends.  In
// host code `scratch` names a host-side stand-in, never the device memory:
// only the address hipGetSymbolAddress returns for the current device is
// passed to kernels.
constexpr size_t kNoAllocScratchBytes = 32ull << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];   // device address of `scratch`, per device

// The current device's copy of `scratch` (looked up once per device, with
// that device current).
int scratch_for_current_device(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return HASTE_ERR_HIP;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return HASTE_ERR_HIP;
        }
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return HASTE_OK;
}

}  // namespace

int haste_step_noalloc(const haste_bf16* h, const int32_t* idx, const haste_bf16* W, const int32_t* y_rowptr,
                       const int32_t* y_col, float scale, float* dW, float* dh, float* Z, double* loss, int64_t B,
                       int64_t H, int64_t K, int64_t G, int64_t F, int dh_mode, hipStream_t stream)
{
    HASTE_TRY(step_check(h, idx, W, nullptr, nullptr, y_rowptr, y_col, scale, dW, dh, Z, loss, B, H, K, G, F,
                         dh_mode));
    const size_t need = layout(HASTE_OP_STEP, B, H, G, F, dh_mode).total;
    if (need > kNoAllocScratchBytes) return HASTE_ERR_WORKSPACE;
    void* ws = nullptr;
    HASTE_TRY(scratch_for_current_device(&ws));
    return step_impl(h, idx, W, nullptr, nullptr, y_rowptr, y_col, scale, dW, dh, Z, loss, B, H, K, G, F, dh_mode,
                     ws, kNoAllocScratchBytes, stream, nullptr);
}

int haste_step(const haste_bf16* h, const int32_t* idx, const haste_bf16* W, const int32_t* y_rowptr,
               const int32_t* y_col, float scale, float* dW, float* dh, float* Z, double* loss, int64_t B,
               int64_t H, int64_t K, int64_t G, int64_t F, int dh_mode, void* workspace, size_t workspace_bytes,
               hipStream_t stream)
{
    return haste_step_timed(h, idx, W, y_rowptr, y_col, scale, dW, dh, Z, loss, B, H, K, G, F, dh_mode, workspace,
                            workspace_bytes, stream, nullptr);
}

int haste_fwd_bce_bwd(const haste_bf16* h, const int32_t* idx, const haste_bf16* W, const int32_t* y_rowptr,
                      const int32_t* y_col, float scale, float* dW, float* dh, float* loss, int mode,
                      void* workspace, size_t workspace_bytes, int64_t B, int64_t H, int64_t K, int64_t G,
                      int64_t F, hipStream_t stream)
{
    if (!W) return HASTE_ERR_NULL;
    if (loss && !aligned16(loss)) return HASTE_ERR_ALIGN;
    // shape and mode first, so that the workspace size below is meaningful
    HASTE_TRY(check_shape(B, H, K, G, F, false));
    if (mode != HASTE_DH_ATOMIC && mode != HASTE_DH_DETERMINISTIC) return HASTE_ERR_UNSUPPORTED;
    const size_t step_ws = layout(HASTE_OP_STEP, B, H, G, F, mode).total;
    HASTE_TRY(check_ws(workspace, workspace_bytes, step_ws + (loss ? 256 : 0)));
    double* acc = loss ? (double*)((char*)workspace + step_ws) : nullptr;
    HASTE_TRY(step_impl(h, idx, W, nullptr, nullptr, y_rowptr, y_col, scale, dW, dh, nullptr, acc, B, H, K, G, F,
                        mode, workspace, step_ws, stream, nullptr));
    if (loss) launch_f64_to_f32(acc, loss, stream);
    return hip_status();
}

int haste_fixed_fwd(const haste_bf16* h, const int32_t* idx1, const haste_bf16* W, float* Z, int64_t B,
                    int64_t H, int64_t L, int64_t F, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!h || !idx1 || !W || !Z) return HASTE_ERR_NULL;
    HASTE_TRY(check_shape(B, H, L, 1, F, true));
    if (!aligned16(h) || !aligned16(idx1) || !aligned16(W) || !aligned16(Z)) return HASTE_ERR_ALIGN;
    const Layout l = layout(HASTE_OP_FIXED_FWD, B, H, 1, F, 0);
    HASTE_TRY(check_ws(workspace, workspace_bytes, l.total));
    uint16_t* hT = at_off<uint16_t>(workspace, l.hT);
    launch_transpose_h(h, hT, B, H, l.Bp, stream);
    FixedArgs a{};
    a.hT = hT; a.Bp = l.Bp; a.B = B; a.H = H; a.idx1 = idx1; a.W = W; a.L = L; a.Z = Z;
    if (!launch_fixed_fwd((int)F, a, 768, stream)) return HASTE_ERR_UNSUPPORTED;
    return hip_status();
}

int haste_fixed_bwd_w(const haste_bf16* h, const int32_t* idx1, const haste_bf16* dZ, float* dW, int64_t B,
                      int64_t H, int64_t L, int64_t F, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!h || !idx1 || !dZ || !dW) return HASTE_ERR_NULL;
    HASTE_TRY(check_shape(B, H, L, 1, F, true));
    if (!aligned16(h) || !aligned16(idx1) || !aligned16(dZ) || !aligned16(dW)) return HASTE_ERR_ALIGN;
    const Layout l = layout(HASTE_OP_FIXED_BWD_W, B, H, 1, F, 0);
    HASTE_TRY(check_ws(workspace, workspace_bytes, l.total));
    uint16_t* hT = at_off<uint16_t>(workspace, l.hT);
    launch_transpose_h(h, hT, B, H, l.Bp, stream);
    FixedArgs a{};
    a.hT = hT; a.Bp = l.Bp; a.B = B; a.H = H; a.idx1 = idx1; a.L = L; a.dZ = dZ; a.dW = dW;
    if (!launch_fixed_bwd_w((int)F, a, 768, stream)) return HASTE_ERR_UNSUPPORTED;
    return hip_status();
}

int haste_fixed_bwd_h(const haste_bf16* dZ, const int32_t* idx1, const haste_bf16* W, float* dh, int64_t B,
                      int64_t H, int64_t L, int64_t F, int dh_mode, void* workspace, size_t workspace_bytes,
                      hipStream_t stream)
{
    if (!dZ || !idx1 || !W || !dh) return HASTE_ERR_NULL;
    HASTE_TRY(check_shape(B, H, L, 1, F, true));
    if (dh_mode != HASTE_DH_ATOMIC && dh_mode != HASTE_DH_DETERMINISTIC) return HASTE_ERR_UNSUPPORTED;
    if (!aligned16(dZ) || !aligned16(idx1) || !aligned16(W) || !aligned16(dh)) return HASTE_ERR_ALIGN;
    const Layout l = layout(HASTE_OP_FIXED_BWD_H, B, H, 1, F, dh_mode);
    HASTE_TRY(check_ws(workspace, workspace_bytes, l.total));
    const bool det = dh_mode == HASTE_DH_DETERMINISTIC;
    FixedArgs a{};
    a.Bp = l.Bp; a.B = B; a.H = H; a.idx1 = idx1; a.W = W; a.L = L; a.dZ = dZ;
    a.nchunks = l.nchunks; a.ntiles = l.ntiles; a.dh = dh; a.part = at_off<float>(workspace, l.part);
    if (!det) launch_fill_f32(dh, B * H, stream);
    if (!launch_fixed_bwd_h((int)F, det, a, stream)) return HASTE_ERR_UNSUPPORTED;
    if (det) launch_dh_reduce(a.part, dh, B, H, l.nchunks, l.ntiles * l.rows, stream);
    return hip_status();
}

int haste_validate_idx(const int32_t* idx, int64_t rows, int64_t F, int64_t H, int32_t* bad, hipStream_t stream)
{
    if (!idx || !bad) return HASTE_ERR_NULL;
    if (rows < 1 || F < 1 || H < 1) return HASTE_ERR_DIM;
    launch_fill_i32(bad, 1, stream);
    launch_validate_idx(idx, rows, F, H, bad, stream);
    return hip_status();
}

int haste_order_slots(int32_t* idx, haste_bf16* W, uint8_t* perm, int64_t K, int64_t G, int64_t F,
                      hipStream_t stream)
{
    if (!idx) return HASTE_ERR_NULL;
    if (K < 1 || G < 1 || F < 1) return HASTE_ERR_DIM;
    if (G != 16 && G != 32 && G != 64) return HASTE_ERR_UNSUPPORTED;
    if (F != 32 && F != 64 && F != 128) return HASTE_ERR_UNSUPPORTED;
    if (K > kMaxLabels / G) return HASTE_ERR_UNSUPPORTED;
    if (!aligned16(idx) || (W && !aligned16(W))) return HASTE_ERR_ALIGN;
    launch_order_slots(idx, reinterpret_cast<uint16_t*>(W), perm, K, (int)G, (int)F, stream);
    return hip_status();
}

int haste_validate_labels(const int32_t* y_rowptr, const int32_t* y_col, int64_t B, int64_t L, int32_t* bad,
                          hipStream_t stream)
{
    if (!y_rowptr || !y_col || !bad) return HASTE_ERR_NULL;
    if (B < 1 || L < 1) return HASTE_ERR_DIM;
    launch_fill_i32(bad, 1, stream);
    launch_validate_labels(y_rowptr, y_col, B, L, bad, stream);
    return hip_status();
}

namespace {

// Head workspace: Z (B x L fp32), stacked dZ hi / lo (2B x L bf16), [h; h]
// (2B x H bf16), hT (H x Bp bf16), the dh partials of the label chunks,
// rocBLAS's workspace.
struct HeadLayout {
    size_t z, dz, hcat, hT, dhcat, blas, total;
    HeadLayout(int64_t B, int64_t H, int64_t L)
    {
        const size_t bl = (size_t)B * (size_t)L, bh = (size_t)B * (size_t)H;
        z = 0;
        dz = z + align256(bl * 4);
        hcat = dz + align256(bl * 4);
        hT = hcat + align256(bh * 4);
        dhcat = hT + align256((size_t)H * (size_t)round_up(B, 32) * 2);
        // partials: 2B x H per rocBLAS chunk, or B x H per matrix-core chunk
        const size_t np = (size_t)head_dh_chunks(L) * 2 > (size_t)head_dh_mfma_chunks(B, H, L)
                              ? (size_t)head_dh_chunks(L) * 2
                              : (size_t)head_dh_mfma_chunks(B, H, L);
        blas = dhcat + align256(bh * 4 * np);
        total = blas + kHeadBlasWorkspace;
    }
};

}  // namespace

size_t haste_head_workspace_size(int64_t B, int64_t H, int64_t L)
{
    if (B < 1 || H < 1 || L < 1) return 0;
    return HeadLayout(B, H, L).total;
}

namespace {

int check_head(const haste_bf16* h, const haste_bf16* W, const int32_t* y_rowptr, const int32_t* y_col,
               float scale, const float* dW, const float* dh, const float* Z, const double* loss, int64_t B,
               int64_t H, int64_t L)
{
    if (!h || !W || !y_rowptr || !y_col || !dW || !dh) return HASTE_ERR_NULL;
    if (B < 1 || H < 1 || L < 1 || !(scale > 0.f)) return HASTE_ERR_DIM;
    // rocBLAS takes 32-bit sizes and leading dimensions
    if (L > kMaxLabels || H > (1 << 20) || B > (1 << 24)) return HASTE_ERR_UNSUPPORTED;
    if (!aligned16(h) || !aligned16(W) || !aligned16(y_rowptr) || !aligned16(y_col) || !aligned16(dW) ||
        !aligned16(dh) || (Z && !aligned16(Z)) || (loss && !aligned16(loss)))
        return HASTE_ERR_ALIGN;
    return HASTE_OK;
}

// The head pass on the workspace of haste_head_workspace_size.
int head_pass(const haste_bf16* h, const haste_bf16* W, const int32_t* y_rowptr, const int32_t* y_col,
              float scale, float* dW, float* dh, float* Z, double* loss, int64_t B, int64_t H, int64_t L,
              bool accumulate, void* workspace, hipStream_t stream)
{
    const HeadLayout l(B, H, L);
    char* w = (char*)workspace;
    float* zbuf = Z ? Z : (float*)(w + l.z);
    if (!run_head(h, W, y_rowptr, y_col, scale, dW, dh, zbuf, Z != nullptr, loss, B, H, L, accumulate, (uint16_t*)(w + l.dz),
                  (uint16_t*)(w + l.hcat), (float*)(w + l.dhcat), (uint16_t*)(w + l.hT), w + l.blas,
                  kHeadBlasWorkspace, stream))
        return HASTE_ERR_HIP;
    return hip_status();
}

}  // namespace

int haste_head_step(const haste_bf16* h, const haste_bf16* W_head, const int32_t* y_rowptr, const int32_t* y_col,
                    float scale, float* dW_head, float* dh, float* Z_head, double* loss, int64_t B, int64_t H,
                    int64_t L_head, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    HASTE_TRY(check_head(h, W_head, y_rowptr, y_col, scale, dW_head, dh, Z_head, loss, B, H, L_head));
    HASTE_TRY(check_ws(workspace, workspace_bytes, haste_head_workspace_size(B, H, L_head)));
    if (loss) launch_fill_f64(loss, 1, stream);
    return head_pass(h, W_head, y_rowptr, y_col, scale, dW_head, dh, Z_head, loss, B, H, L_head, false, workspace,
                     stream);
}

namespace {

// The head pass of the joint step runs on the workspace past the tail's
// status word and hand-off flags, which stay readable after the call.
size_t joint_head_offset(int64_t B, int64_t H, int64_t G, int64_t F, int dh_mode)
{
    return layout(HASTE_OP_STEP, B, H, G, F, dh_mode).hT;
}

}  // namespace

size_t haste_joint_workspace_size(int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, int64_t L_head,
                                  int dh_mode)
{
    if (B < 1 || H < 1) return 0;
    const size_t tail = haste_workspace_size(HASTE_OP_STEP, B, H, K, G, F, dh_mode);
    const size_t head = haste_head_workspace_size(B, H, L_head);
    if (head == 0) return 0;
    const size_t head_end = joint_head_offset(B, H, G, F, dh_mode) + head;
    return tail > head_end ? tail : head_end;
}

int haste_joint_step(const haste_bf16* h, const int32_t* idx, const haste_bf16* W_tail, const int32_t* yt_rowptr,
                     const int32_t* yt_col, const haste_bf16* W_head, const int32_t* yh_rowptr,
                     const int32_t* yh_col, float scale_tail, float scale_head, float* dW_tail, float* dW_head,
                     float* dh, double* loss,
                     int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, int64_t L_head, int dh_mode,
                     void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!idx || !W_tail || !yt_rowptr || !yt_col || !dW_tail) return HASTE_ERR_NULL;
    HASTE_TRY(check_head(h, W_head, yh_rowptr, yh_col, scale_head, dW_head, dh, nullptr, loss, B, H, L_head));
    if (!(scale_tail > 0.f)) return HASTE_ERR_DIM;
    HASTE_TRY(check_shape(B, H, K, G, F, false));
    if (B > kMaxLabelBatch) return HASTE_ERR_UNSUPPORTED;
    if (dh_mode != HASTE_DH_ATOMIC && dh_mode != HASTE_DH_DETERMINISTIC) return HASTE_ERR_UNSUPPORTED;
    if (!aligned16(idx) || !aligned16(W_tail) || !aligned16(yt_rowptr) || !aligned16(yt_col) || !aligned16(dW_tail))
        return HASTE_ERR_ALIGN;
    HASTE_TRY(check_ws(workspace, workspace_bytes, haste_joint_workspace_size(B, H, K, G, F, L_head, dh_mode)));
    // tail: writes dh and clears + accumulates the loss; head: adds to both
    HASTE_TRY(haste_step(h, idx, W_tail, yt_rowptr, yt_col, scale_tail, dW_tail, dh, nullptr, loss, B, H, K, G, F,
                         dh_mode, workspace, workspace_bytes, stream));
    return head_pass(h, W_head, yh_rowptr, yh_col, scale_head, dW_head, dh, nullptr, loss, B, H, L_head, true,
                     (char*)workspace + joint_head_offset(B, H, G, F, dh_mode), stream);
}

size_t haste_rewire_workspace_size(int64_t B, int64_t H, int64_t K, int64_t G, int64_t F)
{
    (void)G;
    (void)F;
    if (B < 1 || H < 1 || K < 1) return 0;
    return align256((size_t)H * (size_t)round_up(B, 32) * 2) + align256((size_t)K * (size_t)H * 4);
}

namespace {

// true when [a, a + na) and [b, b + nb) are the same range or disjoint
bool same_or_disjoint(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return (x == y && na == nb) || x + na <= y || y + nb <= x;
}

}  // namespace

int haste_rewire_timed(const haste_bf16* h, const haste_bf16* dZ, const int32_t* idx, const haste_bf16* W,
                       int64_t n_swap, int32_t* idx_out, haste_bf16* W_out, float* grow_score, float* prune_score,
                       int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, void* workspace,
                       size_t workspace_bytes, hipStream_t stream, hipEvent_t* events)
{
    if (!h || !dZ || !idx || !W || !idx_out || !W_out) return HASTE_ERR_NULL;
    HASTE_TRY(check_shape(B, H, K, G, F, false));
    if (n_swap < 0 || n_swap > F) return HASTE_ERR_DIM;
    if (B > 256) return HASTE_ERR_UNSUPPORTED;
    if (!aligned16(h) || !aligned16(dZ) || !aligned16(idx) || !aligned16(W) || !aligned16(idx_out) ||
        !aligned16(W_out) || (grow_score && !aligned16(grow_score)) || (prune_score && !aligned16(prune_score)))
        return HASTE_ERR_ALIGN;
    const size_t nidx = (size_t)K * (size_t)F * 4, nw = (size_t)K * (size_t)G * (size_t)F * 2;
    if (!same_or_disjoint(idx, nidx, idx_out, nidx) || !same_or_disjoint(W, nw, W_out, nw)) return HASTE_ERR_DIM;
    HASTE_TRY(check_ws(workspace, workspace_bytes, haste_rewire_workspace_size(B, H, K, G, F)));
    const int64_t Bp = round_up(B, 32);
    uint16_t* hT = (uint16_t*)workspace;
    float* grow = grow_score ? grow_score : (float*)((char*)workspace + align256((size_t)H * (size_t)Bp * 2));
    auto mark = [&](int i) {
        if (events) (void)hipEventRecord(events[i], stream);
    };
    mark(0);
    launch_transpose_h(h, hT, B, H, Bp, stream);
    mark(1);
    if (!launch_rewire_score(hT, Bp, B, H, dZ, K * G, (int)G, grow, stream)) return HASTE_ERR_UNSUPPORTED;
    mark(2);
    if (!launch_rewire_select((int)G, (int)F, idx, W, grow, K, H, (int)n_swap, idx_out, W_out, prune_score, stream))
        return HASTE_ERR_UNSUPPORTED;
    mark(3);
    return hip_status();
}

int haste_rewire(const haste_bf16* h, const haste_bf16* dZ, const int32_t* idx, const haste_bf16* W, int64_t n_swap,
                 int32_t* idx_out, haste_bf16* W_out, float* grow_score, float* prune_score, int64_t B, int64_t H,
                 int64_t K, int64_t G, int64_t F, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    return haste_rewire_timed(h, dZ, idx, W, n_swap, idx_out, W_out, grow_score, prune_score, B, H, K, G, F,
                              workspace, workspace_bytes, stream, nullptr);
}

namespace {

int check_emb(int64_t L, int64_t C, int64_t H)
{
    if (L < 1 || C < 1 || H < 8) return HASTE_ERR_DIM;
    if (H % 8 != 0 || H > 1024 || C > L || L > ((int64_t)1 << 30)) return HASTE_ERR_UNSUPPORTED;
    return HASTE_OK;
}

struct KmAssignLayout {
    size_t keys, xpack, mpack, total;
    KmAssignLayout(int64_t n_rows, int64_t C, int64_t H, bool rows)
    {
        const int64_t Hp = kmeans_assign_width(H);
        keys = 0;
        xpack = keys + align256((size_t)n_rows * 8);
        mpack = xpack + ((rows || Hp != H) ? align256((size_t)n_rows * (size_t)Hp * 2) : 0);
        total = mpack + (Hp != H ? align256((size_t)C * (size_t)Hp * 2) : 0);
    }
};

struct GroupLayout {
    size_t keys, start, end, gbase, obase, ng, sim, taken, total;
    GroupLayout(int64_t n, int64_t C, bool greedy)
    {
        keys = 0;
        start = keys + align256((size_t)group_sort_size(n) * 8);
        end = start + align256((size_t)C * 4);
        gbase = end + align256((size_t)C * 4);
        obase = gbase + (greedy ? align256((size_t)C * 4) : 0);
        ng = obase + (greedy ? align256((size_t)C * 4) : 0);
        sim = ng + (greedy ? 256 : 0);
        taken = sim + (greedy ? align256((size_t)n * 4) : 0);
        total = taken + (greedy ? align256((size_t)n) : 0);
    }
};

}  // namespace

size_t haste_kmeans_assign_workspace_size(int64_t n_rows, int64_t C, int64_t H, int with_rows)
{
    if (n_rows < 1 || C < 1 || H < 1) return 0;
    return KmAssignLayout(n_rows, C, H, with_rows != 0).total;
}

int haste_kmeans_assign(const haste_bf16* E, const int32_t* rows, int64_t n_rows, int64_t L, const haste_bf16* M,
                        int64_t C, int64_t H, int32_t* assign, float* score, void* workspace, size_t workspace_bytes,
                        hipStream_t stream)
{
    if (!E || !M || !assign) return HASTE_ERR_NULL;
    HASTE_TRY(check_emb(L, C, H));
    if (n_rows < 1 || (!rows && n_rows != L) || n_rows > L) return HASTE_ERR_DIM;
    if (!aligned16(E) || !aligned16(M) || !aligned16(assign) || (rows && !aligned16(rows)) ||
        (score && !aligned16(score)))
        return HASTE_ERR_ALIGN;
    if (kmeans_assign_tiles(n_rows, C) > ((int64_t)1 << 31)) return HASTE_ERR_UNSUPPORTED;
    const KmAssignLayout l(n_rows, C, H, rows != nullptr);
    HASTE_TRY(check_ws(workspace, workspace_bytes, l.total));
    char* w = (char*)workspace;
    run_kmeans_assign(E, rows, n_rows, M, C, H, assign, score, (uint64_t*)(w + l.keys), (uint16_t*)(w + l.xpack),
                      (uint16_t*)(w + l.mpack), stream);
    return hip_status();
}

int haste_kmeans_init(const haste_bf16* E, const int32_t* init, int64_t L, int64_t C, int64_t H, float* Mc,
                      haste_bf16* Mb, int32_t* counts, hipStream_t stream)
{
    if (!E || !init || !Mc || !Mb || !counts) return HASTE_ERR_NULL;
    HASTE_TRY(check_emb(L, C, H));
    if (!aligned16(E) || !aligned16(init) || !aligned16(Mc) || !aligned16(Mb) || !aligned16(counts))
        return HASTE_ERR_ALIGN;
    run_kmeans_init(E, init, C, H, Mc, Mb, counts, stream);
    return hip_status();
}

size_t haste_kmeans_update_workspace_size(int64_t n, int64_t C)
{
    if (n < 1 || C < 1) return 0;
    return GroupLayout(n, C, false).total;
}

int haste_kmeans_update(const haste_bf16* E, const int32_t* batch, const int32_t* assign, int64_t n, int64_t L,
                        int64_t C, int64_t H, float* Mc, haste_bf16* Mb, int32_t* counts, void* workspace,
                        size_t workspace_bytes, hipStream_t stream)
{
    if (!E || !batch || !assign || !Mc || !Mb || !counts) return HASTE_ERR_NULL;
    HASTE_TRY(check_emb(L, C, H));
    if (n < 1 || n > L) return HASTE_ERR_DIM;
    if (!aligned16(E) || !aligned16(batch) || !aligned16(assign) || !aligned16(Mc) || !aligned16(Mb) ||
        !aligned16(counts))
        return HASTE_ERR_ALIGN;
    const GroupLayout l(n, C, false);
    HASTE_TRY(check_ws(workspace, workspace_bytes, l.total));
    char* w = (char*)workspace;
    run_kmeans_update(E, batch, assign, n, C, H, Mc, Mb, counts, (uint64_t*)(w + l.keys), (int32_t*)(w + l.start),
                      (int32_t*)(w + l.end), stream);
    return hip_status();
}

size_t haste_group_workspace_size(int64_t L, int64_t C)
{
    if (L < 1 || C < 1) return 0;
    return GroupLayout(L, C, true).total;
}

int haste_group_greedy(const haste_bf16* E, const int32_t* assign, int64_t L, int64_t C, int64_t H, int64_t G,
                       int32_t* perm, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!E || !assign || !perm) return HASTE_ERR_NULL;
    HASTE_TRY(check_emb(L, C, H));
    if (G < 1 || G > 64 || L % G != 0) return HASTE_ERR_DIM;
    if (!aligned16(E) || !aligned16(assign) || !aligned16(perm)) return HASTE_ERR_ALIGN;
    const GroupLayout l(L, C, true);
    HASTE_TRY(check_ws(workspace, workspace_bytes, l.total));
    char* w = (char*)workspace;
    run_group_greedy(E, assign, L, C, H, (int)G, perm, (uint64_t*)(w + l.keys), (int32_t*)(w + l.start),
                     (int32_t*)(w + l.end), (int32_t*)(w + l.gbase), (int32_t*)(w + l.obase), (int32_t*)(w + l.ng),
                     (float*)(w + l.sim), (uint8_t*)(w + l.taken), stream);
    return hip_status();
}

void haste_test_set_turn_spins(int spins) { g_turn_spins.store(spins < 0 ? kTurnSpins : spins); }

size_t haste_label_emb_workspace_size(int64_t nnz)
{
    if (nnz < 0) return 0;
    return align256((size_t)group_sort_size(nnz) * 8) + align256((size_t)nnz * 4);
}

int haste_label_emb_accumulate(const haste_bf16* h, const int32_t* y_rowptr, const int32_t* y_col, int64_t nnz,
                               int64_t B, int64_t H, int64_t L, float* S, int32_t* counts, void* workspace,
                               size_t workspace_bytes, hipStream_t stream)
{
    if (!h || !y_rowptr || !S || !counts || (nnz > 0 && !y_col)) return HASTE_ERR_NULL;
    if (B < 1 || nnz < 0) return HASTE_ERR_DIM;
    HASTE_TRY(check_emb(L, 1, H));
    if (nnz > ((int64_t)1 << 30) || B > ((int64_t)1 << 30)) return HASTE_ERR_UNSUPPORTED;
    if (!aligned16(h) || !aligned16(y_rowptr) || (y_col && !aligned16(y_col)) || !aligned16(S) || !aligned16(counts))
        return HASTE_ERR_ALIGN;
    HASTE_TRY(check_ws(workspace, workspace_bytes, haste_label_emb_workspace_size(nnz)));
    uint64_t* keys = (uint64_t*)workspace;
    int32_t* sample = (int32_t*)((char*)workspace + align256((size_t)group_sort_size(nnz) * 8));
    run_label_emb_accumulate(h, y_rowptr, y_col, nnz, B, H, S, counts, keys, sample, stream);
    return hip_status();
}

int haste_label_emb_finalize(const float* S, const int32_t* counts, int64_t L, int64_t H, haste_bf16* E,
                             hipStream_t stream)
{
    if (!S || !counts || !E) return HASTE_ERR_NULL;
    HASTE_TRY(check_emb(L, 1, H));
    if (!aligned16(S) || !aligned16(counts) || !aligned16(E)) return HASTE_ERR_ALIGN;
    run_label_emb_finalize(S, counts, L, H, E, stream);
    return hip_status();
}

int haste_workspace_status(const void* workspace, int32_t* status, hipStream_t stream)
{
    if (!workspace || !status) return HASTE_ERR_NULL;
    if (((uintptr_t)workspace & 255u) != 0) return HASTE_ERR_WORKSPACE;
    if (hipMemcpyAsync(status, workspace, sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess)
        return HASTE_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return HASTE_ERR_HIP;
    return HASTE_OK;
}

const char* haste_status_string(int status)
{
    switch (status) {
    case HASTE_OK: return "ok";
    case HASTE_ERR_NULL: return "a required pointer is NULL";
    case HASTE_ERR_DIM: return "invalid or inconsistent sizes";
    case HASTE_ERR_UNSUPPORTED: return "shape not supported by the gfx950 kernels";
    case HASTE_ERR_ALIGN: return "pointer not 16-byte aligned";
    case HASTE_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case HASTE_ERR_INDEX: return "invalid index set or labels";
    case HASTE_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

const char* haste_version(void) { return "libhaste 0.1 (gfx950)"; }

}  // extern "C"

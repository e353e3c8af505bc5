/*
 * libhaste — group-shared fixed fan-in sparse output layer on AMD MI355X
 * (gfx950), C ABI.
 *
 * Method: "HASTE: Hardware-Aware Dynamic Sparse Training for Large Output
 * Spaces" (papernotes.org notes on the ICML 2026 paper).  L = K*G labels are
 * split into K groups of G labels; the G labels of group k share one fan-in
 * index set I_k of F distinct feature columns out of H ("group-shared fixed
 * fan-in" section), and label l = k*G + g has its own weights W[l, 0..F).
 *
 * Shapes and layouts (all row-major, contiguous):
 *   h    B x H  bf16   features (the encoder output feeding the layer)
 *   idx  K x F  int32  I_k = idx[k, :], entries in [0, H), pairwise distinct, in any
 *                      order (haste_order_slots picks one that suits dh)
 *   W    L x F  bf16   W[l, f] multiplies h[:, idx[l / G, f]]
 *   Z    B x L  fp32   logits
 *   dZ   B x L  bf16   upstream gradient of the logits
 *   dW   L x F  fp32   weight gradient
 *   dh   B x H  fp32   feature gradient
 *   labels: the B x L 0/1 label matrix Y as CSR, y_rowptr[B + 1] and
 *           y_col[y_rowptr[B]]; row b lists the positive label ids of sample
 *           b, strictly increasing (haste_validate_labels checks this).
 * bf16 values are passed as their 16-bit patterns (haste_bf16).
 *
 * Conventions shared by every call:
 *   - All pointers except `workspace` arguments of size 0 and the optional
 *     outputs marked "nullable" are device pointers the caller allocated; the
 *     library never allocates or frees them, keeps no pointer after the call
 *     returns and keeps no state between calls.  Two exceptions, both
 *     process-lifetime and never freed: haste_step_noalloc's static scratch
 *     array (below), and the rocBLAS handle (one per host thread and device,
 *     created on first use; rocBLAS allocates inside it) that haste_head_step
 *     and the joint step create only for head shapes outside their own
 *     kernels (B > 128, H % 64 != 0 or L_head % 8 != 0).  No other call
 *     touches rocBLAS.
 *   - Calls are asynchronous on `stream` (0 = default stream) and return
 *     before the GPU work finishes; outputs are valid after the stream
 *     synchronises.  Outputs are overwritten, never accumulated into.
 *   - Arguments are validated on the host before any HIP call; a negative
 *     haste_status is returned without touching the GPU.  HASTE_ERR_HIP
 *     means a launch failed (hipGetLastError).  Faults inside kernels surface
 *     at the next synchronisation.  The hot calls do not re-validate index
 *     sets or labels: out-of-range or repeated entries are undefined behaviour
 *     (use haste_validate_idx / haste_validate_labels).
 *   - Supported: G in {16, 32, 64} (G = 1 for the haste_fixed_* baseline),
 *     F in {32, 64, 128}, F <= H <= 1024, L = K*G < 2^31 - 64; label-consuming
 *     calls need B <= 256.  Pointers must be 16-byte aligned.  Other shapes
 *     return HASTE_ERR_UNSUPPORTED; the CPU oracle accepts any shape.
 *   - `workspace` is caller-owned device scratch of at least
 *     haste_workspace_size(op, ...) bytes, 256-byte aligned.
 *   - Calls that overlap on one workspace race; separate streams need
 *     separate workspaces.
 *   - Status word: the calls that run the grouped feature gradient
 *     (haste_bwd_h, haste_step and its variants, haste_joint_step) keep an
 *     int32 in the first 4 bytes of their workspace.  The waves of a
 *     feature-gradient workgroup take turns on a shared accumulator; every
 *     wait for a turn is bounded, and a wait that gives up (which a correct
 *     turn sequence never does) skips that wave's update and sets the word
 *     to 1.  The call then still completes, but dh is invalid.  The word is
 *     rewritten by every such call; read it with haste_workspace_status.
 */
#ifndef HASTE_H
#define HASTE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t haste_bf16;

typedef enum {
    HASTE_OK = 0,
    HASTE_ERR_NULL = -1,         /* a required pointer is NULL */
    HASTE_ERR_DIM = -2,          /* a size is < 1, or sizes are inconsistent */
    HASTE_ERR_UNSUPPORTED = -3,  /* valid shape without a kernel (see above) */
    HASTE_ERR_ALIGN = -4,        /* a pointer is not 16-byte aligned */
    HASTE_ERR_WORKSPACE = -5,    /* workspace missing, too small or misaligned */
    HASTE_ERR_INDEX = -6,        /* reserved for validation results */
    HASTE_ERR_HIP = -7           /* a HIP launch failed */
} haste_status;

/* Reduction of the feature gradient across groups. */
typedef enum {
    HASTE_DH_ATOMIC = 0,         /* fp32 atomic adds; summation order varies run to run */
    HASTE_DH_DETERMINISTIC = 1   /* per-chunk partials reduced in fixed order; bitwise reproducible */
} haste_dh_mode;

typedef enum {
    HASTE_OP_FWD = 0,
    HASTE_OP_BWD_W = 1,
    HASTE_OP_BWD_H = 2,
    HASTE_OP_FWD_BCE = 3,
    HASTE_OP_STEP = 4,
    HASTE_OP_FIXED_FWD = 5,
    HASTE_OP_FIXED_BWD_W = 6,
    HASTE_OP_FIXED_BWD_H = 7,
    HASTE_OP_FWD_BCE_BWD = 8
} haste_op;

/* Workspace bytes `op` needs for this shape (K = L and G = 1 for the
 * haste_fixed_* ops).  Returns 0 for an invalid op. */
size_t haste_workspace_size(int op, int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, int dh_mode);

/* Forward logits.  Z[b, l] = sum_f h[b, idx[l/G, f]] * W[l, f]; per group
 * Z_k = H_k W_k^T with H_k = h[:, I_k] ("overall framework" logit formula and
 * "gather-once + dense MMA kernel" section).  Z is B x L fp32. */
int haste_fwd(const haste_bf16* h, const int32_t* idx, const haste_bf16* W, float* Z,
              int64_t B, int64_t H, int64_t K, int64_t G, int64_t F,
              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Weight gradient.  dW[l, f] = sum_b dZ[b, l] * h[b, idx[l/G, f]]; per group
 * dW_k = dZ_k^T H_k ("gather-once + dense MMA kernel").  dW is L x F fp32. */
int haste_bwd_w(const haste_bf16* h, const int32_t* idx, const haste_bf16* dZ, float* dW,
                int64_t B, int64_t H, int64_t K, int64_t G, int64_t F,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Feature gradient.  dh[b, j] = sum over (l, f) with idx[l/G, f] == j of
 * dZ[b, l] * W[l, f]: the per-group products dZ_k W_k added into the
 * overlapping columns I_k and reduced across groups ("gather-once + dense
 * MMA kernel": split-K reduction).  dh is B x H fp32; columns in no index set
 * are 0.  dh_mode selects the cross-workgroup reduction (haste_dh_mode). */
int haste_bwd_h(const haste_bf16* dZ, const int32_t* idx, const haste_bf16* W, float* dh,
                int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, int dh_mode,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes of haste_bwd_h for this shape and dh mode (the same as
 * haste_workspace_size(HASTE_OP_BWD_H, ...)). */
size_t haste_bwd_h_workspace_size(int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, int mode);

/* Forward with the BCE-gradient epilogue: dZ = scale * (sigmoid(Z) - Y)
 * rounded to bf16 (objective of the "head-tail split" section; mean over
 * samples, sum over labels: pass scale = 1/B).  Z (nullable) also receives
 * the fp32 logits.  loss (nullable, 1 double on the device) receives
 * scale * sum_{b,l} [max(z,0) + log(1 + e^-|z|) - y z]. */
int haste_fwd_bce(const haste_bf16* h, const int32_t* idx, const haste_bf16* W,
                  const int32_t* y_rowptr, const int32_t* y_col, float scale,
                  haste_bf16* dZ, float* Z, double* loss,
                  int64_t B, int64_t H, int64_t K, int64_t G, int64_t F,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* One training pass of the layer: forward, BCE gradient, dW and dh, with dZ
 * kept on chip in fp32 (fed to the matrix cores as bf16 hi + lo parts) and
 * never written to memory.  dW (L x F fp32) and dh (B x H fp32) are
 * required; Z (B x L fp32) and loss (1 double) are nullable. */
int haste_step(const haste_bf16* h, const int32_t* idx, const haste_bf16* W,
               const int32_t* y_rowptr, const int32_t* y_col, float scale,
               float* dW, float* dh, float* Z, double* loss,
               int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, int dh_mode,
               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The fused training pass with the argument order of the layer's interface
 * table: forward, BCE gradient dZ = scale * (sigmoid(Z) - Y) kept on chip,
 * dW = dZ^T H_k per group and dh as the split-K scatter of dZ_k W_k
 * ("gather-once + dense MMA kernel" for the three products, "head-tail
 * split" for the BCE objective it differentiates).  The same kernels and
 * results as haste_step (dW and dh bitwise equal to haste_step's with the
 * same mode, shape and loss request: with a loss the forward epilogue forms
 * the sigmoid from e^-|z|, which moves the last bits of dZ); loss
 * (nullable) is 1 fp32 value, scale * sum [max(z,0) +
 * log(1 + e^-|z|) - y z], summed in fp64 and rounded once.  mode is a
 * haste_dh_mode.  Workspace: haste_workspace_size(HASTE_OP_FWD_BCE_BWD, ...)
 * bytes (256 more than haste_step's, for the fp64 loss); its first 4 bytes
 * are the status word.  Errors as haste_step. */
int haste_fwd_bce_bwd(const haste_bf16* h, const int32_t* idx, const haste_bf16* W,
                      const int32_t* y_rowptr, const int32_t* y_col, float scale,
                      float* dW, float* dh, float* loss, int mode,
                      void* workspace, size_t workspace_bytes, int64_t B, int64_t H, int64_t K, int64_t G,
                      int64_t F, hipStream_t stream);

/* haste_step for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same pass,
 * kernels and results (bitwise haste_step's in deterministic mode), with the
 * workspace replaced by a 32 MiB device array inside the library, one per
 * GPU, held until the process ends.  The call allocates nothing: no hipMalloc,
 * hipFree or allocating library routine.  Shapes whose workspace
 * (haste_workspace_size(HASTE_OP_STEP, ...)) exceeds 32 MiB are refused with
 * HASTE_ERR_WORKSPACE before any HIP call (every supported shape with
 * H <= 768 fits; H = 1024 with large B in deterministic mode does not).
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (other streams, other host threads) race and must be serialised by the
 * caller.  The array keeps the last call's contents; every call rewrites or
 * clears what it reads.  Its status word is not exposed; callers that need
 * the checked path use haste_step.  Other arguments and errors as
 * haste_step (HASTE_ERR_HIP also when the array's address cannot be
 * obtained). */
int haste_step_noalloc(const haste_bf16* h, const int32_t* idx, const haste_bf16* W,
                       const int32_t* y_rowptr, const int32_t* y_col, float scale,
                       float* dW, float* dh, float* Z, double* loss,
                       int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, int dh_mode, hipStream_t stream);

/* haste_step with the weight gradient dW_k = dZ_k^T H_k (HASTE page, the
 * "gather-once + dense MMA kernel" section) stored as bf16: dW is L x F
 * bf16, each value the fp32 accumulator of haste_step's dW rounded to nearest even
 * (bitwise that rounding of haste_step's result), so the pass writes half
 * the dW bytes.  The contractions are unchanged (fp32 accumulation, dZ split
 * into bf16 hi + lo parts for the matrix cores), as is dh (fp32); the loss
 * is optional as in haste_step; there is no logits output.  `events` may be
 * NULL, else as in haste_step_timed.  bf16 weights only.  Workspace as
 * haste_workspace_size(HASTE_OP_STEP, ...).  Same errors as haste_step. */
int haste_step_bf16dw(const haste_bf16* h, const int32_t* idx, const haste_bf16* W,
                      const int32_t* y_rowptr, const int32_t* y_col, float scale,
                      haste_bf16* dW, float* dh, double* loss,
                      int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, int dh_mode,
                      void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* events);

/* haste_step plus timing: when `events` is non-NULL, events[0..4] (created
 * by the caller) are recorded on `stream` at the phase boundaries of the
 * pass: [0] start, [1] after the feature-major copy of h and output
 * clearing, [2] after the forward + BCE + dW kernel, [3] after the dh kernel,
 * [4] after the deterministic reduction (same point as [3] in atomic mode).
 * For benchmarks that need per-kernel durations on the caller's stream.
 * Same work, arguments and errors as haste_step. */
int haste_step_timed(const haste_bf16* h, const int32_t* idx, const haste_bf16* W,
                     const int32_t* y_rowptr, const int32_t* y_col, float scale,
                     float* dW, float* dh, float* Z, double* loss,
                     int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, int dh_mode,
                     void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* events);

/* G = 1 baseline: standard fixed fan-in with one index set per label
 * (idx1 is L x F), thin per-label dot products without a shared tile
 * ("background" and "key findings": the micro-benchmark baseline).  Same
 * formulas, shapes and conventions as haste_fwd / haste_bwd_w / haste_bwd_h
 * with K = L and G = 1. */
int haste_fixed_fwd(const haste_bf16* h, const int32_t* idx1, const haste_bf16* W, float* Z,
                    int64_t B, int64_t H, int64_t L, int64_t F,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);
int haste_fixed_bwd_w(const haste_bf16* h, const int32_t* idx1, const haste_bf16* dZ, float* dW,
                      int64_t B, int64_t H, int64_t L, int64_t F,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);
int haste_fixed_bwd_h(const haste_bf16* dZ, const int32_t* idx1, const haste_bf16* W, float* dh,
                      int64_t B, int64_t H, int64_t L, int64_t F, int dh_mode,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Dense head of the head-tail split ("head-tail split" section: the most
 * frequent labels get a dense head, every label seeing all H features, next
 * to the group-shared sparse tail; one BCE objective over both).  One
 * training pass of the head: Z = h W_head^T, dZ = scale * (sigmoid(Z) - Y)
 * (Y: B x L_head 0/1 labels as CSR with sorted, unique, head-local ids),
 * dW_head = dZ^T h and dh = dZ W_head.  W_head is L_head x H bf16
 * row-major, dW_head L_head x H fp32 and dh B x H fp32 (both overwritten),
 * Z_head (nullable) B x L_head fp32, loss (nullable) 1 double, set to
 * scale * sum [max(z,0) + log(1 + e^-|z|) - y z].  Products: bf16 in, fp32
 * accumulate and out.  For B <= 128, H % 64 == 0 and L_head % 8 == 0 all
 * three run on libhaste's matrix-core kernels (the logits fused with the
 * BCE gradient); other shapes run them on rocBLAS (atomics off) with a
 * libhaste BCE kernel between them.  Either way Z, dW_head and dh are
 * bitwise repeatable; the loss is summed with atomics.  dZ reaches the two
 * weight-side products as stacked bf16 hi + lo parts (about 16 significant
 * bits).  The rocBLAS handle is created on the first call of a host thread
 * on a device and kept for the process; each call hands it part of
 * `workspace`.  Limits: B <=
 * 2^24, H <= 2^20, L_head < 2^31 - 64.  Errors as haste_step.  Workspace:
 * haste_head_workspace_size(B, H, L_head) bytes, 256-byte aligned. */
size_t haste_head_workspace_size(int64_t B, int64_t H, int64_t L_head);
int haste_head_step(const haste_bf16* h, const haste_bf16* W_head, const int32_t* y_rowptr, const int32_t* y_col,
                    float scale, float* dW_head, float* dh, float* Z_head, double* loss, int64_t B, int64_t H,
                    int64_t L_head, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Joint head + tail training pass of the head-tail split: haste_step on the
 * group-shared tail (idx, W_tail, tail-local labels yt_*, scale_tail) and the
 * dense head pass (W_head, head-local labels yh_*, scale_head) on the same
 * features h.  With the objective averaged over samples both scales are
 * 1/B; they are separate so that a caller can weight the branches.  dh
 * receives the sum of both branches' feature gradients (tail first, then the
 * head's product added on top, in a fixed order: deterministic when dh_mode
 * is), loss (nullable) the sum of both branches' losses.  Tail shapes and
 * limits as haste_step, head as haste_head_step.  Workspace:
 * haste_joint_workspace_size(...) bytes (the branches run one after the
 * other on `stream` and share it). */
size_t haste_joint_workspace_size(int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, int64_t L_head,
                                  int dh_mode);
int haste_joint_step(const haste_bf16* h, const int32_t* idx, const haste_bf16* W_tail, const int32_t* yt_rowptr,
                     const int32_t* yt_col, const haste_bf16* W_head, const int32_t* yh_rowptr,
                     const int32_t* yh_col, float scale_tail, float scale_head, float* dW_tail, float* dW_head,
                     float* dh, double* loss,
                     int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, int64_t L_head, int dh_mode,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* FP8 weights ("limitations" section: pairing the layer with FP8
 * quantisation is the named next step; the scheme is this library's
 * reading).  W is stored as OCP FP8 E4M3 codes W8 (L x F bytes; 1 sign bit,
 * 4 exponent bits with bias 7, 3 mantissa bits, largest finite 448, no
 * infinities) and one exponent per label group, wexp (K int32): weight
 * [l, f] = decode(W8[l, f]) * 2^wexp[l / G], an exact bf16 value.  The
 * FP8-weight calls compute exactly what haste_fwd / haste_step compute on
 * those bf16 values (bitwise the same results), reading half the weight
 * bytes.  haste_quantize_w8: wexp[k] = the smallest integer e with
 * max |W_k| 2^-e <= 448 (0 for an all-zero group; clamped to [-120, 120])
 * and W8 = the codes of W 2^-e rounded to nearest, ties to the even code.
 * Shapes, limits, workspaces and errors as haste_fwd / haste_step; W8 and
 * wexp 16-byte aligned. */
int haste_quantize_w8(const haste_bf16* W, uint8_t* W8, int32_t* wexp, int64_t K, int64_t G, int64_t F,
                      hipStream_t stream);
int haste_fwd_w8(const haste_bf16* h, const int32_t* idx, const uint8_t* W8, const int32_t* wexp, float* Z,
                 int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, void* workspace, size_t workspace_bytes,
                 hipStream_t stream);
int haste_step_w8(const haste_bf16* h, const int32_t* idx, const uint8_t* W8, const int32_t* wexp,
                  const int32_t* y_rowptr, const int32_t* y_col, float scale, float* dW, float* dh, float* Z,
                  double* loss, int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, int dh_mode, void* workspace,
                  size_t workspace_bytes, hipStream_t stream);
/* haste_step_w8 with the events of haste_step_timed. */
int haste_step_w8_timed(const haste_bf16* h, const int32_t* idx, const uint8_t* W8, const int32_t* wexp,
                        const int32_t* y_rowptr, const int32_t* y_col, float scale, float* dW, float* dh, float* Z,
                        double* loss, int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, int dh_mode,
                        void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* events);

/* Semantic label grouping ("group-shared fixed fan-in" section: labels are
 * grouped by the similarity of their embeddings, approximately, by
 * mini-batch spherical k-means into C ~ L / (beta G) coarse clusters and
 * then, inside each cluster, greedy groups of a seed and its G - 1 nearest
 * neighbours).  Embeddings E: L x H bf16 (H % 8 == 0, H <= 1024), similarity
 * = dot product.  All results are bitwise repeatable.
 *
 * haste_kmeans_assign: assign[i] = argmax_c <E_r, M_c> (lowest c on ties)
 * for r = rows[i] (rows NULL: r = i, n_rows = L); score (nullable) gets
 * the maximum.  M: C x H bf16; rows[] must hold ids in [0, L).  One
 * fused matrix-core kernel computes the products (fp32 accumulate) tile by
 * tile and keeps only each label's best (score, centre), so no score
 * matrix is stored.  The number of 256 x 256 (label, centre) tiles must not
 * exceed 2^31 (HASTE_ERR_UNSUPPORTED).  Workspace:
 * haste_kmeans_assign_workspace_size(n_rows, C, H, rows != NULL): 8 bytes
 * per row, plus, with Hp = H rounded up to 128, the gathered rows (n_rows x
 * Hp bf16) when rows is given or Hp != H, and the centres (C x Hp bf16) when
 * Hp != H.
 * haste_kmeans_init: centre c starts as E[init[c]]: Mc (C x H fp32), Mb
 * (its bf16 copy, the operand of the assignment) and counts[c] = 0.
 * haste_kmeans_update: one mini-batch step (Sculley's update) for the n
 * batch labels batch[] with their centres assign[]: a centre with m batch
 * members becomes mu = (counts[c] Mc[c] + sum of the members, in batch
 * order) / (counts[c] + m), is normalised to unit length, and counts[c] +=
 * m; Mb follows.  Centres without members are unchanged.  Workspace:
 * haste_kmeans_update_workspace_size(n, C).
 * haste_group_greedy: perm (L int32, a permutation of the labels) such
 * that group k = perm[kG .. kG + G): per cluster (assign[] in [0, C)),
 * members in increasing id, the lowest-id ungrouped member seeds a group
 * and the G - 1 ungrouped members with the largest dot product with it
 * (lower id on ties) join; a group lists its members in increasing id;
 * clusters' groups come in cluster order; the members left over (fewer
 * than G per cluster) follow, concatenated in (cluster, id) order and cut
 * into groups of G.  L % G == 0, G <= 64.  Workspace:
 * haste_group_workspace_size(L, C). */
size_t haste_kmeans_assign_workspace_size(int64_t n_rows, int64_t C, int64_t H, int with_rows);
int haste_kmeans_assign(const haste_bf16* E, const int32_t* rows, int64_t n_rows, int64_t L, const haste_bf16* M,
                        int64_t C, int64_t H, int32_t* assign, float* score, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);
int haste_kmeans_init(const haste_bf16* E, const int32_t* init, int64_t L, int64_t C, int64_t H, float* Mc,
                      haste_bf16* Mb, int32_t* counts, hipStream_t stream);
size_t haste_kmeans_update_workspace_size(int64_t n, int64_t C);
int haste_kmeans_update(const haste_bf16* E, const int32_t* batch, const int32_t* assign, int64_t n, int64_t L,
                        int64_t C, int64_t H, float* Mc, haste_bf16* Mb, int32_t* counts, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);
size_t haste_group_workspace_size(int64_t L, int64_t C);
int haste_group_greedy(const haste_bf16* E, const int32_t* assign, int64_t L, int64_t C, int64_t H, int64_t G,
                       int32_t* perm, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Label embeddings for the grouping ("group-shared fixed fan-in" section: a
 * label's embedding is the normalized mean of the encoder features of the
 * samples it is positive for).  S (L x H fp32) and counts (L int32) are the
 * caller's running per-label feature sums and positive counts, zeroed by the
 * caller before the first batch.  haste_label_emb_accumulate adds one batch:
 * for every sample b (features h, B x H bf16) and each positive label l of b
 * (CSR y_rowptr[B + 1] and y_col[nnz], ids in [0, L); nnz = y_rowptr[B],
 * passed by the caller), S[l] += h[b] and counts[l] += 1.  A label's
 * contributions from one batch are summed in sample order and added to S
 * once (no atomics), so S repeats bit for bit for the same batch sequence.
 * haste_label_emb_finalize: E (L x H bf16) = S_l / |S_l| rounded to nearest
 * bf16, and 0 for labels without positives.  8 <= H <= 1024 with H % 8 == 0,
 * L <= 2^30, nnz <= 2^30, B <= 2^30.  Workspace of the accumulation:
 * haste_label_emb_workspace_size(nnz) bytes (sort keys and the entries'
 * sample ids), 256-byte aligned. */
size_t haste_label_emb_workspace_size(int64_t nnz);
int haste_label_emb_accumulate(const haste_bf16* h, const int32_t* y_rowptr, const int32_t* y_col, int64_t nnz,
                               int64_t B, int64_t H, int64_t L, float* S, int32_t* counts, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);
int haste_label_emb_finalize(const float* S, const int32_t* counts, int64_t L, int64_t H, haste_bf16* E,
                             hipStream_t stream);

/* Group-level rewiring of the index sets: the discrete phase of the dynamic
 * sparse training ("loss / training strategy" section: every so many steps
 * the group-level I_k are reselected RigL-style with |I_k| = F kept; the
 * algorithm is not printed, so RigL's steps are taken per group):
 *   grow[k, j]  = sum_g | sum_b dZ[b, kG+g] h[b, j] |   (K x H fp32): the
 *                 dense loss gradient's size on feature column j;
 *   prune[k, f] = sum_g | W[kG+g, f] |                 (K x F fp32);
 *   drop the n_swap slots with the smallest prune score, grow the n_swap
 *   columns with the largest grow score among those not kept (a dropped
 *   column may return), equal scores going to the lower column id; the new
 *   row of idx_out is sorted ascending, a kept column's weights move with it
 *   in W_out and a grown column's weights are zero.
 * h: B x H bf16; dZ: B x L bf16 (e.g. from haste_fwd_bce); idx / W as in
 * haste_fwd; 0 <= n_swap <= F.  idx_out (K x F int32) and W_out (L x F bf16)
 * may be idx and W themselves (in place) or must not overlap them.
 * grow_score (K x H) and prune_score (K x F) are optional fp32 outputs.
 * Scores are fp32 (matrix-core products, fixed summation order), so the
 * result is bitwise repeatable; the selection is exact given the scores.
 * Limits: G in {16, 32, 64}, F in {32, 64, 128}, F <= H <= 1024, B <= 256.
 * Workspace: haste_rewire_workspace_size(B, H, K, G, F) bytes (hT and the
 * K x H grow scores). */
size_t haste_rewire_workspace_size(int64_t B, int64_t H, int64_t K, int64_t G, int64_t F);
int haste_rewire(const haste_bf16* h, const haste_bf16* dZ, const int32_t* idx, const haste_bf16* W, int64_t n_swap,
                 int32_t* idx_out, haste_bf16* W_out, float* grow_score, float* prune_score, int64_t B, int64_t H,
                 int64_t K, int64_t G, int64_t F, void* workspace, size_t workspace_bytes, hipStream_t stream);
/* haste_rewire with timing events (events NULL: no events).  events[0..3]
 * are recorded on `stream` before the feature-major copy of h, before the
 * score kernel, before the selection kernel and after it. */
int haste_rewire_timed(const haste_bf16* h, const haste_bf16* dZ, const int32_t* idx, const haste_bf16* W,
                       int64_t n_swap, int32_t* idx_out, haste_bf16* W_out, float* grow_score, float* prune_score,
                       int64_t B, int64_t H, int64_t K, int64_t G, int64_t F, void* workspace,
                       size_t workspace_bytes, hipStream_t stream, hipEvent_t* events);

/* Bank-balanced slot order, in place.  A group is its index set I_k ("group-
 * shared fixed fan-in" section): the slot at which a column sits does not
 * change any result of the layer as long as column f of W_k moves with it.
 * This call reorders every group's slots for the feature-gradient kernels,
 * whose accumulator holds feature column j's rows in bank group
 * (j >> 1) mod 8 and whose read-add-write instructions each cover a run of 8
 * consecutive slots: per group, the F slots are sorted by that key (equal
 * keys keep their order) and dealt over the F / 8 runs in turn, the p-th
 * sorted slot becoming slot 8 (p mod F/8) + p div F/8.  A key held by at most
 * F / 8 slots of a group then falls in distinct runs (fewer bank conflicts in
 * dh); nothing else depends on the order.
 *   idx   K x F int32, permuted in place (device).
 *   W     L x F bf16 (L = K G), its columns permuted with idx, in place;
 *         NULL to reorder idx alone (e.g. before W is initialised).
 *   perm  K x F uint8 output, perm[k, s] = the old slot now at slot s; NULL
 *         to skip.  Apply it to any other per-slot state the caller keeps
 *         (optimizer moments, FP8 weight codes).
 * Rewiring (haste_rewire) writes sorted rows; order them again afterwards.
 * G in {16, 32, 64}, F in {32, 64, 128}; pointers 16-byte aligned.
 * Asynchronous on `stream`. */
int haste_order_slots(int32_t* idx, haste_bf16* W, uint8_t* perm, int64_t K, int64_t G, int64_t F,
                      hipStream_t stream);

/* Count (into *bad, a device int32 the call zeroes first) the index rows
 * that have an entry outside [0, H) or an entry twice (the order of a row's
 * entries is free). */
int haste_validate_idx(const int32_t* idx, int64_t rows, int64_t F, int64_t H, int32_t* bad,
                       hipStream_t stream);

/* Count (into *bad, zeroed first) the samples whose CSR label row is not
 * non-decreasing in y_rowptr, has an id outside [0, L) or is not strictly
 * increasing. */
int haste_validate_labels(const int32_t* y_rowptr, const int32_t* y_col, int64_t B, int64_t L, int32_t* bad,
                          hipStream_t stream);

/* Copies the status word (first 4 bytes of `workspace`, see the conventions
 * above) of the last feature-gradient call on that workspace into *status
 * (host memory) and synchronises `stream`: 0 = every accumulator hand-off
 * completed, 1 = a bounded turn wait gave up and dh is invalid.  Unlike the
 * other calls this one blocks.  HASTE_ERR_NULL / HASTE_ERR_WORKSPACE
 * (misaligned) / HASTE_ERR_HIP (copy or synchronisation failed). */
int haste_workspace_status(const void* workspace, int32_t* status, hipStream_t stream);

/* Test hook, not for production use: sets the bound (number of polls) of
 * every feature-gradient turn wait launched afterwards in this process, so
 * that a test can force the give-up path on the GPU (0: every wait gives up
 * at once; every kernel still runs to its end) and check that the status
 * word reports it.  A negative value restores the default bound. */
void haste_test_set_turn_spins(int spins);

/* Static text for a haste_status value. */
const char* haste_status_string(int status);

/* Library version string. */
const char* haste_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HASTE_H */

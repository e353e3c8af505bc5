/*
 * CPU oracle for the group-shared fixed fan-in sparse output layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code with
 * the HIP path and must never be used as a fallback for it.
 *
 * Source of every definition: "HASTE: Hardware-Aware Dynamic Sparse Training
 * for Large Output Spaces" (papernotes.org notes on ICML 2026, arXiv
 * 2606.01117).
 *   - logit of label l:  z_l(x) = < w_l , h_{I_g(l)} >, w_l in R^F, I_k a
 *     subset of [H] with |I_k| = F shared by the G labels of group k
 *     ("Method / overall framework" and "group-shared fixed fan-in").
 *   - per group:  Z_k = H_k W_k^T with H_k = h[:, I_k]  ("gather-once + dense
 *     MMA kernel"),  grad W_k = (grad Z_k)^T H_k  (same section),
 *     grad h = the sum over groups of grad Z_k W_k added into the columns I_k
 *     (same section: index sets of different groups overlap and are reduced).
 *   - loss: binary cross-entropy of sigmoid(logit) against 0/1 labels, summed
 *     over labels and averaged over samples ("Head-tail split" objective and
 *     "loss / training strategy").
 *
 * Conventions (the plain reading where the notes are silent):
 *   label l = k*G + g belongs to group k = l / G;
 *   slot f of w_l multiplies feature column idx[k*F + f];
 *   h is B x H, W and dW are L x F, Z and dZ are B x L, dh is B x H, all
 *   row-major; idx is K x F int32;
 *   bf16 inputs are passed as uint16 bit patterns and widened exactly;
 *   all accumulation and all outputs are fp64.
 *
 * Loops are the definitions written out, parallelised with OpenMP over an
 * outer index whose iterations write disjoint outputs, so results do not
 * depend on the thread count.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Threads the OpenMP loops below use (reported next to oracle timings). */
int oracle_num_threads(void)
{
    return omp_get_max_threads();
}

static double bf16_to_double(uint16_t u)
{
    uint32_t bits = (uint32_t)u << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* dZ may be given as bf16 bits (dz16) or as fp64 (dz64); exactly one is set. */
static double dz_at(const uint16_t *dz16, const double *dz64, int64_t i)
{
    return dz64 ? dz64[i] : bf16_to_double(dz16[i]);
}

/* Z[b, l] = sum_f h[b, idx[k, f]] * W[l, f],  k = l / G. */
void oracle_fwd(const uint16_t *h, const int32_t *idx, const uint16_t *W, double *Z,
                int64_t B, int64_t H, int64_t K, int64_t G, int64_t F)
{
    const int64_t L = K * G;
#pragma omp parallel for schedule(static)
    for (int64_t l = 0; l < L; ++l) {
        const int64_t k = l / G;
        for (int64_t b = 0; b < B; ++b) {
            double acc = 0.0;
            for (int64_t f = 0; f < F; ++f)
                acc += bf16_to_double(h[b * H + idx[k * F + f]]) * bf16_to_double(W[l * F + f]);
            Z[b * L + l] = acc;
        }
    }
}

/* dW[l, f] = sum_b dZ[b, l] * h[b, idx[k, f]],  k = l / G. */
static void bwd_w(const uint16_t *h, const int32_t *idx, const uint16_t *dz16, const double *dz64,
                  double *dW, int64_t B, int64_t H, int64_t K, int64_t G, int64_t F)
{
    const int64_t L = K * G;
#pragma omp parallel for schedule(static)
    for (int64_t l = 0; l < L; ++l) {
        const int64_t k = l / G;
        for (int64_t f = 0; f < F; ++f) {
            double acc = 0.0;
            for (int64_t b = 0; b < B; ++b)
                acc += dz_at(dz16, dz64, b * L + l) * bf16_to_double(h[b * H + idx[k * F + f]]);
            dW[l * F + f] = acc;
        }
    }
}

void oracle_bwd_w(const uint16_t *h, const int32_t *idx, const uint16_t *dZ, double *dW,
                  int64_t B, int64_t H, int64_t K, int64_t G, int64_t F)
{
    bwd_w(h, idx, dZ, NULL, dW, B, H, K, G, F);
}

void oracle_bwd_w_f64(const uint16_t *h, const int32_t *idx, const double *dZ, double *dW,
                      int64_t B, int64_t H, int64_t K, int64_t G, int64_t F)
{
    bwd_w(h, idx, NULL, dZ, dW, B, H, K, G, F);
}

/* dh[b, j] = sum over labels l and slots f with idx[l / G, f] == j of
 * dZ[b, l] * W[l, f].  Columns in no index set stay 0. */
static void bwd_h(const uint16_t *dz16, const double *dz64, const int32_t *idx, const uint16_t *W,
                  double *dh, int64_t B, int64_t H, int64_t K, int64_t G, int64_t F)
{
    const int64_t L = K * G;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t j = 0; j < H; ++j)
            dh[b * H + j] = 0.0;
        for (int64_t l = 0; l < L; ++l) {
            const int64_t k = l / G;
            const double d = dz_at(dz16, dz64, b * L + l);
            for (int64_t f = 0; f < F; ++f)
                dh[b * H + idx[k * F + f]] += d * bf16_to_double(W[l * F + f]);
        }
    }
}

void oracle_bwd_h(const uint16_t *dZ, const int32_t *idx, const uint16_t *W, double *dh,
                  int64_t B, int64_t H, int64_t K, int64_t G, int64_t F)
{
    bwd_h(dZ, NULL, idx, W, dh, B, H, K, G, F);
}

void oracle_bwd_h_f64(const double *dZ, const int32_t *idx, const uint16_t *W, double *dh,
                      int64_t B, int64_t H, int64_t K, int64_t G, int64_t F)
{
    bwd_h(NULL, dZ, idx, W, dh, B, H, K, G, F);
}

/*
 * Binary cross-entropy gradient and loss for logits Z (B x L) against the
 * 0/1 label matrix Y given as CSR: row b has Y[b, l] = 1 exactly for the
 * label ids l in y_col[y_rowptr[b] .. y_rowptr[b+1]) (a repeated id is still
 * a single 1).
 *   dZ[b, l] = scale * (sigmoid(Z[b, l]) - Y[b, l]),  sigmoid(x) = 1/(1+e^-x)
 *   loss     = scale * sum_{b,l} [ max(z,0) + log(1 + e^-|z|) - Y z ]
 * The objective sums over labels and averages over samples, so the caller
 * passes scale = 1/B.
 */
void oracle_bce(const double *Z, int64_t B, int64_t L, const int32_t *y_rowptr,
                const int32_t *y_col, double scale, double *dZ, double *loss)
{
    double *row_loss = (double *)calloc((size_t)(B > 0 ? B : 1), sizeof(double));
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < B; ++b) {
        unsigned char *y = (unsigned char *)calloc((size_t)(L > 0 ? L : 1), 1);
        for (int64_t p = y_rowptr[b]; p < y_rowptr[b + 1]; ++p)
            y[y_col[p]] = 1;
        double acc = 0.0;
        for (int64_t l = 0; l < L; ++l) {
            const double z = Z[b * L + l];
            const double yy = y[l] ? 1.0 : 0.0;
            if (dZ)
                dZ[b * L + l] = scale * (1.0 / (1.0 + exp(-z)) - yy);
            acc += (z > 0.0 ? z : 0.0) + log1p(exp(-fabs(z))) - yy * z;
        }
        row_loss[b] = acc;
        free(y);
    }
    if (loss) {
        double s = 0.0;
        for (int64_t b = 0; b < B; ++b)
            s += row_loss[b];
        *loss = scale * s;
    }
    free(row_loss);
}

/*
 * One training pass of the layer: Z = forward, dZ = BCE gradient of Z,
 * then dW and dh from that fp64 dZ (no rounding of dZ).  Any output pointer
 * may be NULL.  Z_work must hold B*L doubles and dZ_work B*L doubles.
 */
void oracle_step(const uint16_t *h, const int32_t *idx, const uint16_t *W,
                 const int32_t *y_rowptr, const int32_t *y_col, double scale,
                 double *Z_work, double *dZ_work, double *dW, double *dh, double *loss,
                 int64_t B, int64_t H, int64_t K, int64_t G, int64_t F)
{
    oracle_fwd(h, idx, W, Z_work, B, H, K, G, F);
    oracle_bce(Z_work, B, K * G, y_rowptr, y_col, scale, dZ_work, loss);
    if (dW)
        oracle_bwd_w_f64(h, idx, dZ_work, dW, B, H, K, G, F);
    if (dh)
        oracle_bwd_h_f64(dZ_work, idx, W, dh, B, H, K, G, F);
}

/*
 * bcq_oracle.c -- plain float64 CPU oracle for the binary-coded quantization
 * (BCQ) product.  TEST INFRASTRUCTURE ONLY: tests, the smoke check and the
 * benchmark's CPU-baseline leg may call it; the library never does.  It shares
 * no code, header, table or helper with the HIP path.
 *
 * What it computes (plain definitions, no blocking, no reordering beyond them):
 *
 *  - BCQ writes a weight matrix as a sum of p binary planes, each plane a
 *    {-1,+1} matrix scaled by its own factor, and computes a p-bit product as p
 *    plane products (AnyBCQ paper notes, "Method / key designs": the BCQ
 *    representation and the direct bit-plane kernel; AnyBCQ abstract on the
 *    mlsanity page: weights kept as bit-planes with scale factors, compute at
 *    bit-plane level).
 *  - The quantization is asymmetric and group-wise with g = 128 columns per
 *    group (AnyBCQ paper notes, "Training strategy"): every (row, group) pair
 *    has its own scale per plane and one offset z.  Reading adopted: the offset
 *    is added to every reconstructed weight of its group, so the product gains
 *    z times the sum of the activations over that group.
 *  - Precision p uses the first p planes of one shared store, and may use its
 *    own scale table (AnyBCQ paper notes, "progressive precision expansion":
 *    earlier planes are frozen and all scales are refit for the new precision).
 *
 * Sign encoding (a reading; the pages only say the planes hold -1/+1): column k
 * of plane i, row m is bit (k mod 32), least significant first, of word
 * signs[(i*M + m)*W + k/32] with W = ceil(K/32); a set bit is +1, clear is -1.
 *
 * Arrays: alpha is the precision-p table [p][M][G], zero is [M][G], G = K/g,
 * x is [K], y is [M], w is [M][K]; all float64, row-major.  Every stored
 * fp16/fp32 value converts to float64 exactly, so the only rounding here is
 * float64 accumulation (relative error ~1e-15 at these sizes).
 */
#include <stddef.h>
#include <stdint.h>

/* +1 or -1 for plane i, row m, column k. */
static int bcq_oracle_sign(const uint32_t *signs, int M, int K, int i, int m, int k)
{
    size_t W = (size_t)(K + 31) / 32;
    uint32_t word = signs[((size_t)i * (size_t)M + (size_t)m) * W + (size_t)(k / 32)];
    return ((word >> (k % 32)) & 1u) ? +1 : -1;
}

/*
 * y[m] = sum over groups j of
 *          sum_{i<p} alpha[i][m][j] * (sum_{k in group j} s_i[m][k] * x[k])
 *        + zero[m][j] * (sum_{k in group j} x[k])
 * i.e. one plane product per plane, each scaled by its per-group factor and
 * accumulated, plus the asymmetric offset times the group's activation sum.
 */
void bcq_oracle_gemv(const uint32_t *signs, int P, int M, int K, int g, int p,
                     const double *alpha, const double *zero, const double *x,
                     double *y)
{
    (void)P;
    int G = K / g;
    for (int m = 0; m < M; ++m) {
        double acc = 0.0;
        for (int j = 0; j < G; ++j) {
            double group_sum = 0.0;
            for (int k = j * g; k < (j + 1) * g; ++k)
                group_sum += x[k];
            for (int i = 0; i < p; ++i) {
                double plane_sum = 0.0; /* add or subtract each activation */
                for (int k = j * g; k < (j + 1) * g; ++k) {
                    if (bcq_oracle_sign(signs, M, K, i, m, k) > 0)
                        plane_sum += x[k];
                    else
                        plane_sum -= x[k];
                }
                acc += alpha[((size_t)i * M + m) * G + j] * plane_sum;
            }
            acc += zero[(size_t)m * G + j] * group_sum;
        }
        y[m] = acc;
    }
}

/*
 * Dense reconstruction at precision p:
 *   w[m][k] = sum_{i<p} alpha[i][m][k/g] * s_i[m][k] + zero[m][k/g]
 */
void bcq_oracle_dequant(const uint32_t *signs, int P, int M, int K, int g, int p,
                        const double *alpha, const double *zero, double *w)
{
    (void)P;
    int G = K / g;
    for (int m = 0; m < M; ++m) {
        for (int k = 0; k < K; ++k) {
            int j = k / g;
            double v = zero[(size_t)m * G + j];
            for (int i = 0; i < p; ++i)
                v += alpha[((size_t)i * M + m) * G + j] *
                     (double)bcq_oracle_sign(signs, M, K, i, m, k);
            w[(size_t)m * K + k] = v;
        }
    }
}

/* Sign of plane i, row m, column k as +1/-1 (for tests of the encoding). */
int bcq_oracle_sign_at(const uint32_t *signs, int M, int K, int i, int m, int k)
{
    return bcq_oracle_sign(signs, M, K, i, m, k);
}

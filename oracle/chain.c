/*
 * Rank-r row delta u = B_rows . A as a fixed chain of fp32 fused multiply-adds.
 *
 * TEST INFRASTRUCTURE ONLY: part of the CPU oracle.  Only the tests, the smoke
 * check and the CPU-baseline leg of the benchmark load this library.
 *
 * The row-wise proxy update (FALQON summary page on shd-paper.top, section on
 * the key design: a row-wise proxy accumulates adapter updates that are merged
 * into the quantized backbone) needs, for each selected backbone row i, the
 * pending adapter delta u_i = B_i . A.  The pages do not say in which order
 * these r products are summed; because the result is later rounded to FP8,
 * any other order can flip a rounding decision, so the order is fixed here:
 *
 *     acc = +0.0f;  for k = 0 .. r-1:  acc = fmaf(B[i,k], A[k,j], acc);
 *     u[i,j] = acc
 *
 * fmaf is the C library's correctly rounded single-precision fused
 * multiply-add.  Rows are independent, so they are spread over OpenMP threads;
 * that changes no arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* u[i*d_in + j] for the rows listed in `rows` (n_rows of them), or for rows
 * 0..n_rows-1 when rows == NULL.  B is [d_out x r], A is [r x d_in], both
 * row-major float32; u is [n_rows x d_in]. */
void orc_rank_chain(const float *B, const float *A, const int64_t *rows,
                    int64_t n_rows, int64_t r, int64_t d_in, float *u)
{
#pragma omp parallel for schedule(static)
    for (int64_t ii = 0; ii < n_rows; ++ii) {
        const int64_t i = rows ? rows[ii] : ii;
        float *ui = u + ii * d_in;
        for (int64_t j = 0; j < d_in; ++j)
            ui[j] = 0.0f;
        for (int64_t k = 0; k < r; ++k) {
            const float b = B[i * r + k];
            const float *ak = A + k * d_in;
            for (int64_t j = 0; j < d_in; ++j)
                ui[j] = fmaf(b, ak[j], ui[j]);
        }
    }
}

/* number of threads an OpenMP parallel region uses here */
int orc_num_threads(void)
{
    int n = 0;
#pragma omp parallel
    {
#pragma omp atomic
        n += 1;
    }
    return n;
}

/* limit the OpenMP threads of later parallel regions (a timing of the oracle
 * on one core); arithmetic is unaffected */
void orc_set_num_threads(int n)
{
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n > 0 ? n : 1);
}

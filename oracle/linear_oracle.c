/* CPU oracle of the quantized linear layer (test infrastructure only: used by tests/, the smoke check and the
 * CPU baseline of the benchmark; the GPU library never includes or links it).
 *
 * Source: the TMAP image-to-video acceleration write-up, section "FFN性能优化", subsection "线性层量化".
 *   - The DiT's weights sit in its linear layers; storing them in 8 bits instead of bf16 saves memory, and
 *     computing in 8 bits as well (W8A8) lowers run time and peak memory.
 *   - Quantization is per block of 128 x 128 elements (the page prefers it to per-tensor and per-channel scales).
 *   - Layers whose quality suffers fall back from W8A8 to W8A16: the weights stay 8-bit, the activations stay
 *     16-bit.
 * The layer is the addmm of the model's FLOP profile (same write-up, section "Attention 性能优化 / 背景"):
 *   y = x W^T + b, with x [M, K] activations, W [N, K] (output features x input features), b [N].
 *
 * Readings (where the page is silent):
 *   - Both operands of W8A8 use 128 x 128 blocks: x in blocks of (128 tokens, 128 input features), W in blocks of
 *     (128 output features, 128 input features).  A ragged edge block holds the remaining rows or columns.
 *   - Each block uses the symmetric INT8 rule of the attention blocks: a = max |v| over the block; a below the
 *     guard gives scale 0 and codes 0; otherwise scale = a/127 and code = clamp(rint(v * (127/a)), -127, 127), all
 *     in fp32 (the rule lives in sattn_oracle.c, orc_quant_i8_rows).
 *   - W8A8: y = sum over 128-wide K blocks kb of s_x[m-block, kb] * s_w[n-block, kb] * S(m, n, kb) + b[n], where
 *     S is the exact integer dot product of the codes over block kb.
 *   - W8A16: y = sum over kb of s_w[n-block, kb] * (x . Wq)(m, n, kb) + b[n]: x is used as given (bf16) and the
 *     weight is its codes times the block scale.
 * Everything after the codes is computed in fp64 (an exact integer S, products and sums in double).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <omp.h>

float orc_bf16_to_f32(uint16_t h);
void orc_quant_i8_rows(const float* x, int rows, int d, int8_t* codes, float* scale);

/* ------------------------------------------------------------------------------------------------ */
/* Per-block INT8 of a bf16 matrix x [rows, cols] (row stride ld, elements) in blocks of br x bc.     */
/* codes: [rows, cols] dense.  scales: [ceil(rows/br), ceil(cols/bc)] row-major.                      */
/* ------------------------------------------------------------------------------------------------ */
void orc_quant_blocks(const uint16_t* x, int rows, int cols, long long ld, int br, int bc, int8_t* codes,
                      float* scales) {
  const int nbr = (rows + br - 1) / br, nbc = (cols + bc - 1) / bc;
#pragma omp parallel
  {
    float* blk = (float*)malloc(sizeof(float) * (size_t)br * bc);
    int8_t* bq = (int8_t*)malloc((size_t)br * bc);
#pragma omp for schedule(dynamic, 1)
    for (int b = 0; b < nbr * nbc; ++b) {
      const int i = b / nbc, j = b % nbc;
      const int r0 = i * br, c0 = j * bc;
      const int nr = (r0 + br < rows ? br : rows - r0), nc = (c0 + bc < cols ? bc : cols - c0);
      for (int r = 0; r < nr; ++r)
        for (int c = 0; c < nc; ++c) blk[r * nc + c] = orc_bf16_to_f32(x[(long long)(r0 + r) * ld + c0 + c]);
      orc_quant_i8_rows(blk, nr, nc, bq, &scales[(long long)i * nbc + j]);
      for (int r = 0; r < nr; ++r)
        for (int c = 0; c < nc; ++c) codes[(long long)(r0 + r) * cols + c0 + c] = bq[r * nc + c];
    }
    free(blk);
    free(bq);
  }
}

/* ------------------------------------------------------------------------------------------------ */
/* W8A8 linear.  xq [M, K] codes with scales sx [ceil(M/blk), K/blk]; wq [N, K] codes with scales         */
/* sw [ceil(N/blk), K/blk]; bias [N] bf16 or NULL.  K is a multiple of blk.                               */
/* out [M, N]: y in fp64.  mag [M, N] (or NULL): sum over kb of |s_x s_w S| plus |b|, the size that rounding */
/* errors of a finite-precision evaluation scale with.                                                   */
/* ------------------------------------------------------------------------------------------------ */
void orc_linear_w8a8(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw, const uint16_t* bias,
                     int M, int N, int K, int blk, double* out, double* mag) {
  const int nkb = K / blk;
#pragma omp parallel for schedule(dynamic, 4)
  for (int m = 0; m < M; ++m) {
    for (int n = 0; n < N; ++n) {
      double y = 0.0, a = 0.0;
      for (int kb = 0; kb < nkb; ++kb) {
        int64_t s = 0;
        const int8_t* xr = xq + (long long)m * K + (long long)kb * blk;
        const int8_t* wr = wq + (long long)n * K + (long long)kb * blk;
        for (int k = 0; k < blk; ++k) s += (int64_t)xr[k] * (int64_t)wr[k];
        const double c = (double)sx[(long long)(m / blk) * nkb + kb] * (double)sw[(long long)(n / blk) * nkb + kb];
        y += c * (double)s;
        a += fabs(c * (double)s);
      }
      if (bias) {
        const double b = (double)orc_bf16_to_f32(bias[n]);
        y += b;
        a += fabs(b);
      }
      out[(long long)m * N + n] = y;
      if (mag) mag[(long long)m * N + n] = a;
    }
  }
}

/* ------------------------------------------------------------------------------------------------ */
/* W8A16 linear.  x [M, K] bf16 (dense); wq, sw, bias, out, mag as above.  mag here is the sum over kb of  */
/* |s_w| * sum_k |x wq| plus |b| (the partial sums inside a block are also rounded by a finite-precision  */
/* evaluation).                                                                                           */
/* ------------------------------------------------------------------------------------------------ */
void orc_linear_w8a16(const uint16_t* x, const int8_t* wq, const float* sw, const uint16_t* bias, int M, int N,
                      int K, int blk, double* out, double* mag) {
  const int nkb = K / blk;
#pragma omp parallel
  {
    double* xr = (double*)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(dynamic, 4)
    for (int m = 0; m < M; ++m) {
      for (int k = 0; k < K; ++k) xr[k] = (double)orc_bf16_to_f32(x[(long long)m * K + k]);
      for (int n = 0; n < N; ++n) {
        double y = 0.0, a = 0.0;
        for (int kb = 0; kb < nkb; ++kb) {
          double p = 0.0, pa = 0.0;
          const int8_t* wr = wq + (long long)n * K + (long long)kb * blk;
          for (int k = 0; k < blk; ++k) {
            const double t = xr[kb * blk + k] * (double)wr[k];
            p += t;
            pa += fabs(t);
          }
          const double s = (double)sw[(long long)(n / blk) * nkb + kb];
          y += s * p;
          a += fabs(s) * pa;
        }
        if (bias) {
          const double b = (double)orc_bf16_to_f32(bias[n]);
          y += b;
          a += fabs(b);
        }
        out[(long long)m * N + n] = y;
        if (mag) mag[(long long)m * N + n] = a;
      }
    }
    free(xr);
  }
}

/*
 * sattn_oracle.c -- plain, slow CPU oracle for SageAttention-style quantized attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library.  The GPU library never links, includes or calls it, and it shares
 * no code, header, table or constant generator with the GPU kernels.
 *
 * What it computes (sources are the web pages on quantized attention for video DiTs):
 *   - The operator being replaced is PyTorch's scaled-dot-product flash attention, softmax(c*Q*K^T)*V
 *     (TMAP image-to-video acceleration write-up, ai.aiking123.com/155823, section
 *     "Attention 性能优化 / 背景", per-operator FLOP table).
 *   - It is replaced by SageAttention, an 8-bit quantized attention (same page, section "attention量化");
 *     on Wan the whole self-attention computation goes from 16 to 8 bits (same page, section
 *     "显存优化 / 量化").
 *   - A quantization scale computed from an all-zero channel divides by zero and poisons the output with
 *     NaN; the page reports fixing it (section "优化算子细节").  Every scale below is guarded.
 *   - Attention precision is switched per layer (section "保持视频质量"): the three modes below.
 *   - The score matrix is never materialised; softmax is computed online over key tiles (page
 *     "视频生成推理加速实战:从基线到27倍", step 3 "引擎级优化", item "算子融合与高效注意力").
 *   - Block-sparse attention computes only the regions a sparse block mask selects (page
 *     "视频生成模型的高效推理加速机制解析", section "核心组成与关键能力", item 3 "稀疏注意力", and step 3 of
 *     "工作原理与执行流程").
 * The pages give no formulas for the quantizer; the readings taken here (K smoothing by its per-channel
 * mean, symmetric per-block INT8 with scale amax/127, per-channel E4M3 for V with scale amax/448, the
 * guard threshold 2^-100, P quantized relative to the running max) are the plainest ones consistent with
 * the pages and are listed with their reasons in the design notes.
 *
 * Precision: every step whose result is an integer code (K mean, scales, INT8 codes, E4M3 codes) is done
 * in IEEE fp32 with round-to-nearest-even and no contraction (build with -ffp-contract=off), because the
 * GPU kernel takes that decision in fp32.  Integer scores are exact int64.  Everything else (exponentials,
 * the softmax sum and the P*V accumulation) is fp64.
 *
 * Parity pins: every function here is pinned by tests/test_oracle_*.py against closed forms, library
 * routines (torch's bf16 / float8_e4m3fn casts, numpy int64 matmul), invariants and brute force.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_GUARD 0x1p-100f /* an amax below this is treated as an all-zero block or channel */

/* ------------------------------------------------------------------------------------------------ */
/* Number formats                                                                                    */
/* ------------------------------------------------------------------------------------------------ */

/* bfloat16 keeps the top 16 bits of an IEEE fp32; rounding is to nearest, ties to even. */
uint16_t orc_bf16_from_f32(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t lower = u & 0xFFFFu, upper = u >> 16;
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
  return (uint16_t)upper;
}

float orc_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* OCP 8-bit floating point, E4M3FN flavour: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits,
 * no infinities, S.1111.111 is NaN, largest finite magnitude 448, smallest subnormal 2^-9. */
float orc_e4m3_decode(uint8_t c) {
  int sign = c >> 7, e = (c >> 3) & 0xF, m = c & 0x7;
  if (e == 0xF && m == 0x7) return NAN;
  double v = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return (float)(sign ? -v : v);
}

/* Nearest E4M3FN value, ties to the even code (= even mantissa), magnitudes >= 448 saturate to 448
 * ("satfinite"), NaN maps to the NaN code.  Found by bisection over the 127 non-negative finite codes,
 * whose decoded values increase with the code. */
uint8_t orc_e4m3_encode(float x) {
  if (isnan(x)) return 0x7F;
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs((double)x);
  if (a >= 448.0) return sign | 0x7E;
  int lo = 0, hi = 0x7E; /* largest code c with value(c) <= a */
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if ((double)orc_e4m3_decode((uint8_t)mid) <= a) lo = mid; else hi = mid - 1;
  }
  double below = orc_e4m3_decode((uint8_t)lo), above = orc_e4m3_decode((uint8_t)(lo + 1));
  int c;
  if (a - below < above - a) c = lo;
  else if (a - below > above - a) c = lo + 1;
  else c = (lo & 1) ? lo + 1 : lo;
  return sign | (uint8_t)c;
}

/* ------------------------------------------------------------------------------------------------ */
/* Step 1: per-channel mean of K over the tokens (the smoothing vector).                             */
/* Order is fixed so the result is one exact fp32 number: within each run of 64 consecutive tokens   */
/* the values are added one after another in token order; the run sums are then added one after     */
/* another in run order; the total is divided by the token count (IEEE division).                    */
/* k: bf16 [n, d] with row stride ld (elements).  mu: [d].                                           */
/* ------------------------------------------------------------------------------------------------ */
void orc_k_mean(const uint16_t* k, int n, int d, long long ld, float* mu) {
  for (int c = 0; c < d; ++c) {
    float total = 0.0f;
    for (int t0 = 0; t0 < n; t0 += 64) {
      int t1 = t0 + 64 < n ? t0 + 64 : n;
      float run = 0.0f;
      for (int t = t0; t < t1; ++t) run = run + orc_bf16_to_f32(k[(long long)t * ld + c]);
      total = total + run;
    }
    mu[c] = total / (float)n;
  }
}

/* ------------------------------------------------------------------------------------------------ */
/* Steps 3/4: symmetric INT8 quantization of one block of rows (all d channels).                     */
/* a = max |x|; a < 2^-100 -> scale 0 and all codes 0 (the zero-channel/zero-block guard);           */
/* otherwise inv = 127/a, scale = a/127, code = clamp(rint(x*inv), -127, 127), rint ties to even.    */
/* x: fp32 [rows, d] dense.  codes: [rows, d].                                                        */
/* ------------------------------------------------------------------------------------------------ */
void orc_quant_i8_rows(const float* x, int rows, int d, int8_t* codes, float* scale) {
  float a = 0.0f;
  for (long long i = 0; i < (long long)rows * d; ++i) {
    float v = fabsf(x[i]);
    if (v > a) a = v;
  }
  if (!(a >= ORC_GUARD)) {
    *scale = 0.0f;
    memset(codes, 0, (size_t)rows * d);
    return;
  }
  float inv = 127.0f / a;
  *scale = a / 127.0f;
  for (long long i = 0; i < (long long)rows * d; ++i) {
    float q = rintf(x[i] * inv);
    if (q > 127.0f) q = 127.0f;
    if (q < -127.0f) q = -127.0f;
    codes[i] = (int8_t)q;
  }
}

/* Q quantization: blocks of blk consecutive rows; the last block holds the remaining rows.
 * q: bf16 [n, d] (row stride ld).  codes: [nblk*blk, d] (pad rows are 0).  scales: [nblk]. */
void orc_quant_q(const uint16_t* q, int n, int d, long long ld, int blk, int8_t* codes, float* scales) {
  int nblk = (n + blk - 1) / blk;
  float* x = (float*)malloc(sizeof(float) * (size_t)blk * d);
  memset(codes, 0, (size_t)nblk * blk * d);
  for (int b = 0; b < nblk; ++b) {
    int r0 = b * blk, rows = (n - r0) < blk ? (n - r0) : blk;
    for (int r = 0; r < rows; ++r)
      for (int c = 0; c < d; ++c) x[(long long)r * d + c] = orc_bf16_to_f32(q[(long long)(r0 + r) * ld + c]);
    orc_quant_i8_rows(x, rows, d, codes + (long long)r0 * d, &scales[b]);
  }
  free(x);
}

/* Step 2 + step 4: smoothed K' = float(K) - mu (fp32, not re-rounded), then block quantization. */
void orc_quant_k(const uint16_t* k, int n, int d, long long ld, const float* mu, int blk, int8_t* codes,
                 float* scales) {
  int nblk = (n + blk - 1) / blk;
  float* x = (float*)malloc(sizeof(float) * (size_t)blk * d);
  memset(codes, 0, (size_t)nblk * blk * d);
  for (int b = 0; b < nblk; ++b) {
    int r0 = b * blk, rows = (n - r0) < blk ? (n - r0) : blk;
    for (int r = 0; r < rows; ++r)
      for (int c = 0; c < d; ++c)
        x[(long long)r * d + c] = orc_bf16_to_f32(k[(long long)(r0 + r) * ld + c]) - mu[c];
    orc_quant_i8_rows(x, rows, d, codes + (long long)r0 * d, &scales[b]);
  }
  free(x);
}

/* Step 5 (8-bit P*V mode only): per-channel E4M3 quantization of V.
 * a_c = max over tokens |V[:,c]|; guard as above; inv = 448/a_c, scale = a_c/448,
 * code = e4m3(V*inv).  v: bf16 [n, d] (row stride ld).  codes: [n, d] natural layout.  scales: [d]. */
void orc_quant_v(const uint16_t* v, int n, int d, long long ld, uint8_t* codes, float* scales) {
  for (int c = 0; c < d; ++c) {
    float a = 0.0f;
    for (int t = 0; t < n; ++t) {
      float x = fabsf(orc_bf16_to_f32(v[(long long)t * ld + c]));
      if (x > a) a = x;
    }
    if (!(a >= ORC_GUARD)) {
      scales[c] = 0.0f;
      for (int t = 0; t < n; ++t) codes[(long long)t * d + c] = 0;
      continue;
    }
    float inv = 448.0f / a;
    scales[c] = a / 448.0f;
    for (int t = 0; t < n; ++t) codes[(long long)t * d + c] = orc_e4m3_encode(orc_bf16_to_f32(v[(long long)t * ld + c]) * inv);
  }
}

/* ------------------------------------------------------------------------------------------------ */
/* Step 6: integer scores S[r, j] = sum_c qc[r, c] * kc[j, c], exact in int64.                        */
/* ------------------------------------------------------------------------------------------------ */
void orc_qk_int(const int8_t* qc, int nq, const int8_t* kc, int nk, int d, int64_t* s) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < nq; ++r)
    for (int j = 0; j < nk; ++j) {
      int64_t acc = 0;
      for (int c = 0; c < d; ++c) acc += (int64_t)qc[(long long)r * d + c] * (int64_t)kc[(long long)j * d + c];
      s[(long long)r * nk + j] = acc;
    }
}

/* ------------------------------------------------------------------------------------------------ */
/* Steps 7-9: the quantized attention, replayed step by step with the online softmax over key tiles  */
/* of width `tile` (ascending).  Modes:                                                              */
/*   0  bf16 exact: x = fp32(sum_c q*k in fp64) * (c*log2 e); P rounded to bf16; V is bf16.          */
/*   1  INT8 QK^T + bf16 PV: x = fp32(S_int) * ((s_q*s_k)*(c*log2 e)); P rounded to bf16; V bf16.    */
/*   2  INT8 QK^T + FP8 PV: as 1, but P^ = e4m3(p*448) and V^ = the V codes; the epilogue multiplies */
/*      by s_v[c]/448.                                                                               */
/* For each tile: m' = max(m, max x); alpha = 2^(m - m') (0 for the first tile); p = 2^(x - m')       */
/* (fp64, stored as fp32); l = alpha*l + sum p (unquantized p); acc = alpha*acc + sum P^*V^; m = m'.  */
/* Output O = acc / l (mode 2: acc * s_v[c] / (448*l)), rounded to fp32 and then to bf16.             */
/*                                                                                                   */
/* Row r uses Q block r/blk_q; key j uses K block j/blk_k.  Only `rows` (nrows indices) are computed. */
/* All matrices dense row-major: q_bf16/k_bf16/v_bf16 [n, d] bf16; q_codes [.., d]; k_codes [.., d];  */
/* v_codes [nkv, d].  out: bf16 [nrows, d]; out_f32 (may be NULL): [nrows, d] fp32 before rounding.   */
/*                                                                                                   */
/* Block-sparse variant (page "视频生成模型的高效推理加速机制解析", section "核心组成与关键能力", item 3, and */
/* step 3 of "工作原理与执行流程": the attention layer computes only the regions its sparse mask selects):  */
/* keep, when not NULL, is a [ceil(rows/mask_qblk), nkb] byte mask over query blocks of mask_qblk rows and */
/* key blocks of ORC_MASK_KBLK keys (nkb = ceil(nkv / ORC_MASK_KBLK)); key j counts for row r only if     */
/* keep[(r / mask_qblk) * nkb + j / ORC_MASK_KBLK] != 0.  Keys that do not count are left out of every    */
/* step (the running max, l and acc); a tile without such keys changes nothing; a row with none gets 0.  */
/* ------------------------------------------------------------------------------------------------ */
#define ORC_MASK_KBLK 64
void orc_attn_emulate_masked(int mode, int nkv, int d, int blk_q, int blk_k, int tile, float sm_scale,
                             const uint16_t* q_bf16, const uint16_t* k_bf16, const int8_t* q_codes,
                             const float* q_scales, const int8_t* k_codes, const float* k_scales,
                             const uint16_t* v_bf16, const uint8_t* v_codes, const float* v_scales,
                             const int* rows, int nrows, const uint8_t* keep, int mask_qblk, uint16_t* out,
                             float* out_f32) {
  const int nkb = (nkv + ORC_MASK_KBLK - 1) / ORC_MASK_KBLK;
  const float clog2e = sm_scale * 1.4426950408889634f; /* c * log2(e) in fp32 */
  /* V^ as numbers: the bf16 values (modes 0/1) or the decoded E4M3 codes (mode 2) */
  float* vhat = (float*)malloc(sizeof(float) * (size_t)nkv * d);
  for (long long i = 0; i < (long long)nkv * d; ++i)
    vhat[i] = (mode == 2) ? orc_e4m3_decode(v_codes[i]) : orc_bf16_to_f32(v_bf16[i]);
  /* mode 0 reads the keys as numbers */
  float* kf = NULL;
  if (mode == 0) {
    kf = (float*)malloc(sizeof(float) * (size_t)nkv * d);
    for (long long i = 0; i < (long long)nkv * d; ++i) kf[i] = orc_bf16_to_f32(k_bf16[i]);
  }
#pragma omp parallel
  {
    float* x = (float*)malloc(sizeof(float) * (size_t)tile);
    double* acc = (double*)malloc(sizeof(double) * (size_t)d);
    float* qrow = (float*)malloc(sizeof(float) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
    for (int ri = 0; ri < nrows; ++ri) {
      const int r = rows[ri];
      if (mode == 0)
        for (int c = 0; c < d; ++c) qrow[c] = orc_bf16_to_f32(q_bf16[(long long)r * d + c]);
      float m = -INFINITY;
      double l = 0.0;
      for (int c = 0; c < d; ++c) acc[c] = 0.0;
      const uint8_t* keep_row = keep ? keep + (long long)(r / mask_qblk) * nkb : NULL;
      for (int j0 = 0; j0 < nkv; j0 += tile) {
        const int j1 = (j0 + tile) < nkv ? (j0 + tile) : nkv;
        /* step 7: dequantized, pre-scaled logits of this tile (keys left out by the mask: x = -inf) */
        float tmax = -INFINITY;
        for (int j = j0; j < j1; ++j) {
          if (keep_row && !keep_row[j / ORC_MASK_KBLK]) {
            x[j - j0] = -INFINITY;
            continue;
          }
          float xv;
          if (mode == 0) {
            double s = 0.0;
            for (int c = 0; c < d; ++c) s += (double)qrow[c] * (double)kf[(long long)j * d + c];
            xv = (float)s * clog2e;
          } else {
            int64_t s = 0;
            for (int c = 0; c < d; ++c) s += (int64_t)q_codes[(long long)r * d + c] * (int64_t)k_codes[(long long)j * d + c];
            const float f = (q_scales[r / blk_q] * k_scales[j / blk_k]) * clog2e;
            xv = (float)s * f;
          }
          x[j - j0] = xv;
          if (xv > tmax) tmax = xv;
        }
        if (tmax == -INFINITY) continue; /* no key of this tile counts for this row */
        /* step 8: online softmax update */
        const float mnew = tmax > m ? tmax : m;
        const double alpha = (m == -INFINITY) ? 0.0 : (double)(float)exp2((double)m - (double)mnew);
        double psum = 0.0;
        for (int c = 0; c < d; ++c) acc[c] *= alpha;
        for (int j = j0; j < j1; ++j) {
          if (x[j - j0] == -INFINITY) continue;
          const float p = (float)exp2((double)x[j - j0] - (double)mnew);
          psum += (double)p;
          const double ph = (mode == 2) ? (double)orc_e4m3_decode(orc_e4m3_encode(p * 448.0f))
                                        : (double)orc_bf16_to_f32(orc_bf16_from_f32(p));
          const float* vj = vhat + (long long)j * d;
          for (int c = 0; c < d; ++c) acc[c] += ph * (double)vj[c];
        }
        l = alpha * l + psum;
        m = mnew;
      }
      /* step 9: epilogue (a row whose mask keeps no key: O = 0) */
      for (int c = 0; c < d; ++c) {
        double o = (l == 0.0) ? 0.0 : (mode == 2) ? acc[c] * (double)v_scales[c] / (448.0 * l) : acc[c] / l;
        float of = (float)o;
        if (out_f32) out_f32[(long long)ri * d + c] = of;
        out[(long long)ri * d + c] = orc_bf16_from_f32(of);
      }
    }
    free(x);
    free(acc);
    free(qrow);
  }
  free(vhat);
  free(kf);
}

void orc_attn_emulate(int mode, int nkv, int d, int blk_q, int blk_k, int tile, float sm_scale,
                      const uint16_t* q_bf16, const uint16_t* k_bf16, const int8_t* q_codes,
                      const float* q_scales, const int8_t* k_codes, const float* k_scales,
                      const uint16_t* v_bf16, const uint8_t* v_codes, const float* v_scales,
                      const int* rows, int nrows, uint16_t* out, float* out_f32) {
  orc_attn_emulate_masked(mode, nkv, d, blk_q, blk_k, tile, sm_scale, q_bf16, k_bf16, q_codes, q_scales, k_codes,
                          k_scales, v_bf16, v_codes, v_scales, rows, nrows, NULL, 1, out, out_f32);
}

/* ------------------------------------------------------------------------------------------------ */
/* Exact attention in fp64 from the bf16 inputs: O = softmax(c * q * K^T) * V, the operator that the  */
/* quantized modes approximate.  out: fp64 [nrows, d].  With keep (as in orc_attn_emulate_masked),    */
/* the softmax runs over the keys the mask keeps for the row; a row with none gets 0.                 */
/* ------------------------------------------------------------------------------------------------ */
void orc_attn_ref_fp64_masked(int nkv, int d, double sm_scale, const uint16_t* q_bf16, const uint16_t* k_bf16,
                              const uint16_t* v_bf16, const int* rows, int nrows, const uint8_t* keep,
                              int mask_qblk, double* out) {
  const int nkb = (nkv + ORC_MASK_KBLK - 1) / ORC_MASK_KBLK;
  double* kd = (double*)malloc(sizeof(double) * (size_t)nkv * d);
  double* vd = (double*)malloc(sizeof(double) * (size_t)nkv * d);
  for (long long i = 0; i < (long long)nkv * d; ++i) {
    kd[i] = orc_bf16_to_f32(k_bf16[i]);
    vd[i] = orc_bf16_to_f32(v_bf16[i]);
  }
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)nkv);
    double* qd = (double*)malloc(sizeof(double) * (size_t)d);
    double* num = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
    for (int ri = 0; ri < nrows; ++ri) {
      const int r = rows[ri];
      for (int c = 0; c < d; ++c) qd[c] = orc_bf16_to_f32(q_bf16[(long long)r * d + c]);
      const uint8_t* keep_row = keep ? keep + (long long)(r / mask_qblk) * nkb : NULL;
      double mx = -INFINITY;
      for (int j = 0; j < nkv; ++j) {
        if (keep_row && !keep_row[j / ORC_MASK_KBLK]) {
          s[j] = -INFINITY;
          continue;
        }
        double dot = 0.0;
        for (int c = 0; c < d; ++c) dot += qd[c] * kd[(long long)j * d + c];
        s[j] = sm_scale * dot;
        if (s[j] > mx) mx = s[j];
      }
      double den = 0.0;
      for (int c = 0; c < d; ++c) num[c] = 0.0;
      for (int j = 0; j < nkv; ++j) {
        if (s[j] == -INFINITY) continue;
        const double w = exp(s[j] - mx);
        den += w;
        for (int c = 0; c < d; ++c) num[c] += w * vd[(long long)j * d + c];
      }
      for (int c = 0; c < d; ++c) out[(long long)ri * d + c] = (den == 0.0) ? 0.0 : num[c] / den;
    }
    free(s);
    free(qd);
    free(num);
  }
  free(kd);
  free(vd);
}

void orc_attn_ref_fp64(int nkv, int d, double sm_scale, const uint16_t* q_bf16, const uint16_t* k_bf16,
                       const uint16_t* v_bf16, const int* rows, int nrows, double* out) {
  orc_attn_ref_fp64_masked(nkv, d, sm_scale, q_bf16, k_bf16, v_bf16, rows, nrows, NULL, 1, out);
}

int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

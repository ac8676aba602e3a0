/* The CPU oracle (oracle/sattn_oracle.c, oracle/linear_oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer: every function runs on small inputs whose buffers are allocated at exactly the size the
 * function's contract names (ragged blocks and tiles, all three modes, masks with empty rows, zero blocks), so any
 * read or write outside them, and any undefined arithmetic, aborts the program.  A few invariants are checked on the
 * way (finite outputs, codes in range).  Exits 0 when all hold. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

uint16_t orc_bf16_from_f32(float x);
float orc_bf16_to_f32(uint16_t h);
float orc_e4m3_decode(uint8_t c);
uint8_t orc_e4m3_encode(float x);
void orc_k_mean(const uint16_t* k, int n, int d, long long ld, float* mu);
void orc_quant_q(const uint16_t* q, int n, int d, long long ld, int blk, int8_t* codes, float* scales);
void orc_quant_k(const uint16_t* k, int n, int d, long long ld, const float* mu, int blk, int8_t* codes,
                 float* scales);
void orc_quant_v(const uint16_t* v, int n, int d, long long ld, uint8_t* codes, float* scales);
void orc_qk_int(const int8_t* qc, int nq, const int8_t* kc, int nk, int d, int64_t* s);
void orc_attn_emulate_masked(int mode, int nkv, int d, int blk_q, int blk_k, int tile, float sm_scale,
                             const uint16_t* q_bf16, const uint16_t* k_bf16, const int8_t* q_codes,
                             const float* q_scales, const int8_t* k_codes, const float* k_scales,
                             const uint16_t* v_bf16, const uint8_t* v_codes, const float* v_scales, const int* rows,
                             int nrows, const uint8_t* keep, int mask_qblk, uint16_t* out, float* out_f32);
void orc_attn_ref_fp64_masked(int nkv, int d, double sm_scale, const uint16_t* q_bf16, const uint16_t* k_bf16,
                              const uint16_t* v_bf16, const int* rows, int nrows, const uint8_t* keep,
                              int mask_qblk, double* out);
void orc_quant_blocks(const uint16_t* x, int rows, int cols, long long ld, int br, int bc, int8_t* codes,
                      float* scales);
void orc_linear_w8a8(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw, const uint16_t* bias,
                     int M, int N, int K, int blk, double* out, double* mag);
void orc_linear_w8a16(const uint16_t* x, const int8_t* wq, const float* sw, const uint16_t* bias, int M, int N,
                      int K, int blk, double* out, double* mag);

static int failures = 0;
#define EXPECT(c)                                                   \
  do {                                                              \
    if (!(c)) {                                                     \
      fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #c);        \
      ++failures;                                                   \
    }                                                               \
  } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double uniform(void) { /* xorshift64*, in [0, 1) */
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return (double)((rng * 0x2545F4914F6CDD1Dull) >> 11) * 0x1p-53;
}
static uint16_t* bf16_array(long long n, double scale, double offset) {
  uint16_t* a = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)n);
  for (long long i = 0; i < n; ++i) a[i] = orc_bf16_from_f32((float)(offset + scale * (2.0 * uniform() - 1.0)));
  return a;
}
static int cdiv(int a, int b) { return (a + b - 1) / b; }

static void check_codecs(void) {
  for (int c = 0; c < 256; ++c) {
    const float v = orc_e4m3_decode((uint8_t)c);
    if ((c & 0x7F) != 0x7F) EXPECT(orc_e4m3_encode(v) == (uint8_t)c || v == 0.0f);
  }
  for (int i = 0; i < 65536; ++i) {
    const float f = orc_bf16_to_f32((uint16_t)i);
    if (!isnan(f)) EXPECT(orc_bf16_from_f32(f) == (uint16_t)i);
  }
}

static void check_attention(int n_q, int n_kv, int d, int blk_q, int tile) {
  const int blk_k = 64, nqb = cdiv(n_q, blk_q), nkb = cdiv(n_kv, blk_k);
  uint16_t* q = bf16_array((long long)n_q * d, 1.0, 0.0);
  uint16_t* k = bf16_array((long long)n_kv * d, 1.0, 0.5);
  uint16_t* v = bf16_array((long long)n_kv * d, 1.0, 0.0);
  for (int c = 0; c < d && n_kv > 64; ++c) k[64 * d + c] = 0; /* part of a zero key block */
  float* mu = (float*)malloc(sizeof(float) * d);
  int8_t* qc = (int8_t*)malloc((size_t)nqb * blk_q * d); /* padded to whole blocks, as the contract says */
  float* qs = (float*)malloc(sizeof(float) * nqb);
  int8_t* kc = (int8_t*)malloc((size_t)nkb * blk_k * d);
  float* ks = (float*)malloc(sizeof(float) * nkb);
  uint8_t* vc = (uint8_t*)malloc((size_t)n_kv * d);
  float* vs = (float*)malloc(sizeof(float) * d);
  orc_k_mean(k, n_kv, d, d, mu);
  orc_quant_q(q, n_q, d, d, blk_q, qc, qs);
  orc_quant_k(k, n_kv, d, d, mu, blk_k, kc, ks);
  orc_quant_v(v, n_kv, d, d, vc, vs);
  for (long long i = 0; i < (long long)nqb * blk_q * d; ++i) EXPECT(qc[i] >= -127 && (i < (long long)n_q * d || !qc[i]));
  int64_t* s = (int64_t*)malloc(sizeof(int64_t) * (size_t)n_q * n_kv);
  orc_qk_int(qc, n_q, kc, n_kv, d, s);
  int* rows = (int*)malloc(sizeof(int) * n_q);
  for (int r = 0; r < n_q; ++r) rows[r] = r;
  /* mask over (128-row, 64-key) blocks: random, with the first query block left empty */
  const int mq = 128, nmq = cdiv(n_q, mq);
  uint8_t* keep = (uint8_t*)malloc((size_t)nmq * nkb);
  for (int i = 0; i < nmq * nkb; ++i) keep[i] = (i >= nkb) && uniform() < 0.6;
  uint16_t* out = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)n_q * d);
  float* out_f = (float*)malloc(sizeof(float) * (size_t)n_q * d);
  double* ref = (double*)malloc(sizeof(double) * (size_t)n_q * d);
  for (int masked = 0; masked < 2; ++masked) {
    for (int mode = 0; mode < 3; ++mode) {
      orc_attn_emulate_masked(mode, n_kv, d, blk_q, blk_k, tile, 1.0f / sqrtf((float)d), q, k, qc, qs, kc, ks, v, vc,
                              vs, rows, n_q, masked ? keep : NULL, mq, out, out_f);
      for (long long i = 0; i < (long long)n_q * d; ++i) EXPECT(isfinite(out_f[i]));
    }
    orc_attn_ref_fp64_masked(n_kv, d, 1.0 / sqrt((double)d), q, k, v, rows, n_q, masked ? keep : NULL, mq, ref);
    for (long long i = 0; i < (long long)n_q * d; ++i) EXPECT(isfinite(ref[i]));
  }
  free(q); free(k); free(v); free(mu); free(qc); free(qs); free(kc); free(ks); free(vc); free(vs); free(s);
  free(rows); free(keep); free(out); free(out_f); free(ref);
}

static void check_linear(int M, int N, int K) {
  const int blk = 128, mb = cdiv(M, blk), nb = cdiv(N, blk), kb = K / blk;
  uint16_t* x = bf16_array((long long)M * K, 3.0, 0.0);
  uint16_t* w = bf16_array((long long)N * K, 0.1, 0.0);
  uint16_t* b = bf16_array(N, 0.02, 0.0);
  int8_t* xq = (int8_t*)malloc((size_t)M * K);
  float* sx = (float*)malloc(sizeof(float) * mb * kb);
  int8_t* wq = (int8_t*)malloc((size_t)N * K);
  float* sw = (float*)malloc(sizeof(float) * nb * kb);
  double* y = (double*)malloc(sizeof(double) * (size_t)M * N);
  double* mag = (double*)malloc(sizeof(double) * (size_t)M * N);
  orc_quant_blocks(x, M, K, K, blk, blk, xq, sx);
  orc_quant_blocks(w, N, K, K, blk, blk, wq, sw);
  orc_linear_w8a8(xq, sx, wq, sw, b, M, N, K, blk, y, mag);
  for (long long i = 0; i < (long long)M * N; ++i) EXPECT(isfinite(y[i]) && mag[i] >= 0.0);
  orc_linear_w8a16(x, wq, sw, NULL, M, N, K, blk, y, mag);
  for (long long i = 0; i < (long long)M * N; ++i) EXPECT(isfinite(y[i]));
  free(x); free(w); free(b); free(xq); free(sx); free(wq); free(sw); free(y); free(mag);
}

int main(void) {
  check_codecs();
  check_attention(1, 1, 64, 64, 64);
  check_attention(65, 63, 64, 64, 7);
  check_attention(200, 197, 128, 128, 64);
  check_attention(300, 130, 64, 64, 32);
  check_linear(1, 8, 128);
  check_linear(130, 136, 384);
  if (failures) return 1;
  printf("oracle host checks: ok\n");
  return 0;
}

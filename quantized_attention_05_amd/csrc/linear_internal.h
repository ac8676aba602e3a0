// Internal interface between the C ABI (api.cpp) and the quantized linear-layer kernels (linear.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace sattn {

constexpr int kLinBlk = 128;  // edge of the square quantization blocks of activations and weights

// y[M, N] = x[M, K] W[N, K]^T + bias, on quantized operands.
//   W8A8 : a = activation codes (int8, row stride lda bytes), sx its block scales [ceil(M/128), K/128];
//   W8A16: a = activations (bf16, row stride lda bytes), sx unused.
//   b = weight codes, int8 (W8A8) or the same codes stored as bf16 (W8A16), row stride ldb bytes;
//   sw = weight block scales [ceil(N/128), K/128].
struct LinearArg {
  const uint8_t* a;
  int64_t lda;
  const uint8_t* b;
  int64_t ldb;
  const float* sx;
  const float* sw;
  const uint16_t* bias;  // bf16 [N] or null
  uint16_t* y;           // bf16, row stride ldy elements
  int64_t ldy;
  int M, N, K;
};

hipError_t launch_quant_blocks(const uint16_t* x, int rows, int cols, int64_t ld, int8_t* codes, float* scales,
                               hipStream_t s);
hipError_t launch_codes_to_bf16(const int8_t* codes, uint16_t* out, int64_t n, hipStream_t s);
hipError_t launch_linear(bool w8a8, const LinearArg& p, hipStream_t s);
// Per-call set-up of the GEMM kernels a call may launch (their dynamic LDS limit); enqueues nothing.
hipError_t prepare_linear(bool w8a8);

}  // namespace sattn

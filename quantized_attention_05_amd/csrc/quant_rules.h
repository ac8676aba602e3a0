// Device-side rules of the per-block INT8 code shared by the quantization pass (quant.hip) and the attention kernel
// that quantizes its own Q block (attn.hip), so that both produce the same codes bit for bit: fp32, round to nearest
// even, no contraction (a multiply followed by a rounding, nothing to fuse).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sattn {

__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// 8 bf16 values (16 bytes) -> 8 floats
__device__ __forceinline__ void unpack8(const uint4& u, float* f) {
  f[0] = bf2f(u.x & 0xFFFFu); f[1] = bf2f(u.x >> 16);
  f[2] = bf2f(u.y & 0xFFFFu); f[3] = bf2f(u.y >> 16);
  f[4] = bf2f(u.z & 0xFFFFu); f[5] = bf2f(u.z >> 16);
  f[6] = bf2f(u.w & 0xFFFFu); f[7] = bf2f(u.w >> 16);
}

// code = clamp(rint(x * (127 / amax)), -127, 127), with inv = 127 / amax computed once per block
__device__ __forceinline__ int8_t code_i8(float x, float inv) {
  float q = rintf(x * inv);
  q = fminf(fmaxf(q, -127.0f), 127.0f);
  return (int8_t)(int)q;
}

}  // namespace sattn

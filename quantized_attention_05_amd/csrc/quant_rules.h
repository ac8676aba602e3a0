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

// The codes of four values of one block, packed into a word (the first value in the lowest byte):
// code = clamp(rint(x * inv), -127, 127) with inv = 127 / amax computed once per block (0 for an all-zero block).
// The clamp never acts: |x| <= amax and inv = fl(127 / amax) keep fl(x * inv) within 127 (1 + 2^-24)^2 < 127.5.
// Adding 1.5 * 2^23 to fl(x * inv) rounds it to an integer, ties to even (the sum's spacing is 1 and 1.5 * 2^23 is
// even), and leaves that integer in two's complement in the low byte of the sum's bits.  The multiply and the add
// round separately (no fused multiply-add), as rint(fl(x * inv)) does.
__device__ __forceinline__ uint32_t codes4(const float* x, float inv) {
#pragma clang fp contract(off)
  uint32_t b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float y = x[i] * inv;
    b[i] = __float_as_uint(y + 12582912.0f);
  }
  return (b[0] & 0xFFu) | ((b[1] & 0xFFu) << 8) | ((b[2] & 0xFFu) << 16) | (b[3] << 24);
}

}  // namespace sattn

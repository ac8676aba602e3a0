// Quantization pass of libsattn (HBM-bound): Q per-block INT8, K smoothing + per-block INT8, V per-channel
// E4M3 (or the bf16 V transpose that the bf16 P*V path reads).
//
// Every decision that produces a code is taken in IEEE fp32, round-to-nearest-even, without contraction,
// so the codes and scales are bit-identical to a plain sequential CPU evaluation of the same formulas:
//   K mean: 64-token runs summed in token order, run sums added in run order, one division by Nkv.
//   block quant: a = max|x|; a < 2^-100 -> scale 0, codes 0 (the zero-channel guard whose absence turned
//   whole videos black, TMAP I2V write-up, section "优化算子细节"); else scale = a/127 and
//   code = clamp(rint(x * (127/a)), -127, 127).
//   V: per-channel a_c over all tokens; scale = a_c/448, code = E4M3(v * (448/a_c)), RNE, saturating.
#pragma clang fp contract(off)

#include "quant_rules.h"
#include "sattn_internal.h"

namespace sattn {
namespace {

// max over the 256 threads of a block (4 waves of 64)
__device__ __forceinline__ float block_max256(float v, float* red) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return v;
}

// ---------------------------------------------------------------------------------------------- Q blocks
// grid (nqb, H, B), 256 threads; thread owns 8 consecutive channels of rows r = tid / TPR + pass * RPP.
template <int D, int BQ>
__global__ void __launch_bounds__(256) quant_q_kernel(TensorArg q, QuantArg qa) {
  constexpr int TPR = D / 8;          // threads per row
  constexpr int RPP = 256 / TPR;      // rows per pass
  constexpr int PASSES = BQ / RPP;
  __shared__ float red[4];
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int r0 = blk * BQ;
  const int rows = min(BQ, qa.Nq - r0);
  const int c0 = (threadIdx.x % TPR) * 8;
  const int rr = threadIdx.x / TPR;
  const uint16_t* src = q.ptr + b * q.sb + h * q.sh;
  float x[PASSES][8];
  float a = 0.0f;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int r = rr + p * RPP;
    if (r < rows) {
      const uint4 u = *reinterpret_cast<const uint4*>(src + (int64_t)(r0 + r) * q.sn + c0);
      unpack8(u, x[p]);
#pragma unroll
      for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(x[p][i]));
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[p][i] = 0.0f;
    }
  }
  a = block_max256(a, red);
  const bool zero = !(a >= kGuard);
  const float inv = zero ? 0.0f : 127.0f / a;
  int8_t* dst = qa.q_codes + (((int64_t)b * qa.H + h) * qa.nqb * BQ + r0) * D;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int r = rr + p * RPP;
    uint32_t lo = 0, hi = 0;
    if (!zero && r < rows) {
      lo = codes4(x[p], inv);
      hi = codes4(x[p] + 4, inv);
    }
    *reinterpret_cast<uint2*>(dst + (int64_t)r * D + c0) = make_uint2(lo, hi);
  }
  if (threadIdx.x == 0) qa.q_scales[((int64_t)b * qa.H + h) * qa.nqb + blk] = zero ? 0.0f : a / 127.0f;
}

// ---------------------------------------------------------------------------------------------- K/V stats
// Rows t0 .. t1-1 of 8 bf16 channels folded into acc in row order: fp32 sum, or (MAXABS) max |x|.  The loads of
// kStatBatch rows are issued together, then folded one after another, so the order of the additions is the plain
// sequential one while a thread has many loads in flight (a run is all the parallelism one thread has, and a
// short sequence gives few runs).
constexpr int kStatBatch = 16;
template <bool MAXABS>
__device__ __forceinline__ void run_reduce(const uint16_t* p, int64_t sn, int t0, int t1, float (&acc)[8]) {
  auto fold = [&](const uint4& u) {
    float f[8];
    unpack8(u, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = MAXABS ? fmaxf(acc[i], fabsf(f[i])) : acc[i] + f[i];
  };
  int t = t0;
  for (; t + kStatBatch <= t1; t += kStatBatch) {
    uint4 u[kStatBatch];
#pragma unroll
    for (int j = 0; j < kStatBatch; ++j) u[j] = *reinterpret_cast<const uint4*>(p + (int64_t)(t + j) * sn);
#pragma unroll
    for (int j = 0; j < kStatBatch; ++j) fold(u[j]);
  }
  for (; t < t1; ++t) fold(*reinterpret_cast<const uint4*>(p + (int64_t)t * sn));
}

// Per 64-token run and channel: sequential fp32 sum of K, and max |V| (mode 2).  Thread owns 8 channels of
// one run; grid (ceil(nkb / RUNS), H, B) with RUNS runs per 256-thread block.
template <int D>
__global__ void __launch_bounds__(256) kv_stats_kernel(TensorArg k, TensorArg v, bool with_v, QuantArg qa, float* ksum,
                                                       float* vmax) {
  constexpr int TPR = D / 8;
  constexpr int RUNS = 256 / TPR;
  const int h = blockIdx.y, b = blockIdx.z;
  const int run = blockIdx.x * RUNS + threadIdx.x / TPR;
  if (run >= qa.nkb) return;
  const int c0 = (threadIdx.x % TPR) * 8;
  const int t0 = run * kChunk;
  const int t1 = min(t0 + kChunk, qa.Nkv);
  const uint16_t* ks = k.ptr + b * k.sb + h * k.sh + c0;
  float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  run_reduce<false>(ks, k.sn, t0, t1, s);
  const int64_t o = (((int64_t)b * qa.H + h) * qa.nkb + run) * D + c0;
  *reinterpret_cast<float4*>(ksum + o) = make_float4(s[0], s[1], s[2], s[3]);
  *reinterpret_cast<float4*>(ksum + o + 4) = make_float4(s[4], s[5], s[6], s[7]);
  if (with_v) {
    const uint16_t* vs = v.ptr + b * v.sb + h * v.sh + c0;
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    run_reduce<true>(vs, v.sn, t0, t1, m);
    *reinterpret_cast<float4*>(vmax + o) = make_float4(m[0], m[1], m[2], m[3]);
    *reinterpret_cast<float4*>(vmax + o + 4) = make_float4(m[4], m[5], m[6], m[7]);
  }
}

// Threads [0, B*H*d): one per (b, h, c), run sums added in run order -> K mean.  Threads [B*H*d, 2*B*H*d) (with V):
// one per (b, h, c), V maxima -> scale and reciprocal.  Both are bound by the latency of their loads, so 64 are
// issued together; the K additions stay one after another in run order.
__global__ void __launch_bounds__(128) kv_finalize_kernel(QuantArg qa, bool with_v, const float* ksum, const float* vmax,
                                                          float* vinv) {
  constexpr int kBatch = 64;
  const int d = qa.d;
  const int64_t n = (int64_t)qa.B * qa.H * d;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool vpart = i >= n;
  if (vpart) i -= n;
  if (i >= n || (vpart && !with_v)) return;
  const int64_t bh = i / d;
  const int c = (int)(i % d);
  int r = 0;
  if (!vpart) {
    const float* ps = ksum + bh * qa.nkb * d + c;
    float total = 0.0f;
    for (; r + kBatch <= qa.nkb; r += kBatch) {
      float x[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) x[u] = ps[(int64_t)(r + u) * d];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) total = total + x[u];
    }
    for (; r < qa.nkb; ++r) total = total + ps[(int64_t)r * d];
    qa.k_mean[i] = total / (float)qa.Nkv;
  } else {
    const float* pm = vmax + bh * qa.nkb * d + c;
    float a = 0.0f;
    for (; r + kBatch <= qa.nkb; r += kBatch) {
      float x[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) x[u] = pm[(int64_t)(r + u) * d];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) a = fmaxf(a, x[u]);
    }
    for (; r < qa.nkb; ++r) a = fmaxf(a, pm[(int64_t)r * d]);
    const bool zero = !(a >= kGuard);
    qa.v_scales[i] = zero ? 0.0f : a / 448.0f;
    vinv[i] = zero ? 0.0f : 448.0f / a;
  }
}

// ---------------------------------------------------------------------------------------------- K'/V blocks
// grid (nkb, H, B), 256 threads.  K' = K - mean, per-block INT8 (modes 1, 2).  V: E4M3 codes (mode 2) or
// bf16 (modes 0, 1) written transposed per 64-key tile ([d][64], keys contiguous) through LDS.
template <int D, int MODE>
__global__ void __launch_bounds__(256) kv_quant_kernel(TensorArg k, TensorArg v, QuantArg qa, const float* vinv) {
  constexpr int TPR = D / 8;
  constexpr int RPP = 256 / TPR;
  constexpr int PASSES = kTile / RPP;
  constexpr int VB = (MODE == 2) ? 1 : 2;          // bytes per transposed V element
  constexpr int LROW = kTile * VB + 16;            // padded LDS row (one channel)
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) uint8_t vt[D * LROW];
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t0 = blk * kTile;
  const int rows = min(kTile, qa.Nkv - t0);
  const int c0 = (threadIdx.x % TPR) * 8;
  const int rr = threadIdx.x / TPR;
  const int64_t bh = (int64_t)b * qa.H + h;

  if (MODE != 0) {
    const uint16_t* src = k.ptr + b * k.sb + h * k.sh;
    float mu[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) mu[i] = qa.k_mean[bh * D + c0 + i];
    float x[PASSES][8];
    float a = 0.0f;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int r = rr + p * RPP;
      if (r < rows) {
        float f[8];
        unpack8(*reinterpret_cast<const uint4*>(src + (int64_t)(t0 + r) * k.sn + c0), f);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          x[p][i] = f[i] - mu[i];
          a = fmaxf(a, fabsf(x[p][i]));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[p][i] = 0.0f;
      }
    }
    a = block_max256(a, red);
    const bool zero = !(a >= kGuard);
    const float inv = zero ? 0.0f : 127.0f / a;
    int8_t* dst = qa.k_codes + (bh * qa.nkb * kTile + t0) * D;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int r = rr + p * RPP;
      uint32_t lo = 0, hi = 0;
      if (!zero && r < rows) {
        lo = codes4(x[p], inv);
        hi = codes4(x[p] + 4, inv);
      }
      *reinterpret_cast<uint2*>(dst + (int64_t)r * D + c0) = make_uint2(lo, hi);
    }
    if (threadIdx.x == 0) qa.k_scales[bh * qa.nkb + blk] = zero ? 0.0f : a / 127.0f;
  }

  // V: load rows, convert, scatter transposed into LDS, then write [D][64] rows to global.
  {
    const uint16_t* src = v.ptr + b * v.sb + h * v.sh;
    float vi[8];
    if (MODE == 2) {
#pragma unroll
      for (int i = 0; i < 8; ++i) vi[i] = vinv[bh * D + c0 + i];
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int r = rr + p * RPP;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (r < rows) u = *reinterpret_cast<const uint4*>(src + (int64_t)(t0 + r) * v.sn + c0);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
      if (MODE == 2) {
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          // a guarded channel (scale 0) gets code 0 even for -0.0 inputs
          const float f0 = vi[i] == 0.0f ? 0.0f : bf2f(w[i / 2] & 0xFFFFu) * vi[i];
          const float f1 = vi[i + 1] == 0.0f ? 0.0f : bf2f(w[i / 2] >> 16) * vi[i + 1];
          const uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
          vt[(c0 + i) * LROW + r] = (uint8_t)(pk & 0xFFu);
          vt[(c0 + i + 1) * LROW + r] = (uint8_t)((pk >> 8) & 0xFFu);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          *reinterpret_cast<uint16_t*>(&vt[(c0 + i) * LROW + 2 * r]) = (uint16_t)(w[i / 2] & 0xFFFFu);
          *reinterpret_cast<uint16_t*>(&vt[(c0 + i + 1) * LROW + 2 * r]) = (uint16_t)(w[i / 2] >> 16);
        }
      }
    }
    __syncthreads();
    // D rows of 64*VB bytes; 16-byte pieces
    constexpr int PIECES = D * kTile * VB / 16;
    constexpr int PPR = kTile * VB / 16;  // pieces per row
    uint8_t* dst = (MODE == 2) ? qa.v_codes : reinterpret_cast<uint8_t*>(qa.v_t);
    dst += ((bh * qa.nkb + blk) * D) * (int64_t)(kTile * VB);
    for (int pc = threadIdx.x; pc < PIECES; pc += 256) {
      const int row = pc / PPR, col = (pc % PPR) * 16;
      *reinterpret_cast<uint4*>(dst + (int64_t)row * kTile * VB + col) = *reinterpret_cast<const uint4*>(&vt[row * LROW + col]);
    }
  }
}

}  // namespace

hipError_t launch_quant_q(const TensorArg& q, const QuantArg& qa, hipStream_t s) {
  dim3 grid(qa.nqb, qa.H, qa.B);
  if (qa.d == 128 && qa.blk_q == 128) quant_q_kernel<128, 128><<<grid, 256, 0, s>>>(q, qa);
  else if (qa.d == 128 && qa.blk_q == 64) quant_q_kernel<128, 64><<<grid, 256, 0, s>>>(q, qa);
  else if (qa.d == 64 && qa.blk_q == 128) quant_q_kernel<64, 128><<<grid, 256, 0, s>>>(q, qa);
  else quant_q_kernel<64, 64><<<grid, 256, 0, s>>>(q, qa);
  return hipGetLastError();
}

hipError_t launch_kv_stats(const TensorArg& k, const TensorArg& v, bool with_v, const QuantArg& qa, float* ksum,
                           float* vmax, hipStream_t s) {
  const int runs = 256 / (qa.d / 8);
  dim3 grid(cdiv(qa.nkb, runs), qa.H, qa.B);
  if (qa.d == 128) kv_stats_kernel<128><<<grid, 256, 0, s>>>(k, v, with_v, qa, ksum, vmax);
  else kv_stats_kernel<64><<<grid, 256, 0, s>>>(k, v, with_v, qa, ksum, vmax);
  return hipGetLastError();
}

hipError_t launch_kv_finalize(const QuantArg& qa, bool with_v, const float* ksum, const float* vmax, float* vinv,
                              hipStream_t s) {
  const int64_t n = (int64_t)qa.B * qa.H * qa.d * (with_v ? 2 : 1);
  kv_finalize_kernel<<<(unsigned)((n + 127) / 128), 128, 0, s>>>(qa, with_v, ksum, vmax, vinv);
  return hipGetLastError();
}

hipError_t launch_kv_quant(const TensorArg& k, const TensorArg& v, int mode, const QuantArg& qa, const float* vinv,
                           hipStream_t s) {
  dim3 grid(qa.nkb, qa.H, qa.B);
  if (qa.d == 128) {
    if (mode == 0) kv_quant_kernel<128, 0><<<grid, 256, 0, s>>>(k, v, qa, vinv);
    else if (mode == 1) kv_quant_kernel<128, 1><<<grid, 256, 0, s>>>(k, v, qa, vinv);
    else kv_quant_kernel<128, 2><<<grid, 256, 0, s>>>(k, v, qa, vinv);
  } else {
    if (mode == 0) kv_quant_kernel<64, 0><<<grid, 256, 0, s>>>(k, v, qa, vinv);
    else if (mode == 1) kv_quant_kernel<64, 1><<<grid, 256, 0, s>>>(k, v, qa, vinv);
    else kv_quant_kernel<64, 2><<<grid, 256, 0, s>>>(k, v, qa, vinv);
  }
  return hipGetLastError();
}

}  // namespace sattn

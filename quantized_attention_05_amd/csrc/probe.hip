// Per-head error statistics of an attention output against a reference output: the attention-error probe
// behind layer-selective quantization (TMAP I2V write-up, section "保持视频质量": the attention error of each layer
// over the denoising iterations decides which layers keep full precision).
//
// Two launches with a fixed summation order, so the result depends on the shape alone:
//   1. stats_partial_kernel: each (batch, head) is cut into G row chunks (G = error_stats_chunks(N), at most 64);
//      one workgroup per chunk sums its rows in fp64 with a fixed thread -> element assignment (per-thread sums,
//      then a fixed tree over the workgroup) and writes 4 partial sums to the caller's workspace;
//   2. stats_final_kernel: one 64-lane workgroup per (batch, head) adds the G partials with a fixed tree.
// The probe reads each output once (2 x 2 bytes per element) and is HBM-bound; G chunks per head spread a 40-head
// 720p output over 2560 workgroups, where one workgroup per head would use 40 of the 256 compute units.
#include "probe_internal.h"

namespace sattn {
namespace {

constexpr int kStatsThreads = 256;
constexpr int kStatsUnroll = 4;  // 16-byte vectors of each operand in flight per thread

__device__ __forceinline__ double bf16_lo(uint32_t w) { return (double)__uint_as_float(w << 16); }
__device__ __forceinline__ double bf16_hi(uint32_t w) { return (double)__uint_as_float(w & 0xffff0000u); }

struct Sums {
  double dd, rr, ar, aa;
};

__device__ __forceinline__ void accumulate(Sums& s, uint4 va, uint4 vr) {
  const uint32_t wa[4] = {va.x, va.y, va.z, va.w}, wr[4] = {vr.x, vr.y, vr.z, vr.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double x = (e & 1) ? bf16_hi(wa[e / 2]) : bf16_lo(wa[e / 2]);
    const double y = (e & 1) ? bf16_hi(wr[e / 2]) : bf16_lo(wr[e / 2]);
    const double dlt = x - y;
    s.dd += dlt * dlt;
    s.rr += y * y;
    s.ar += x * y;
    s.aa += x * x;
  }
}

template <int D>
__global__ void __launch_bounds__(kStatsThreads) stats_partial_kernel(TensorArg a, TensorArg r, int H, int N, int G,
                                                                      double* part) {
  const int g = blockIdx.x, bh = blockIdx.y;
  const int b = bh / H, h = bh % H;
  const int rows = (N + G - 1) / G;  // as the host sized the chunks
  const int r0 = g * rows;
  const int r1 = min(N, r0 + rows);
  constexpr int VEC = 8;  // 8 bf16 = 16 bytes per load
  constexpr int PER_ROW = D / VEC;
  const uint16_t* pa = a.ptr + b * a.sb + h * a.sh + (int64_t)r0 * a.sn;
  const uint16_t* pr = r.ptr + b * r.sb + h * r.sh + (int64_t)r0 * r.sn;
  // < 2^31: a chunk holds at most ceil(N / 64) rows once N > 16128
  const int total = r1 > r0 ? (r1 - r0) * PER_ROW : 0;
  Sums s{0.0, 0.0, 0.0, 0.0};
  int i = threadIdx.x;
  // Element order per thread: i, i + T, i + 2T, ...; the unrolled body loads kStatsUnroll vectors first and then
  // adds them in that same order.
  for (; i + (kStatsUnroll - 1) * kStatsThreads < total; i += kStatsUnroll * kStatsThreads) {
    uint4 va[kStatsUnroll], vr[kStatsUnroll];
#pragma unroll
    for (int u = 0; u < kStatsUnroll; ++u) {
      const int j = i + u * kStatsThreads;
      const int row = j / PER_ROW, c = (j % PER_ROW) * VEC;
      va[u] = *reinterpret_cast<const uint4*>(pa + (int64_t)row * a.sn + c);
      vr[u] = *reinterpret_cast<const uint4*>(pr + (int64_t)row * r.sn + c);
    }
#pragma unroll
    for (int u = 0; u < kStatsUnroll; ++u) accumulate(s, va[u], vr[u]);
  }
  for (; i < total; i += kStatsThreads) {
    const int row = i / PER_ROW, c = (i % PER_ROW) * VEC;
    accumulate(s, *reinterpret_cast<const uint4*>(pa + (int64_t)row * a.sn + c),
               *reinterpret_cast<const uint4*>(pr + (int64_t)row * r.sn + c));
  }
  __shared__ double red[4][kStatsThreads];
  red[0][threadIdx.x] = s.dd;
  red[1][threadIdx.x] = s.rr;
  red[2][threadIdx.x] = s.ar;
  red[3][threadIdx.x] = s.aa;
  __syncthreads();
  for (int w = kStatsThreads / 2; w > 0; w /= 2) {
    if ((int)threadIdx.x < w) {
#pragma unroll
      for (int k = 0; k < 4; ++k) red[k][threadIdx.x] += red[k][threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x < 4) part[((int64_t)bh * G + g) * 4 + threadIdx.x] = red[threadIdx.x][0];
}

// One wave per (batch, head): lane t holds partial t (0 beyond G), then a fixed tree over the 64 lanes.
__global__ void __launch_bounds__(64) stats_final_kernel(const double* part, int G, double* out) {
  const int bh = blockIdx.x, t = threadIdx.x;
  __shared__ double red[4][64];
#pragma unroll
  for (int k = 0; k < 4; ++k) red[k][t] = t < G ? part[((int64_t)bh * G + t) * 4 + k] : 0.0;
  __syncthreads();
  for (int w = 32; w > 0; w /= 2) {
    if (t < w) {
#pragma unroll
      for (int k = 0; k < 4; ++k) red[k][t] += red[k][t + w];
    }
    __syncthreads();
  }
  if (t < 4) out[(int64_t)bh * 4 + t] = red[t][0];
}

}  // namespace

hipError_t launch_error_stats(const TensorArg& a, const TensorArg& r, int B, int H, int N, int d, double* part,
                              double* out, hipStream_t s) {
  const int G = error_stats_chunks(N);
  const dim3 grid(G, B * H);
  if (d == 128) stats_partial_kernel<128><<<grid, kStatsThreads, 0, s>>>(a, r, H, N, G, part);
  else stats_partial_kernel<64><<<grid, kStatsThreads, 0, s>>>(a, r, H, N, G, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  stats_final_kernel<<<B * H, 64, 0, s>>>(part, G, out);
  return hipGetLastError();
}

}  // namespace sattn

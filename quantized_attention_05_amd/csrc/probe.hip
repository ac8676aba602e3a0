// Per-head error statistics of an attention output against a reference output: the attention-error probe
// behind layer-selective quantization (TMAP I2V write-up, section "保持视频质量": the attention error of each layer
// over the denoising iterations decides which layers keep full precision).
//
// One workgroup per (batch, head) walks all rows of that head with a fixed thread -> element assignment and sums
// in fp64 in a fixed order (per-thread sums, then a fixed tree over the workgroup), so the result is deterministic
// and needs no workspace.  The probe reads each output once (2 x 2 bytes per element); it is not on the hot path.
#include "sattn_internal.h"

namespace sattn {
namespace {

constexpr int kProbeThreads = 512;

__device__ __forceinline__ double bf16_value(uint16_t h) { return (double)__uint_as_float((uint32_t)h << 16); }

template <int D>
__global__ void __launch_bounds__(kProbeThreads) error_stats_kernel(TensorArg a, TensorArg r, int H, int N,
                                                                    double* out) {
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh % H;
  const uint16_t* pa = a.ptr + b * a.sb + h * a.sh;
  const uint16_t* pr = r.ptr + b * r.sb + h * r.sh;
  constexpr int VEC = 8;                   // 8 bf16 = 16 bytes per load
  constexpr int PER_ROW = D / VEC;
  double s_dd = 0.0, s_rr = 0.0, s_ar = 0.0, s_aa = 0.0;
  const int64_t total = (int64_t)N * PER_ROW;
  for (int64_t i = threadIdx.x; i < total; i += kProbeThreads) {
    const int row = (int)(i / PER_ROW), c = (int)(i % PER_ROW) * VEC;
    const uint4 va = *reinterpret_cast<const uint4*>(pa + (int64_t)row * a.sn + c);
    const uint4 vr = *reinterpret_cast<const uint4*>(pr + (int64_t)row * r.sn + c);
    const uint32_t wa[4] = {va.x, va.y, va.z, va.w}, wr[4] = {vr.x, vr.y, vr.z, vr.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double x = bf16_value((uint16_t)(wa[e / 2] >> (16 * (e & 1))));
      const double y = bf16_value((uint16_t)(wr[e / 2] >> (16 * (e & 1))));
      const double dlt = x - y;
      s_dd += dlt * dlt;
      s_rr += y * y;
      s_ar += x * y;
      s_aa += x * x;
    }
  }
  __shared__ double red[4][kProbeThreads];
  red[0][threadIdx.x] = s_dd;
  red[1][threadIdx.x] = s_rr;
  red[2][threadIdx.x] = s_ar;
  red[3][threadIdx.x] = s_aa;
  __syncthreads();
  for (int w = kProbeThreads / 2; w > 0; w /= 2) {
    if ((int)threadIdx.x < w) {
#pragma unroll
      for (int k = 0; k < 4; ++k) red[k][threadIdx.x] += red[k][threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x < 4) out[(int64_t)bh * 4 + threadIdx.x] = red[threadIdx.x][0];
}

}  // namespace

hipError_t launch_error_stats(const TensorArg& a, const TensorArg& r, int B, int H, int N, int d, double* out,
                              hipStream_t s) {
  if (d == 128) error_stats_kernel<128><<<B * H, kProbeThreads, 0, s>>>(a, r, H, N, out);
  else error_stats_kernel<64><<<B * H, kProbeThreads, 0, s>>>(a, r, H, N, out);
  return hipGetLastError();
}

}  // namespace sattn

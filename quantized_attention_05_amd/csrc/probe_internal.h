// Internal declarations of the error-statistics probe (not part of the C ABI).
#pragma once

#include "sattn_internal.h"

namespace sattn {

// Row chunks per (batch, head) of the error-statistics reduction: one per 256 rows, at most 64.  A function of N
// alone, so the summation order, and every bit of the result, depends on the shape only.
constexpr int kStatsMaxChunks = 64;
inline int error_stats_chunks(int N) {
  const int g = cdiv(N, 256);
  return g < kStatsMaxChunks ? g : kStatsMaxChunks;
}

// Enqueues the two reduction launches.  part: B*H*error_stats_chunks(N)*4 doubles of workspace for the per-chunk
// partial sums; out: B*H*4 doubles.  Returns hipGetLastError().
hipError_t launch_error_stats(const TensorArg& a, const TensorArg& r, int B, int H, int N, int d, double* part,
                              double* out, hipStream_t s);

}  // namespace sattn

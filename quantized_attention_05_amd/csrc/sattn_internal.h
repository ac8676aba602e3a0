// Internal declarations shared by the HIP translation units of libsattn (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sattn.h"

namespace sattn {

constexpr int kTile = 64;          // keys per softmax tile == K quantization block == V tile
constexpr int kChunk = 64;         // tokens per run of the K-mean / V-amax first pass
constexpr float kGuard = 0x1p-100f; // amax below this: all-zero block or channel (scale 0, codes 0)
constexpr int kMaskQRows = SATTN_MASK_QBLK;  // block-sparse mask: query rows per mask row
constexpr int kMaxSparseTiles = 32768;       // block-sparse: key tiles per mask row the kernel can list in LDS

inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// Strided view of a bf16 tensor [B, H, N, d] (element strides; channel stride 1).
struct TensorArg {
  const uint16_t* ptr;
  int64_t sb, sh, sn;
};

inline TensorArg tensor_arg(const sattn_tensor* t) {
  return TensorArg{reinterpret_cast<const uint16_t*>(t->ptr), t->stride_b, t->stride_h, t->stride_n};
}

// Dense quantized operands (see sattn_quant in sattn.h) plus sizes.
struct QuantArg {
  int B, H, Nq, Nkv, d, blk_q, nqb, nkb;
  int8_t* q_codes;
  float* q_scales;
  int8_t* k_codes;
  float* k_scales;
  float* k_mean;
  uint8_t* v_codes;
  float* v_scales;
  uint16_t* v_t;
};

// Per-call set-up of the attention kernel a call will launch (its dynamic LDS limit); enqueues nothing.
hipError_t prepare_attn(int mode, int d, bool sparse, bool fuse_q);
// Query rows of one attention workgroup (the grid has ceil(Nq / rows) * H * B workgroups).
int attn_rows_per_workgroup();

// Launchers (enqueue only; return hipGetLastError()).
hipError_t launch_quant_q(const TensorArg& q, const QuantArg& qa, hipStream_t s);
hipError_t launch_kv_stats(const TensorArg& k, const TensorArg& v, bool with_v, const QuantArg& qa, float* ksum,
                           float* vmax, hipStream_t s);
hipError_t launch_kv_finalize(const QuantArg& qa, bool with_v, const float* ksum, const float* vmax, float* vinv,
                              hipStream_t s);
hipError_t launch_kv_quant(const TensorArg& k, const TensorArg& v, int mode, const QuantArg& qa, const float* vinv,
                           hipStream_t s);
// mask: nullptr for dense attention, else the block-sparse mask [B, H, ceil(Nq/128), ceil(Nkv/64)] (device bytes).
// fuse_q (modes 1 and 2): quantize Q from the bf16 tensor q inside the kernel instead of reading qa's Q codes.
hipError_t launch_attn(int mode, const TensorArg& q, const TensorArg& k, const QuantArg& qa, uint16_t* o, int64_t osb,
                       int64_t osh, int64_t osn, float sm_scale, const uint8_t* mask, bool fuse_q, hipStream_t s);
hipError_t launch_debug_qk(const QuantArg& qa, int b, int h, int q0, int nq, int k0, int nk, int32_t* out,
                           hipStream_t s);

}  // namespace sattn

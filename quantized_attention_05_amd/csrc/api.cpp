// C ABI of libsattn: argument checks, workspace carving, mode dispatch.  Allocates nothing, synchronises
// nothing, keeps no state; every kernel is enqueued on the caller's stream.  The operations are declared and cited
// in include/sattn.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "linear_internal.h"
#include "probe_internal.h"
#include "sattn_internal.h"

using namespace sattn;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool valid_mode(int m) { return m == SATTN_MODE_BF16 || m == SATTN_MODE_I8_BF16 || m == SATTN_MODE_I8_FP8; }

// Shape checks shared by every entry point: INVALID_ARG for nonsense, UNSUPPORTED for sensible shapes the
// kernels are not built for.
sattn_status check_shape(int B, int H, int Nq, int Nkv, int d, int blk_q, int blk_k, int mode) {
  if (B <= 0 || H <= 0 || Nq <= 0 || Nkv <= 0 || d <= 0 || blk_q <= 0 || blk_k <= 0) return SATTN_ERR_INVALID_ARG;
  if (!valid_mode(mode)) return SATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return SATTN_ERR_UNSUPPORTED;
  if (blk_q != 64 && blk_q != 128) return SATTN_ERR_UNSUPPORTED;
  if (blk_k != kTile) return SATTN_ERR_UNSUPPORTED;
  // keep every element offset of the padded code arrays inside int64 and every grid dimension in range (the
  // attention grid has one workgroup per query tile and head)
  if ((int64_t)B * H > 65535 || Nq > (1 << 28) || Nkv > (1 << 28)) return SATTN_ERR_UNSUPPORTED;
  if ((int64_t)cdiv(Nq, attn_rows_per_workgroup()) * B * H > INT32_MAX) return SATTN_ERR_UNSUPPORTED;
  return SATTN_OK;
}

// An error left pending by earlier, unrelated HIP calls of this thread would otherwise be read back by this call's
// launch check and reported as its own: take it off before the first launch.
void clear_pending_error() { (void)hipGetLastError(); }

struct Sizes {
  int nqb, nkb;
  size_t q_codes, q_scales, k_codes, k_scales, k_mean, v_codes, v_scales, v_t, total;
};

// Sizes of the quantized operands.  with_q = false leaves out the Q codes and scales: the drop-in calls quantize Q
// inside the attention kernel and keep only K and V in the workspace.
Sizes sizes(int B, int H, int Nq, int Nkv, int d, int blk_q, int mode, bool with_q = true) {
  Sizes s;
  const size_t bh = (size_t)B * H;
  s.nqb = cdiv(Nq, blk_q);
  s.nkb = cdiv(Nkv, kTile);
  const bool quant = mode != SATTN_MODE_BF16;
  s.q_codes = quant && with_q ? align_up(bh * s.nqb * blk_q * d) : 0;
  s.q_scales = quant && with_q ? align_up(bh * s.nqb * sizeof(float)) : 0;
  s.k_codes = quant ? align_up(bh * (size_t)s.nkb * kTile * d) : 0;
  s.k_scales = quant ? align_up(bh * s.nkb * sizeof(float)) : 0;
  s.k_mean = quant ? align_up(bh * d * sizeof(float)) : 0;
  s.v_codes = mode == SATTN_MODE_I8_FP8 ? align_up(bh * (size_t)s.nkb * kTile * d) : 0;
  s.v_scales = mode == SATTN_MODE_I8_FP8 ? align_up(bh * d * sizeof(float)) : 0;
  s.v_t = mode != SATTN_MODE_I8_FP8 ? align_up(bh * (size_t)s.nkb * kTile * d * 2) : 0;
  s.total = s.q_codes + s.q_scales + s.k_codes + s.k_scales + s.k_mean + s.v_codes + s.v_scales + s.v_t;
  return s;
}

size_t scratch_bytes(int B, int H, int Nkv, int d, int mode) {
  if (mode == SATTN_MODE_BF16) return 0;
  const size_t runs = (size_t)B * H * cdiv(Nkv, kChunk) * d * sizeof(float);
  size_t bytes = align_up(runs);                                   // K run sums
  if (mode == SATTN_MODE_I8_FP8) bytes += align_up(runs) + align_up((size_t)B * H * d * sizeof(float));  // V
  return bytes;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

sattn_status check_tensor(const sattn_tensor* t, int B, int H, int N, int d) {
  if (!t || !t->ptr) return SATTN_ERR_INVALID_ARG;
  if (t->B != B || t->H != H || t->N != N || t->d != d) return SATTN_ERR_INVALID_ARG;
  if (!aligned16(t->ptr)) return SATTN_ERR_INVALID_ARG;
  if (t->stride_b % 8 || t->stride_h % 8 || t->stride_n % 8) return SATTN_ERR_INVALID_ARG;
  if (t->stride_b < 0 || t->stride_h < 0 || t->stride_n < d) return SATTN_ERR_INVALID_ARG;
  return SATTN_OK;
}

// mode 0 reads K rows of a 64-key tile at 32-bit byte offsets row * stride_n * 2
sattn_status check_k_rows(const sattn_tensor* k, int mode) {
  return (mode == SATTN_MODE_BF16 && k->stride_n >= (int64_t{1} << 24)) ? SATTN_ERR_UNSUPPORTED : SATTN_OK;
}

QuantArg quant_arg(const sattn_quant& q) {
  QuantArg a;
  a.B = q.B;
  a.H = q.H;
  a.Nq = q.Nq;
  a.Nkv = q.Nkv;
  a.d = q.d;
  a.blk_q = q.blk_q;
  a.nqb = cdiv(q.Nq, q.blk_q);
  a.nkb = cdiv(q.Nkv, kTile);
  a.q_codes = q.q_codes;
  a.q_scales = q.q_scales;
  a.k_codes = q.k_codes;
  a.k_scales = q.k_scales;
  a.k_mean = q.k_mean;
  a.v_codes = q.v_codes;
  a.v_scales = q.v_scales;
  a.v_t = q.v_t;
  return a;
}

sattn_status check_quant(const sattn_quant* q, int mode) {
  if (!q) return SATTN_ERR_INVALID_ARG;
  sattn_status st = check_shape(q->B, q->H, q->Nq, q->Nkv, q->d, q->blk_q, q->blk_k, mode);
  if (st != SATTN_OK) return st;
  if (q->mode != mode) return SATTN_ERR_INVALID_ARG;
  if (mode != SATTN_MODE_BF16) {
    if (!q->q_codes || !q->q_scales || !q->k_codes || !q->k_scales || !q->k_mean) return SATTN_ERR_INVALID_ARG;
    if (!aligned16(q->q_codes) || !aligned16(q->k_codes)) return SATTN_ERR_INVALID_ARG;
  }
  if (mode == SATTN_MODE_I8_FP8) {
    if (!q->v_codes || !q->v_scales || !aligned16(q->v_codes)) return SATTN_ERR_INVALID_ARG;
  } else {
    if (!q->v_t || !aligned16(q->v_t)) return SATTN_ERR_INVALID_ARG;
  }
  return SATTN_OK;
}

sattn_status hip_status(hipError_t e) { return e == hipSuccess ? SATTN_OK : SATTN_ERR_HIP; }

// The quantization pass; with_q = false skips the Q blocks (the attention kernel of the drop-in calls quantizes them).
sattn_status do_quantize(const sattn_tensor* q, const sattn_tensor* k, const sattn_tensor* v, int mode,
                         const sattn_quant* out, void* scratch, size_t scratch_bytes_, hipStream_t s,
                         bool with_q = true) {
  const QuantArg qa = quant_arg(*out);
  const TensorArg kt = tensor_arg(k), vt = tensor_arg(v);
  hipError_t e = hipSuccess;
  if (mode != SATTN_MODE_BF16) {
    const size_t runs = align_up((size_t)qa.B * qa.H * cdiv(qa.Nkv, kChunk) * qa.d * sizeof(float));
    float* ksum = reinterpret_cast<float*>(scratch);
    float* vmax = mode == SATTN_MODE_I8_FP8 ? reinterpret_cast<float*>(static_cast<char*>(scratch) + runs) : nullptr;
    float* vinv = mode == SATTN_MODE_I8_FP8 ? reinterpret_cast<float*>(static_cast<char*>(scratch) + 2 * runs) : nullptr;
    (void)scratch_bytes_;
    const bool with_v = mode == SATTN_MODE_I8_FP8;
    if (with_q && (e = launch_quant_q(tensor_arg(q), qa, s)) != hipSuccess) return hip_status(e);
    if ((e = launch_kv_stats(kt, vt, with_v, qa, ksum, vmax, s)) != hipSuccess) return hip_status(e);
    if ((e = launch_kv_finalize(qa, with_v, ksum, vmax, vinv, s)) != hipSuccess) return hip_status(e);
    e = launch_kv_quant(kt, vt, mode, qa, vinv, s);
  } else {
    e = launch_kv_quant(kt, vt, mode, qa, nullptr, s);
  }
  return hip_status(e);
}

sattn_status layout(int B, int H, int Nq, int Nkv, int d, int blk_q, int blk_k, int mode, void* base, sattn_quant* out,
                    bool with_q = true) {
  const Sizes z = sizes(B, H, Nq, Nkv, d, blk_q, mode, with_q);
  std::memset(out, 0, sizeof(*out));
  out->B = B;
  out->H = H;
  out->Nq = Nq;
  out->Nkv = Nkv;
  out->d = d;
  out->blk_q = blk_q;
  out->blk_k = blk_k;
  out->mode = mode;
  char* p = static_cast<char*>(base);
  auto take = [&](size_t n) -> char* {
    if (n == 0) return nullptr;
    char* r = p;
    p += n;
    return r;
  };
  out->q_codes = reinterpret_cast<int8_t*>(take(z.q_codes));
  out->q_scales = reinterpret_cast<float*>(take(z.q_scales));
  out->k_codes = reinterpret_cast<int8_t*>(take(z.k_codes));
  out->k_scales = reinterpret_cast<float*>(take(z.k_scales));
  out->k_mean = reinterpret_cast<float*>(take(z.k_mean));
  out->v_codes = reinterpret_cast<uint8_t*>(take(z.v_codes));
  out->v_scales = reinterpret_cast<float*>(take(z.v_scales));
  out->v_t = reinterpret_cast<uint16_t*>(take(z.v_t));
  return SATTN_OK;
}

sattn_status fwd_common(const sattn_tensor* q, const sattn_tensor* k, const sattn_tensor* v, const sattn_tensor* o,
                        float sm_scale, int mode, int blk_q, int blk_k, void* ws, size_t ws_bytes,
                        const uint8_t* mask, hipStream_t s) {
  if (!q || !k || !v || !o) return SATTN_ERR_INVALID_ARG;
  const int B = q->B, H = q->H, Nq = q->N, Nkv = k->N, d = q->d;
  sattn_status st;
  // consistency of the four tensors first (INVALID_ARG), then what the kernels support (UNSUPPORTED)
  if ((st = check_tensor(q, B, H, Nq, d)) != SATTN_OK) return st;
  if ((st = check_tensor(k, B, H, Nkv, d)) != SATTN_OK) return st;
  if ((st = check_tensor(v, B, H, Nkv, d)) != SATTN_OK) return st;
  if ((st = check_tensor(o, B, H, Nq, d)) != SATTN_OK) return st;
  if ((st = check_shape(B, H, Nq, Nkv, d, blk_q, blk_k, mode)) != SATTN_OK) return st;
  if ((st = check_k_rows(k, mode)) != SATTN_OK) return st;
  if (!(std::isfinite(sm_scale))) return SATTN_ERR_INVALID_ARG;
  // Q is quantized inside the attention kernel (modes 1 and 2): the workspace holds K, V and the partial sums only
  const Sizes z = sizes(B, H, Nq, Nkv, d, blk_q, mode, false);
  const size_t need = z.total + scratch_bytes(B, H, Nkv, d, mode);
  if (!ws || ws_bytes < need) return SATTN_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) % kAlign) != 0) return SATTN_ERR_INVALID_ARG;
  sattn_quant qk;
  layout(B, H, Nq, Nkv, d, blk_q, blk_k, mode, ws, &qk, false);
  void* scratch = static_cast<char*>(ws) + z.total;
  const bool fuse_q = mode != SATTN_MODE_BF16;
  clear_pending_error();
  if ((st = hip_status(prepare_attn(mode, d, mask != nullptr, fuse_q))) != SATTN_OK) return st;
  st = do_quantize(q, k, v, mode, &qk, scratch, need - z.total, s, false);
  if (st != SATTN_OK) return st;
  const float c = sm_scale > 0.0f ? sm_scale : 1.0f / std::sqrt((float)d);
  const TensorArg ot = tensor_arg(o);
  return hip_status(launch_attn(mode, tensor_arg(q), tensor_arg(k), quant_arg(qk), const_cast<uint16_t*>(ot.ptr), ot.sb,
                                ot.sh, ot.sn, c, mask, fuse_q, s));
}

}  // namespace

extern "C" {

const char* sattn_status_string(int st) {
  switch (st) {
    case SATTN_OK: return "ok";
    case SATTN_ERR_INVALID_ARG: return "invalid argument";
    case SATTN_ERR_UNSUPPORTED: return "unsupported shape or block size";
    case SATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case SATTN_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int sattn_kv_tile(int d, int mode) {
  (void)d;
  (void)mode;
  return kTile;
}

size_t sattn_quant_bytes(int B, int H, int Nq, int Nkv, int d, int blk_q, int blk_k, int mode) {
  if (check_shape(B, H, Nq, Nkv, d, blk_q, blk_k, mode) != SATTN_OK) return 0;
  return sizes(B, H, Nq, Nkv, d, blk_q, mode).total;
}

sattn_status sattn_quant_layout(int B, int H, int Nq, int Nkv, int d, int blk_q, int blk_k, int mode, void* base,
                                sattn_quant* out) {
  if (!out || !base) return SATTN_ERR_INVALID_ARG;
  sattn_status st = check_shape(B, H, Nq, Nkv, d, blk_q, blk_k, mode);
  if (st != SATTN_OK) return st;
  if ((reinterpret_cast<uintptr_t>(base) % kAlign) != 0) return SATTN_ERR_INVALID_ARG;
  return layout(B, H, Nq, Nkv, d, blk_q, blk_k, mode, base, out);
}

size_t sattn_quantize_scratch_bytes(int B, int H, int Nkv, int d, int mode) {
  if (check_shape(B, H, 1, Nkv, d, 64, kTile, mode) != SATTN_OK) return 0;
  return scratch_bytes(B, H, Nkv, d, mode);
}

size_t sattn_workspace_bytes(int B, int H, int Nq, int Nkv, int d, int blk_q, int blk_k, int mode) {
  if (check_shape(B, H, Nq, Nkv, d, blk_q, blk_k, mode) != SATTN_OK) return 0;
  return sizes(B, H, Nq, Nkv, d, blk_q, mode, false).total + scratch_bytes(B, H, Nkv, d, mode);
}

sattn_status sattn_quantize(const sattn_tensor* q, const sattn_tensor* k, const sattn_tensor* v, int mode,
                            const sattn_quant* out, void* scratch, size_t scratch_bytes_, sattn_stream_t stream) {
  sattn_status st = check_quant(out, mode);
  if (st != SATTN_OK) return st;
  const int B = out->B, H = out->H, d = out->d;
  if (mode != SATTN_MODE_BF16 && (st = check_tensor(q, B, H, out->Nq, d)) != SATTN_OK) return st;
  if ((st = check_tensor(k, B, H, out->Nkv, d)) != SATTN_OK) return st;
  if ((st = check_tensor(v, B, H, out->Nkv, d)) != SATTN_OK) return st;
  const size_t need = scratch_bytes(B, H, out->Nkv, d, mode);
  if (need > 0 && (!scratch || scratch_bytes_ < need)) return SATTN_ERR_WORKSPACE;
  clear_pending_error();
  return do_quantize(q, k, v, mode, out, scratch, scratch_bytes_, reinterpret_cast<hipStream_t>(stream));
}

sattn_status sattn_fwd_quantized(const sattn_tensor* q, const sattn_tensor* k, const sattn_quant* qk,
                                 const sattn_tensor* o, float sm_scale, int mode, sattn_stream_t stream) {
  sattn_status st = check_quant(qk, mode);
  if (st != SATTN_OK) return st;
  if ((st = check_tensor(o, qk->B, qk->H, qk->Nq, qk->d)) != SATTN_OK) return st;
  if (mode == SATTN_MODE_BF16) {
    if ((st = check_tensor(q, qk->B, qk->H, qk->Nq, qk->d)) != SATTN_OK) return st;
    if ((st = check_tensor(k, qk->B, qk->H, qk->Nkv, qk->d)) != SATTN_OK) return st;
    if ((st = check_k_rows(k, mode)) != SATTN_OK) return st;
  }
  if (!(std::isfinite(sm_scale))) return SATTN_ERR_INVALID_ARG;
  const float c = sm_scale > 0.0f ? sm_scale : 1.0f / std::sqrt((float)qk->d);
  const TensorArg ot = tensor_arg(o);
  const TensorArg none{nullptr, 0, 0, 0};
  const TensorArg qt = mode == SATTN_MODE_BF16 ? tensor_arg(q) : none;
  const TensorArg kt = mode == SATTN_MODE_BF16 ? tensor_arg(k) : none;
  clear_pending_error();
  if ((st = hip_status(prepare_attn(mode, qk->d, false, false))) != SATTN_OK) return st;
  return hip_status(launch_attn(mode, qt, kt, quant_arg(*qk), const_cast<uint16_t*>(ot.ptr), ot.sb, ot.sh, ot.sn, c,
                                nullptr, false, reinterpret_cast<hipStream_t>(stream)));
}

sattn_status sattn_fwd(const sattn_tensor* q, const sattn_tensor* k, const sattn_tensor* v, const sattn_tensor* o,
                       float sm_scale, int mode, int blk_q, int blk_k, void* ws, size_t ws_bytes,
                       sattn_stream_t stream) {
  return fwd_common(q, k, v, o, sm_scale, mode, blk_q, blk_k, ws, ws_bytes, nullptr,
                    reinterpret_cast<hipStream_t>(stream));
}

sattn_status sattn_fwd_block_sparse(const sattn_tensor* q, const sattn_tensor* k, const sattn_tensor* v,
                                    const sattn_tensor* o, const uint8_t* block_mask, float sm_scale, int mode,
                                    int blk_q, int blk_k, void* ws, size_t ws_bytes, sattn_stream_t stream) {
  if (!block_mask || !k) return SATTN_ERR_INVALID_ARG;
  if (k->N > 0 && cdiv(k->N, SATTN_MASK_KBLK) > kMaxSparseTiles) return SATTN_ERR_UNSUPPORTED;
  return fwd_common(q, k, v, o, sm_scale, mode, blk_q, blk_k, ws, ws_bytes, block_mask,
                    reinterpret_cast<hipStream_t>(stream));
}

sattn_status sattn_cross_fwd(const sattn_tensor* q, const sattn_tensor* k, const sattn_tensor* v,
                             const sattn_tensor* o, float sm_scale, int mode, void* ws, size_t ws_bytes,
                             sattn_stream_t stream) {
  return fwd_common(q, k, v, o, sm_scale, mode, 128, kTile, ws, ws_bytes, nullptr, reinterpret_cast<hipStream_t>(stream));
}

size_t sattn_error_stats_workspace_bytes(int B, int H, int N) {
  if (B <= 0 || H <= 0 || N <= 0) return 0;
  return align_up((size_t)B * H * error_stats_chunks(N) * 4 * sizeof(double));
}

sattn_status sattn_error_stats(const sattn_tensor* a, const sattn_tensor* ref, double* out, void* ws, size_t ws_bytes,
                               sattn_stream_t stream) {
  if (!a || !ref || !out) return SATTN_ERR_INVALID_ARG;
  if (a->B <= 0 || a->H <= 0 || a->N <= 0) return SATTN_ERR_INVALID_ARG;
  sattn_status st;
  if ((st = check_tensor(a, a->B, a->H, a->N, a->d)) != SATTN_OK) return st;
  if ((st = check_tensor(ref, a->B, a->H, a->N, a->d)) != SATTN_OK) return st;
  if (reinterpret_cast<uintptr_t>(out) % 8 != 0) return SATTN_ERR_INVALID_ARG;
  if ((a->d != 64 && a->d != 128) || (int64_t)a->B * a->H > 65535) return SATTN_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < sattn_error_stats_workspace_bytes(a->B, a->H, a->N)) return SATTN_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % 8 != 0) return SATTN_ERR_INVALID_ARG;
  clear_pending_error();
  return hip_status(launch_error_stats(tensor_arg(a), tensor_arg(ref), a->B, a->H, a->N, a->d,
                                       static_cast<double*>(ws), out, reinterpret_cast<hipStream_t>(stream)));
}

sattn_status sattn_debug_qk_int32(const sattn_quant* qk, int b, int h, int q0, int nq, int k0, int nk, int32_t* out,
                                  sattn_stream_t stream) {
  if (!qk || !out) return SATTN_ERR_INVALID_ARG;
  sattn_status st = check_quant(qk, qk->mode);
  if (st != SATTN_OK) return st;
  if (qk->mode == SATTN_MODE_BF16) return SATTN_ERR_INVALID_ARG;
  if (b < 0 || b >= qk->B || h < 0 || h >= qk->H || nq <= 0 || nk <= 0 || q0 < 0 || k0 < 0)
    return SATTN_ERR_INVALID_ARG;
  const int nq_pad = cdiv(qk->Nq, qk->blk_q) * qk->blk_q, nk_pad = cdiv(qk->Nkv, kTile) * kTile;
  if ((int64_t)q0 + nq > nq_pad || (int64_t)k0 + nk > nk_pad) return SATTN_ERR_INVALID_ARG;
  clear_pending_error();
  return hip_status(launch_debug_qk(quant_arg(*qk), b, h, q0, nq, k0, nk, out, reinterpret_cast<hipStream_t>(stream)));
}

// ---- quantized linear layer
sattn_status sattn_quantize_blocks(const void* x, int rows, int cols, int64_t ld, int8_t* codes, float* scales,
                                   sattn_stream_t stream) {
  if (!x || !codes || !scales || rows < 1 || cols < 1) return SATTN_ERR_INVALID_ARG;
  if (cols % kLinBlk != 0 || rows > (1 << 28) || cols > (1 << 28)) return SATTN_ERR_UNSUPPORTED;
  if (ld < cols || ld % 8 != 0 || !aligned16(x) || !aligned16(codes) || reinterpret_cast<uintptr_t>(scales) % 4)
    return SATTN_ERR_INVALID_ARG;
  clear_pending_error();
  return hip_status(launch_quant_blocks(static_cast<const uint16_t*>(x), rows, cols, ld, codes, scales,
                                        reinterpret_cast<hipStream_t>(stream)));
}

size_t sattn_linear_workspace_bytes(int M, int N, int K, int mode) {
  if (M < 1 || N < 1 || K < kLinBlk || K % kLinBlk != 0) return 0;
  if (mode == SATTN_LINEAR_W8A8) return align_up((size_t)M * K) + align_up((size_t)cdiv(M, kLinBlk) * (K / kLinBlk) * 4);
  if (mode == SATTN_LINEAR_W8A16) return align_up((size_t)N * K * 2);
  return 0;
}

}  // extern "C"

namespace {

// Shape and output checks shared by the linear entry points.
sattn_status check_linear(const void* y, int64_t ldy, int M, int N, int K, const void* bias) {
  if (!y || M < 1 || N < 1 || K < 1) return SATTN_ERR_INVALID_ARG;
  if (K % kLinBlk != 0 || K > (1 << 20) || M > (1 << 28) || N > (1 << 28)) return SATTN_ERR_UNSUPPORTED;
  if ((int64_t)cdiv(M, kLinBlk) * cdiv(N, kLinBlk) > INT32_MAX) return SATTN_ERR_UNSUPPORTED;
  if (ldy < N || reinterpret_cast<uintptr_t>(y) % 2) return SATTN_ERR_INVALID_ARG;
  if (bias && reinterpret_cast<uintptr_t>(bias) % 2) return SATTN_ERR_INVALID_ARG;
  return SATTN_OK;
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace

extern "C" {

sattn_status sattn_linear_quantized(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw,
                                    const void* bias, void* y, int64_t ldy, int M, int N, int K, sattn_stream_t stream) {
  if (!xq || !sx || !wq || !sw) return SATTN_ERR_INVALID_ARG;
  sattn_status st = check_linear(y, ldy, M, N, K, bias);
  if (st != SATTN_OK) return st;
  if (!aligned16(xq) || !aligned16(wq) || !aligned4(sx) || !aligned4(sw)) return SATTN_ERR_INVALID_ARG;
  LinearArg p{reinterpret_cast<const uint8_t*>(xq), K, reinterpret_cast<const uint8_t*>(wq), K, sx, sw,
              static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(y), ldy, M, N, K};
  clear_pending_error();
  if ((st = hip_status(prepare_linear(true))) != SATTN_OK) return st;
  return hip_status(launch_linear(true, p, reinterpret_cast<hipStream_t>(stream)));
}

sattn_status sattn_linear(const void* x, int64_t ldx, const int8_t* wq, const float* sw, const void* bias, void* y,
                          int64_t ldy, int M, int N, int K, int mode, void* ws, size_t ws_bytes, sattn_stream_t stream) {
  if (!x || !wq || !sw) return SATTN_ERR_INVALID_ARG;
  if (mode != SATTN_LINEAR_W8A8 && mode != SATTN_LINEAR_W8A16) return SATTN_ERR_INVALID_ARG;
  sattn_status st = check_linear(y, ldy, M, N, K, bias);
  if (st != SATTN_OK) return st;
  if (ldx < K || ldx % 8 != 0 || !aligned16(x) || !aligned16(wq) || !aligned4(sw)) return SATTN_ERR_INVALID_ARG;
  if (ldx >= (int64_t{1} << 23)) return SATTN_ERR_UNSUPPORTED;  // a 128-row tile of x must span below 2^31 bytes
  const size_t need = sattn_linear_workspace_bytes(M, N, K, mode);
  if (!ws || ws_bytes < need) return SATTN_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return SATTN_ERR_INVALID_ARG;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint8_t* base = static_cast<uint8_t*>(ws);
  clear_pending_error();
  if ((st = hip_status(prepare_linear(mode == SATTN_LINEAR_W8A8))) != SATTN_OK) return st;
  hipError_t e;
  if (mode == SATTN_LINEAR_W8A8) {
    int8_t* xq = reinterpret_cast<int8_t*>(base);
    float* sx = reinterpret_cast<float*>(base + align_up((size_t)M * K));
    if ((e = launch_quant_blocks(static_cast<const uint16_t*>(x), M, K, ldx, xq, sx, s)) != hipSuccess)
      return hip_status(e);
    LinearArg p{reinterpret_cast<const uint8_t*>(xq), K, reinterpret_cast<const uint8_t*>(wq), K, sx, sw,
                static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(y), ldy, M, N, K};
    return hip_status(launch_linear(true, p, s));
  }
  uint16_t* wb = reinterpret_cast<uint16_t*>(base);
  if ((e = launch_codes_to_bf16(wq, wb, (int64_t)N * K, s)) != hipSuccess) return hip_status(e);
  LinearArg p{static_cast<const uint8_t*>(x), ldx * 2, reinterpret_cast<const uint8_t*>(wb), (int64_t)K * 2, nullptr,
              sw, static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(y), ldy, M, N, K};
  return hip_status(launch_linear(false, p, s));
}

}  // extern "C"

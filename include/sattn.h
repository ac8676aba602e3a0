/*
 * sattn.h -- C ABI of libsattn: SageAttention-style quantized attention for video diffusion
 * transformers, hand-written HIP for AMD Instinct MI355X (gfx950).
 *
 * What the library computes, and where the pages describe it:
 *   - Attention O = softmax(c * Q K^T) V per (batch, head) with no mask: the scaled-dot-product flash
 *     attention operator that dominates the FLOP profile of a Wan-class image-to-video DiT (TMAP I2V
 *     acceleration write-up, ai.aiking123.com/155823, section "Attention 性能优化 / 背景", FLOP table).
 *   - It is replaced by an 8-bit quantized operator (same page, section "attention量化": SageAttention),
 *     with the whole self-attention computation in 8 bits on Wan (section "显存优化 / 量化").
 *   - Precision is chosen per attention layer (section "保持视频质量": layer-selective quantization),
 *     which here is the per-call `mode` argument.
 *   - Scales computed from an all-zero channel must not divide by zero (section "优化算子细节"): every
 *     scale is guarded (amax < 2^-100 -> scale 0, codes 0).
 *   - The score matrix is never materialised (tutorial "视频生成推理加速实战:从基线到27倍", step 3,
 *     item "算子融合与高效注意力"): the softmax runs online over 64-key tiles.
 *
 * Quantization (modes 1 and 2), all in IEEE fp32 with round-to-nearest-even:
 *   mean[c]   = per-channel mean of K over the Nkv tokens.  Summation order is fixed: 64-token runs summed
 *               one value after another, then the run sums one after another, then one division by Nkv.
 *   K'        = float(K) - mean  (not re-rounded)
 *   Q, K'     : blocks of blk_q (Q) / blk_k (K') consecutive tokens of one (batch, head), all d channels;
 *               a = max|x| over the block's valid tokens; a < 2^-100 -> scale 0 and codes 0; otherwise
 *               scale = a/127, code = clamp(rint(x * (127/a)), -127, 127).
 *   V (mode 2): per channel a_c = max over tokens |V[:,c]|; guard as above; scale = a_c/448,
 *               code = E4M3FN(v * (448/a_c)) rounded to nearest even, saturating at 448.
 * Attention (per 64-key tile, ascending): x = S_int * (s_q*s_k*c*log2 e) (mode 0: x = (q.k)*c*log2 e);
 *   m' = max(m, max x); alpha = 2^(m-m'); p = 2^(x-m'); l = alpha*l + sum p;
 *   acc = alpha*acc + P^ V^ with P^ = bf16(p) (modes 0/1) or E4M3(448 p) (mode 2) and V^ = V (bf16) or
 *   the V codes (mode 2); O = acc / l (mode 2: acc * scale_v[c] / (448 l)), rounded to bf16.
 *
 * Conventions for every entry point:
 *   - Pointers inside the structs are DEVICE pointers; the structs themselves and every other pointer
 *     argument are HOST memory, read only during the call.
 *   - Nothing is allocated and nothing is synchronised.  All work is enqueued on `stream` (0 = the null
 *     stream) and the call returns.  Faults inside kernels surface at the caller's next synchronisation.
 *   - The caller owns every buffer.  The library keeps no state between calls (no flags, caches or handles;
 *     per-kernel launch attributes are set on the current device by every call), so it is re-entrant and
 *     serves every GPU of a process alike; concurrent calls need distinct workspaces and outputs.  Outputs
 *     must not alias inputs.  The one exception is sattn_fwd_noalloc, whose workspace is the library's own
 *     per-GPU array (its device address is looked up once per device and kept).
 *   - Errors: arguments are checked on the host before any launch.  A bad argument returns
 *     SATTN_ERR_INVALID_ARG, a valid but unsupported shape SATTN_ERR_UNSUPPORTED, a too small workspace
 *     SATTN_ERR_WORKSPACE; in these cases nothing has been enqueued.  SATTN_ERR_HIP reports a failure of
 *     the HIP runtime: when the per-call set-up fails, nothing has been enqueued; when a launch fails, the
 *     kernels this call enqueued before it (which write only the workspace and the call's outputs) may
 *     still run, and the outputs are undefined.  An error left pending by earlier, unrelated HIP calls of
 *     the calling thread is cleared on entry and not reported.  No C++ exception crosses this interface.
 *   - NaN or Inf inputs are outside the contract.  Zero blocks and zero channels are inside it and give
 *     finite outputs.
 *   - Empty shapes (B, H, N, rows or columns below 1) are SATTN_ERR_INVALID_ARG, not a silent no-op: a
 *     softmax over no keys has no value, and a call with no queries is refused the same way.
 */
#ifndef SATTN_H
#define SATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* sattn_stream_t; /* a hipStream_t */

typedef enum {
  SATTN_OK = 0,
  SATTN_ERR_INVALID_ARG = 1,
  SATTN_ERR_UNSUPPORTED = 2,
  SATTN_ERR_WORKSPACE = 3,
  SATTN_ERR_HIP = 4
} sattn_status;

typedef enum {
  SATTN_MODE_BF16 = 0,    /* exact bf16 attention (bf16 QK^T and P*V, fp32 accumulation)        */
  SATTN_MODE_I8_BF16 = 1, /* INT8 QK^T with int32 accumulation, bf16 P*V                         */
  SATTN_MODE_I8_FP8 = 2   /* INT8 QK^T with int32 accumulation, FP8-E4M3 P*V                     */
} sattn_mode;

/* A bf16 activation tensor [B, H, N, d] addressed as ptr + b*stride_b + h*stride_h + n*stride_n + c
 * (strides in elements; the channel stride is 1).  Both [B,H,N,d] and [B,N,H,d] storage fit.
 * Requirements: ptr 16-byte aligned; stride_b, stride_h, stride_n multiples of 8; d in {64, 128}.
 * In mode 0 (bf16 scores) the attention kernel addresses the K rows of a 64-key tile with 32-bit offsets, so
 * K's stride_n must be below 2^24 elements there (else SATTN_ERR_UNSUPPORTED). */
typedef struct {
  void* ptr;
  int B, H, N, d;
  int64_t stride_b, stride_h, stride_n;
} sattn_tensor;

/* Quantized operands of one attention call.  nqb = ceil(Nq/blk_q), nkb = ceil(Nkv/64) (blk_k is 64),
 * nq_pad = nqb*blk_q, nk_pad = nkb*64.  All arrays dense, device memory, owned by the caller.
 *   q_codes  int8  [B, H, nq_pad, d]    row-major per token; pad tokens hold 0
 *   q_scales fp32  [B, H, nqb]
 *   k_codes  int8  [B, H, nk_pad, d]    codes of K' = K - mean; pad tokens hold 0
 *   k_scales fp32  [B, H, nkb]
 *   k_mean   fp32  [B, H, d]
 *   v_codes  uint8 [B, H, nkb, d, 64]   mode 2: E4M3 codes of V, transposed per 64-key tile (element
 *                                       (tile t, channel c, j) is key 64t+j); pad keys hold 0.  NULL otherwise.
 *   v_scales fp32  [B, H, d]            mode 2 only (NULL otherwise)
 *   v_t      bf16  [B, H, nkb, d, 64]   modes 0/1: V transposed per 64-key tile, same order as v_codes;
 *                                       pad keys hold 0.  NULL in mode 2.
 * sattn_quant_layout() fills every pointer from one base address. */
typedef struct {
  int B, H, Nq, Nkv, d, blk_q, blk_k, mode;
  int8_t* q_codes;
  float* q_scales;
  int8_t* k_codes;
  float* k_scales;
  float* k_mean;
  uint8_t* v_codes;
  float* v_scales;
  uint16_t* v_t;
} sattn_quant;

/* Status text for `st` (host pointer to static storage; never NULL). */
const char* sattn_status_string(int st);

/* Width of the key tiles over which the online softmax rescales (64 for every mode and d). */
int sattn_kv_tile(int d, int mode);

/* Bytes needed for the quantized operands of one call (the arrays of sattn_quant, each 256-byte
 * aligned), or 0 if the shape is invalid. */
size_t sattn_quant_bytes(int B, int H, int Nq, int Nkv, int d, int blk_q, int blk_k, int mode);

/* Lays out the arrays of a sattn_quant inside `base` (device memory of at least sattn_quant_bytes).
 * Pure host arithmetic, no device access.  Returns SATTN_ERR_INVALID_ARG for an invalid shape. */
sattn_status sattn_quant_layout(int B, int H, int Nq, int Nkv, int d, int blk_q, int blk_k, int mode, void* base,
                                sattn_quant* out);

/* Workspace bytes for sattn_fwd / sattn_cross_fwd / sattn_fwd_block_sparse: the quantized K and V operands of
 * sattn_quant (the Q codes are left out: these calls quantize each Q block inside the attention kernel, with the
 * same rule and the same codes as sattn_quantize) plus the per-64-token partial sums of the K-mean and V-amax
 * passes; or 0 if the shape is invalid. */
size_t sattn_workspace_bytes(int B, int H, int Nq, int Nkv, int d, int blk_q, int blk_k, int mode);

/* Scratch bytes needed by sattn_quantize (per-64-token K partial sums and V partial maxima). */
size_t sattn_quantize_scratch_bytes(int B, int H, int Nkv, int d, int mode);

/* Quantization of one attention call (modes 1 and 2), or the V transpose alone (mode 0).
 * q: [B,H,Nq,d] bf16, k and v: [B,H,Nkv,d] bf16 (q may be NULL in mode 0).  `out` must describe
 * buffers for the same shape and mode (e.g. from sattn_quant_layout).  `scratch` holds
 * sattn_quantize_scratch_bytes bytes of device memory.  blk_q in {64, 128}; blk_k must be 64. */
sattn_status sattn_quantize(const sattn_tensor* q, const sattn_tensor* k, const sattn_tensor* v, int mode,
                            const sattn_quant* out, void* scratch, size_t scratch_bytes, sattn_stream_t stream);

/* Attention on prepared operands: modes 1/2 read the codes in `qk` (q and k may be NULL); mode 0 reads
 * q and k (bf16) and qk->v_t.  o: [B,H,Nq,d] bf16 output.  sm_scale <= 0 selects 1/sqrt(d). */
sattn_status sattn_fwd_quantized(const sattn_tensor* q, const sattn_tensor* k, const sattn_quant* qk,
                                 const sattn_tensor* o, float sm_scale, int mode, sattn_stream_t stream);

/* Drop-in self-attention: quantize K and V (or transpose V for mode 0) into `ws`, then attend; in modes 1 and 2
 * the attention kernel quantizes each blk_q-row Q block itself (the codes of sattn_quantize, bit for bit), so the
 * result equals sattn_quantize + sattn_fwd_quantized exactly.
 * q, o: [B,H,Nq,d]; k, v: [B,H,Nkv,d]; ws: sattn_workspace_bytes(...) bytes of device memory. */
sattn_status sattn_fwd(const sattn_tensor* q, const sattn_tensor* k, const sattn_tensor* v, const sattn_tensor* o,
                       float sm_scale, int mode, int blk_q, int blk_k, void* ws, size_t ws_bytes,
                       sattn_stream_t stream);

/* sattn_fwd without a caller workspace, for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The workspace is a fixed array of
 * SATTN_NOALLOC_SCRATCH_BYTES bytes inside the library: every GPU the library runs on holds its own copy until the
 * process ends; the call itself allocates nothing.  Arguments and results as sattn_fwd;
 * a shape whose sattn_workspace_bytes exceeds SATTN_NOALLOC_SCRATCH_BYTES returns SATTN_ERR_WORKSPACE (nothing is
 * enqueued).  Every call on one GPU shares that GPU's array and leaves its contents behind (nothing in it needs to
 * start at zero): calls that overlap on one GPU, on concurrent streams or from several host threads, race and must
 * be serialised by the caller.  256 MiB holds, e.g., every mode of a Wan-1.3B 480p self-attention call (H 12,
 * N 32 760, d 128) and a 720p cross-attention call over 769 keys in mode 0. */
#define SATTN_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
sattn_status sattn_fwd_noalloc(const sattn_tensor* q, const sattn_tensor* k, const sattn_tensor* v,
                               const sattn_tensor* o, float sm_scale, int mode, int blk_q, int blk_k,
                               sattn_stream_t stream);

/* Cross-attention of the video tokens (Nq long) over a short key sequence (Nkv small: e.g. 512 text +
 * 257 image tokens of a Wan I2V block, one softmax over their concatenation).  Same arithmetic and
 * workspace as sattn_fwd with blk_q = 128 and blk_k = 64. */
sattn_status sattn_cross_fwd(const sattn_tensor* q, const sattn_tensor* k, const sattn_tensor* v,
                             const sattn_tensor* o, float sm_scale, int mode, void* ws, size_t ws_bytes,
                             sattn_stream_t stream);

/* Block-sparse self-attention: the attention layer computes only the regions a sparse block mask selects
 * (page "视频生成模型的高效推理加速机制解析", section "核心组成与关键能力", item 3 "稀疏注意力", and step 3 of
 * "工作原理与执行流程").  As sattn_fwd, except that the query rows of mask block i (rows SATTN_MASK_QBLK*i ..
 * SATTN_MASK_QBLK*(i+1)-1) attend only to the keys of the key blocks j (keys SATTN_MASK_KBLK*j ..) with
 *   block_mask[((b*H + h)*nqm + i)*nkm + j] != 0,   nqm = ceil(Nq / SATTN_MASK_QBLK), nkm = ceil(Nkv / SATTN_MASK_KBLK).
 * Keys left out take no part in the softmax; query rows whose mask row keeps nothing get O = 0.  Quantization
 * (K mean, scales) still uses every key.  block_mask: device bytes, read only, B*H*nqm*nkm of them.
 * Errors: SATTN_ERR_INVALID_ARG for a NULL mask, SATTN_ERR_UNSUPPORTED for nkm > 32768, else as sattn_fwd. */
#define SATTN_MASK_QBLK 128
#define SATTN_MASK_KBLK 64
sattn_status sattn_fwd_block_sparse(const sattn_tensor* q, const sattn_tensor* k, const sattn_tensor* v,
                                    const sattn_tensor* o, const uint8_t* block_mask, float sm_scale, int mode,
                                    int blk_q, int blk_k, void* ws, size_t ws_bytes, sattn_stream_t stream);

/* Attention-error probe of layer-selective quantization (TMAP I2V write-up, section "保持视频质量": the error of each
 * attention layer over the denoising iterations, against the original precision, decides which layers keep it).
 * For two outputs a and ref of the same shape [B,H,N,d] (bf16, e.g. a quantized-mode call and the mode-0 call on the
 * same inputs), writes per (b, h) the fp64 sums over rows and channels
 *   out[(b*H + h)*4 + 0..3] = sum (a - ref)^2, sum ref^2, sum a*ref, sum a^2
 * (relative L2 error = sqrt(out0 / out1), cosine = out2 / sqrt(out1 * out3)).  out: device memory, 8-byte aligned,
 * B*H*4 doubles.  ws: device memory, 8-byte aligned, at least sattn_error_stats_workspace_bytes(B, H, N) bytes, for
 * the per-chunk partial sums (each head's rows are summed in up to 64 chunks, then the chunks are added).
 * Deterministic: the summation order depends on the shape alone.  Errors: SATTN_ERR_INVALID_ARG for NULL or
 * mismatched tensors or a misaligned out or ws, SATTN_ERR_UNSUPPORTED for d outside {64, 128} or B*H > 65535,
 * SATTN_ERR_WORKSPACE for a NULL or too small ws. */
size_t sattn_error_stats_workspace_bytes(int B, int H, int N); /* 0 for an empty shape */
sattn_status sattn_error_stats(const sattn_tensor* a, const sattn_tensor* ref, double* out, void* ws, size_t ws_bytes,
                               sattn_stream_t stream);

/* ---------------------------------------------------------------------------------------------------------------
 * Quantized linear layer (TMAP I2V write-up, section "FFN性能优化", subsection "线性层量化"): the weights of the
 * linear layers are stored in INT8 with one scale per 128 x 128 block.  W8A8 also quantizes the activations per
 * 128 x 128 block and multiplies in 8 bits; W8A16, the fallback for layers whose quality suffers, keeps bf16
 * activations against the same 8-bit weights.  The layer is y = x W^T + b with x [M, K], W [N, K] (output x input
 * features) and b [N]: the addmm of the model's FLOP profile (section "Attention 性能优化 / 背景").
 * --------------------------------------------------------------------------------------------------------------- */
#define SATTN_LINEAR_BLK 128

typedef enum { SATTN_LINEAR_W8A8 = 0, SATTN_LINEAR_W8A16 = 1 } sattn_linear_mode;

/* Per-block INT8 of a bf16 matrix x [rows, cols] (row stride ld elements).  For every 128 x 128 block (the last row
 * block may be shorter): a = max |v|; a < 2^-100 gives scale 0 and codes 0, else scale = a/127 and
 * code = clamp(rint(v * (127/a)), -127, 127) in fp32 with ties to even.  codes: int8 [rows, cols] dense; scales:
 * float [ceil(rows/128), cols/128] row-major.  Device memory; x and codes 16-byte aligned, scales 4-byte aligned.
 * Prepares a weight once, ahead of the calls that use it.  Errors: SATTN_ERR_INVALID_ARG for a NULL or misaligned
 * pointer, rows < 1, ld < cols or ld not a multiple of 8; SATTN_ERR_UNSUPPORTED for cols not a positive multiple of
 * 128, or rows or cols above 2^28. */
sattn_status sattn_quantize_blocks(const void* x, int rows, int cols, int64_t ld, int8_t* codes, float* scales,
                                   sattn_stream_t stream);

/* Workspace of sattn_linear in bytes: W8A8 the activation codes and their scales (M*K, then
 * 4*ceil(M/128)*(K/128), each part 256-byte aligned), W8A16 the weight codes widened to bf16 (2*N*K).  0 for an
 * invalid shape or mode. */
size_t sattn_linear_workspace_bytes(int M, int N, int K, int mode);

/* W8A8 linear on prepared operands: y[m, n] = sum over the 128-wide K blocks kb of
 * (sx[m/128, kb] * sw[n/128, kb]) * (the exact int32 dot product of the codes over kb) + bias[n], accumulated in
 * fp32 in K-block order and rounded to bf16.  xq: int8 [M, K] dense with sx [ceil(M/128), K/128]; wq: int8 [N, K]
 * dense with sw [ceil(N/128), K/128] (both as written by sattn_quantize_blocks); bias: bf16 [N] or NULL; y: bf16
 * [M, N], row stride ldy (>= N), 2-byte aligned (rows that start 16-byte aligned are written 16 bytes at a time).  K: a positive multiple of 128, at most 2^20.
 * Device memory throughout; allocates nothing.  Errors: SATTN_ERR_INVALID_ARG for NULL or misaligned pointers or a
 * bad stride; SATTN_ERR_UNSUPPORTED for a K outside the above, M or N above 2^28, or more than 2^31 - 1 output
 * tiles of 128 x 128. */
sattn_status sattn_linear_quantized(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw,
                                    const void* bias, void* y, int64_t ldy, int M, int N, int K, sattn_stream_t stream);

/* The quantized linear layer y = x W^T + bias for bf16 activations x [M, K] (row stride ldx, a multiple of 8;
 * 16-byte aligned) and a weight prepared by sattn_quantize_blocks (wq [N, K], sw).
 *   SATTN_LINEAR_W8A8 : x is quantized per 128 x 128 block into the workspace, then as sattn_linear_quantized.
 *   SATTN_LINEAR_W8A16: y[m, n] = sum over kb of sw[n/128, kb] * (x . wq over kb, fp32) + bias[n]; the weight codes
 *                       are widened to bf16 in the workspace (exact), x is used as given.
 * ws: device, 256-byte aligned, at least sattn_linear_workspace_bytes(M, N, K, mode) bytes.  Errors: as
 * sattn_linear_quantized (ldx above 2^23 is SATTN_ERR_UNSUPPORTED), plus SATTN_ERR_INVALID_ARG for an unknown mode
 * and SATTN_ERR_WORKSPACE for a missing or small workspace. */
sattn_status sattn_linear(const void* x, int64_t ldx, const int8_t* wq, const float* sw, const void* bias, void* y,
                          int64_t ldy, int M, int N, int K, int mode, void* ws, size_t ws_bytes, sattn_stream_t stream);

/* Test hook: the int32 scores S = q_codes . k_codes^T of one (b, h) for query rows [q0, q0+nq) and keys
 * [k0, k0+nk), computed with the same INT8 matrix-core path as the attention kernel.
 * out: device int32 [nq, nk] row-major.  Rows/keys must lie inside the padded code arrays. */
sattn_status sattn_debug_qk_int32(const sattn_quant* qk, int b, int h, int q0, int nq, int k0, int nk,
                                  int32_t* out, sattn_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SATTN_H */

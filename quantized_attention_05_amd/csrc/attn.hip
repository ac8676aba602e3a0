// Fused attention kernel of libsattn for CDNA4 (gfx950).
//
// One workgroup = 4 waves = 128 query rows of one (batch, head); each wave owns 32 rows.  The workgroup
// streams 64-key tiles of K and V through LDS and every wave, per tile:
//   1. S^T = K Q^T on the matrix cores: INT8 v_mfma_i32_32x32x32_i8 with int32 accumulation (modes 1, 2),
//      or bf16 v_mfma_f32_32x32x16_bf16 (mode 0).  Computing the transpose puts one query per lane
//      (lanes n and n+32 share query n), so the softmax row statistics are lane-local plus one swap.
//      The rows of the K operand are fed in a permuted order so that lane (n, g) ends up holding keys
//      32g .. 32g+31 of the tile in register order.
//   2. Dequantize and run the online softmax in fp32 (base-2 exponent with c*log2(e) folded into the
//      per-tile scale s_q*s_k*c*log2 e), skipping the O rescale when no running max moved.
//   3. Round P (bf16, or E4M3 of 448*p) straight into the B operand of the P*V matrix-core op
//      (v_mfma_f32_32x32x16_bf16 or v_mfma_f32_32x32x64_f8f6f4 reading E4M3), accumulating O^T in fp32.
// The loop is software-pipelined: the matrix ops of the neighbouring tiles (scores of tile t+1, P*V of tile
// t-1) are interleaved with the softmax of tile t.  K/V tiles move HBM -> LDS with buffer loads that write LDS
// directly (no register staging) into a ring of LDS stages, several tiles ahead, one barrier per tile; the LDS
// rows are XOR-swizzled in 16-byte granules so that every matrix-operand read is free of bank conflicts.  The
// score matrix never leaves registers (tutorial "视频生成推理加速实战:从基线到27倍", step 3, item
// "算子融合与高效注意力"); 8-bit Q*K^T and P*V follow the TMAP I2V write-up (sections "attention量化",
// "显存优化 / 量化"); the per-call mode is its layer-selective precision (section "保持视频质量").
#include <type_traits>

#include "quant_rules.h"
#include "sattn_internal.h"

namespace sattn {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kRowsPerWave = 32;

struct AttnArg {
  TensorArg q, k;      // bf16 inputs (mode 0 only)
  QuantArg qa;         // codes / scales / transposed V
  uint16_t* o;
  int64_t osb, osh, osn;
  float clog2e;        // sm_scale * log2(e)
  int nqt;             // query tiles (32 rows per wave of a workgroup) per (b, h)
  const uint8_t* mask; // block-sparse: [B, H, nqt, nkb] bytes, nonzero = attend to that key tile (else unused)
};

// Operand row slot i (0..31) of a 32-row block, i = 8a + 4g + t, is fed the element that lands in
// register 4a + t of lane half g of the 32x32 output, so lane (n, g) holds elements 32g.. (keys) or
// (D/2)g.. (channels) in register order.
__device__ __forceinline__ int slot_key(int i, int bm) {  // key inside a 64-key tile, 32-key block bm
  return 32 * ((i >> 2) & 1) + 16 * bm + 4 * (i >> 3) + (i & 3);
}
template <int D>
__device__ __forceinline__ int slot_channel(int i, int cb) {  // channel, 32-channel output block cb
  return (D / 2) * ((i >> 2) & 1) + 16 * cb + 4 * (i >> 3) + (i & 3);
}

// XOR swizzles of the 16-byte granules of an LDS row (G granules per row).  For the row sets that the 16
// lanes of a quarter-wave (and the 8 lanes of an eighth) read together, they map equal logical granules
// to distinct bank groups, for 32 and for 64 LDS banks.
template <int G>
__device__ __forceinline__ int kswz(int key) {
  if (G == 4) return (((key >> 1) & 1) ^ ((key >> 2) & 1)) | (((key >> 5) & 1) << 1);
  if (G == 8) return ((key & 1) ^ ((key >> 2) & 1)) | (((key >> 1) & 1) << 1) | (((key >> 5) & 1) << 2);
  return (key & 3) | (((key >> 5) & 1) << 2) | (((key >> 2) & 1) << 3);
}
template <int G, int D>
__device__ __forceinline__ int vswz(int ch) {
  constexpr int gb = (D == 128) ? 6 : 5;  // channel bit that selects the lane half
  if (G == 4) return (((ch >> 1) & 1) ^ ((ch >> 2) & 1)) | (((ch >> gb) & 1) << 1);
  return ((ch & 1) ^ ((ch >> 2) & 1)) | (((ch >> 1) & 1) << 1) | (((ch >> gb) & 1) << 2);
}

template <int MODE, int D>
struct Geo {
  static constexpr int KB = (MODE == 0) ? 2 : 1;  // bytes per K element
  static constexpr int VB = (MODE == 2) ? 1 : 2;  // bytes per V element
  static constexpr int KROW = D * KB;             // bytes of one key row
  static constexpr int VROW = kTile * VB;         // bytes of one (transposed) V channel row
  static constexpr int KG = KROW / 16;            // granules per K row
  static constexpr int VG = VROW / 16;            // granules per V row
  static constexpr int KBYTES = kTile * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int KSTEPS = (MODE == 0) ? D / 16 : D / 32;  // k-steps of the Q*K^T op
  static constexpr int CB = D / 32;                              // 32-channel output blocks
  static constexpr int VREADS = (MODE == 2) ? 2 : 4;             // 16-byte V reads per output block
  static_assert(2 * STAGE <= 65536, "LDS offsets must fit the 16-bit instruction offset");
};

// The workgroup -> (query tile, head, batch) map.  Workgroups are handed to the 8 XCDs round-robin; this
// renumbering gives every XCD one contiguous range of tiles (consecutive query tiles of the same head), so
// the workgroups resident on one XCD stream the same K/V tiles through that XCD's L2.
__device__ __forceinline__ int xcd_remap(int wg, int nwg) {
  const int q = nwg / 8, r = nwg % 8;
  const int xcd = wg % 8, slot = wg / 8;
  return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// ---------------------------------------------------------------------------------------------------------
// The software-pipelined key loop.  Iteration t issues, on the matrix cores, P(t-1) V(t-1) and the scores
// S(t+1) = K(t+1) Q^T, and on the vector ALU the softmax of S(t); the matrix ops are spread through the vector
// instruction stream, so one wave keeps both units busy.  Tiles stream through an LDS ring (Ring below) whose
// loads run DIST iterations ahead of their use.

// Raw buffer over one tile (out-of-range loads return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
// 16 bytes per lane from buffer offset voff into LDS at dst + 16 * lane.
__device__ __forceinline__ void lds_load16_buf(__amdgpu_buffer_rsrc_t r, int voff, uint8_t* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 16, voff, 0, 0, 0);
}
// 4 bytes per lane from buffer offset voff into LDS at dst + 4 * lane.
__device__ __forceinline__ void lds_load4_buf(__amdgpu_buffer_rsrc_t r, int voff, uint8_t* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 4, voff, 0, 0, 0);
}
// Workgroup barrier of the pipelined loop, without the memory-model waits of __syncthreads (whose workgroup
// release would wait for every tile load in flight).  Inside the loop LDS is written only by the tile loads,
// which each wave waits for explicitly (vmcnt) before the barrier.  Every LDS read of a stage must have returned
// before the barrier that precedes its overwrite: the compiler may place the wait for a read's data (at its first
// use) after the barrier, hence the explicit lgkmcnt(0).  The wavefront-scope fences only stop the compiler from
// moving LDS accesses across the barrier.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}
// LDS ring of the pipelined kernel with W waves: R stages of one K tile + one V tile (four when the stages fit the
// 64 KiB that 16-bit LDS instruction offsets reach), loads DIST = R - 1 iterations ahead, one K-scale slot per stage.
template <int MODE, int D, int W>
struct Ring {
  using G = Geo<MODE, D>;
  static constexpr int THREADS = 64 * W;
  static constexpr int KIPW = G::KBYTES / (16 * THREADS);  // 16-byte-per-lane loads per wave: K tile
  static constexpr int VIPW = G::VBYTES / (16 * THREADS);  // V tile
  static constexpr int IPW = KIPW + VIPW;
  static_assert(KIPW * 16 * THREADS == G::KBYTES && VIPW * 16 * THREADS == G::VBYTES, "tiles split into whole loads");
  static constexpr int R = (4 * G::STAGE <= 65536) ? 4 : 2;
  static constexpr int DIST = R - 1;
  static constexpr int SLOT = 256;          // 64 lanes x 4 B (every lane loads the same scale)
  static constexpr int OPS = IPW + (MODE != 0);  // loads per wave per iteration (+ the K scale of the 8-bit modes)
  static constexpr int BYTES = R * G::STAGE + R * SLOT;
  // block-sparse: after the ring, the count of kept key tiles (16 bytes) and their indices (uint16 each)
  static constexpr int LIST_OFF = BYTES;
  static constexpr int MAX_LIST = kMaxSparseTiles;
  static constexpr int SPARSE_BYTES = BYTES + 16 + ((2 * MAX_LIST + 15) / 16) * 16;
};
// Waves per workgroup of the pipelined kernel (two per SIMD either way).  Eight waves would share every K/V tile
// among 256 query rows, but the barrier then couples the two waves of a SIMD and it measured slower than four.
template <int MODE, int D>
constexpr int pipe_waves() {
  return 4;
}
// max / sum of a value over lanes n and n + 32 (one v_permlane32_swap)
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Non-template wrappers of the E4M3 builtins (in template-dependent code the host pass would drop the kernel's
// launch stub).
__device__ __forceinline__ v16f mfma_e4m3(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ int pack_e4m3(float lo0, float lo1, float hi0, float hi1) {
  // the two conversions write the low and the high half of the word, so its prior content is never read: start
  // from whatever the register holds instead of a zeroed one
  int w;
  asm volatile("" : "=v"(w));
  w = __builtin_amdgcn_cvt_pk_fp8_f32(lo0, lo1, w, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(hi0, hi1, w, true);
}

// P of one tile as the B operand of the P*V ops: E4M3 of 448 p (mode 2) or bf16 p (mode 1), keys 32g.. of lane (n, g)
template <int MODE>
struct PTile {
  v8bf b[4];
};
template <>
struct PTile<2> {
  v8i w;
};

// FUSEQ (modes 1 and 2): the kernel quantizes its own Q block from the bf16 Q tensor instead of reading the codes of
// a separate pass.  The workgroup's 128 query rows are exactly one Q block when blk_q = 128 (two when it is 64), so the
// block's amax is one workgroup reduction, and codes and scale follow the same rule as the quantization pass
// (quant_rules.h): a = max|Q| over the block's valid rows, a < 2^-100 -> scale 0 and codes 0, else
// scale = a/127 and code = clamp(rint(x * (127/a)), -127, 127).
template <int MODE, int D, int W, bool SPARSE, bool FUSEQ>
__global__ void __launch_bounds__(64 * W, 8 / W) attn_pipe_kernel(AttnArg a) {
  using G = Geo<MODE, D>;
  using RG = Ring<MODE, D, W>;
  static_assert(!SPARSE || W * kRowsPerWave == kMaskQRows, "one mask row per workgroup query tile");
  static_assert(!FUSEQ || (MODE != 0 && W * kRowsPerWave == 128), "a workgroup quantizes one 128-row Q block");
  using SAcc = std::conditional_t<MODE == 0, v16f, v16i>;  // scores: fp32 (bf16 op) or biased int32 (INT8 op)
  constexpr int CB = G::CB;
  constexpr int KS = G::KSTEPS;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = logical % a.nqt;
  const int h = (logical / a.nqt) % a.qa.H;
  const int b = logical / (a.nqt * a.qa.H);
  const int64_t bh = (int64_t)b * a.qa.H + h;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: LDS load targets stay scalar
  const int n = lane & 31;
  const int g = lane >> 5;
  const int q0 = qt * (W * kRowsPerWave) + wave * kRowsPerWave;
  const bool active = q0 < a.qa.Nq;
  const int nkb = a.qa.nkb;
  const int Nkv = a.qa.Nkv;

  // ---- per-lane load plan: instruction j of this wave fills LDS granules [(W j + wave) * 64, +64)
  int ld_off[RG::IPW];
#pragma unroll
  for (int j = 0; j < RG::IPW; ++j) {
    const int slot = (W * j + wave) * 64 + lane;
    if (j < RG::KIPW) {
      const int key = slot / G::KG, phys = slot % G::KG;
      const int col = (phys ^ kswz<G::KG>(key)) * 16;
      ld_off[j] = (MODE == 0) ? key * (int)a.k.sn * 2 + col : key * G::KROW + col;
    } else {
      const int s = slot - G::KBYTES / 16;
      const int ch = s / G::VG, phys = s % G::VG;
      ld_off[j] = ch * G::VROW + (phys ^ vswz<G::VG, D>(ch)) * 16;
    }
  }
  const uint8_t* ksrc = (MODE == 0) ? reinterpret_cast<const uint8_t*>(a.k.ptr + b * a.k.sb + h * a.k.sh)
                                    : reinterpret_cast<const uint8_t*>(a.qa.k_codes) + bh * nkb * (int64_t)G::KBYTES;
  const uint8_t* vsrc = ((MODE == 2) ? a.qa.v_codes : reinterpret_cast<const uint8_t*>(a.qa.v_t)) +
                        bh * nkb * (int64_t)G::VBYTES;
  auto issue_k = [&](int t, uint8_t* stage) {
    // mode 0: 64 rows of the bf16 K tensor; the buffer ends after the last row in the sequence, so the rows of a
    // ragged tile past it read as zero (their scores are masked)
    const auto r = (MODE == 0) ? tile_rsrc(ksrc + (int64_t)t * kTile * a.k.sn * 2,
                                           ((min(kTile, Nkv - t * kTile) - 1) * (int)a.k.sn + D) * 2)
                               : tile_rsrc(ksrc + (int64_t)t * G::KBYTES, G::KBYTES);
#pragma unroll
    for (int j = 0; j < RG::KIPW; ++j) lds_load16_buf(r, ld_off[j], stage + (W * j + wave) * 1024);
  };
  auto issue_v = [&](int t, uint8_t* stage) {
    const auto r = tile_rsrc(vsrc + (int64_t)t * G::VBYTES, G::VBYTES);
#pragma unroll
    for (int j = RG::KIPW; j < RG::IPW; ++j) lds_load16_buf(r, ld_off[j], stage + (W * j + wave) * 1024);
  };

  // ---- per-lane LDS read offsets of the matrix operands (within a stage)
  int k_rd[2][KS];
#pragma unroll
  for (int bm = 0; bm < 2; ++bm) {
    const int key = slot_key(n, bm);
#pragma unroll
    for (int s = 0; s < KS; ++s) k_rd[bm][s] = key * G::KROW + (((2 * s + g) ^ kswz<G::KG>(key)) * 16);
  }
  int v_rd[CB][G::VREADS];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int ch = slot_channel<D>(n, cb);
#pragma unroll
    for (int e = 0; e < G::VREADS; ++e) {
      const int c = (MODE == 2) ? 2 * g + e : 4 * g + e;
      v_rd[cb][e] = G::KBYTES + ch * G::VROW + ((c ^ vswz<G::VG, D>(ch)) * 16);
    }
  }

  // ---- Q fragment (B operand of S^T = K Q^T), resident for the whole key loop
  v4i qf8[MODE == 0 ? 1 : KS];
  v8bf qfb[MODE == 0 ? KS : 1];
  float fq = 0.0f;  // (s_q *) c * log2(e)
  if constexpr (MODE == 0) {
    const int row = q0 + n;
    const uint16_t* src = a.q.ptr + b * a.q.sb + h * a.q.sh + (int64_t)row * a.q.sn;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (active && row < a.qa.Nq) qfb[s] = *reinterpret_cast<const v8bf*>(src + 16 * s + 8 * g);
      else qfb[s] = (v8bf){};
    }
    fq = a.clog2e;
  } else if constexpr (!FUSEQ) {
    if (active) {
      const int8_t* src = a.qa.q_codes + (bh * a.qa.nqb * a.qa.blk_q + q0 + n) * D;
#pragma unroll
      for (int s = 0; s < KS; ++s) qf8[s] = *reinterpret_cast<const v4i*>(src + 32 * s + 16 * g);
      fq = a.qa.q_scales[bh * a.qa.nqb + q0 / a.qa.blk_q] * a.clog2e;
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) qf8[s] = (v4i){};
    }
  }
  // FUSEQ: this lane's bf16 Q values (row q0 + n, channels 32 s + 16 g ..), loaded now and used once the prologue's
  // tile loads are in flight too (their latencies overlap): the amax goes through LDS, the codes follow the barrier
  __shared__ float qred[FUSEQ ? W : 1];
  uint4 qraw[FUSEQ ? 2 * KS : 1];
  if constexpr (FUSEQ) {
    // a row past the sequence loads the last row instead (always in bounds; no branch around the loads) and is left
    // out of the amax and the codes
    const int row = min(q0 + n, a.qa.Nq - 1);
    const uint16_t* src = a.q.ptr + b * a.q.sb + h * a.q.sh + (int64_t)row * a.q.sn + 16 * g;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qraw[2 * s] = *reinterpret_cast<const uint4*>(src + 32 * s);
      qraw[2 * s + 1] = *reinterpret_cast<const uint4*>(src + 32 * s + 8);
    }
  }
  const float* kscale = (MODE == 0) ? nullptr : a.qa.k_scales + bh * nkb;

  v16f oacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) oacc[cb] = (v16f){};
  float m = -INFINITY;  // running max of x for query n (identical in both lane halves)
  float l = 0.0f;       // this lane's half of the running sum of p (mode 2: of 448 p)

  // The score accumulators start from the bit pattern of the float 1/(2 pi).  |S| <= 128 * 127^2 keeps the
  // int32 sum inside that float's binade [1/8, 1/4), so the result read as a float is 1/(2 pi) + S * 2^-26 and
  // one exact subtraction (Sterbenz) leaves S * 2^-26: cheaper than an int -> float conversion.  Biased values
  // keep the order of S, so the max runs on the integers.
  constexpr int kBias = 0x3E22F983;
  const float bias_f = __int_as_float(kBias);

  // INT8 modes: the bias block lives in registers for the whole loop (the empty asm hides that it is a constant,
  // so the compiler feeds it to the first matrix op of each tile instead of rebuilding it every tile)
  v16i bias_acc = {kBias, kBias, kBias, kBias, kBias, kBias, kBias, kBias,
                   kBias, kBias, kBias, kBias, kBias, kBias, kBias, kBias};
#if defined(__HIP_DEVICE_COMPILE__)
  if constexpr (MODE != 0) asm volatile("" : "+v"(bias_acc));
#endif
  auto qk = [&](const uint8_t* st, SAcc (&acc)[2]) {
    if constexpr (MODE == 0) {
      acc[0] = (v16f){};
      acc[1] = (v16f){};
      // the operands of two k-steps are read before their four matrix ops, so that reads stay in flight while the
      // matrix cores run (read by read, every op waited for its own operand; four k-steps at once spill)
      constexpr int GRP = 2;
#pragma unroll
      for (int s0 = 0; s0 < KS; s0 += GRP) {
        v8bf kv[GRP][2];
#pragma unroll
        for (int s = 0; s < GRP; ++s)
#pragma unroll
          for (int bm = 0; bm < 2; ++bm) kv[s][bm] = *reinterpret_cast<const v8bf*>(st + k_rd[bm][s0 + s]);
#pragma unroll
        for (int s = 0; s < GRP; ++s)
#pragma unroll
          for (int bm = 0; bm < 2; ++bm)
            acc[bm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv[s][bm], qfb[s0 + s], acc[bm], 0, 0, 0);
      }
    } else {
      acc[0] = bias_acc;
      acc[1] = bias_acc;
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int bm = 0; bm < 2; ++bm) {
          const v4i kv = *reinterpret_cast<const v4i*>(st + k_rd[bm][s]);
          acc[bm] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kv, qf8[s], acc[bm], 0, 0, 0);
        }
    }
  };
  auto pv = [&](const uint8_t* st, const PTile<MODE>& p) {
    if constexpr (MODE == 2) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const v4i lo = *reinterpret_cast<const v4i*>(st + v_rd[cb][0]);
        const v4i hi = *reinterpret_cast<const v4i*>(st + v_rd[cb][1]);
        const v8i vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        oacc[cb] = mfma_e4m3(vv, p.w, oacc[cb]);
      }
    } else if constexpr (MODE == 0) {
      // (bf16 scores: the four V reads of a channel block go out before its four matrix ops, as in the scores above)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        v8bf vv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) vv[j] = *reinterpret_cast<const v8bf*>(st + v_rd[cb][j]);
#pragma unroll
        for (int j = 0; j < 4; ++j) oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv[j], p.b[j], oacc[cb], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v8bf vv = *reinterpret_cast<const v8bf*>(st + v_rd[cb][j]);
          oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, p.b[j], oacc[cb], 0, 0, 0);
        }
    }
  };
  // Online softmax (base 2) of one tile: updates m and l, writes P, returns alpha = 2^(m_old - m_new).
  // x = S*f with f >= 0; rounding is monotone, so the tile max of x is f times the max of S.  A lane half
  // without keys in the sequence contributes a value <= 0 that never exceeds the other half's.
  auto softmax = [&](const SAcc (&acc)[2], float f, int valid, PTile<MODE>& p, auto tail_tag) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    auto in_seq = [&](int bm, int r) { return !TAIL || (32 * g + 16 * bm + r < valid); };
    // the score of element (bm, r) as a float: S (bf16 op) or S * 2^-26 (unbiased INT8 result, exact).  Folding the
    // bias into the FMA's addend instead would round that addend (about 2^23 units of S) once per tile; the
    // resulting shift flips E4M3 roundings of P often enough to be visible in O, so the subtraction stays exact.
    auto score = [&](int bm, int r) {
      if constexpr (MODE == 0) return acc[bm][r];
      else return __int_as_float(acc[bm][r]) - bias_f;
    };
    float smax;  // tile max of S (in S units); a lane half without keys in the sequence gives a value <= 0
    if constexpr (MODE == 0) {
      float fm[4] = {-3.0e38f, -3.0e38f, -3.0e38f, -3.0e38f};
#pragma unroll
      for (int bm = 0; bm < 2; ++bm)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (in_seq(bm, r)) fm[(2 * bm + r) & 3] = fmaxf(fm[(2 * bm + r) & 3], acc[bm][r]);
      smax = fmaxf(fmaxf(fm[0], fm[1]), fmaxf(fm[2], fm[3]));
    } else {
      int im[4] = {kBias - (1 << 30), kBias - (1 << 30), kBias - (1 << 30), kBias - (1 << 30)};
#pragma unroll
      for (int bm = 0; bm < 2; ++bm)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (in_seq(bm, r)) im[(2 * bm + r) & 3] = max(im[(2 * bm + r) & 3], acc[bm][r]);
      smax = (float)(max(max(im[0], im[1]), max(im[2], im[3])) - kBias);
    }
    const float xmax = halves_max(smax * f);
    const float mnew = fmaxf(m, xmax);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);  // 0 on the first tile (m = -inf), 1 if m is unchanged
    const float fe = (MODE == 0) ? f : f * 0x1p26f;         // scale of the stored scores
    // mode 2 keeps 448 p (= 2^(x - m + log2 448)) so that the E4M3 conversion needs no multiply
    const float nb = ((MODE == 2) ? 8.807354922057604f : 0.0f) - mnew;
    float lp[4];
    if constexpr (MODE == 2) {
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int bm = w >> 2, r0 = 4 * (w & 3);
        float pe[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(score(bm, r0 + e), fe, nb));
          if (!in_seq(bm, r0 + e)) pe[e] = 0.0f;
          lp[e] = (w == 0) ? pe[e] : lp[e] + pe[e];
        }
        p.w[w] = pack_e4m3(pe[0], pe[1], pe[2], pe[3]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int bm = j >> 1, r0 = 8 * (j & 1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(score(bm, r0 + e), fe, nb));
          if (!in_seq(bm, r0 + e)) pe = 0.0f;
          lp[e & 3] = (j == 0 && e < 4) ? pe : lp[e & 3] + pe;
          p.b[j][e] = (__bf16)pe;
        }
      }
    }
    l = l * alpha + ((lp[0] + lp[1]) + (lp[2] + lp[3]));
    m = mnew;
    return alpha;
  };

  // ---- the key tiles this workgroup attends to, in ascending order: all nkb of them, or (block-sparse) the tiles
  // its mask row keeps, listed in LDS by wave 0.  Iteration i of the loop below handles tile tile_of(i).
  int ntile = nkb;
  const uint16_t* list = reinterpret_cast<const uint16_t*>(smem + RG::LIST_OFF + 16);
  if constexpr (SPARSE) {
    if (wave == 0) {
      uint16_t* wlist = reinterpret_cast<uint16_t*>(smem + RG::LIST_OFF + 16);
      const uint8_t* mrow = a.mask + ((int64_t)bh * a.nqt + qt) * nkb;
      int cnt = 0;
      for (int base = 0; base < nkb; base += 64) {
        const int j = base + lane;
        const bool keep = j < nkb && mrow[j] != 0;
        const uint64_t bal = __ballot(keep);
        if (keep) wlist[cnt + __popcll(bal & ((1ull << lane) - 1ull))] = (uint16_t)j;
        cnt += __popcll(bal);
      }
      if (lane == 0) *reinterpret_cast<int*>(smem + RG::LIST_OFF) = cnt;
    }
    __syncthreads();
    ntile = __builtin_amdgcn_readfirstlane(*reinterpret_cast<const int*>(smem + RG::LIST_OFF));
    if (ntile == 0) {  // nothing to attend to: O = 0 (uniform over the workgroup, no load in flight)
      const int row = q0 + n;
      if (active && row < a.qa.Nq) {
        uint4* dst = reinterpret_cast<uint4*>(a.o + b * a.osb + h * a.osh + (int64_t)row * a.osn + (D / 2) * g);
#pragma unroll
        for (int i = 0; i < D / 16; ++i) dst[i] = make_uint4(0, 0, 0, 0);
      }
      return;
    }
  }
  auto tile_of = [&](int i) -> int {
    if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane(list[i]);
    else return i;
  };

  // ---- LDS ring of R stages.  Iteration i reads stage i % R: K and the K block scale of tile_of(i+1) and V of
  // tile_of(i-1); it loads K and the scale of tile_of(i+1+DIST) and V of tile_of(i-1+DIST) into stage
  // (i+DIST) % R, whose last reader was iteration i-1.  The loads of a stage therefore have DIST iterations to land.
  constexpr int R = RG::R, DIST = RG::DIST;
  uint8_t* const slots = smem + R * G::STAGE;  // per-stage K scale slots (RG::SLOT bytes each)
  auto issue_s = [&](int t, uint8_t* slot) {
    if constexpr (MODE != 0) lds_load4_buf(tile_rsrc(kscale + t, 4), 0, slot);
  };
  auto wait_loads = [&]() {  // every load issued before the last DIST - 1 iterations has landed
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((DIST - 1) * RG::OPS) : "memory");
  };

  // ---- one iteration: P V of the previous tile, S of the next one (if NEXT) and the softmax of this one, then
  // the O rescale
  float ks = 0.0f;  // K block scale of the tile whose softmax comes next
  auto step = [&](int i, int srd, const SAcc (&scur)[2], SAcc (&snext)[2], const PTile<MODE>& pprev,
                  PTile<MODE>& pcur, auto tail_tag, auto next_tag) __attribute__((always_inline)) {
    constexpr bool NEXT = decltype(next_tag)::value;
    const float f = fq * ks;  // (also completes this wave's read of the scale slot that is reloaded below)
    wait_loads();
    ring_barrier();  // stage srd is visible to every wave; every wave is done with stage (srd + DIST) % R
    const int swr = (srd + DIST) % R;
    // past the end these reload the last tile, which nothing reads again
    issue_k(tile_of(min(i + 1 + DIST, ntile - 1)), smem + swr * G::STAGE);
    issue_v(tile_of(min(i - 1 + DIST, ntile - 1)), smem + swr * G::STAGE);
    issue_s(tile_of(min(i + 1 + DIST, ntile - 1)), slots + swr * RG::SLOT);
    const uint8_t* rd = smem + srd * G::STAGE;
    if constexpr (NEXT && MODE != 0) ks = *reinterpret_cast<const float*>(slots + srd * RG::SLOT);
    pv(rd, pprev);
    if constexpr (NEXT) qk(rd, snext);
    const float mold = m;
    const float alpha = softmax(scur, f, Nkv - tile_of(i) * kTile, pcur, tail_tag);
    // Keep P and l computed here, in the same scheduling region as the matrix ops above, rather than sunk past
    // the rescale branch (an empty asm reading them; device pass only, its register constraints are the GPU's).
    // Within the region the compiler's own scheduler interleaves the matrix ops with the softmax; explicit
    // scheduling groups measured slower.
#if defined(__HIP_DEVICE_COMPILE__)
    if constexpr (MODE == 2) asm volatile("" ::"v"(pcur.w), "v"(l));
    else asm volatile("" ::"v"(pcur.b[0]), "v"(pcur.b[1]), "v"(pcur.b[2]), "v"(pcur.b[3]), "v"(l));
#endif
    if (i > 0 && __any(m != mold)) {  // (on the first tile the accumulator is still zero)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
    }
  };

  if constexpr (MODE == 0 && D == 128 && !SPARSE) {
    // ---- dense bf16 at d = 128: one tile per iteration, without the software pipeline.  Stage i % R holds K and V
    // of tile i; iteration i loads tile i + DIST into stage (i + DIST) % R, whose last reader was iteration i - 1.
    // At this instance's register count the compiler issues a step's matrix ops ahead of its softmax whichever form
    // the loop takes, so the pipeline's second score and P buffers (48 registers) bought nothing here.  (At d = 64
    // and with a block-sparse mask this form takes more registers than the pipelined one.)
#pragma unroll
    for (int j = 0; j < DIST; ++j) {
      issue_k(tile_of(min(j, ntile - 1)), smem + j * G::STAGE);
      issue_v(tile_of(min(j, ntile - 1)), smem + j * G::STAGE);
    }
    // iteration `it` from stage SRD (TAIL: the sequence's ragged last tile)
    auto one = [&](int it, auto slot_tag, auto tail_tag) __attribute__((always_inline)) {
      constexpr int SRD = decltype(slot_tag)::value;
      constexpr int SWR = (SRD + DIST) % R;
      wait_loads();
      ring_barrier();  // stage SRD is visible to every wave; every wave is done with stage SWR
      // past the end these reload the last tile, which nothing reads again
      issue_k(tile_of(min(it + DIST, ntile - 1)), smem + SWR * G::STAGE);
      issue_v(tile_of(min(it + DIST, ntile - 1)), smem + SWR * G::STAGE);
      const uint8_t* rd = smem + SRD * G::STAGE;
      SAcc sc[2];
      qk(rd, sc);
      PTile<MODE> pc;
      const float mold = m;
      const float alpha = softmax(sc, fq, Nkv - tile_of(it) * kTile, pc, tail_tag);
      if (it > 0 && __any(m != mold)) {  // (on the first tile the accumulator is still zero)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
      }
      pv(rd, pc);
    };
    auto at_slot = [&](int it, auto tail_tag) __attribute__((always_inline)) {
      static_assert(R <= 4, "stage offsets are compile-time for up to four stages");
      const int sl = it % R;
      if (sl == 0) one(it, std::integral_constant<int, 0>{}, tail_tag);
      else if (sl == 1) one(it, std::integral_constant<int, 1 % R>{}, tail_tag);
      else if (sl == 2) one(it, std::integral_constant<int, 2 % R>{}, tail_tag);
      else one(it, std::integral_constant<int, 3 % R>{}, tail_tag);
    };
    // groups of R iterations with constant stage offsets, the rest one by one; only the sequence's last tile can be
    // ragged
    const int nlast = ntile - 1;
    int it = 0;
    static_assert(R == 2 || R == 4, "two or four stages");
    for (; it + R <= nlast; it += R) {
      one(it, std::integral_constant<int, 0>{}, std::false_type{});
      one(it + 1, std::integral_constant<int, 1>{}, std::false_type{});
      if constexpr (R == 4) {
        one(it + 2, std::integral_constant<int, 2 % R>{}, std::false_type{});
        one(it + 3, std::integral_constant<int, 3 % R>{}, std::false_type{});
      }
    }
    for (; it < nlast; ++it) at_slot(it, std::false_type{});
    if (Nkv % kTile && tile_of(it) == nkb - 1) at_slot(it, std::true_type{});
    else at_slot(it, std::false_type{});
  } else {
    // ---- prologue.  The V half of stage 0 ("tile -1", read with P = 0 by the first iteration) is zeroed before any
    // tile load is in flight: an LDS store issued while a direct-to-LDS load is pending would wait for all of them.
    // Then K of the first tile and its scale go to stage DIST, first, so that the first scores wait for them alone,
    // and then stages 0 .. DIST-1 as iterations 0 .. DIST-1 expect them.
    static_assert(G::VBYTES % (16 * RG::THREADS) == 0, "the V tile splits into whole 16-byte stores per thread");
  #pragma unroll
    for (int j = 0; j < G::VBYTES / (16 * RG::THREADS); ++j)
      *reinterpret_cast<uint4*>(smem + G::KBYTES + 16 * (j * RG::THREADS + (int)threadIdx.x)) = make_uint4(0, 0, 0, 0);
    issue_k(tile_of(0), smem + DIST * G::STAGE);
    issue_s(tile_of(0), slots + DIST * RG::SLOT);
  #pragma unroll
    for (int j = 0; j < DIST; ++j) {
      issue_k(tile_of(min(j + 1, ntile - 1)), smem + j * G::STAGE);
      if (j > 0) issue_v(tile_of(min(j - 1, ntile - 1)), smem + j * G::STAGE);
      issue_s(tile_of(min(j + 1, ntile - 1)), slots + j * RG::SLOT);
    }
    // loads of this wave issued after the first K tile and its scale: stage 0 (K and scale), stages 1 .. DIST-1
    constexpr int kAfterFirst = RG::KIPW + (MODE != 0) + (DIST - 1) * RG::OPS;
    static_assert(kAfterFirst < 64, "the wait count fits vmcnt");
    PTile<MODE> pa = {}, pb = {};
    SAcc sa[2], sb[2];
    if constexpr (FUSEQ) {  // the wave's part of the Q block's amax
      // (nothing moves above this point: the use of the Q values, and the wait for them, stays after the tile loads
      // above are issued)
      __builtin_amdgcn_sched_barrier(0);
      float am = 0.0f;
  #pragma unroll
      for (int j = 0; j < 2 * KS; ++j) {
        float f[8];
        unpack8(qraw[j], f);
  #pragma unroll
        for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(f[i]));
      }
      if (q0 + n >= a.qa.Nq) am = 0.0f;  // (a row past the sequence holds a copy of the last row)
  #pragma unroll
      for (int off = 32; off > 0; off >>= 1) am = fmaxf(am, __shfl_xor(am, off, 64));
      if (lane == 0) qred[wave] = am;  // read after the barrier below
    }
    // this wave's loads up to the first K tile and its scale (and the Q rows before them) have landed; after the
    // barrier, every wave's have
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kAfterFirst) : "memory");
    ring_barrier();
    if constexpr (FUSEQ) {
      // the block's amax: all W waves (blk_q = 128) or this wave's pair (blk_q = 64, two blocks per workgroup)
      float am;
      if (a.qa.blk_q == 128) {
        am = qred[0];
  #pragma unroll
        for (int w = 1; w < W; ++w) am = fmaxf(am, qred[w]);
      } else {
        am = fmaxf(qred[wave & ~1], qred[wave | 1]);
      }
      const bool zero = !(am >= kGuard);
      const float inv = zero ? 0.0f : 127.0f / am;
      fq = (zero ? 0.0f : am / 127.0f) * a.clog2e;
      const bool row_ok = !zero && q0 + n < a.qa.Nq;
  #pragma unroll
      for (int s = 0; s < KS; ++s) {
        int wv[4];
  #pragma unroll
        for (int j = 0; j < 2; ++j) {
          float f[8];
          unpack8(qraw[2 * s + j], f);
          uint32_t lo = 0, hi = 0;
          if (row_ok) {
            lo = codes4(f, inv);
            hi = codes4(f + 4, inv);
          }
          wv[2 * j] = (int)lo;
          wv[2 * j + 1] = (int)hi;
        }
        qf8[s] = (v4i){wv[0], wv[1], wv[2], wv[3]};
      }
    }
    ks = (MODE == 0) ? 1.0f : *reinterpret_cast<const float*>(slots + DIST * RG::SLOT);
    qk(smem + DIST * G::STAGE, sa);

    // ---- iterations 0 .. ntile-2 have a next tile; groups of R run with constant stage offsets
    const int nmain = ntile - 1;
    int i = 0;
    for (; i + R <= nmain; i += R) {
      step(i, 0, sa, sb, pa, pb, std::false_type{}, std::true_type{});
      step(i + 1, 1, sb, sa, pb, pa, std::false_type{}, std::true_type{});
      if constexpr (R == 4) {
        step(i + 2, 2, sa, sb, pa, pb, std::false_type{}, std::true_type{});
        step(i + 3, 3, sb, sa, pb, pa, std::false_type{}, std::true_type{});
      }
    }
    for (; i < nmain; ++i) {
      step(i, i % R, sa, sb, pa, pb, std::false_type{}, std::true_type{});
      sa[0] = sb[0];
      sa[1] = sb[1];
      pa = pb;
    }
    // i = ntile - 1: the last tile; only the sequence's last tile can be ragged
    if (Nkv % kTile && tile_of(i) == nkb - 1) step(i, i % R, sa, sb, pa, pb, std::true_type{}, std::false_type{});
    else step(i, i % R, sa, sb, pa, pb, std::false_type{}, std::false_type{});
    wait_loads();
    ring_barrier();
    pv(smem + (ntile % R) * G::STAGE, pb);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no tile load may still be writing LDS when the wave exits

  // ---------------- epilogue: O = acc / l  (mode 2: acc * s_v[c] / (448 l)), bf16, lane writes D/2 channels
  const float ltot = halves_sum(l);
  const int row = q0 + n;
  if (!active || row >= a.qa.Nq) return;
  const float inv = 1.0f / ltot;
  uint16_t* dst = a.o + b * a.osb + h * a.osh + (int64_t)row * a.osn + (D / 2) * g;
  const float* vs = (MODE == 2) ? a.qa.v_scales + bh * D + (D / 2) * g : nullptr;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    uint32_t w[8];
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      float o0 = oacc[cb][e] * inv, o1 = oacc[cb][e + 1] * inv;
      if (MODE == 2) {
        o0 *= vs[16 * cb + e];
        o1 *= vs[16 * cb + e + 1];
      }
      const __bf16 h0 = (__bf16)o0, h1 = (__bf16)o1;
      w[e / 2] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    }
    *reinterpret_cast<uint4*>(dst + 16 * cb) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint4*>(dst + 16 * cb + 8) = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

// Int32 scores of a window, through the same operand layout as attn_pipe_kernel (one wave per 32x64 block).
template <int D>
__global__ void __launch_bounds__(64) debug_qk_kernel(QuantArg qa, int64_t bh, int q0, int nq, int k0, int nk,
                                                       int32_t* out) {
  constexpr int KSTEPS = D / 32;
  constexpr int KROW = D + 16;
  __shared__ __attribute__((aligned(16))) uint8_t kl[kTile * KROW];
  const int lane = threadIdx.x, n = lane & 31, g = lane >> 5;
  const int rq = q0 + blockIdx.x * 32;  // first query row of this block
  const int rk = k0 + blockIdx.y * 64;  // first key of this block
  const int nq_pad = qa.nqb * qa.blk_q, nk_pad = qa.nkb * kTile;
  // K rows -> LDS (rows outside the padded array read as zero)
  for (int p = lane; p < kTile * D / 16; p += 64) {
    const int key = p / (D / 16), col = (p % (D / 16)) * 16;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (rk + key < nk_pad) v = *reinterpret_cast<const uint4*>(qa.k_codes + (bh * nk_pad + rk + key) * D + col);
    *reinterpret_cast<uint4*>(kl + key * KROW + col) = v;
  }
  __syncthreads();
  v4i qf[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    qf[s] = (v4i){};
    if (rq + n < nq_pad) qf[s] = *reinterpret_cast<const v4i*>(qa.q_codes + (bh * nq_pad + rq + n) * D + 32 * s + 16 * g);
  }
#pragma unroll
  for (int bm = 0; bm < 2; ++bm) {
    const int key = slot_key(n, bm);
    v16i acc = {};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const v4i kv = *reinterpret_cast<const v4i*>(kl + key * KROW + 32 * s + 16 * g);
      acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kv, qf[s], acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qi = blockIdx.x * 32 + n, kj = blockIdx.y * 64 + 32 * g + 16 * bm + r;
      if (qi < nq && kj < nk) out[(int64_t)qi * nk + kj] = acc[r];
    }
  }
}

// The kernel instance of a call: dense or block-sparse, Q codes read or quantized in the kernel (modes 1 and 2).
template <int MODE, int D>
const void* attn_kernel_for(bool sparse, bool fuse_q) {
  constexpr int W = pipe_waves<MODE, D>();
  if constexpr (MODE == 0) {
    return sparse ? reinterpret_cast<const void*>(&attn_pipe_kernel<MODE, D, W, true, false>)
                  : reinterpret_cast<const void*>(&attn_pipe_kernel<MODE, D, W, false, false>);
  } else {
    if (sparse)
      return fuse_q ? reinterpret_cast<const void*>(&attn_pipe_kernel<MODE, D, W, true, true>)
                    : reinterpret_cast<const void*>(&attn_pipe_kernel<MODE, D, W, true, false>);
    return fuse_q ? reinterpret_cast<const void*>(&attn_pipe_kernel<MODE, D, W, false, true>)
                  : reinterpret_cast<const void*>(&attn_pipe_kernel<MODE, D, W, false, false>);
  }
}

template <int MODE, int D>
hipError_t launch_attn_t(AttnArg a, bool fuse_q, hipStream_t s) {
  constexpr int W = pipe_waves<MODE, D>();
  using RG = Ring<MODE, D, W>;
  const bool sparse = a.mask != nullptr;
  // dense: the ring; block-sparse: the ring + the tile list (sized for this call's key tiles)
  const int bytes = sparse ? RG::LIST_OFF + 16 + cdiv(2 * a.qa.nkb, 16) * 16 : RG::BYTES;
  a.nqt = cdiv(a.qa.Nq, W * kRowsPerWave);
  const int64_t nwg = (int64_t)a.nqt * a.qa.H * a.qa.B;  // below 2^31 by the host's shape checks
  void* args[] = {&a};
  const hipError_t e = hipLaunchKernel(attn_kernel_for<MODE, D>(sparse, fuse_q), dim3((unsigned)nwg), dim3(64 * W),
                                       args, bytes, s);
  return e != hipSuccess ? e : hipGetLastError();
}

// The dynamic LDS limit of the kernel a call will launch (more than the default 64 KiB in mode 2), set on the current
// device before anything is enqueued.  Set on every call rather than remembered, so that no state is kept and a
// second GPU of the process gets it too.
template <int MODE, int D>
hipError_t prepare_attn_t(bool sparse, bool fuse_q) {
  using RG = Ring<MODE, D, pipe_waves<MODE, D>()>;
  return hipFuncSetAttribute(attn_kernel_for<MODE, D>(sparse, fuse_q), hipFuncAttributeMaxDynamicSharedMemorySize,
                             sparse ? RG::SPARSE_BYTES : RG::BYTES);
}

}  // namespace

hipError_t launch_attn(int mode, const TensorArg& q, const TensorArg& k, const QuantArg& qa, uint16_t* o, int64_t osb,
                       int64_t osh, int64_t osn, float sm_scale, const uint8_t* mask, bool fuse_q, hipStream_t s) {
  AttnArg a;
  a.q = q;
  a.k = k;
  a.qa = qa;
  a.o = o;
  a.osb = osb;
  a.osh = osh;
  a.osn = osn;
  a.clog2e = sm_scale * 1.4426950408889634f;
  a.mask = mask;
  if (qa.d == 128) {
    if (mode == 0) return launch_attn_t<0, 128>(a, fuse_q, s);
    if (mode == 1) return launch_attn_t<1, 128>(a, fuse_q, s);
    return launch_attn_t<2, 128>(a, fuse_q, s);
  }
  if (mode == 0) return launch_attn_t<0, 64>(a, fuse_q, s);
  if (mode == 1) return launch_attn_t<1, 64>(a, fuse_q, s);
  return launch_attn_t<2, 64>(a, fuse_q, s);
}

hipError_t prepare_attn(int mode, int d, bool sparse, bool fuse_q) {
  if (d == 128) {
    if (mode == 0) return prepare_attn_t<0, 128>(sparse, fuse_q);
    if (mode == 1) return prepare_attn_t<1, 128>(sparse, fuse_q);
    return prepare_attn_t<2, 128>(sparse, fuse_q);
  }
  if (mode == 0) return prepare_attn_t<0, 64>(sparse, fuse_q);
  if (mode == 1) return prepare_attn_t<1, 64>(sparse, fuse_q);
  return prepare_attn_t<2, 64>(sparse, fuse_q);
}

int attn_rows_per_workgroup() { return 4 * kRowsPerWave; }

hipError_t launch_debug_qk(const QuantArg& qa, int b, int h, int q0, int nq, int k0, int nk, int32_t* out,
                           hipStream_t s) {
  dim3 grid(cdiv(nq, 32), cdiv(nk, 64));
  const int64_t bh = (int64_t)b * qa.H + h;
  if (qa.d == 128) debug_qk_kernel<128><<<grid, 64, 0, s>>>(qa, bh, q0, nq, k0, nk, out);
  else debug_qk_kernel<64><<<grid, 64, 0, s>>>(qa, bh, q0, nq, k0, nk, out);
  return hipGetLastError();
}

}  // namespace sattn

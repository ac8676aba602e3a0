// Fused attention kernels of libsattn for CDNA4 (gfx950).
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
// K/V tiles move HBM -> LDS with global_load_lds_dwordx4 (no register staging), two stages, one barrier
// per tile; the LDS rows are XOR-swizzled in 16-byte granules so that every matrix-operand read is free of
// bank conflicts.  The score matrix never leaves registers (tutorial "视频生成推理加速实战:从基线到27倍",
// step 3, item "算子融合与高效注意力"); 8-bit Q*K^T and P*V follow the TMAP I2V write-up (sections
// "attention量化", "显存优化 / 量化"); the per-call mode is its layer-selective precision (section
// "保持视频质量").
#include <type_traits>

#include "sattn_internal.h"

namespace sattn {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerWG = kWaves * kRowsPerWave;  // 128

struct AttnArg {
  TensorArg q, k;      // bf16 inputs (mode 0 only)
  QuantArg qa;         // codes / scales / transposed V
  uint16_t* o;
  int64_t osb, osh, osn;
  float clog2e;        // sm_scale * log2(e)
  int nqt;             // query tiles of 128 rows per (b, h)
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
  static constexpr int KIPW = KBYTES / (16 * 256);  // load instructions per wave for K (4 waves x 64 lanes)
  static constexpr int VIPW = VBYTES / (16 * 256);
  static constexpr int IPW = KIPW + VIPW;
  static constexpr int KSTEPS = (MODE == 0) ? D / 16 : D / 32;  // k-steps of the Q*K^T op
  static constexpr int CB = D / 32;                              // 32-channel output blocks
  static constexpr int VREADS = (MODE == 2) ? 2 : 4;             // 16-byte V reads per output block
  static_assert(KBYTES % (16 * 256) == 0 && VBYTES % (16 * 256) == 0, "tiles split into whole instructions");
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

template <int MODE, int D>
__global__ void __launch_bounds__(256, 2) attn_kernel(AttnArg a) {
  using G = Geo<MODE, D>;
  constexpr int CB = G::CB;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = logical % a.nqt;
  const int h = (logical / a.nqt) % a.qa.H;
  const int b = logical / (a.nqt * a.qa.H);
  const int64_t bh = (int64_t)b * a.qa.H + h;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 31;  // query of this lane inside the wave's 32 rows
  const int g = lane >> 5;  // lane half
  const int q0 = qt * kRowsPerWG + wave * kRowsPerWave;
  const bool active = q0 < a.qa.Nq;
  const int nkb = a.qa.nkb;
  const int Nkv = a.qa.Nkv;

  // ---- per-lane load plan: instruction j of this wave fills LDS granules [(4j + wave) * 64, +64)
  int ld_off[G::IPW];  // byte offset inside the tile's source (K rows of mode 0: key and column instead)
  int ld_key[G::KIPW];
#pragma unroll
  for (int j = 0; j < G::IPW; ++j) {
    const int slot = (4 * j + wave) * 64 + lane;
    if (j < G::KIPW) {
      const int key = slot / G::KG, phys = slot % G::KG;
      const int col = phys ^ kswz<G::KG>(key);
      ld_key[j] = key;
      ld_off[j] = (MODE == 0) ? col * 16 : key * G::KROW + col * 16;
    } else {
      const int s = slot - G::KBYTES / 16;
      const int ch = s / G::VG, phys = s % G::VG;
      const int col = phys ^ vswz<G::VG, D>(ch);
      ld_off[j] = ch * G::VROW + col * 16;
    }
  }
  const uint8_t* ksrc = (MODE == 0) ? reinterpret_cast<const uint8_t*>(a.k.ptr + b * a.k.sb + h * a.k.sh)
                                    : reinterpret_cast<const uint8_t*>(a.qa.k_codes) + bh * nkb * (int64_t)G::KBYTES;
  const uint8_t* vsrc = ((MODE == 2) ? a.qa.v_codes : reinterpret_cast<const uint8_t*>(a.qa.v_t)) +
                        bh * nkb * (int64_t)G::VBYTES;

  auto issue_tile = [&](int t, int stage) {
    uint8_t* dst = smem + stage * G::STAGE;
#pragma unroll
    for (int j = 0; j < G::IPW; ++j) {
      const uint8_t* src;
      if (j < G::KIPW) {
        if (MODE == 0) {
          const int row = min(t * kTile + ld_key[j], Nkv - 1);  // rows past the sequence are masked later
          src = ksrc + (int64_t)row * a.k.sn * 2 + ld_off[j];
        } else {
          src = ksrc + (int64_t)t * G::KBYTES + ld_off[j];
        }
      } else {
        src = vsrc + (int64_t)t * G::VBYTES + ld_off[j];
      }
      __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(dst + (4 * j + wave) * 64 * 16), 16, 0, 0);
    }
  };

  // ---- per-lane LDS read offsets of the matrix operands (within a stage)
  int k_rd[2][G::KSTEPS];
#pragma unroll
  for (int bm = 0; bm < 2; ++bm) {
    const int key = slot_key(n, bm);
#pragma unroll
    for (int s = 0; s < G::KSTEPS; ++s) k_rd[bm][s] = key * G::KROW + (((2 * s + g) ^ kswz<G::KG>(key)) * 16);
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
  v4i qf8[MODE == 0 ? 1 : G::KSTEPS];
  v8bf qfb[MODE == 0 ? G::KSTEPS : 1];
  float fq = 0.0f;  // s_q * c * log2(e)
  if (MODE == 0) {
    const int row = q0 + n;
    const uint16_t* src = a.q.ptr + b * a.q.sb + h * a.q.sh + (int64_t)row * a.q.sn;
#pragma unroll
    for (int s = 0; s < G::KSTEPS; ++s) {
      if (active && row < a.qa.Nq) qfb[s] = *reinterpret_cast<const v8bf*>(src + 16 * s + 8 * g);
      else qfb[s] = (v8bf){};
    }
    fq = a.clog2e;
  } else {
    if (active) {
      const int8_t* src = a.qa.q_codes + (bh * a.qa.nqb * a.qa.blk_q + q0 + n) * D;
#pragma unroll
      for (int s = 0; s < G::KSTEPS; ++s) qf8[s] = *reinterpret_cast<const v4i*>(src + 32 * s + 16 * g);
      fq = a.qa.q_scales[bh * a.qa.nqb + q0 / a.qa.blk_q] * a.clog2e;
    } else {
#pragma unroll
      for (int s = 0; s < G::KSTEPS; ++s) qf8[s] = (v4i){};
    }
  }
  const float* kscale = a.qa.k_scales + bh * nkb;

  v16f oacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) oacc[cb] = (v16f){};
  float m = -INFINITY;  // running max of x for query n (identical in both lane halves)
  float l = 0.0f;       // this lane's half of the running sum of p (mode 2: of 448 p)

  auto process = [&](const uint8_t* st, int t, auto tail_tag) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    const int valid = Nkv - t * kTile;  // keys of this tile inside the sequence (>= 64 unless TAIL)
    auto in_seq = [&](int bm, int r) { return !TAIL || (32 * g + 16 * bm + r < valid); };

    // ---------------- 1. scores of 64 keys x 32 queries: two independent accumulation chains
    float sf[2][16];
    float smax;
    if (MODE == 0) {
      v16f acc[2] = {(v16f){}, (v16f){}};
#pragma unroll
      for (int s = 0; s < G::KSTEPS; ++s)
#pragma unroll
        for (int bm = 0; bm < 2; ++bm) {
          const v8bf kv = *reinterpret_cast<const v8bf*>(st + k_rd[bm][s]);
          acc[bm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, qfb[s], acc[bm], 0, 0, 0);
        }
      smax = -3.0e38f;
#pragma unroll
      for (int bm = 0; bm < 2; ++bm)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sf[bm][r] = acc[bm][r];
          if (in_seq(bm, r)) smax = fmaxf(smax, sf[bm][r]);
        }
    } else {
      v16i acc[2] = {(v16i){}, (v16i){}};
#pragma unroll
      for (int s = 0; s < G::KSTEPS; ++s)
#pragma unroll
        for (int bm = 0; bm < 2; ++bm) {
          const v4i kv = *reinterpret_cast<const v4i*>(st + k_rd[bm][s]);
          acc[bm] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kv, qf8[s], acc[bm], 0, 0, 0);
        }
      int imax = -0x7FFFFFFF;
#pragma unroll
      for (int bm = 0; bm < 2; ++bm)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (in_seq(bm, r)) imax = max(imax, acc[bm][r]);
#pragma unroll
      for (int bm = 0; bm < 2; ++bm)
#pragma unroll
        for (int r = 0; r < 16; ++r) sf[bm][r] = (float)acc[bm][r];  // exact: |S| < 2^24
      smax = (float)imax;  // a half with no key in the sequence gives -2^31, scaled below like the rest
    }

    // ---------------- 2. online softmax (base 2).  x = S*f with f >= 0; rounding is monotone, so the
    // tile max of x is f times the max of S.  A lane half without keys contributes a value <= 0 that never
    // exceeds the other half's (for f = 0 every x is 0).
    const float f = (MODE == 0) ? fq : fq * kscale[t];
    float xmax = smax * f;
    xmax = fmaxf(xmax, __shfl_xor(xmax, 32, 64));
    const float mnew = fmaxf(m, xmax);
    if (__any(mnew != m)) {
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);  // 0 on the first tile (m = -inf)
      l *= alpha;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
    }
    m = mnew;
    // mode 2 keeps 448 p (= 2^(x - m + log2 448)) so that the E4M3 conversion needs no multiply
    const float nb = ((MODE == 2) ? 8.807354922057604f : 0.0f) - mnew;
    float lp[4] = {0.0f, 0.0f, 0.0f, 0.0f};

    // ---------------- 3. P rounded into the P*V operand, then P*V
    if (MODE == 2) {
      v8i pf;  // E4M3 of 448 p for keys 32g .. 32g+31 (byte j <-> key 32g + j)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int bm = w >> 2, r0 = 4 * (w & 3);
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sf[bm][r0 + e], f, nb));
          if (!in_seq(bm, r0 + e)) p[e] = 0.0f;
          lp[e] += p[e];
        }
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], word, true);
        pf[w] = word;
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const v4i lo = *reinterpret_cast<const v4i*>(st + v_rd[cb][0]);
        const v4i hi = *reinterpret_cast<const v4i*>(st + v_rd[cb][1]);
        const v8i vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        oacc[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vv, pf, oacc[cb], 0, 0, 0, 0, 0, 0);
      }
    } else {
      v8bf pb[4];  // bf16 p: operand j holds keys 32g + 8j .. 32g + 8j + 7
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int bm = j >> 1, r0 = 8 * (j & 1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sf[bm][r0 + e], f, nb));
          if (!in_seq(bm, r0 + e)) p = 0.0f;
          lp[e & 3] += p;
          pb[j][e] = (__bf16)p;
        }
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v8bf vv = *reinterpret_cast<const v8bf*>(st + v_rd[cb][j]);
          oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pb[j], oacc[cb], 0, 0, 0);
        }
    }
    l += (lp[0] + lp[1]) + (lp[2] + lp[3]);
  };

  // ---- main loop over the tiles that lie wholly inside the sequence (one barrier per tile; the next
  // tile's loads fly while this one is computed), then the ragged last tile, if any, on its own path
  const int nfull = Nkv / kTile;
  issue_tile(0, 0);
  for (int t = 0; t < nfull; ++t) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // tile t visible to all waves; everyone is done with the other stage
    if (t + 1 < nkb) issue_tile(t + 1, (t + 1) & 1);
    process(smem + (t & 1) * G::STAGE, t, std::false_type{});
  }
  if (nfull < nkb) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    process(smem + (nfull & 1) * G::STAGE, nfull, std::true_type{});
  }

  // ---------------- epilogue: O = acc / l  (mode 2: acc * s_v[c] / (448 l)), bf16, lane writes D/2 channels
  const float ltot = l + __shfl_xor(l, 32, 64);
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

// Int32 scores of a window, through the same operand layout as attn_kernel (one wave per 32x64 block).
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

template <int MODE, int D>
hipError_t launch_attn_t(const AttnArg& a, int nwg, hipStream_t s) {
  constexpr int bytes = 2 * Geo<MODE, D>::STAGE;
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_kernel<MODE, D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    configured = true;
  }
  attn_kernel<MODE, D><<<nwg, 256, bytes, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(int mode, const TensorArg& q, const TensorArg& k, const QuantArg& qa, uint16_t* o, int64_t osb,
                       int64_t osh, int64_t osn, float sm_scale, hipStream_t s) {
  AttnArg a;
  a.q = q;
  a.k = k;
  a.qa = qa;
  a.o = o;
  a.osb = osb;
  a.osh = osh;
  a.osn = osn;
  a.clog2e = sm_scale * 1.4426950408889634f;
  a.nqt = cdiv(qa.Nq, kRowsPerWG);
  const int64_t nwg64 = (int64_t)a.nqt * qa.H * qa.B;
  if (nwg64 > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int nwg = (int)nwg64;
  if (qa.d == 128) {
    if (mode == 0) return launch_attn_t<0, 128>(a, nwg, s);
    if (mode == 1) return launch_attn_t<1, 128>(a, nwg, s);
    return launch_attn_t<2, 128>(a, nwg, s);
  }
  if (mode == 0) return launch_attn_t<0, 64>(a, nwg, s);
  if (mode == 1) return launch_attn_t<1, 64>(a, nwg, s);
  return launch_attn_t<2, 64>(a, nwg, s);
}

hipError_t launch_debug_qk(const QuantArg& qa, int b, int h, int q0, int nq, int k0, int nk, int32_t* out,
                           hipStream_t s) {
  dim3 grid(cdiv(nq, 32), cdiv(nk, 64));
  const int64_t bh = (int64_t)b * qa.H + h;
  if (qa.d == 128) debug_qk_kernel<128><<<grid, 64, 0, s>>>(qa, bh, q0, nq, k0, nk, out);
  else debug_qk_kernel<64><<<grid, 64, 0, s>>>(qa, bh, q0, nq, k0, nk, out);
  return hipGetLastError();
}

}  // namespace sattn

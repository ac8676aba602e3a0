// Quantized linear layer y = x W^T + b with 128 x 128 per-block INT8 (TMAP I2V write-up, section "FFN性能优化",
// subsection "线性层量化": 8-bit linear weights in 128 x 128 blocks; W8A8 computes in 8 bits, W8A16 keeps the 8-bit
// weights and 16-bit activations for the layers that need it).
//
// Kernels:
//   quant_blocks_kernel   one workgroup per 128 x 128 block of a bf16 matrix: block max, INT8 codes, block scale
//                         (the symmetric rule of the attention blocks: scale a/127, codes rint(v * 127/a)).
//   codes_to_bf16_kernel  INT8 codes to bf16 (exact: |code| <= 127 needs 7 bits), the W8A16 weight operand.
//   linear_kernel<A8,WR>  the GEMM.  A workgroup owns a (64 WR) x 128 output tile: 128 x 128 with 4 waves (W8A8, and
//                         W8A16 on one row block) or 256 x 128 with 8 waves (W8A16).  Each wave computes 64 x 64,
//                         which lies in one (row block, column block) pair of scale blocks, so every 128-wide K
//                         block has one scale factor per wave: s_x s_w (W8A8) or s_w (W8A16).  The wave's 64 x 64 is
//                         2 x 2 blocks of 32 x 32 on the matrix cores (v_mfma_i32_32x32x32_i8, or
//                         v_mfma_f32_32x32x16_bf16).  The matrix cores accumulate one K block exactly (int32) or in
//                         fp32; at its end the partial sums are scaled and added to the fp32 accumulators (INT8: the
//                         int32 sums start from a float's bit pattern, so that one exact subtraction replaces the
//                         int-to-float conversion).  Operands stream through LDS rings of 128-byte row slices
//                         (direct-to-LDS buffer loads, one or two stages ahead); the fold of one K block overlaps the
//                         next one's matrix ops.
#include <algorithm>
#include <climits>
#include <numeric>
#include <type_traits>

#include "linear_internal.h"
#include "sattn_internal.h"

namespace sattn {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kLinThreads = 256;

__device__ __forceinline__ float bf16_value(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint32_t code_i8(float x, float inv) {
  float q = rintf(x * inv);
  q = fminf(fmaxf(q, -127.0f), 127.0f);
  return (uint32_t)(uint8_t)(int8_t)q;
}

// ---------------------------------------------------------------------------------------------------------
// Per-block INT8.  Thread t covers columns [8 (t % 16), +8) of rows t / 16 + 16 i, i = 0..7, of its block.
__global__ void __launch_bounds__(kLinThreads) quant_blocks_kernel(const uint16_t* __restrict__ x, int rows,
                                                                   int64_t ld, int8_t* __restrict__ codes, int cols,
                                                                   float* __restrict__ scales) {
  const int bj = blockIdx.x, bi = blockIdx.y;
  const int r0 = bi * kLinBlk, c0 = bj * kLinBlk;
  const int nr = min(kLinBlk, rows - r0);
  const int cg = threadIdx.x & 15, rr = threadIdx.x >> 4;
  uint4 raw[8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = rr + 16 * i;
    raw[i] = (r < nr) ? *reinterpret_cast<const uint4*>(x + (int64_t)(r0 + r) * ld + c0 + 8 * cg)
                      : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(bf16_value((w[e / 2] >> (16 * (e & 1))) & 0xFFFFu)));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  __shared__ float wmax[kLinThreads / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  const float a = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const bool zero = !(a >= kGuard);
  const float inv = zero ? 0.0f : 127.0f / a;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = rr + 16 * i;
    if (r >= nr) continue;
    const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo |= code_i8(bf16_value((w[e / 2] >> (16 * (e & 1))) & 0xFFFFu), inv) << (8 * e);
      hi |= code_i8(bf16_value((w[2 + e / 2] >> (16 * (e & 1))) & 0xFFFFu), inv) << (8 * e);
    }
    *reinterpret_cast<uint2*>(codes + (int64_t)(r0 + r) * cols + c0 + 8 * cg) = make_uint2(lo, hi);
  }
  if (threadIdx.x == 0) scales[(int64_t)bi * (cols / kLinBlk) + bj] = zero ? 0.0f : a / 127.0f;
}

// ---------------------------------------------------------------------------------------------------------
// INT8 codes -> bf16, 16 codes per thread and step.
__global__ void __launch_bounds__(kLinThreads) codes_to_bf16_kernel(const int8_t* __restrict__ c,
                                                                    uint16_t* __restrict__ out, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * kLinThreads + threadIdx.x; i < n16; i += (int64_t)gridDim.x * kLinThreads) {
    const uint4 v = reinterpret_cast<const uint4*>(c)[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int sh = 16 * (q & 1);
      const float lo = (float)(int8_t)(w[q >> 1] >> sh), hi = (float)(int8_t)(w[q >> 1] >> (sh + 8));
      o[q] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
    }
    uint4* dst = reinterpret_cast<uint4*>(out) + 2 * i;
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
}

// ---------------------------------------------------------------------------------------------------------
// The GEMM.
constexpr int kLinRow = 128;  // bytes of one operand row per LDS stage
constexpr int kLinLdsMax = 160 * 1024;  // LDS of a compute unit

// The INT8 partial sums of a K block start from the bit pattern of the float 1/(2 pi) (an inline constant of the
// matrix-core instruction).  A K block's sum obeys |S| <= 128 * 127^2 < 2^21, and adding S to that pattern stays in
// the binade [2^-3, 2^-2), whose spacing is 2^-26: read as a float the result is 1/(2 pi) + S 2^-26 exactly, and
// subtracting 1/(2 pi) gives S 2^-26 exactly (Sterbenz).  The fp32 accumulators therefore hold y 2^-26, and the
// epilogue scales them back by 2^26 exactly.  Every rounding is the one of the unscaled sum while the scaled values
// stay normal (|y| above about 2^-100).
[[maybe_unused]] constexpr int kI8Bias = 0x3E22F983;
[[maybe_unused]] constexpr float kI8BiasF = 0.15915494309189535f;  // the float with those bits
[[maybe_unused]] constexpr float kI8Unit = 67108864.0f;            // 2^26

// Tile geometry.  WR rows x 2 columns of waves, each wave computing 64 x 64: WR = 4 gives a 256 x 128 tile (8 waves,
// one workgroup per compute unit, a 3-stage ring loaded two stages ahead), WR = 2 a 128 x 128 tile (4 waves, two
// workgroups per compute unit, a 2-stage ring loaded one stage ahead).  Both keep about 64-96 KiB of tile loads in
// flight per compute unit; the wide tile streams a quarter fewer operand bytes per matrix op.
//
// A stage holds HALVES 128-row activation slices and one 128-row weight slice of ROW bytes each.  Each slice has a
// ring of its own in LDS (R slots of 16 KiB), then come the per-K-block scale lists (one per 128-row block of the
// tile): a wave's operands then lie in two rings whose slots sit at most 32 KiB apart, within the 16-bit immediate
// offset of an LDS read.
template <bool A8, int WR>
struct LinGeo {
  static constexpr int NW = 2 * WR;                 // waves
  static constexpr int THREADS = 64 * NW;
  static constexpr int TM = 64 * WR;                // activation (output) rows of a tile
  static constexpr int HALVES = TM / kLinBlk;       // 128-row activation slices (row blocks) of a tile
  static constexpr int EB = A8 ? 1 : 2;             // bytes per operand element
  static constexpr int ROW = kLinRow;               // bytes of one operand row per stage (granules of 16 B)
  static constexpr int G16 = ROW / 16;              // granules per row
  static constexpr int SPB = kLinBlk * EB / ROW;    // stages per 128-wide K block
  static constexpr int KSTEPS = ROW / 32;           // matrix-core k-steps per stage, 32 bytes of K each
  static constexpr int SL = kLinBlk * ROW;          // one slice of a stage: 128 rows x ROW bytes
  static constexpr int R = WR == 4 ? 3 : 2;         // ring stages
  static constexpr int DIST = R - 1;                // a stage is loaded this many stages ahead of its use
  static constexpr int RING = R * SL;               // the ring of one slice
  static constexpr int NSL = HALVES + 1;            // slices per stage
  static constexpr int BOFF = HALVES * RING;        // the weight ring follows the activation rings
  static constexpr int BYTES = NSL * RING;          // the scale lists follow
  static constexpr int LPS = SL / (16 * THREADS);   // 16-byte loads per thread per slice
  static constexpr int OPS = NSL * LPS;             // loads per thread per stage
  static constexpr int SETS = A8 ? 2 : 1;           // partial-sum register sets
  // K blocks after which the pattern of (first ring slot, register set) repeats
  static constexpr int PERIOD = std::lcm(R / std::gcd(R, SPB), SETS);
  static constexpr int MAX_KB = (kLinLdsMax - BYTES) / (4 * HALVES);  // K blocks the scale lists have room for
  static_assert(LPS * 16 * THREADS == SL, "slices split into whole loads");
  static_assert((R - 1) * SL < 65536, "slot offsets fit the immediate offset of an LDS read");
  static_assert(NW * 64 * 64 * 2 <= BYTES, "the epilogue stages the bf16 tile in the rings");
  static_assert((DIST - 1) * OPS < 64, "the wait count fits vmcnt");
};

// XOR swizzles of the 16-byte granules of an LDS row (4 or 8 granules).  The 16 lanes of a quarter-wave read 16
// consecutive rows at one logical granule (and the 8 lanes of an eighth, 8 rows); these maps send them to distinct
// bank groups for 64 and for 32 LDS banks.
template <int G16>
__device__ __forceinline__ int lswz(int row) {
  if (G16 == 4) return ((row >> 1) & 3) ^ ((row >> 3) & 1);
  return ((row >> 1) & 7) ^ ((row & 1) << 2);
}

// Workgroups are handed to the 8 XCDs round-robin; renumber them so that each XCD gets one contiguous range.
__device__ __forceinline__ int xcd_order(int wg, int nwg) {
  const int q = nwg / 8, r = nwg % 8;
  const int xcd = wg % 8, slot = wg / 8;
  return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Workgroup barrier of the K loop.  The slot of the previous stage is refilled right after it, so every LDS read this
// wave issued must have returned first: the compiler may place the wait for a read's data (at its first use) after
// the barrier, hence the explicit lgkmcnt(0).  The wavefront-scope fences keep the compiler from moving LDS accesses
// across the barrier; without a workgroup fence the barrier does not wait for the tile loads in flight.
__device__ __forceinline__ void ring_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

__device__ __forceinline__ v16i mma_i8(const v4i& a, const v4i& b, const v16i& c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v16f mma_bf16(const v8bf& a, const v8bf& b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// The K loop runs stage by stage: wait for the stage, barrier, load stage t + DIST into the slot stage t - 1 used, run
// the stage's k-steps on the matrix cores.  The partial sums of consecutive K blocks alternate between two register
// sets (INT8), so the scaled fold of K block kb - 1 into the fp32 accumulators is independent of the matrix ops of K
// block kb and sits in the same scheduling region: the vector ALU works while the matrix cores run.  Ring slots and
// register sets are compile-time: the loop body covers PERIOD K blocks.
template <bool A8, int WR>
__global__ void __launch_bounds__(128 * WR, 4 / WR) linear_kernel(LinearArg p) {
  // (the body is device code only: the host pass needs just the signature for the launch stub, and it would drop the
  // stub over the target builtins and register constraints below)
#if defined(__HIP_DEVICE_COMPILE__)
  using G = LinGeo<A8, WR>;
  using Part = std::conditional_t<A8, v16i, v16f>;  // one K block's partial sums of a 32 x 32 block
  using Opnd = std::conditional_t<A8, v4i, v8bf>;
  constexpr int R = G::R, NW = G::NW, G16 = G::G16;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int n32 = lane & 31, g = lane >> 5;
  const int mtiles = (p.M + G::TM - 1) / G::TM, ntiles = (p.N + kLinBlk - 1) / kLinBlk;
  const int nkb = p.K / kLinBlk;

  // output tile: XCD-contiguous ranges, then groups of 4 row tiles walked column tile by column tile, so the
  // workgroups that run together share both their activation and their weight slices in L2
  constexpr int GM = 4;
  const int logical = xcd_order(blockIdx.x, gridDim.x);
  const int grp = logical / (GM * ntiles);
  const int first = grp * GM;
  const int gm = min(GM, mtiles - first);
  const int within = logical - grp * GM * ntiles;
  const int mt = first + within % gm, nt = within / gm;
  const int m0 = mt * G::TM, n0 = nt * kLinBlk;

  // the scale factor of every K block, for each 128-row block of the tile (0 for a block past M: its rows are zero
  // and never stored), after the rings; each wave uses the list of its own row block
  const int mblocks = (p.M + kLinBlk - 1) / kLinBlk;
  float* cs = reinterpret_cast<float*>(smem + G::BYTES);
  for (int e = threadIdx.x; e < G::HALVES * nkb; e += G::THREADS) {
    const int h = e / nkb, kb = e - h * nkb, rb = mt * G::HALVES + h;
    float v = p.sw[(int64_t)nt * nkb + kb];
    if constexpr (A8) v = (rb < mblocks) ? p.sx[(int64_t)rb * nkb + kb] * v : 0.0f;
    cs[e] = v;
  }
  const int half = G::HALVES > 1 ? (64 * wm) / kLinBlk : 0;  // this wave's activation slice
  const float* csw = cs + half * nkb;
  __syncthreads();  // a full workgroup barrier: the lists are written with ordinary LDS stores (no tile load yet)

  // the slices' rows: a stage reads them through a buffer that starts at its K offset and ends after the last row in
  // the matrix, so rows past M (N) read as zero (an activation slice wholly past M has an empty buffer)
  const int arows = min(G::TM, p.M - m0), brows = min(kLinBlk, p.N - n0);
  const uint8_t* abase = p.a + (int64_t)m0 * p.lda;
  const uint8_t* bbase = p.b + (int64_t)n0 * p.ldb;
  // load plan: load j of this wave fills LDS granules [(NW j + wave) * 64, +64) of a slice; LDS granule q holds row
  // q / G16, logical granule (q % G16) ^ lswz(row).  The K offset of a stage goes in the buffer base.
  int la[G::LPS], lb[G::LPS];
#pragma unroll
  for (int j = 0; j < G::LPS; ++j) {
    const int q = (NW * j + wave) * 64 + lane;
    const int row = q / G16, lg = (q % G16) ^ lswz<G16>(row);
    la[j] = row * (int)p.lda + 16 * lg;
    lb[j] = row * (int)p.ldb + 16 * lg;
  }
  const int T = nkb * G::SPB;  // stages
  // loads of stage t's data (clamped to the last stage: the tail reloads it into a free slot, so that no branch
  // splits the loop body) into ring slot SLOT
  auto issue = [&](int t, auto slot_tag) __attribute__((always_inline)) {
    constexpr int SLOT = decltype(slot_tag)::value;
    const int kbyte = min(t, T - 1) * G::ROW;
    // (a row's bytes from kbyte on stay inside the buffer: kbyte + ROW <= K * EB <= ld)
    const auto rb = rows_rsrc(bbase + kbyte, brows * (int)p.ldb - kbyte);
#pragma unroll
    for (int h = 0; h < G::HALVES; ++h) {
      const int hrows = min(kLinBlk, arows - kLinBlk * h);
      const auto ra = rows_rsrc(abase + (int64_t)kLinBlk * h * p.lda + kbyte, max(hrows * (int)p.lda - kbyte, 0));
      uint8_t* sa = smem + h * G::RING + SLOT * G::SL;
#pragma unroll
      for (int j = 0; j < G::LPS; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(sa + (NW * j + wave) * 1024), 16, la[j], 0, 0, 0);
    }
    uint8_t* sb = smem + G::BOFF + SLOT * G::SL;
#pragma unroll
    for (int j = 0; j < G::LPS; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(sb + (NW * j + wave) * 1024), 16, lb[j], 0, 0, 0);
  };
  // operand reads: 32-row block i of this wave, k-step s: row (64 w + 32 i + lane % 32) of its slice, logical granule
  // 2 s + lane / 32.  Where ring and slot offsets together would pass the 16-bit immediate offset of an LDS read (the
  // wide tile), the addresses carry the offset of their ring, kept opaque to the compiler, and the immediate is only
  // the slot's.
  int ard[2][G::KSTEPS], brd[2][G::KSTEPS];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int arow = 64 * wm + 32 * i + n32 - kLinBlk * half, brow = 64 * wn + 32 * i + n32;
#pragma unroll
    for (int s = 0; s < G::KSTEPS; ++s) {
      ard[i][s] = half * G::RING + arow * G::ROW + 16 * ((2 * s + g) ^ lswz<G16>(arow));
      brd[i][s] = G::BOFF + brow * G::ROW + 16 * ((2 * s + g) ^ lswz<G16>(brow));
      if constexpr (G::BOFF + (R - 1) * G::SL + G::SL > 65536) asm("" : "+v"(ard[i][s]), "+v"(brd[i][s]));
    }
  }

  v16f acc[2][2];
  Part part[2][2][2];  // [register set][i][j]
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using I0 = std::integral_constant<int, 0>;
  using I2 = std::integral_constant<int, 2>;
  // fold rows-block range [I0, I1) of register set SET (scale factor fc) into the accumulators
  auto fold = [&](float fc, auto set_tag, auto i0_tag, auto i1_tag) __attribute__((always_inline)) {
    constexpr int SET = decltype(set_tag)::value, FI0 = decltype(i0_tag)::value, FI1 = decltype(i1_tag)::value;
#pragma unroll
    for (int i = FI0; i < FI1; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if constexpr (A8)
            acc[i][j][r] = __builtin_fmaf(fc, __int_as_float(part[SET][i][j][r]) - kI8BiasF, acc[i][j][r]);
          else
            acc[i][j][r] = __builtin_fmaf(fc, part[SET][i][j][r], acc[i][j][r]);
        }
  };
  // stage t (ring slot SLOT) into register set SET: wait until the stage has landed for every wave, refill the slot
  // of stage t - 1 with stage t + DIST, run the k-steps (FRESH: the first stage of a K block, from its start value),
  // and fold the part [FI0, FI1) of the other register set (the previous K block, scale factor fc)
  auto stage = [&](int t, auto slot_tag, auto set_tag, auto fresh_tag, auto fi0_tag, auto fi1_tag, float fc)
      __attribute__((always_inline)) {
    constexpr int SLOT = decltype(slot_tag)::value, SET = decltype(set_tag)::value;
    constexpr bool FRESH = decltype(fresh_tag)::value;
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((G::DIST - 1) * G::OPS) : "memory");  // this wave's loads of stage t
    ring_sync();  // ... and every other wave's; all reads of stage t - 1 are done, so its slot can be refilled
    issue(t + G::DIST, std::integral_constant<int, (SLOT + G::DIST) % R>{});
    const uint8_t* st = smem + SLOT * G::SL;  // (the read addresses include the offset of their ring)
#pragma unroll
    for (int s = 0; s < G::KSTEPS; ++s) {
      Opnd av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        av[i] = *reinterpret_cast<const Opnd*>(st + ard[i][s]);
        bv[i] = *reinterpret_cast<const Opnd*>(st + brd[i][s]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          Part c0 = part[SET][i][j];
          if (FRESH && s == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              if constexpr (A8) c0[r] = kI8Bias;
              else c0[r] = 0.0f;
            }
          }
          if constexpr (A8) part[SET][i][j] = mma_i8(av[i], bv[j], c0);
          else part[SET][i][j] = mma_bf16(av[i], bv[j], c0);
        }
    }
    fold(fc, std::integral_constant<int, SET ^ 1>{}, fi0_tag, fi1_tag);
  };
  // K block kb, at position PH of the period (kb = PH mod PERIOD): its first stage sits in ring slot PH SPB mod R and
  // its partial sums go to register set PH mod 2 (INT8; set 1 for bf16).  With FOLD, the previous K block (the other
  // set) is folded in halves over its first two stages, or all at once in its only stage.
  auto kblock = [&](int kb, auto ph_tag, auto fold_tag) __attribute__((always_inline)) {
    constexpr int PH = decltype(ph_tag)::value;
    constexpr int SLOT0 = (PH * G::SPB) % R, SET = A8 ? PH % 2 : 1;
    constexpr bool FOLD = decltype(fold_tag)::value;
    using FI1 = std::integral_constant<int, FOLD ? (G::SPB >= 2 ? 1 : 2) : 0>;
    using FI2 = std::integral_constant<int, FOLD ? 2 : 0>;
    using SetT = std::integral_constant<int, SET>;
    const float fc = FOLD ? csw[kb - 1] : 0.0f;
    stage(kb * G::SPB, std::integral_constant<int, SLOT0>{}, SetT{}, std::true_type{}, I0{}, FI1{}, fc);
    static_for<1, G::SPB>([&](auto u_tag) __attribute__((always_inline)) {
      constexpr int U = decltype(u_tag)::value;
      using Lo = std::integral_constant<int, U == 1 ? FI1::value : 0>;
      using Hi = std::integral_constant<int, U == 1 ? FI2::value : 0>;
      stage(kb * G::SPB + U, std::integral_constant<int, (SLOT0 + U) % R>{}, SetT{}, std::false_type{}, Lo{}, Hi{},
            U == 1 ? fc : 0.0f);
    });
  };
  // prologue: stages 0 .. DIST-1 into slots 0 .. DIST-1
  issue(0, S0{});
  if constexpr (G::DIST > 1) issue(1, S1{});
  static_assert(G::DIST <= 2, "the prologue issues DIST stages");
  constexpr int P = G::PERIOD;
  if constexpr (A8) {
    // INT8: the fold costs as much vector work as a K block's matrix ops; two register sets overlap them
    kblock(0, I0{}, std::false_type{});
    int kb = 1;
    if constexpr (P == 2) {
      // (the plain two-block form: the compiler interleaves the fold with the matrix ops of both blocks)
      for (; kb + 1 < nkb; kb += 2) {
        kblock(kb, S1{}, std::true_type{});
        kblock(kb + 1, S0{}, std::true_type{});
      }
      if (kb < nkb) {
        kblock(kb, S1{}, std::true_type{});
        fold(csw[nkb - 1], S1{}, I0{}, I2{});
      } else {
        fold(csw[nkb - 1], S0{}, I0{}, I2{});
      }
    } else {
      for (; kb + P <= nkb; kb += P)
        static_for<1, P + 1>([&](auto u_tag) __attribute__((always_inline)) {
          constexpr int U = decltype(u_tag)::value;
          kblock(kb + U - 1, std::integral_constant<int, U % P>{}, std::true_type{});
        });
      const int rest = nkb - kb;  // 0 .. P - 1 more K blocks, at positions 1 .. rest
      static_for<1, P>([&](auto u_tag) __attribute__((always_inline)) {
        constexpr int U = decltype(u_tag)::value;
        if (U <= rest) kblock(kb + U - 1, std::integral_constant<int, U>{}, std::true_type{});
      });
      if ((nkb - 1) & 1) fold(csw[nkb - 1], S1{}, I0{}, I2{});
      else fold(csw[nkb - 1], S0{}, I0{}, I2{});
    }
  } else {
    // bf16: four times the matrix work per fold and one register set (two would not fit with the wider operands)
    int kb = 0;
    for (; kb + P <= nkb; kb += P)
      static_for<0, P>([&](auto u_tag) __attribute__((always_inline)) {
        constexpr int U = decltype(u_tag)::value;
        kblock(kb + U, std::integral_constant<int, U>{}, std::false_type{});
        fold(csw[kb + U], S1{}, I0{}, I2{});
      });
    const int rest = nkb - kb;
    static_for<0, P - 1>([&](auto u_tag) __attribute__((always_inline)) {
      constexpr int U = decltype(u_tag)::value;
      if (U < rest) {
        kblock(kb + U, std::integral_constant<int, U>{}, std::false_type{});
        fold(csw[kb + U], S1{}, I0{}, I2{});
      }
    });
  }

  // epilogue through LDS (the rings are free once every wave is past its last stage and the extra loads of the last
  // stage have landed): the wave writes its 64 x 64 block as bf16 rows of 128 bytes, then stores them 16 bytes per
  // lane.  Lane holds column 32 j + lane % 32 of the block; register r of block i is row
  // 32 i + 8 (r / 4) + 4 (lane / 32) + r % 4.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  uint16_t* ot = reinterpret_cast<uint16_t*>(smem) + wave * 64 * 64;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int cl = 32 * j + n32;
    const int n = n0 + 64 * wn + cl;
    const float bias = (p.bias && n < p.N) ? bf16_value(p.bias[n]) : 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
        const __bf16 h = (__bf16)(A8 ? __builtin_fmaf(acc[i][j][r], kI8Unit, bias) : acc[i][j][r] + bias);
        ot[rl * 64 + cl] = __builtin_bit_cast(uint16_t, h);
      }
  }
  __syncthreads();
  // 64 rows x 8 granules of 16 bytes per wave block: lane reads granule lane % 8 of rows lane / 8 + 8 q
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int rl = lane / 8 + 8 * q, gc = lane % 8;
    const int m = m0 + 64 * wm + rl, n = n0 + 64 * wn + 8 * gc;
    if (m >= p.M || n >= p.N) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(ot + rl * 64 + 8 * gc);
    uint16_t* dst = p.y + (int64_t)m * p.ldy + n;
    if (n + 8 <= p.N && (reinterpret_cast<uintptr_t>(dst) & 15u) == 0) {
      *reinterpret_cast<uint4*>(dst) = v;
    } else {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      const int cnt = min(8, p.N - n);
      for (int e = 0; e < cnt; ++e) dst[e] = (uint16_t)(w[e / 2] >> (16 * (e & 1)));
    }
  }
#endif
}

template <bool A8, int WR>
hipError_t launch_linear_t(const LinearArg& p, hipStream_t s) {
  using G = LinGeo<A8, WR>;
  const int mtiles = (p.M + G::TM - 1) / G::TM, ntiles = (p.N + kLinBlk - 1) / kLinBlk;
  const size_t bytes = G::BYTES + (size_t)G::HALVES * (p.K / kLinBlk) * sizeof(float);
  linear_kernel<A8, WR><<<(unsigned)(mtiles * ntiles), G::THREADS, bytes, s>>>(p);
  return hipGetLastError();
}

template <bool A8, int WR>
hipError_t prepare_linear_t() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&linear_kernel<A8, WR>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, kLinLdsMax);
}

}  // namespace

hipError_t launch_quant_blocks(const uint16_t* x, int rows, int cols, int64_t ld, int8_t* codes, float* scales,
                               hipStream_t s) {
  const dim3 grid((unsigned)(cols / kLinBlk), (unsigned)((rows + kLinBlk - 1) / kLinBlk));
  quant_blocks_kernel<<<grid, kLinThreads, 0, s>>>(x, rows, ld, codes, cols, scales);
  return hipGetLastError();
}

hipError_t launch_codes_to_bf16(const int8_t* codes, uint16_t* out, int64_t n, hipStream_t s) {
  const int64_t n16 = n / 16;
  const int64_t blocks = std::min<int64_t>((n16 + kLinThreads - 1) / kLinThreads, 8192);
  codes_to_bf16_kernel<<<(unsigned)std::max<int64_t>(blocks, 1), kLinThreads, 0, s>>>(codes, out, n16);
  return hipGetLastError();
}

// The dynamic LDS limit of every GEMM variant a call may launch, set on the current device before anything is
// enqueued (on every call: no state is kept, and each GPU of the process gets it).
hipError_t prepare_linear(bool w8a8) {
  if (w8a8) return prepare_linear_t<true, 2>();
  const hipError_t e = prepare_linear_t<false, 4>();
  return e != hipSuccess ? e : prepare_linear_t<false, 2>();
}

hipError_t launch_linear(bool w8a8, const LinearArg& p, hipStream_t s) {
  // INT8 keeps the 128-row tile: its fold hides best under the matrix ops of the other workgroup's wave on the same
  // SIMD, and the 8-wave tile (two waves of one workgroup per SIMD, in step) measured no faster.  bf16 takes the
  // 256-row tile once there is more than one row block, its scale lists fit beside the rings, and 256 activation rows
  // span less than 2^31 bytes (the buffer offsets and extents are 32-bit).
  if (w8a8) return launch_linear_t<true, 2>(p, s);
  if (p.M > kLinBlk && p.lda * 256 <= INT32_MAX && p.K / kLinBlk <= LinGeo<false, 4>::MAX_KB)
    return launch_linear_t<false, 4>(p, s);
  return launch_linear_t<false, 2>(p, s);
}

}  // namespace sattn

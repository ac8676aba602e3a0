// Host-side check of libsattn's C ABI layer (csrc/api.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer:
// api.cpp is built for the host alone and linked against stand-ins for the kernel launchers that record each call
// and never touch memory, so every size, layout and argument check runs for real while no GPU is needed.  Exits 0
// when every expectation holds; any sanitizer report aborts the program.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "../../quantized_attention_05_amd/csrc/linear_internal.h"
#include "../../quantized_attention_05_amd/csrc/probe_internal.h"
#include "../../quantized_attention_05_amd/csrc/sattn_internal.h"

namespace {
std::vector<std::string> g_log;      // launcher calls, in order
std::string g_fail;                  // the launcher that returns an error, if any
int g_last_error_reads = 0;          // hipGetLastError calls (the entry points clear a pending error)
int g_failures = 0;

hipError_t record(const char* name) {
  g_log.push_back(name);
  return g_fail == name ? hipErrorLaunchFailure : hipSuccess;
}
void expect(bool ok, const char* what, int line) {
  if (!ok) {
    std::fprintf(stderr, "FAILED line %d: %s\n", line, what);
    ++g_failures;
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)
}  // namespace

extern "C" hipError_t hipGetLastError(void) {
  ++g_last_error_reads;
  return hipSuccess;
}

namespace sattn {
hipError_t launch_quant_q(const TensorArg&, const QuantArg&, hipStream_t) { return record("quant_q"); }
hipError_t launch_kv_stats(const TensorArg&, const TensorArg&, bool, const QuantArg&, float*, float*, hipStream_t) {
  return record("kv_stats");
}
hipError_t launch_kv_finalize(const QuantArg&, bool, const float*, const float*, float*, hipStream_t) {
  return record("kv_finalize");
}
hipError_t launch_kv_quant(const TensorArg&, const TensorArg&, int, const QuantArg&, const float*, hipStream_t) {
  return record("kv_quant");
}
hipError_t launch_attn(int, const TensorArg&, const TensorArg&, const QuantArg&, uint16_t*, int64_t, int64_t, int64_t,
                       float, const uint8_t*, bool, hipStream_t) {
  return record("attn");
}
hipError_t launch_error_stats(const TensorArg&, const TensorArg&, int, int, int, int, double*, double*, hipStream_t) {
  return record("error_stats");
}
hipError_t launch_debug_qk(const QuantArg&, int, int, int, int, int, int, int32_t*, hipStream_t) {
  return record("debug_qk");
}
hipError_t prepare_attn(int, int, bool, bool) { return record("prepare_attn"); }
int attn_rows_per_workgroup() { return 128; }
hipError_t launch_quant_blocks(const uint16_t*, int, int, int64_t, int8_t*, float*, hipStream_t) {
  return record("quant_blocks");
}
hipError_t launch_codes_to_bf16(const int8_t*, uint16_t*, int64_t, hipStream_t) { return record("codes_to_bf16"); }
hipError_t launch_linear(bool, const LinearArg&, hipStream_t) { return record("linear"); }
hipError_t prepare_linear(bool) { return record("prepare_linear"); }
}  // namespace sattn

namespace {
constexpr uintptr_t kFake = uintptr_t{1} << 40;  // an aligned address that is never dereferenced

sattn_tensor tensor(int B, int H, int N, int d, int64_t sn = 0) {
  if (!sn) sn = d;
  return sattn_tensor{reinterpret_cast<void*>(kFake), B, H, N, d, (int64_t)H * N * sn, (int64_t)N * sn, sn};
}

std::string joined() {
  std::string s;
  for (auto& x : g_log) s += (s.empty() ? "" : ",") + x;
  return s;
}

void check_sizes() {
  // every valid shape: the quantized operands fit in the workspace, grow with every size and carve into aligned,
  // disjoint arrays inside [base, base + bytes)
  const int shapes[][5] = {{1, 1, 1, 1, 64}, {1, 2, 256, 256, 64}, {2, 3, 300, 170, 128}, {1, 40, 75600, 75600, 128},
                           {1, 40, 75600, 769, 128}, {3, 7, 65, 129, 64}, {1, 65535, 1, 1, 128},
                           {1, 1, 1 << 28, 1 << 28, 128}, {255, 257, 1000, 333, 64}};
  for (auto& sh : shapes)
    for (int blk_q : {64, 128})
      for (int mode = 0; mode < 3; ++mode) {
        const int B = sh[0], H = sh[1], Nq = sh[2], Nkv = sh[3], d = sh[4];
        const size_t qb = sattn_quant_bytes(B, H, Nq, Nkv, d, blk_q, 64, mode);
        const size_t wb = sattn_workspace_bytes(B, H, Nq, Nkv, d, blk_q, 64, mode);
        EXPECT(qb > 0 && wb > 0);
        EXPECT(mode != 0 || wb >= qb);
        const size_t codes = (size_t)B * H * d * ((size_t)(Nq + blk_q - 1) / blk_q * blk_q);
        EXPECT(mode == 0 || qb >= codes);
        // the drop-in workspace leaves out the Q codes (quantized inside the attention kernel)
        EXPECT(mode == 0 || wb + codes <= qb + sattn_quantize_scratch_bytes(B, H, Nkv, d, mode) + 512);
        EXPECT(sattn_workspace_bytes(B, H, Nq + 1, Nkv, d, blk_q, 64, mode) >= wb || Nq == (1 << 28));
        sattn_quant q;
        const uintptr_t base = uintptr_t{1} << 44;
        EXPECT(sattn_quant_layout(B, H, Nq, Nkv, d, blk_q, 64, mode, reinterpret_cast<void*>(base), &q) == SATTN_OK);
        const uintptr_t ptrs[] = {(uintptr_t)q.q_codes, (uintptr_t)q.q_scales, (uintptr_t)q.k_codes,
                                  (uintptr_t)q.k_scales, (uintptr_t)q.k_mean, (uintptr_t)q.v_codes,
                                  (uintptr_t)q.v_scales, (uintptr_t)q.v_t};
        uintptr_t prev = 0;
        for (uintptr_t p : ptrs) {
          if (!p) continue;
          EXPECT(p >= base && p < base + qb && p % 256 == 0 && p > prev);
          prev = p;
        }
      }
  // shapes the kernels are not built for, or whose grids would not fit, give 0 rather than wrapping around
  EXPECT(sattn_workspace_bytes(1, 65536, 256, 256, 64, 64, 64, 2) == 0);
  EXPECT(sattn_workspace_bytes(1, 65535, 1 << 28, 256, 64, 64, 64, 2) == 0);
  EXPECT(sattn_workspace_bytes(1, 1, (1 << 28) + 1, 256, 64, 64, 64, 2) == 0);
  EXPECT(sattn_workspace_bytes(-1, 1, 256, 256, 64, 64, 64, 2) == 0);
  EXPECT(sattn_workspace_bytes(1, 1, 256, 256, 96, 64, 64, 2) == 0);
  EXPECT(sattn_quantize_scratch_bytes(1, 40, 75600, 128, 2) > 0 && sattn_quantize_scratch_bytes(1, 40, 75600, 128, 0) == 0);
  for (int mode = 0; mode < 2; ++mode)
    EXPECT(sattn_linear_workspace_bytes(75600, 13824, 5120, mode) > 0);
  EXPECT(sattn_linear_workspace_bytes(1 << 28, 1 << 28, 1 << 20, 0) > 0);  // size_t arithmetic, no int overflow
}

void check_fwd() {
  for (int mode = 0; mode < 3; ++mode) {
    const sattn_tensor q = tensor(1, 40, 75600, 128), k = tensor(1, 40, 769, 128), o = tensor(1, 40, 75600, 128);
    const size_t ws = sattn_workspace_bytes(1, 40, 75600, 769, 128, 128, 64, mode);
    auto call = [&](const sattn_tensor* qq, size_t wsb, void* wsp) {
      g_log.clear();
      return sattn_fwd(qq, &k, &k, &o, 0.0f, mode, 128, 64, wsp, wsb, nullptr);
    };
    const int reads = g_last_error_reads;
    EXPECT(call(&q, ws, reinterpret_cast<void*>(kFake)) == SATTN_OK);
    EXPECT(g_last_error_reads > reads);  // a pending error is cleared before the first launch
    // the drop-in call quantizes Q inside the attention kernel: no separate Q pass
    const std::string want = mode == 0 ? "prepare_attn,kv_quant,attn" : "prepare_attn,kv_stats,kv_finalize,kv_quant,attn";
    EXPECT(joined() == want);
    // host-side errors enqueue nothing
    EXPECT(call(&q, ws - 1, reinterpret_cast<void*>(kFake)) == SATTN_ERR_WORKSPACE && g_log.empty());
    EXPECT(call(&q, ws, reinterpret_cast<void*>(kFake + 16)) == SATTN_ERR_INVALID_ARG && g_log.empty());
    const sattn_tensor bad_stride = tensor(1, 40, 75600, 128, 132);
    EXPECT(call(&bad_stride, ws, reinterpret_cast<void*>(kFake)) == SATTN_ERR_INVALID_ARG && g_log.empty());
    EXPECT(call(nullptr, ws, reinterpret_cast<void*>(kFake)) == SATTN_ERR_INVALID_ARG && g_log.empty());
    // a failing set-up enqueues nothing; a failing launch stops the sequence there
    g_fail = "prepare_attn";
    EXPECT(call(&q, ws, reinterpret_cast<void*>(kFake)) == SATTN_ERR_HIP && joined() == "prepare_attn");
    g_fail = "kv_quant";
    EXPECT(call(&q, ws, reinterpret_cast<void*>(kFake)) == SATTN_ERR_HIP);
    EXPECT(g_log.back() == "kv_quant");
    g_fail.clear();
  }
  // prepared operands, cross-attention, block-sparse and the probe through the same checks
  sattn_quant qd;
  EXPECT(sattn_quant_layout(1, 2, 256, 256, 64, 64, 64, 2, reinterpret_cast<void*>(kFake), &qd) == SATTN_OK);
  const sattn_tensor o = tensor(1, 2, 256, 64);
  g_log.clear();
  EXPECT(sattn_fwd_quantized(nullptr, nullptr, &qd, &o, 0.0f, 2, nullptr) == SATTN_OK);
  EXPECT(joined() == "prepare_attn,attn");
  g_log.clear();
  EXPECT(sattn_fwd_quantized(nullptr, nullptr, &qd, &o, 0.0f, 1, nullptr) == SATTN_ERR_INVALID_ARG && g_log.empty());
  const size_t ws = sattn_workspace_bytes(1, 2, 256, 256, 64, 64, 64, 2);
  g_log.clear();
  EXPECT(sattn_fwd_block_sparse(&o, &o, &o, &o, reinterpret_cast<const uint8_t*>(kFake), 0.0f, 2, 64, 64,
                                reinterpret_cast<void*>(kFake), ws, nullptr) == SATTN_OK);
  EXPECT(g_log.back() == "attn");
  g_log.clear();
  EXPECT(sattn_fwd_block_sparse(&o, &o, &o, &o, nullptr, 0.0f, 2, 64, 64, reinterpret_cast<void*>(kFake), ws,
                                nullptr) == SATTN_ERR_INVALID_ARG && g_log.empty());
  g_log.clear();
  const size_t ws_es = sattn_error_stats_workspace_bytes(1, 2, 256);
  EXPECT(sattn_error_stats(&o, &o, reinterpret_cast<double*>(kFake), reinterpret_cast<void*>(kFake), ws_es, nullptr) ==
         SATTN_OK && joined() == "error_stats");
  g_log.clear();
  EXPECT(sattn_error_stats(&o, &o, reinterpret_cast<double*>(kFake), reinterpret_cast<void*>(kFake), ws_es - 1,
                           nullptr) == SATTN_ERR_WORKSPACE && g_log.empty());
  g_log.clear();
  EXPECT(sattn_debug_qk_int32(&qd, 0, 1, 0, 256, 0, 256, reinterpret_cast<int32_t*>(kFake), nullptr) == SATTN_OK);
  EXPECT(sattn_debug_qk_int32(&qd, 0, 2, 0, 4, 0, 4, reinterpret_cast<int32_t*>(kFake), nullptr) ==
         SATTN_ERR_INVALID_ARG);
}

void check_linear() {
  void* P = reinterpret_cast<void*>(kFake);
  const int8_t* c = reinterpret_cast<const int8_t*>(kFake);
  const float* f = reinterpret_cast<const float*>(kFake);
  for (int mode = 0; mode < 2; ++mode) {
    const size_t ws = sattn_linear_workspace_bytes(300, 136, 384, mode);
    g_log.clear();
    EXPECT(sattn_linear(P, 384, c, f, nullptr, P, 136, 300, 136, 384, mode, P, ws, nullptr) == SATTN_OK);
    EXPECT(joined() == (mode == 0 ? "prepare_linear,quant_blocks,linear" : "prepare_linear,codes_to_bf16,linear"));
    g_log.clear();
    EXPECT(sattn_linear(P, 384, c, f, nullptr, P, 136, 300, 136, 384, mode, P, ws - 1, nullptr) ==
               SATTN_ERR_WORKSPACE && g_log.empty());
  }
  g_log.clear();
  EXPECT(sattn_linear_quantized(c, f, c, f, nullptr, P, 128, 1 << 28, 1 << 28, 128, nullptr) ==
             SATTN_ERR_UNSUPPORTED && g_log.empty());
  EXPECT(sattn_quantize_blocks(P, 256, 384, 384, reinterpret_cast<int8_t*>(kFake), reinterpret_cast<float*>(kFake),
                               nullptr) == SATTN_OK);
}
}  // namespace

int main() {
  check_sizes();
  check_fwd();
  check_linear();
  if (g_failures) return 1;
  std::printf("api host checks: ok\n");
  return 0;
}

// C ABI of the layer (declared in include/macaq.h): host-side argument
// validation, workspace sizing and dispatch to the gfx950 kernels.
// Validation happens before any HIP call, so argument errors are reported
// the same way with or without a device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "macaq.h"
#include "macaq_probe.h"

namespace macaq {
hipError_t launch_act_quant(const void* x, bool x_f32, bool reciprocal, const float* s,
                            const int32_t* offsets, int E, int64_t rows_per_expert, int64_t M,
                            int64_t K, uint8_t* codes, uint8_t* scales, hipStream_t stream);
hipError_t launch_encode_e2m1(const float* v, int64_t n, uint8_t* codes, hipStream_t stream);
hipError_t launch_quant_plain(const void* x, bool x_f32, int64_t M, int64_t K, uint8_t* codes, uint8_t* scales,
                              hipStream_t stream);
hipError_t launch_gemm(const uint8_t* A, const uint8_t* As, const int32_t* offsets, int E,
                       const uint8_t* B, const uint8_t* Bs, int64_t M, int64_t N, int64_t K,
                       void* Y, int mode, hipStream_t stream);
hipError_t launch_linear_fused(const void* x, bool x_f32, const float* s, const uint8_t* B,
                               const uint8_t* Bs, int64_t M, int64_t N, int64_t K, void* Y, int mode,
                               void* ws, hipStream_t stream);
size_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K, bool fused);
bool linear_fused_supported(int64_t M, int64_t N, int64_t K, int64_t E);
bool decode_supported(int64_t M, int64_t N, int64_t K, int64_t E);
hipError_t launch_hessian(const void* x, bool x_f32, const float* s, const int32_t* offsets, int E, int64_t T,
                          int64_t K, float* H, hipStream_t stream);
hipError_t launch_prep_hessian(const void* w, bool w_f32, const float* s, const float* H, int E, int64_t N,
                               int64_t K, uint8_t* codes, uint8_t* scales, hipStream_t stream);
hipError_t launch_flip_grad(const void* w, bool w_f32, const float* s, const float* H, const uint8_t* codes,
                            const uint8_t* scales, int E, int64_t row0, int64_t rows, int64_t N, int64_t K,
                            double* G, hipStream_t stream);
hipError_t launch_flip_rounds(const float* H, int E, int64_t row0, int64_t rows, int64_t N, int64_t K,
                              int max_rounds, const double* G, uint8_t* codes, const uint8_t* scales, int32_t* moves,
                              hipStream_t stream);
hipError_t launch_decode_gemm(const uint8_t* A, const uint8_t* As, const uint8_t* W, const uint8_t* Ws, int64_t M,
                              int64_t N, int64_t K, void* Y, int mode, float* part_ws, hipStream_t stream);
hipError_t launch_gemm_tiled(const uint8_t* A, const uint8_t* As, const int32_t* offsets, int E, const uint8_t* B,
                             const uint8_t* Bs, int64_t M, int64_t N, int64_t K, void* Y, int mode, bool a_tiled,
                             hipStream_t stream);
hipError_t launch_act_quant_tiled(const void* x, bool x_f32, const float* s, const int32_t* offsets, int E, int64_t M,
                                  int64_t K, uint8_t* codes, uint8_t* scales, hipStream_t stream);
hipError_t launch_probe_mfma(const void* src, int64_t blocks, int waves, int iters, float* out, hipStream_t stream);
hipError_t launch_probe_stream(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes, int64_t blocks,
                               uint32_t* out, hipStream_t stream);
hipError_t launch_tile_weights(const uint8_t* wc, const uint8_t* ws, int64_t E, int64_t N, int64_t K, uint8_t* tc,
                               uint8_t* ts, hipStream_t stream);
// output mode bits of the GEMM kernels (mx_common.h)
constexpr int kOutBf16 = 1;
constexpr int kOutSwiGLU = 2;

// Tuning overrides of the launchers (macaq_set_tuning); 0 = automatic.
namespace {
std::atomic<int> g_tuning[MACAQ_TUNE_COUNT];
}
int tuning(int knob) { return g_tuning[knob].load(std::memory_order_relaxed); }
}  // namespace macaq

namespace {

constexpr int kVersion = 10000;  // 1.0.0
constexpr int64_t kMaxFusedM = 2;  // AUTO takes the fused path up to this M
// ... and for small layers: every 32-row block of the fused kernel repeats
// the transform of the whole activation, which below this many repeated
// values costs less than the second launch of the unfused path
constexpr int64_t kMaxFusedRepeat = int64_t(1) << 20;

thread_local std::string g_last_error;

int fail(int status, const std::string& what) {
  g_last_error = what;
  return status;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

std::atomic<int> g_device_ok{0};

int check_device() {
  if (g_device_ok.load(std::memory_order_relaxed)) return MACAQ_OK;
  int n = 0;
  const hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess || n <= 0)
    return fail(MACAQ_ERR_NO_DEVICE, std::string("no HIP device: ") +
                                         (e == hipSuccess ? "device count is 0" : hipGetErrorString(e)));
  g_device_ok.store(1, std::memory_order_relaxed);
  return MACAQ_OK;
}

int hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return MACAQ_OK;
  return fail(MACAQ_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---- MACAQ_CHECK=1: the debug mode.  Before launching, the entry point waits
// for its stream and checks the device-side preconditions it can read back
// cheaply (expert offsets start at 0, never decrease and end at the row
// count; every factor of s is finite and > 0); after launching, it waits for
// the stream again, so that a kernel fault surfaces as MACAQ_ERR_HIP of the
// call that caused it.  Without it no entry point synchronizes.
bool check_mode() {
  const char* v = std::getenv("MACAQ_CHECK");
  return v != nullptr && v[0] == '1';
}

int check_inputs(const char* fn, hipStream_t stream, const int32_t* offsets, int64_t E, int64_t rows,
                 const float* s, int64_t s_count) {
  if (!check_mode()) return MACAQ_OK;
  if (int st = hip_status(hipStreamSynchronize(stream), fn)) return st;
  if (offsets != nullptr && E > 1) {
    std::vector<int32_t> off((size_t)E + 1);
    if (int st = hip_status(hipMemcpy(off.data(), offsets, off.size() * sizeof(int32_t), hipMemcpyDeviceToHost), fn))
      return st;
    if (off[0] != 0 || (int64_t)off[(size_t)E] != rows)
      return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": expert_offsets must start at 0 and end at " +
                                             std::to_string(rows) + " (MACAQ_CHECK)");
    for (int64_t e = 0; e < E; ++e)
      if (off[(size_t)e + 1] < off[(size_t)e])
        return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": expert_offsets decrease at expert " +
                                               std::to_string(e) + " (MACAQ_CHECK)");
  }
  if (s != nullptr && s_count > 0) {
    std::vector<float> h((size_t)s_count);
    if (int st = hip_status(hipMemcpy(h.data(), s, h.size() * sizeof(float), hipMemcpyDeviceToHost), fn)) return st;
    for (size_t i = 0; i < h.size(); ++i)
      if (!(std::isfinite(h[i]) && h[i] > 0.0f))
        return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": s[" + std::to_string(i) +
                                               "] is not a finite positive factor (MACAQ_CHECK)");
  }
  return MACAQ_OK;
}

// The status of a call that has enqueued its kernels; under MACAQ_CHECK a
// fault while they run is reported here.
int finish(const char* fn, hipStream_t stream, int status) {
  if (status != MACAQ_OK || !check_mode()) return status;
  return hip_status(hipStreamSynchronize(stream), fn);
}

int check_dtype(macaq_dtype d, const char* name) {
  if (d != MACAQ_BF16 && d != MACAQ_F32)
    return fail(MACAQ_ERR_UNSUPPORTED, std::string(name) + ": dtype must be MACAQ_BF16 or MACAQ_F32");
  return MACAQ_OK;
}

int check_k(int64_t K, const char* fn) {
  if (K < 32 || K % 32 != 0)
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": K must be a positive multiple of 32 (got " +
                                           std::to_string(K) + ")");
  return MACAQ_OK;
}

// Output of the GEMM-based entry points: dtype and epilogue -> kernel mode.
int output_mode(macaq_dtype y_dtype, uint32_t epilogue, int64_t N, const void* y, const char* fn, int* mode) {
  if (y_dtype != MACAQ_F32 && y_dtype != MACAQ_BF16)
    return fail(MACAQ_ERR_UNSUPPORTED, std::string(fn) + ": y dtype must be MACAQ_F32 or MACAQ_BF16");
  if (epilogue != MACAQ_EPI_NONE && epilogue != MACAQ_EPI_SWIGLU)
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": unknown epilogue");
  if (epilogue == MACAQ_EPI_SWIGLU && N % 2 != 0)
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": SwiGLU needs an even N (gate/up row pairs)");
  if (!aligned(y, y_dtype == MACAQ_F32 ? 4 : 2))
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": y misaligned for its dtype");
  *mode = (y_dtype == MACAQ_BF16 ? macaq::kOutBf16 : 0) | (epilogue == MACAQ_EPI_SWIGLU ? macaq::kOutSwiGLU : 0);
  return MACAQ_OK;
}

int validate_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const int32_t* offsets, int64_t E,
                  const uint8_t* w_codes, const uint8_t* w_scales, int64_t M, int64_t N, int64_t K,
                  const void* y, const char* fn) {
  if (E < 1) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": E must be >= 1");
  if (E > 1 && offsets == nullptr)
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": expert_offsets required when E > 1");
  if (M < 0 || N < 1) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": need M >= 0 and N >= 1");
  if (int st = check_k(K, fn)) return st;
  if (K % 128 != 0)
    return fail(MACAQ_ERR_UNSUPPORTED, std::string(fn) + ": K must be a multiple of 128 for the MFMA GEMM");
  if (M > 0 && (!a_codes || !a_scales || !y))
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": null activation or output pointer");
  if (!w_codes || !w_scales) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": null weight pointer");
  if (!aligned(a_codes, 16) || !aligned(w_codes, 16))
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": code pointers must be 16-byte aligned");
  if (!aligned(a_scales, 4) || !aligned(w_scales, 4))
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": scale pointers must be 4-byte aligned");
  if (M > INT32_MAX || N > INT32_MAX || E > 4096)
    return fail(MACAQ_ERR_UNSUPPORTED, std::string(fn) + ": sizes beyond the supported range");
  return MACAQ_OK;
}

// Shape rule of the tiled W' layout.
int check_tiled(int64_t N, int64_t K, const char* fn) {
  if (N % 32 != 0 || K % 128 != 0)
    return fail(MACAQ_ERR_UNSUPPORTED, std::string(fn) + ": tiled weights need N % 32 == 0 and K % 128 == 0");
  return MACAQ_OK;
}

}  // namespace

extern "C" {

int macaq_version(void) { return kVersion; }

int macaq_probe_mfma(const void* src, int64_t blocks, int waves_per_block, int iters, float* out, void* stream) {
  const char* fn = "macaq_probe_mfma";
  if (src == nullptr || out == nullptr) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": null pointer");
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": src not 16-byte aligned");
  if (blocks < 1 || blocks > (int64_t(1) << 20)) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": blocks out of range");
  if (waves_per_block != 4 && waves_per_block != 8)
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": waves_per_block must be 4 or 8");
  if (iters < 1) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": iters must be >= 1");
  if (int st = check_device()) return st;
  return hip_status(macaq::launch_probe_mfma(src, blocks, waves_per_block, iters, out, (hipStream_t)stream), fn);
}

int macaq_probe_stream(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes, int64_t blocks,
                       uint32_t* out, void* stream) {
  const char* fn = "macaq_probe_stream";
  if (read_bytes < 0 || write_bytes < 0 || read_bytes % 16 != 0 || write_bytes % 16 != 0)
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": sizes must be non-negative multiples of 16");
  if (read_bytes == 0 && write_bytes == 0) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": nothing to stream");
  if ((read_bytes > 0 && (src == nullptr || reinterpret_cast<uintptr_t>(src) % 16 != 0)) ||
      (write_bytes > 0 && (dst == nullptr || reinterpret_cast<uintptr_t>(dst) % 16 != 0)))
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": src / dst missing or not 16-byte aligned");
  if (read_bytes > 0 && write_bytes > 0 && read_bytes % write_bytes != 0)
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": read_bytes must be a whole multiple of write_bytes");
  if (blocks < 1 || blocks > (int64_t(1) << 20)) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": blocks out of range");
  if (out == nullptr) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": out is null");
  if (int st = check_device()) return st;
  return hip_status(macaq::launch_probe_stream(src, read_bytes, dst, write_bytes, blocks, out, (hipStream_t)stream), fn);
}

int macaq_set_tuning(int knob, int value) {
  static const int kMax[MACAQ_TUNE_COUNT] = {3, 64, 64, 2, 8, 4, 64, 64, 16, 64};
  if (knob < 0 || knob >= MACAQ_TUNE_COUNT)
    return fail(MACAQ_ERR_INVALID_ARG, "macaq_set_tuning: unknown knob " + std::to_string(knob));
  if (value < 0 || value > kMax[knob])
    return fail(MACAQ_ERR_INVALID_ARG, "macaq_set_tuning: value " + std::to_string(value) + " out of range for knob " +
                                           std::to_string(knob));
  return macaq::g_tuning[knob].exchange(value, std::memory_order_relaxed);
}

const char* macaq_status_string(int status) {
  switch (status) {
    case MACAQ_OK: return "ok";
    case MACAQ_ERR_INVALID_ARG: return "invalid argument";
    case MACAQ_ERR_UNSUPPORTED: return "unsupported";
    case MACAQ_ERR_NO_DEVICE: return "no device";
    case MACAQ_ERR_HIP: return "HIP error";
    case MACAQ_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

const char* macaq_last_error(void) { return g_last_error.c_str(); }

int macaq_prepare_weights(const void* w, macaq_dtype w_dtype, const float* s, int64_t E, int64_t N,
                          int64_t K, uint8_t* w_codes, uint8_t* w_scales, void* stream) {
  const char* fn = "macaq_prepare_weights";
  if (int st = check_dtype(w_dtype, fn)) return st;
  if (E < 1 || N < 1) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": need E >= 1 and N >= 1");
  if (int st = check_k(K, fn)) return st;
  if (!w || !s || !w_codes || !w_scales) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": null pointer");
  if (!aligned(w, 16) || !aligned(w_codes, 16) || !aligned(s, 16))
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": w, s and w_codes must be 16-byte aligned");
  if (int st = check_device()) return st;
  if (int st = check_inputs(fn, (hipStream_t)stream, nullptr, E, E * N, s, E * K)) return st;
  return finish(fn, (hipStream_t)stream,
                hip_status(macaq::launch_act_quant(w, w_dtype == MACAQ_F32, true, s, nullptr, (int)E, N, E * N, K,
                                                   w_codes, w_scales, (hipStream_t)stream),
                           fn));
}

int macaq_hessian(const void* x, macaq_dtype x_dtype, const float* s, const int32_t* expert_offsets, int64_t E,
                  int64_t T, int64_t K, float* h, void* stream) {
  const char* fn = "macaq_hessian";
  if (int st = check_dtype(x_dtype, fn)) return st;
  if (E < 1 || T < 0) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": need E >= 1 and T >= 0");
  if (E > 1 && expert_offsets == nullptr)
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": expert_offsets required when E > 1");
  if (int st = check_k(K, fn)) return st;
  if (K % 128 != 0)
    return fail(MACAQ_ERR_UNSUPPORTED, std::string(fn) + ": K must be a multiple of 128 (Hessian tile)");
  if (!s || !h || (T > 0 && !x)) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": null pointer");
  if ((T > 0 && !aligned(x, 16)) || !aligned(s, 16) || !aligned(h, 4))
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": x and s must be 16-byte aligned, h 4-byte aligned");
  if (E > 4096 || K > (1 << 20))
    return fail(MACAQ_ERR_UNSUPPORTED, std::string(fn) + ": sizes beyond the supported range");
  if (int st = check_device()) return st;
  if (int st = check_inputs(fn, (hipStream_t)stream, expert_offsets, E, T, s, E * K)) return st;
  return finish(fn, (hipStream_t)stream,
                hip_status(macaq::launch_hessian(x, x_dtype == MACAQ_F32, s, E > 1 ? expert_offsets : nullptr, (int)E,
                                                 T, K, h, (hipStream_t)stream),
                           fn));
}

int macaq_prepare_weights_hessian(const void* w, macaq_dtype w_dtype, const float* s, const float* h, int64_t E,
                                  int64_t N, int64_t K, uint8_t* w_codes, uint8_t* w_scales, void* stream) {
  const char* fn = "macaq_prepare_weights_hessian";
  if (int st = check_dtype(w_dtype, fn)) return st;
  if (E < 1 || N < 1) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": need E >= 1 and N >= 1");
  if (int st = check_k(K, fn)) return st;
  if (!w || !s || !h || !w_codes || !w_scales)
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": null pointer");
  if (!aligned(w, 16) || !aligned(w_codes, 16) || !aligned(s, 16) || !aligned(h, 4))
    return fail(MACAQ_ERR_INVALID_ARG,
                std::string(fn) + ": w, s and w_codes must be 16-byte aligned, h 4-byte aligned");
  if (E > 4096 || K / 32 > 65535 || N > INT32_MAX)
    return fail(MACAQ_ERR_UNSUPPORTED, std::string(fn) + ": sizes beyond the supported range");
  if (int st = check_device()) return st;
  if (int st = check_inputs(fn, (hipStream_t)stream, nullptr, E, E * N, s, E * K)) return st;
  return finish(fn, (hipStream_t)stream,
                hip_status(macaq::launch_prep_hessian(w, w_dtype == MACAQ_F32, s, h, (int)E, N, K, w_codes, w_scales,
                                                      (hipStream_t)stream),
                           fn));
}

int macaq_quant_act(const void* x, macaq_dtype x_dtype, const float* s, const int32_t* expert_offsets,
                    int64_t E, int64_t M, int64_t K, uint8_t* a_codes, uint8_t* a_scales, void* stream) {
  const char* fn = "macaq_quant_act";
  if (int st = check_dtype(x_dtype, fn)) return st;
  if (E < 1 || M < 0) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": need E >= 1 and M >= 0");
  if (E > 1 && expert_offsets == nullptr)
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": expert_offsets required when E > 1");
  if (int st = check_k(K, fn)) return st;
  if (M == 0) return MACAQ_OK;
  if (!x || !s || !a_codes || !a_scales) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": null pointer");
  if (!aligned(x, 16) || !aligned(a_codes, 16) || !aligned(s, 16))
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": x, s and a_codes must be 16-byte aligned");
  if (E > INT32_MAX) return fail(MACAQ_ERR_UNSUPPORTED, std::string(fn) + ": too many experts");
  if (int st = check_device()) return st;
  if (int st = check_inputs(fn, (hipStream_t)stream, expert_offsets, E, M, s, E * K)) return st;
  return finish(fn, (hipStream_t)stream,
                hip_status(macaq::launch_act_quant(x, x_dtype == MACAQ_F32, false, s, E > 1 ? expert_offsets : nullptr,
                                                   (int)E, 0, M, K, a_codes, a_scales, (hipStream_t)stream),
                           fn));
}

int macaq_quant_act_tiled(const void* x, macaq_dtype x_dtype, const float* s, const int32_t* expert_offsets, int64_t E,
                          int64_t M, int64_t K, uint8_t* a_codes, uint8_t* a_scales, void* stream) {
  const char* fn = "macaq_quant_act_tiled";
  if (int st = check_dtype(x_dtype, fn)) return st;
  if (E < 1 || M < 0) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": need E >= 1 and M >= 0");
  if (E > 1 && expert_offsets == nullptr)
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": expert_offsets required when E > 1");
  if (int st = check_k(K, fn)) return st;
  if (K % 128 != 0) return fail(MACAQ_ERR_UNSUPPORTED, std::string(fn) + ": the tiled layout needs K % 128 == 0");
  if (M == 0) return MACAQ_OK;
  if (!x || !s || !a_codes || !a_scales) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": null pointer");
  if (!aligned(x, 16) || !aligned(a_codes, 16) || !aligned(s, 16))
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": x, s and a_codes must be 16-byte aligned");
  if (E > 4096) return fail(MACAQ_ERR_UNSUPPORTED, std::string(fn) + ": too many experts");
  if (int st = check_device()) return st;
  if (int st = check_inputs(fn, (hipStream_t)stream, expert_offsets, E, M, s, E * K)) return st;
  return finish(fn, (hipStream_t)stream,
                hip_status(macaq::launch_act_quant_tiled(x, x_dtype == MACAQ_F32, s, E > 1 ? expert_offsets : nullptr,
                                                         (int)E, M, K, a_codes, a_scales, (hipStream_t)stream),
                           fn));
}

size_t macaq_quant_act_tiled_rows(int64_t M, int64_t E) {
  if (M <= 0 || E <= 0) return 0;
  return (size_t)(E == 1 ? (M + 31) / 32 * 32 : (M + 31 * E + 31) / 32 * 32);
}

size_t macaq_quant_act_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0) return 0;
  return round_up((size_t)M * (size_t)K / 2, 256) + round_up((size_t)M * (size_t)K / 32, 256);
}

size_t macaq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t E) {
  // the decode GEMM's K-split partial sums (row-major weights, M <= 32, few row tiles)
  if (M <= 0 || N <= 0 || K <= 0 || E != 1 || !macaq::decode_supported(M, N, K, E)) return 0;
  return round_up(macaq::decode_workspace_bytes(M, N, K, false), 256);
}

int macaq_linear_path(int64_t M, int64_t N, int64_t K, int64_t E, uint32_t flags) {
  const bool tiled = (flags & MACAQ_W_TILED) != 0;
  flags &= ~MACAQ_W_TILED;
  if (flags > MACAQ_PATH_UNFUSED) return fail(MACAQ_ERR_INVALID_ARG, "macaq_linear_path: unknown flags");
  if (tiled) return MACAQ_PATH_UNFUSED;   // tiled weights: transform kernel, then the prefill / grouped GEMM
  if (flags != MACAQ_PATH_AUTO) return (int)flags;
  if (!macaq::linear_fused_supported(M, N, K, E)) return MACAQ_PATH_UNFUSED;
  const int64_t repeat = (N + 31) / 32 * M * K;
  return (M <= kMaxFusedM || repeat <= kMaxFusedRepeat) ? MACAQ_PATH_FUSED : MACAQ_PATH_UNFUSED;
}

}  // extern "C"

namespace {
// The unfused path of a layer with tiled weights stages the activation in the
// same tiled layout (whole 32-row blocks, each expert starting a block);
// every other unfused path stages it row-major.
bool stage_tiled(uint32_t flags) { return (flags & MACAQ_W_TILED) != 0; }

// Staging of the activation codes and scales: their bytes, and where the
// scales start.
int64_t stage_rows(int64_t M, int64_t E, bool tiled) { return tiled ? (int64_t)macaq_quant_act_tiled_rows(M, E) : M; }
size_t stage_code_bytes(int64_t M, int64_t E, int64_t K, bool tiled) {
  return round_up((size_t)stage_rows(M, E, tiled) * (size_t)K / 2, 256);
}
size_t stage_bytes(int64_t M, int64_t E, int64_t K, bool tiled) {
  return stage_code_bytes(M, E, K, tiled) + round_up((size_t)stage_rows(M, E, tiled) * (size_t)K / 32, 256);
}
}  // namespace

extern "C" {

size_t macaq_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t E, uint32_t flags) {
  if (M <= 0 || N <= 0 || K <= 0 || E <= 0) return 0;   // (MACAQ_W_TILED: the unfused path's workspace)
  const int path = macaq_linear_path(M, N, K, E, flags);
  if (path == MACAQ_PATH_FUSED) return round_up(macaq::decode_workspace_bytes(M, N, K, true), 256);
  if (path == MACAQ_PATH_UNFUSED) return stage_bytes(M, E, K, stage_tiled(flags)) + macaq_gemm_workspace_bytes(M, N, K, E);
  return 0;
}

namespace {
int run_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const int32_t* expert_offsets, int64_t E,
             const uint8_t* w_codes, const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, void* y, int mode,
             void* workspace, hipStream_t stream, const char* fn, bool w_tiled = false, bool a_tiled = false) {
  if (w_tiled)
    return hip_status(macaq::launch_gemm_tiled(a_codes, a_scales, E > 1 ? expert_offsets : nullptr, (int)E, w_codes,
                                               w_scales, M, N, K, y, mode, a_tiled, stream),
                      fn);
  if (macaq::decode_supported(M, N, K, E))
    return hip_status(macaq::launch_decode_gemm(a_codes, a_scales, w_codes, w_scales, M, N, K, y, mode,
                                                static_cast<float*>(workspace), stream),
                      fn);
  return hip_status(macaq::launch_gemm(a_codes, a_scales, E > 1 ? expert_offsets : nullptr, (int)E, w_codes,
                                       w_scales, M, N, K, y, mode, stream),
                    fn);
}

int check_workspace(void* workspace, size_t have, size_t need, const char* fn) {
  if (need == 0) return MACAQ_OK;
  if (workspace == nullptr || have < need)
    return fail(MACAQ_ERR_WORKSPACE, std::string(fn) + ": workspace of " + std::to_string(need) +
                                         " bytes required, got " + std::to_string(workspace ? have : 0));
  if (!aligned(workspace, 256))
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": workspace must be 256-byte aligned");
  return MACAQ_OK;
}
}  // namespace

int macaq_gemm_ex(const uint8_t* a_codes, const uint8_t* a_scales, const int32_t* expert_offsets, int64_t E,
                  const uint8_t* w_codes, const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, void* y,
                  macaq_dtype y_dtype, uint32_t epilogue, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "macaq_gemm";
  const bool w_tiled = (epilogue & MACAQ_W_TILED) != 0;
  const bool a_tiled = (epilogue & MACAQ_A_TILED) != 0;
  epilogue &= ~(MACAQ_W_TILED | MACAQ_A_TILED);
  if (a_tiled && !w_tiled)
    return fail(MACAQ_ERR_UNSUPPORTED, std::string(fn) + ": tiled activations need tiled weights");
  if (int st = validate_gemm(a_codes, a_scales, expert_offsets, E, w_codes, w_scales, M, N, K, y, fn)) return st;
  int mode = 0;
  if (int st = output_mode(y_dtype, epilogue, N, y, fn, &mode)) return st;
  if (w_tiled)
    if (int st = check_tiled(N, K, fn)) return st;
  if (M == 0) return MACAQ_OK;
  if (int st = check_workspace(workspace, workspace_bytes, macaq_gemm_workspace_bytes(M, N, K, E), fn)) return st;
  if (int st = check_device()) return st;
  if (int st = check_inputs(fn, (hipStream_t)stream, expert_offsets, E, M, nullptr, 0)) return st;
  return finish(fn, (hipStream_t)stream,
                run_gemm(a_codes, a_scales, expert_offsets, E, w_codes, w_scales, M, N, K, y, mode, workspace,
                         (hipStream_t)stream, fn, w_tiled, a_tiled));
}

int macaq_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const int32_t* expert_offsets, int64_t E,
               const uint8_t* w_codes, const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, float* y,
               void* workspace, size_t workspace_bytes, void* stream) {
  return macaq_gemm_ex(a_codes, a_scales, expert_offsets, E, w_codes, w_scales, M, N, K, y, MACAQ_F32,
                       MACAQ_EPI_NONE, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---- static scratch of the allocation-free entry point.  The unfused
// path's staging (the activation codes and scales between its two kernels)
// lives in this file-scope device array instead of a caller's workspace; each
// device holds its own copy for the life of the process.  In host code
// `scratch` only names the symbol: its device address is looked up once per
// device with hipGetSymbolAddress, and only that address is handed to
// kernels.
namespace {
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[MACAQ_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device (nullptr until looked up)

int scratch_for_current_device(void** out, const char* fn) {
  int dev = -1;
  if (int st = hip_status(hipGetDevice(&dev), fn)) return st;
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MACAQ_ERR_UNSUPPORTED, std::string(fn) + ": device index " + std::to_string(dev) + " out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (int st = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), fn)) return st;
    if (p == nullptr) return fail(MACAQ_ERR_HIP, std::string(fn) + ": no device address for the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MACAQ_OK;
}

int linear_impl(const void* x, macaq_dtype x_dtype, const float* s, const int32_t* expert_offsets, int64_t E,
                const uint8_t* w_codes, const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, void* y,
                macaq_dtype y_dtype, uint32_t epilogue, void* workspace, size_t workspace_bytes, uint32_t flags,
                void* stream, const char* fn, bool noalloc) {
  if (int st = check_dtype(x_dtype, fn)) return st;
  const bool w_tiled = (flags & MACAQ_W_TILED) != 0;
  if ((flags & ~MACAQ_W_TILED) > MACAQ_PATH_UNFUSED)
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": unknown flags");
  if (!x && M > 0) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": null x");
  if (!s) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": null s");
  if (M > 0 && (!aligned(x, 16) || !aligned(s, 16)))
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": x and s must be 16-byte aligned");
  // the GEMM's rules (E, offsets, K, weights, y); activation buffers are internal
  const uint8_t* dummy = reinterpret_cast<const uint8_t*>(w_codes);
  if (int st = validate_gemm(dummy, w_scales, expert_offsets, E, w_codes, w_scales, M, N, K, y, fn)) return st;
  int mode = 0;
  if (int st = output_mode(y_dtype, epilogue, N, y, fn, &mode)) return st;
  if (w_tiled) {
    if (int st = check_tiled(N, K, fn)) return st;
    if ((flags & ~MACAQ_W_TILED) == MACAQ_PATH_FUSED)
      return fail(MACAQ_ERR_UNSUPPORTED, std::string(fn) + ": the fused decode path reads row-major weights");
  }
  if (M == 0) return MACAQ_OK;
  if (flags == MACAQ_PATH_FUSED && !macaq::linear_fused_supported(M, N, K, E))
    return fail(MACAQ_ERR_UNSUPPORTED, std::string(fn) + ": the fused path serves E == 1, M <= 32, K % 256 == 0");
  const bool fused = macaq_linear_path(M, N, K, E, flags) == MACAQ_PATH_FUSED;
  const size_t need = macaq_linear_workspace_bytes(M, N, K, E, flags);
  if (noalloc) {   // staging in the static scratch array instead of a workspace
    if (need > (size_t)MACAQ_NOALLOC_SCRATCH_BYTES)
      return fail(MACAQ_ERR_WORKSPACE, std::string(fn) + ": this shape needs " + std::to_string(need) +
                                           " bytes of staging, more than the " +
                                           std::to_string((size_t)MACAQ_NOALLOC_SCRATCH_BYTES) +
                                           " of the static scratch array; use macaq_linear_ex with a workspace");
    if (int st = check_device()) return st;
    workspace = nullptr;
    workspace_bytes = 0;
    if (need > 0) {
      if (int st = scratch_for_current_device(&workspace, fn)) return st;
      workspace_bytes = need;
    }
  }
  if (int st = check_workspace(workspace, workspace_bytes, need, fn)) return st;
  if (int st = check_device()) return st;
  hipStream_t st = (hipStream_t)stream;
  if (int r = check_inputs(fn, st, expert_offsets, E, M, s, E * K)) return r;
  if (fused)
    return finish(fn, st,
                  hip_status(macaq::launch_linear_fused(x, x_dtype == MACAQ_F32, s, w_codes, w_scales, M, N, K, y,
                                                        mode, workspace, st),
                             "macaq_linear (fused)"));
  const bool a_tiled = stage_tiled(flags);
  uint8_t* a_codes = static_cast<uint8_t*>(workspace);
  uint8_t* a_scales = a_codes + stage_code_bytes(M, E, K, a_tiled);
  const int32_t* off = E > 1 ? expert_offsets : nullptr;
  if (int r = hip_status(a_tiled ? macaq::launch_act_quant_tiled(x, x_dtype == MACAQ_F32, s, off, (int)E, M, K, a_codes,
                                                                 a_scales, st)
                                 : macaq::launch_act_quant(x, x_dtype == MACAQ_F32, false, s, off, (int)E, 0, M, K,
                                                           a_codes, a_scales, st),
                         "macaq_linear (transform)"))
    return r;
  void* gemm_ws = static_cast<uint8_t*>(workspace) + stage_bytes(M, E, K, a_tiled);
  return finish(fn, st,
                run_gemm(a_codes, a_scales, off, E, w_codes, w_scales, M, N, K, y, mode, gemm_ws, st,
                         "macaq_linear (gemm)", w_tiled, a_tiled));
}

}  // namespace

extern "C" {

int macaq_linear_ex(const void* x, macaq_dtype x_dtype, const float* s, const int32_t* expert_offsets, int64_t E,
                    const uint8_t* w_codes, const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, void* y,
                    macaq_dtype y_dtype, uint32_t epilogue, void* workspace, size_t workspace_bytes, uint32_t flags,
                    void* stream) {
  return linear_impl(x, x_dtype, s, expert_offsets, E, w_codes, w_scales, M, N, K, y, y_dtype, epilogue, workspace,
                     workspace_bytes, flags, stream, "macaq_linear", false);
}

int macaq_linear_noalloc(const void* x, macaq_dtype x_dtype, const float* s, const int32_t* expert_offsets,
                         int64_t E, const uint8_t* w_codes, const uint8_t* w_scales, int64_t M, int64_t N, int64_t K,
                         void* y, macaq_dtype y_dtype, uint32_t epilogue, uint32_t flags, void* stream) {
  return linear_impl(x, x_dtype, s, expert_offsets, E, w_codes, w_scales, M, N, K, y, y_dtype, epilogue, nullptr, 0,
                     flags, stream, "macaq_linear_noalloc", true);
}

int macaq_linear(const void* x, macaq_dtype x_dtype, const float* s, const int32_t* expert_offsets, int64_t E,
                 const uint8_t* w_codes, const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, float* y,
                 void* workspace, size_t workspace_bytes, uint32_t flags, void* stream) {
  return macaq_linear_ex(x, x_dtype, s, expert_offsets, E, w_codes, w_scales, M, N, K, y, MACAQ_F32, MACAQ_EPI_NONE,
                         workspace, workspace_bytes, flags, stream);
}

int macaq_tile_weights(const uint8_t* w_codes, const uint8_t* w_scales, int64_t E, int64_t N, int64_t K,
                       uint8_t* t_codes, uint8_t* t_scales, void* stream) {
  const char* fn = "macaq_tile_weights";
  if (E < 1 || N < 1) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": need E >= 1 and N >= 1");
  if (int st = check_k(K, fn)) return st;
  if (int st = check_tiled(N, K, fn)) return st;
  if (!w_codes || !w_scales || !t_codes || !t_scales)
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": null pointer");
  if (!aligned(w_codes, 16) || !aligned(t_codes, 16) || !aligned(w_scales, 4) || !aligned(t_scales, 4))
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": code pointers must be 16-byte, scale pointers 4-byte aligned");
  if (E > 4096 || E * N > INT32_MAX)
    return fail(MACAQ_ERR_UNSUPPORTED, std::string(fn) + ": sizes beyond the supported range");
  const uint8_t* wc_end = w_codes + (size_t)E * N * (K / 2);
  const uint8_t* tc_end = t_codes + (size_t)E * N * (K / 2);
  if (t_codes < wc_end && w_codes < tc_end)
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": t_codes must not overlap w_codes");
  if (int st = check_device()) return st;
  if (int st = check_inputs(fn, (hipStream_t)stream, nullptr, 1, 0, nullptr, 0)) return st;
  return finish(fn, (hipStream_t)stream,
                hip_status(macaq::launch_tile_weights(w_codes, w_scales, E, N, K, t_codes, t_scales,
                                                      (hipStream_t)stream),
                           fn));
}

int macaq_quant_mxfp4(const void* x, macaq_dtype x_dtype, int64_t M, int64_t K, uint8_t* codes, uint8_t* scales,
                      void* stream) {
  const char* fn = "macaq_quant_mxfp4";
  if (int st = check_dtype(x_dtype, fn)) return st;
  if (M < 0) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": need M >= 0");
  if (int st = check_k(K, fn)) return st;
  if (M == 0) return MACAQ_OK;
  if (!x || !codes || !scales) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": null pointer");
  if (!aligned(x, 16) || !aligned(codes, 16))
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": x and codes must be 16-byte aligned");
  if (int st = check_device()) return st;
  if (int st = check_inputs(fn, (hipStream_t)stream, nullptr, 1, M, nullptr, 0)) return st;
  return finish(fn, (hipStream_t)stream,
                hip_status(macaq::launch_quant_plain(x, x_dtype == MACAQ_F32, M, K, codes, scales,
                                                     (hipStream_t)stream),
                           fn));
}

int macaq_encode_e2m1(const float* v, int64_t n, uint8_t* codes, void* stream) {
  const char* fn = "macaq_encode_e2m1";
  if (n < 0) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": n must be >= 0");
  if (n == 0) return MACAQ_OK;
  if (!v || !codes) return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": null pointer");
  if (int st = check_device()) return st;
  if (int st = check_inputs(fn, (hipStream_t)stream, nullptr, 1, 0, nullptr, 0)) return st;
  return finish(fn, (hipStream_t)stream, hip_status(macaq::launch_encode_e2m1(v, n, codes, (hipStream_t)stream), fn));
}

size_t macaq_flip_refine_workspace_bytes(int64_t rows, int64_t K) {
  if (rows <= 0 || K <= 0) return 0;
  return (size_t)((rows + 127) / 128 * 128) * (size_t)K * sizeof(double);
}

int macaq_flip_refine(const void* w, macaq_dtype w_dtype, const float* s, const float* h, int64_t E, int64_t N,
                      int64_t K, int32_t max_rounds, uint8_t* w_codes, const uint8_t* w_scales, int32_t* moves,
                      void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "macaq_flip_refine";
  if (int st = check_dtype(w_dtype, fn)) return st;
  if (E < 1 || N < 1 || max_rounds < 0)
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": need E >= 1, N >= 1 and max_rounds >= 0");
  if (int st = check_k(K, fn)) return st;
  if (K % 128 != 0 || K > 32640)
    return fail(MACAQ_ERR_UNSUPPORTED, std::string(fn) + ": K must be a multiple of 128 and at most 32640");
  if (!w || !s || !h || !w_codes || !w_scales)
    return fail(MACAQ_ERR_INVALID_ARG, std::string(fn) + ": null pointer");
  if (!aligned(w, 16) || !aligned(w_codes, 16) || !aligned(s, 16) || !aligned(h, 4))
    return fail(MACAQ_ERR_INVALID_ARG,
                std::string(fn) + ": w, s and w_codes must be 16-byte aligned, h 4-byte aligned");
  if (E > 4096 || N > INT32_MAX)
    return fail(MACAQ_ERR_UNSUPPORTED, std::string(fn) + ": sizes beyond the supported range");
  const size_t row_bytes = (size_t)K * sizeof(double);
  if (int st = check_workspace(workspace, workspace_bytes, macaq_flip_refine_workspace_bytes(128, K), fn))
    return st;
  if (int st = check_device()) return st;
  if (int st = check_inputs(fn, (hipStream_t)stream, nullptr, E, E * N, s, E * K)) return st;
  const int64_t fit = (int64_t)(workspace_bytes / row_bytes);   // gradient rows the workspace holds
  const bool f32 = w_dtype == MACAQ_F32;
  hipStream_t st = (hipStream_t)stream;
  double* G = static_cast<double*>(workspace);
  if (fit >= E * N) {   // all experts in one pair of launches
    if (int r = hip_status(macaq::launch_flip_grad(w, f32, s, h, w_codes, w_scales, (int)E, 0, N, N, K, G, st),
                           "macaq_flip_refine (gradient)"))
      return r;
    return finish(fn, st,
                  hip_status(macaq::launch_flip_rounds(h, (int)E, 0, N, N, K, max_rounds, G, w_codes, w_scales,
                                                       moves, st),
                             "macaq_flip_refine (rounds)"));
  }
  // else expert by expert, in chunks of rows that fit (a multiple of 128)
  const int64_t chunk = std::min<int64_t>(fit / 128 * 128, (N + 127) / 128 * 128);
  const size_t eb = f32 ? 4 : 2;
  for (int64_t e = 0; e < E; ++e) {
    const void* we = static_cast<const uint8_t*>(w) + (size_t)e * N * K * eb;
    const float* se = s + e * K;
    const float* he = h + e * K * K;
    uint8_t* ce = w_codes + e * N * (K / 2);
    const uint8_t* sce = w_scales + e * N * (K / 32);
    int32_t* me = moves ? moves + e * N : nullptr;
    for (int64_t r0 = 0; r0 < N; r0 += chunk) {
      const int64_t rows = std::min(chunk, N - r0);
      if (int r = hip_status(macaq::launch_flip_grad(we, f32, se, he, ce, sce, 1, r0, rows, N, K, G, st),
                             "macaq_flip_refine (gradient)"))
        return r;
      if (int r = hip_status(macaq::launch_flip_rounds(he, 1, r0, rows, N, K, max_rounds, G, ce, sce, me, st),
                             "macaq_flip_refine (rounds)"))
        return r;
    }
  }
  return finish(fn, st, MACAQ_OK);
}

}  // extern "C"

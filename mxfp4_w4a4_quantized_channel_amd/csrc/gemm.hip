// Launcher of the MXFP4 GEMM (kernel template in gemm_kernel.h).
#include <cstdlib>
#include <cstring>

#include "gemm_kernel.h"

namespace macaq {

namespace {

template <int BM, int BN, int WM, int WN, int BK, int S>
hipError_t launch_pipe(const uint8_t* A, const uint8_t* As, const int32_t* offsets, int E, const uint8_t* B,
                       const uint8_t* Bs, int64_t M, int64_t N, int64_t K, float* Y, hipStream_t stream) {
  using L = PipeLayout<BM, BN, BK, 1>;
  constexpr int lds = S * L::kStage;
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)gemm_mxfp4_pipe_kernel<BM, BN, WM, WN, BK, S>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  const int tiles_n = (int)ceil_div(N, BN);
  int64_t tiles_m = ceil_div(M, BM);
  if (offsets != nullptr) tiles_m += E;  // each expert may add one partial row tile
  const int64_t blocks = tiles_m * tiles_n;
  gemm_mxfp4_pipe_kernel<BM, BN, WM, WN, BK, S><<<dim3((unsigned)blocks), dim3(64 * WM * WN), lds, stream>>>(
      A, As, B, Bs, offsets, E, M, N, K, Y, (int)tiles_m, tiles_n, 4);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint8_t* A, const uint8_t* As, const int32_t* offsets, int E,
                       const uint8_t* B, const uint8_t* Bs, int64_t M, int64_t N, int64_t K,
                       float* Y, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  // Tile choice: the largest tile that still gives about one tile per CU.
  // MACAQ_GEMM_TILE=256x256 | 256x128 | 128x128 forces one (tests use it to
  // cover every kernel on small shapes).
  int64_t t256 = ceil_div(M, 256) * ceil_div(N, 256);
  int64_t t128 = ceil_div(M, 256) * ceil_div(N, 128);
  if (const char* force = getenv("MACAQ_GEMM_TILE")) {
    const bool f256 = strcmp(force, "256x256") == 0, f128 = strcmp(force, "256x128") == 0;
    t256 = f256 ? INT64_MAX : 0;
    t128 = f128 ? INT64_MAX : 0;
  }
  if (K % 256 == 0) {
    if (t256 >= 240) return launch_pipe<256, 256, 2, 2, 256, 2>(A, As, offsets, E, B, Bs, M, N, K, Y, stream);
    if (t128 >= 120) return launch_pipe<256, 128, 2, 2, 256, 2>(A, As, offsets, E, B, Bs, M, N, K, Y, stream);
  } else {
    if (t256 >= 240) return launch_pipe<256, 256, 2, 2, 128, 4>(A, As, offsets, E, B, Bs, M, N, K, Y, stream);
    if (t128 >= 120) return launch_pipe<256, 128, 2, 2, 128, 4>(A, As, offsets, E, B, Bs, M, N, K, Y, stream);
  }
  constexpr int BM = 128, BN = 128;
  const int n_tiles_n = (int)ceil_div(N, BN);
  int64_t m_slots = ceil_div(M, BM);
  if (offsets != nullptr) m_slots += E;  // each expert may add one partial tile
  const int64_t blocks = m_slots * n_tiles_n;
  gemm_mxfp4_kernel<BM, BN, 2, 2><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
      A, As, B, Bs, offsets, E, M, N, K, Y, n_tiles_n);
  return hipGetLastError();
}

}  // namespace macaq

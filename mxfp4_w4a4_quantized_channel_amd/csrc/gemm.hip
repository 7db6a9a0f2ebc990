// Launcher of the MXFP4 GEMM (kernel template in gemm_kernel.h).
#include "gemm_kernel.h"

namespace macaq {

namespace {

template <int BM, int BN, int WM, int WN, int BK, int S, int MINB, int OUT, bool BT, bool AT>
hipError_t launch_pipe_out(const uint8_t* A, const uint8_t* As, const int32_t* offsets, int E, const uint8_t* B,
                           const uint8_t* Bs, int64_t M, int64_t N, int64_t K, void* Y, hipStream_t stream) {
  using L = PipeLayout<BM, BN, BK, 1>;
  constexpr int lds = S * L::kStage;
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)gemm_mxfp4_pipe_kernel<BM, BN, WM, WN, BK, S, MINB, OUT, BT, AT>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  const int tiles_n = (int)ceil_div(N, BN);
  int64_t tiles_m = ceil_div(M, BM);
  if (offsets != nullptr) tiles_m += E;  // each expert may add one partial row tile
  const int64_t blocks = tiles_m * tiles_n;
  // tile rows per XCD group (blocks of a group share A and W' panels in one L2)
  const int group_m = tuning(MACAQ_TUNE_GEMM_GROUP_M) > 0 ? tuning(MACAQ_TUNE_GEMM_GROUP_M) : 4;
  gemm_mxfp4_pipe_kernel<BM, BN, WM, WN, BK, S, MINB, OUT, BT, AT>
      <<<dim3((unsigned)blocks), dim3(64 * WM * WN), lds, stream>>>(A, As, B, Bs, offsets, E, M, N, K, Y,
                                                                    (int)tiles_m, tiles_n, group_m);
  return hipGetLastError();
}

// output mode (run time) -> kernel instantiation
template <int BM, int BN, int WM, int WN, int BK, int S, int MINB = 1, bool BT = false, bool AT = false>
hipError_t launch_pipe(const uint8_t* A, const uint8_t* As, const int32_t* offsets, int E, const uint8_t* B,
                       const uint8_t* Bs, int64_t M, int64_t N, int64_t K, void* Y, int mode, hipStream_t stream) {
  switch (mode) {
    case 0:
      return launch_pipe_out<BM, BN, WM, WN, BK, S, MINB, 0, BT, AT>(A, As, offsets, E, B, Bs, M, N, K, Y, stream);
    case kOutBf16:
      return launch_pipe_out<BM, BN, WM, WN, BK, S, MINB, kOutBf16, BT, AT>(A, As, offsets, E, B, Bs, M, N, K, Y,
                                                                            stream);
    case kOutSwiGLU:
      return launch_pipe_out<BM, BN, WM, WN, BK, S, MINB, kOutSwiGLU, BT, AT>(A, As, offsets, E, B, Bs, M, N, K, Y,
                                                                              stream);
    default:
      return launch_pipe_out<BM, BN, WM, WN, BK, S, MINB, kOutBf16 | kOutSwiGLU, BT, AT>(A, As, offsets, E, B, Bs, M,
                                                                                          N, K, Y, stream);
  }
}

// Repack of prepared W' (row-major codes [E][N][K/2], scales [E][N][K/32])
// into the tiled layout: per expert, for each 32-row group g and 128-wide
// K-tile t, 2 KiB of codes (row r of the group at byte 64 r, its 16-byte
// chunk c at position c ^ ((r >> 2) & 3)) and 128 bytes of scales (row r's
// 4 bytes at 4 r).  One thread per 16-byte code chunk (and per 4 scale bytes).
__global__ void tile_weights_kernel(const uint8_t* __restrict__ wc, const uint8_t* __restrict__ ws, int64_t rows,
                                    int64_t K, uint8_t* __restrict__ tc, uint8_t* __restrict__ ts) {
  const int64_t KT = K >> 7;                       // K-tiles per row
  const int64_t chunks = rows * (K >> 5);          // 16-byte code chunks (= 32-value groups)
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < chunks) {
    const int64_t row = i / (K >> 5), c_all = i % (K >> 5);    // row over all experts (N % 32 == 0)
    const int64_t t = c_all >> 2;
    const int c = (int)(c_all & 3);
    const int r = (int)(row & 31);
    const int64_t dst = ((row >> 5) * KT + t) * 2048 + r * 64 + ((c ^ ((r >> 2) & 3)) << 4);
    *reinterpret_cast<uint4*>(tc + dst) = *reinterpret_cast<const uint4*>(wc + row * (K >> 1) + c_all * 16);
  }
  if (i < rows * KT) {   // 4-byte scale words: (row, K-tile)
    const int64_t row = i / KT, t = i % KT;
    const int64_t dst = ((row >> 5) * KT + t) * 128 + (row & 31) * 4;
    *reinterpret_cast<uint32_t*>(ts + dst) = *reinterpret_cast<const uint32_t*>(ws + row * (K >> 5) + t * 4);
  }
}

}  // namespace

hipError_t launch_tile_weights(const uint8_t* wc, const uint8_t* ws, int64_t E, int64_t N, int64_t K, uint8_t* tc,
                               uint8_t* ts, hipStream_t stream) {
  const int64_t rows = E * N;
  const int64_t threads = rows * (K >> 5);   // >= the scale words rows * K / 128
  if (threads <= 0) return hipSuccess;
  tile_weights_kernel<<<dim3((unsigned)ceil_div(threads, 256)), dim3(256), 0, stream>>>(wc, ws, rows, K, tc, ts);
  return hipGetLastError();
}

// GEMM with W' in the tiled layout (N % 32 == 0, K % 128 == 0): 128-wide
// K-tiles in a 4-deep ring (the tiled copies are contiguous, so the shorter
// tiles cost no copy efficiency and keep three tiles in flight); 256x256
// when that gives about one tile per CU, else 128x128 with two blocks per
// CU.  a_tiled: the activation codes and scales are in the same tiled
// layout (expert-padded for grouped layers); there the grouped 128x128
// tiles run three blocks per CU with 3-deep rings (MoE E64 T8192 N1024
// K3072: 24.7 against 27.2 us with two blocks of 4-deep rings, whose 528
// tiles took one round of 512 slots and a tail of 16; per-token routing
// 45.8 against 45.0), dense ones two per CU (attn-proj 24.1 against 25.3);
// same box, operands rotated past the Infinity Cache.
hipError_t launch_gemm_tiled(const uint8_t* A, const uint8_t* As, const int32_t* offsets, int E, const uint8_t* B,
                             const uint8_t* Bs, int64_t M, int64_t N, int64_t K, void* Y, int mode, bool a_tiled,
                             hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  const int64_t t256 = ceil_div(M, 256) * ceil_div(N, 256);
  int choice = (offsets == nullptr && t256 >= 240) ? 0 : 2;
  if (const int force = tuning(MACAQ_TUNE_GEMM_TILE)) choice = force - 1;
  if (a_tiled) {
    switch (choice) {
      case 0: return launch_pipe<256, 256, 2, 2, 128, 4, 1, true, true>(A, As, offsets, E, B, Bs, M, N, K, Y, mode, stream);
      case 1: return launch_pipe<256, 128, 2, 2, 128, 4, 1, true, true>(A, As, offsets, E, B, Bs, M, N, K, Y, mode, stream);
      default:
        if (offsets != nullptr)
          return launch_pipe<128, 128, 2, 2, 128, 3, 3, true, true>(A, As, offsets, E, B, Bs, M, N, K, Y, mode, stream);
        return launch_pipe<128, 128, 2, 2, 128, 4, 2, true, true>(A, As, offsets, E, B, Bs, M, N, K, Y, mode, stream);
    }
  }
  switch (choice) {
    case 0: return launch_pipe<256, 256, 2, 2, 128, 4, 1, true>(A, As, offsets, E, B, Bs, M, N, K, Y, mode, stream);
    case 1: return launch_pipe<256, 128, 2, 2, 128, 4, 1, true>(A, As, offsets, E, B, Bs, M, N, K, Y, mode, stream);
    default: return launch_pipe<128, 128, 2, 2, 128, 4, 2, true>(A, As, offsets, E, B, Bs, M, N, K, Y, mode, stream);
  }
}

hipError_t launch_gemm(const uint8_t* A, const uint8_t* As, const int32_t* offsets, int E,
                       const uint8_t* B, const uint8_t* Bs, int64_t M, int64_t N, int64_t K,
                       void* Y, int mode, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  // Tile choice (measured on MI355X): 256x256 when that still gives about one
  // tile per CU (largest tiles, least LDS and L2 traffic per FLOP); else
  // 256x128; grouped layers and small shapes use 128x128 with two blocks per
  // CU, whose finer granularity keeps ragged experts from leaving CUs idle.
  // macaq_set_tuning(MACAQ_TUNE_GEMM_TILE) forces one.
  const int64_t t256 = ceil_div(M, 256) * ceil_div(N, 256);
  const int64_t t128 = ceil_div(M, 256) * ceil_div(N, 128);
  int choice;  // 0: 256x256, 1: 256x128, 2: 128x128
  if (offsets != nullptr) choice = 2;
  else if (t256 >= 240) choice = 0;
  else if (t128 >= 200) choice = 1;
  else choice = 2;
  if (const int force = tuning(MACAQ_TUNE_GEMM_TILE)) choice = force - 1;
  const bool k256 = K % 256 == 0;
  switch (choice) {
    case 0:
      return k256 ? launch_pipe<256, 256, 2, 2, 256, 2>(A, As, offsets, E, B, Bs, M, N, K, Y, mode, stream)
                  : launch_pipe<256, 256, 2, 2, 128, 4>(A, As, offsets, E, B, Bs, M, N, K, Y, mode, stream);
    case 1:
      return k256 ? launch_pipe<256, 128, 2, 2, 256, 2>(A, As, offsets, E, B, Bs, M, N, K, Y, mode, stream)
                  : launch_pipe<256, 128, 2, 2, 128, 4>(A, As, offsets, E, B, Bs, M, N, K, Y, mode, stream);
    default:
      return k256 ? launch_pipe<128, 128, 2, 2, 256, 2, 2>(A, As, offsets, E, B, Bs, M, N, K, Y, mode, stream)
                  : launch_pipe<128, 128, 2, 2, 128, 4, 2>(A, As, offsets, E, B, Bs, M, N, K, Y, mode, stream);
  }
}

}  // namespace macaq

// MXFP4 x MXFP4 GEMM on CDNA4 block-scaled MFMA, dense and grouped.
//
// Sources: "MACaQ Enables Streaming W4A4 Quantization with 32.5GB GPU
// Memory", section "Quantization mechanism" (the transformed, quantized
// activation goes through an FP4 matrix multiplication with the offline
// weight, y = x W^T); "华为开源MACaQ:本地量化提速3倍", section
// "现在还不能把它当成通用量化工厂" (dense and grouped W4A4 matmul operators).
//
// y[m][n] = sum_k a(m,k) w(e(m),n,k), both operands MXFP4 row-major along K
// (codes [rows][K/2], E8M0 scales [rows][K/32]).
//
// Instruction: v_mfma_scale_f32_32x32x64_f8f6f4 with both operands FP4.
// Each lane feeds 16 bytes = 32 FP4 values of one row and the E8M0 byte of
// exactly those 32 values, so one lane's operand is one MXFP4 group and the
// row-major MXFP4 layout is the MFMA operand layout.  The sum over K is
// invariant under a permutation of K applied to both operands, so within a
// K-tile of 256 (8 groups) lane half h (lanes 32h..32h+31) of sub-step j
// takes group 4h + j: a lane's four sub-steps read one contiguous 64-byte
// run of its row and one scale dword whose byte j the instruction's op_sel
// picks.
//
// Tiling: a block computes a BM x BN tile of y with WAVES_M x WAVES_N waves;
// each wave owns a (BM/WAVES_M) x (BN/WAVES_N) sub-tile of 32x32 MFMA
// blocks with fp32 accumulators in registers.  K-tiles of 256 are staged in
// LDS, double-buffered: the global loads of tile k+1 are in flight while
// tile k feeds the MFMAs.  In LDS each 128-byte tile row holds 8 chunks of
// 16 bytes, chunk c of row r stored at position c ^ (r & 7), so the
// fragment reads of 8 consecutive rows hit 8 different bank groups.
//
// Grouped (mixture-of-experts) operation: rows are sorted by expert and the
// block index enumerates (expert, row-tile) pairs on the device from the
// expert offsets, so no host synchronization is needed; slots past the last
// expert's tiles exit at once.
#include "mx_common.h"

namespace macaq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v8i as_operand(const uint4& q) {
  v8i r;
  r[0] = (int)q.x; r[1] = (int)q.y; r[2] = (int)q.z; r[3] = (int)q.w;
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}

template <int BM, int BN, int WAVES_M, int WAVES_N>
struct GemmTile {
  static constexpr int kThreads = 64 * WAVES_M * WAVES_N;
  static constexpr int kTM = BM / WAVES_M;
  static constexpr int kTN = BN / WAVES_N;
  static constexpr int kFM = kTM / 32;
  static constexpr int kFN = kTN / 32;
  static constexpr int kAChunks = BM * 8 / kThreads;
  static constexpr int kBChunks = BN * 8 / kThreads;
  static constexpr int kASc = (BM * 2 + kThreads - 1) / kThreads;
  static constexpr int kBSc = (BN * 2 + kThreads - 1) / kThreads;
  static_assert(kTM % 32 == 0 && kTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(BM * 8 % kThreads == 0 && BN * 8 % kThreads == 0, "chunks must divide evenly");
};

template <int J, int FM, int FN>
__device__ __forceinline__ void mfma_substep(v16f (&acc)[FM][FN], const uint4 (&fa)[FM],
                                             const uint4 (&fb)[FN], const uint32_t (&sa)[FM],
                                             const uint32_t (&sb)[FN]) {
#pragma unroll
  for (int mi = 0; mi < FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < FN; ++ni)
      acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          as_operand(fa[mi]), as_operand(fb[ni]), acc[mi][ni], 4, 4, J, (int)sa[mi], J, (int)sb[ni]);
}

template <int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_mxfp4_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, const int32_t* __restrict__ offsets, int E, int64_t M,
    int64_t N, int64_t K, float* __restrict__ Y, int n_tiles_n) {
  using T = GemmTile<BM, BN, WAVES_M, WAVES_N>;
  __shared__ __attribute__((aligned(16))) uint8_t smA[2][BM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t smB[2][BN * 128];
  __shared__ uint32_t smAs[2][BM * 2];
  __shared__ uint32_t smBs[2][BN * 2];

  // ---- tile -> (expert, rows, columns)
  const int tn = (int)(blockIdx.x % (unsigned)n_tiles_n);
  int64_t slot = blockIdx.x / (unsigned)n_tiles_n;
  int e = 0;
  int64_t row_begin = 0, row_end = M;
  if (offsets != nullptr) {
    for (e = 0; e < E; ++e) {
      const int64_t b = offsets[e], en = offsets[e + 1];
      const int64_t t = (en - b + BM - 1) / BM;
      if (slot < t) {
        row_begin = b + slot * BM;
        row_end = en;
        break;
      }
      slot -= t;
    }
    if (e == E) return;
  } else {
    row_begin = slot * BM;
    if (row_begin >= M) return;
  }
  const int64_t n0 = (int64_t)tn * BN;
  const int64_t KB = K >> 1;   // code bytes per row
  const int64_t KG = K >> 5;   // groups (scale bytes) per row
  const uint8_t* Bx = B + (int64_t)e * N * KB;
  const uint8_t* Bsx = Bs + (int64_t)e * N * KG;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  const int r32 = lane & 31;
  const int h = lane >> 5;

  // ---- per-thread global source offsets (rows clamped into the valid range)
  int64_t offA[T::kAChunks], offB[T::kBChunks];
  int ldsA[T::kAChunks], ldsB[T::kBChunks];
#pragma unroll
  for (int i = 0; i < T::kAChunks; ++i) {
    const int idx = tid + i * T::kThreads;
    const int row = idx >> 3;
    int64_t gr = row_begin + row;
    if (gr >= row_end) gr = row_end - 1;
    offA[i] = gr * KB + (idx & 7) * 16;
    ldsA[i] = row * 128 + (((idx & 7) ^ (row & 7)) << 4);
  }
#pragma unroll
  for (int i = 0; i < T::kBChunks; ++i) {
    const int idx = tid + i * T::kThreads;
    const int row = idx >> 3;
    int64_t gn = n0 + row;
    if (gn >= N) gn = N - 1;
    offB[i] = gn * KB + (idx & 7) * 16;
    ldsB[i] = row * 128 + (((idx & 7) ^ (row & 7)) << 4);
  }
  // chunk c of a thread is the same for all its chunks: idx & 7 == tid & 7
  const int my_c = tid & 7;
  int64_t offAs[T::kASc], offBs[T::kBSc];
#pragma unroll
  for (int i = 0; i < T::kASc; ++i) {
    const int idx = tid + i * T::kThreads;
    const int row = idx < BM * 2 ? (idx >> 1) : 0;
    int64_t gr = row_begin + row;
    if (gr >= row_end) gr = row_end - 1;
    offAs[i] = gr * KG + (idx & 1) * 4;
  }
#pragma unroll
  for (int i = 0; i < T::kBSc; ++i) {
    const int idx = tid + i * T::kThreads;
    const int row = idx < BN * 2 ? (idx >> 1) : 0;
    int64_t gn = n0 + row;
    if (gn >= N) gn = N - 1;
    offBs[i] = gn * KG + (idx & 1) * 4;
  }
  const int my_half = tid & 1;

  uint4 ra[T::kAChunks], rb[T::kBChunks];
  uint32_t ras[T::kASc], rbs[T::kBSc];

#define MACAQ_LOAD_TILE(KT)                                                                          \
  {                                                                                                  \
    const int64_t g0 = (int64_t)(KT) * 8;                                                            \
    const bool cok = g0 + my_c < KG;                                                                 \
    const bool sok = g0 + my_half * 4 < KG;                                                          \
    _Pragma("unroll") for (int i = 0; i < T::kAChunks; ++i) {                                        \
      ra[i] = cok ? *reinterpret_cast<const uint4*>(A + offA[i] + g0 * 16) : make_uint4(0, 0, 0, 0); \
    }                                                                                                \
    _Pragma("unroll") for (int i = 0; i < T::kBChunks; ++i) {                                        \
      rb[i] = cok ? *reinterpret_cast<const uint4*>(Bx + offB[i] + g0 * 16) : make_uint4(0, 0, 0, 0); \
    }                                                                                                \
    _Pragma("unroll") for (int i = 0; i < T::kASc; ++i) {                                            \
      ras[i] = sok ? *reinterpret_cast<const uint32_t*>(As + offAs[i] + g0) : 0u;                    \
    }                                                                                                \
    _Pragma("unroll") for (int i = 0; i < T::kBSc; ++i) {                                            \
      rbs[i] = sok ? *reinterpret_cast<const uint32_t*>(Bsx + offBs[i] + g0) : 0u;                   \
    }                                                                                                \
  }
#define MACAQ_STORE_TILE(ST)                                                                         \
  {                                                                                                  \
    _Pragma("unroll") for (int i = 0; i < T::kAChunks; ++i)                                          \
        *reinterpret_cast<uint4*>(&smA[ST][ldsA[i]]) = ra[i];                                        \
    _Pragma("unroll") for (int i = 0; i < T::kBChunks; ++i)                                          \
        *reinterpret_cast<uint4*>(&smB[ST][ldsB[i]]) = rb[i];                                        \
    _Pragma("unroll") for (int i = 0; i < T::kASc; ++i) {                                            \
      if (tid + i * T::kThreads < BM * 2) smAs[ST][tid + i * T::kThreads] = ras[i];                  \
    }                                                                                                \
    _Pragma("unroll") for (int i = 0; i < T::kBSc; ++i) {                                            \
      if (tid + i * T::kThreads < BN * 2) smBs[ST][tid + i * T::kThreads] = rbs[i];                  \
    }                                                                                                \
  }

  v16f acc[T::kFM][T::kFN];
#pragma unroll
  for (int mi = 0; mi < T::kFM; ++mi)
#pragma unroll
    for (int ni = 0; ni < T::kFN; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  const int nk = (int)((K + 255) / 256);
  MACAQ_LOAD_TILE(0)
  MACAQ_STORE_TILE(0)
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) MACAQ_LOAD_TILE(kt + 1)

    uint32_t sa[T::kFM], sb[T::kFN];
    int rowA[T::kFM], rowB[T::kFN];
#pragma unroll
    for (int mi = 0; mi < T::kFM; ++mi) {
      rowA[mi] = wm * T::kTM + mi * 32 + r32;
      sa[mi] = smAs[st][rowA[mi] * 2 + h];
    }
#pragma unroll
    for (int ni = 0; ni < T::kFN; ++ni) {
      rowB[ni] = wn * T::kTN + ni * 32 + r32;
      sb[ni] = smBs[st][rowB[ni] * 2 + h];
    }
    const int sw = r32 & 7;
    uint4 fa[T::kFM], fb[T::kFN];
#define MACAQ_SUBSTEP(J)                                                                      \
  {                                                                                           \
    _Pragma("unroll") for (int mi = 0; mi < T::kFM; ++mi) fa[mi] =                            \
        *reinterpret_cast<const uint4*>(&smA[st][rowA[mi] * 128 + (((4 * h + (J)) ^ sw) << 4)]); \
    _Pragma("unroll") for (int ni = 0; ni < T::kFN; ++ni) fb[ni] =                            \
        *reinterpret_cast<const uint4*>(&smB[st][rowB[ni] * 128 + (((4 * h + (J)) ^ sw) << 4)]); \
    mfma_substep<J>(acc, fa, fb, sa, sb);                                                     \
  }
    MACAQ_SUBSTEP(0)
    MACAQ_SUBSTEP(1)
    MACAQ_SUBSTEP(2)
    MACAQ_SUBSTEP(3)
#undef MACAQ_SUBSTEP

    if (kt + 1 < nk) MACAQ_STORE_TILE(st ^ 1)
    __syncthreads();
  }

#undef MACAQ_LOAD_TILE
#undef MACAQ_STORE_TILE

  // ---- epilogue: lane (r32, h) of 32x32 block holds column r32 and rows
  // 8*(r/4) + 4*h + (r%4) for accumulator register r.
#pragma unroll
  for (int mi = 0; mi < T::kFM; ++mi) {
#pragma unroll
    for (int ni = 0; ni < T::kFN; ++ni) {
      const int64_t n = n0 + wn * T::kTN + ni * 32 + r32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = row_begin + wm * T::kTM + mi * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (m < row_end && n < N) Y[m * N + n] = acc[mi][ni][r];
      }
    }
  }
}

hipError_t launch_gemm(const uint8_t* A, const uint8_t* As, const int32_t* offsets, int E,
                       const uint8_t* B, const uint8_t* Bs, int64_t M, int64_t N, int64_t K,
                       float* Y, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
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

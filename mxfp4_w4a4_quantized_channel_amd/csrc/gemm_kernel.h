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
// blocks with fp32 accumulators in registers.  K-tiles are staged in an LDS
// ring filled by direct-to-LDS copies (see gemm_mxfp4_pipe_kernel below).
//
// Grouped (mixture-of-experts) operation: rows are sorted by expert and the
// block index enumerates (expert, row-tile) pairs on the device from the
// expert offsets, so no host synchronization is needed; slots past the last
// expert's tiles exit at once.
#pragma once

#include <type_traits>

#include "mx_common.h"

namespace macaq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// y is written once and never read back by the GEMM: its stores are
// non-temporal, so they stream past the caches instead of evicting the A and
// W' panels the other blocks are still reading (measured: attn-proj 33.2 ->
// 28.4 us, down-prefill 144 -> 125 us, MoE 39.9 -> 36.0 us).

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

// fp32 epilogue of a wave's FM x FN block of 32x32 accumulators whose first
// row is m0 and first column n0 (rows below row_end and columns below N are
// stored): lane (r32, h) holds column r32 and rows 8*(r/4) + 4*h + (r%4) of
// accumulator register r.
template <int FM, int FN>
__device__ __forceinline__ void store_wave_tile_f32(const v16f (&acc)[FM][FN], void* __restrict__ Y, int64_t m0,
                                                    int64_t row_end, int64_t n0, int64_t N, int r32, int h) {
  const bool interior = (m0 + FM * 32 <= row_end) && (n0 + FN * 32 <= N);
  if (interior) {
#pragma unroll
    for (int mi = 0; mi < FM; ++mi)
#pragma unroll
      for (int ni = 0; ni < FN; ++ni) {
        float* yp = reinterpret_cast<float*>(Y) + (m0 + mi * 32 + 4 * h) * N + n0 + ni * 32 + r32;
#pragma unroll
        for (int r = 0; r < 16; ++r) __builtin_nontemporal_store(acc[mi][ni][r], &yp[(8 * (r >> 2) + (r & 3)) * N]);
      }
    return;
  }
#pragma unroll
  for (int mi = 0; mi < FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) {
      const int64_t n = n0 + ni * 32 + r32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + mi * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (m < row_end && n < N) __builtin_nontemporal_store(acc[mi][ni][r], reinterpret_cast<float*>(Y) + m * N + n);
      }
    }
}

// bf16 / SwiGLU epilogue staged through LDS (the pipelined kernel's stages
// are free after its K loop): per 32x32 accumulator block, the wave writes
// its values to a [32][36]-float LDS tile (row-major, rows padded to keep
// 16-byte alignment), then each lane reads 8 consecutive columns of one row
// (two such pieces per lane) and stores them as 8 bf16 values (one 16-byte
// store) or, for SwiGLU, the 4 results silu(gate) * up of those 4 (gate, up)
// column pairs.  Two tiles per wave alternate, so one block's reads overlap
// the next block's writes; the wave's LDS accesses complete in order, so a
// tile is reused without a barrier.
constexpr int kEpiStride = 36;                        // floats per LDS tile row
constexpr int kEpiLdsBytes = 2 * 32 * kEpiStride * 4;  // per wave (two tiles)

// One 8-column piece of one output row from the LDS tile: 8 bf16 values (one
// 16-byte store), or for SwiGLU the 4 results of its 4 (gate, up) pairs.
// CHECKED handles rows past row_end, columns past N and unaligned rows; the
// unchecked form is for wave tiles that lie wholly inside y with 16-byte
// aligned rows.
template <int OUT, bool CHECKED>
__device__ __forceinline__ void store_epi_piece(const float* __restrict__ src, void* __restrict__ Y, int64_t m,
                                                int64_t n, int64_t row_end, int64_t N) {
  const float4 p0 = *reinterpret_cast<const float4*>(src);
  const float4 p1 = *reinterpret_cast<const float4*>(src + 4);
  const float v[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
  if (CHECKED && (m >= row_end || n >= N)) return;
  if constexpr ((OUT & kOutSwiGLU) != 0) {
    const int64_t ldo = N >> 1, j0 = n >> 1;   // 4 output columns j0..j0+3
    float o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = silu_times(v[2 * k], v[2 * k + 1]);
    if constexpr ((OUT & kOutBf16) != 0) {
      uint16_t* yp = reinterpret_cast<uint16_t*>(Y) + m * ldo + j0;
      if (!CHECKED || (n + 8 <= N && (reinterpret_cast<uintptr_t>(yp) & 7) == 0)) {
        __builtin_nontemporal_store(u32x2{pk_bf16_rne(o[0], o[1]), pk_bf16_rne(o[2], o[3])},
                                    reinterpret_cast<u32x2*>(yp));
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (n + 2 * k < N) yp[k] = f32_to_bf16_rne(o[k]);
      }
    } else {
      float* yp = reinterpret_cast<float*>(Y) + m * ldo + j0;
      if (!CHECKED || (n + 8 <= N && (reinterpret_cast<uintptr_t>(yp) & 15) == 0)) {
        __builtin_nontemporal_store(f32x4{o[0], o[1], o[2], o[3]}, reinterpret_cast<f32x4*>(yp));
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (n + 2 * k < N) yp[k] = o[k];
      }
    }
  } else {   // bf16
    uint16_t* yp = reinterpret_cast<uint16_t*>(Y) + m * N + n;
    if (!CHECKED || (n + 8 <= N && (reinterpret_cast<uintptr_t>(yp) & 15) == 0)) {
      __builtin_nontemporal_store(u32x4{pk_bf16_rne(v[0], v[1]), pk_bf16_rne(v[2], v[3]), pk_bf16_rne(v[4], v[5]),
                                        pk_bf16_rne(v[6], v[7])},
                                  reinterpret_cast<u32x4*>(yp));
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (n + k < N) yp[k] = f32_to_bf16_rne(v[k]);
    }
  }
}

template <int OUT, bool CHECKED, int FM, int FN>
__device__ __forceinline__ void store_wave_tile_lds_impl(const v16f (&acc)[FM][FN], float* __restrict__ t,
                                                         void* __restrict__ Y, int64_t m0, int64_t row_end,
                                                         int64_t n0, int64_t N, int lane) {
  const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int mi = 0; mi < FM; ++mi) {
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) {
      float* tt = static_cast<float*>(__builtin_assume_aligned(t + ((mi * FN + ni) & 1) * (32 * kEpiStride), 16));
#pragma unroll
      for (int r = 0; r < 16; ++r) tt[(8 * (r >> 2) + 4 * h + (r & 3)) * kEpiStride + r32] = acc[mi][ni][r];
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int item = lane + 64 * it;        // 32 rows x 4 pieces of 8 columns
        const int row = item >> 2, c = (item & 3) * 8;
        store_epi_piece<OUT, CHECKED>(tt + row * kEpiStride + c, Y, m0 + mi * 32 + row, n0 + ni * 32 + c, row_end, N);
      }
    }
  }
}

template <int OUT, int FM, int FN>
__device__ __forceinline__ void store_wave_tile_lds(const v16f (&acc)[FM][FN], float* __restrict__ t,
                                                    void* __restrict__ Y, int64_t m0, int64_t row_end, int64_t n0,
                                                    int64_t N, int lane) {
  static_assert(OUT != 0, "fp32 output is stored from the registers");
  // Unchecked when the wave tile lies inside y and every piece's store is
  // aligned: with N % 8 == 0 and a 16-byte aligned y, the 16-byte bf16
  // pieces, the 8-byte SwiGLU bf16 pieces and the 16-byte SwiGLU fp32 pieces
  // all start on their own size (piece columns are multiples of 8).
  const bool interior = (m0 + FM * 32 <= row_end) && (n0 + FN * 32 <= N) && (N % 8) == 0 &&
                        (reinterpret_cast<uintptr_t>(Y) & 15) == 0;
  if (interior)
    store_wave_tile_lds_impl<OUT, false>(acc, t, Y, m0, row_end, n0, N, lane);
  else
    store_wave_tile_lds_impl<OUT, true>(acc, t, Y, m0, row_end, n0, N, lane);
}

// ---------------------------------------------------------------------------
// Pipelined kernel: a ring of STAGES LDS buffers of K-tiles of BK (128 or
// 256) filled by direct-to-LDS copies issued with inline assembly.  The
// copies have no register results; their completion is tracked explicitly
// with s_waitcnt vmcnt(n) (the builtin form makes the compiler wait for
// every outstanding copy before any LDS read, which serializes the ring).
//
// Schedule of a K-tile (NSUB = BK/64 MFMA sub-steps): the MFMAs of sub-step
// j run while the fragments of sub-step j+1 are read from LDS into a second
// register set.  In the last sub-step every wave already holds its
// fragments, so the stage is free: the wave waits for the next tile's
// copies, meets the others at the one barrier of the tile, issues the copy
// of tile kt+STAGES into the freed stage and reads the next tile's scales
// and first fragments, all interleaved with that sub-step's MFMAs.  Past the
// last tile the freed stages receive copies of the last tile again, so that
// every wait counts the same number of outstanding copies.
//
// LDS row of a K-tile: BK/2 bytes = CPR chunks of 16 bytes (CPR = BK/32
// groups); chunk c of row r sits at position c ^ f(r), f(r) = (r / (8/CPR))
// mod CPR, so the 16-byte fragment reads of 8 consecutive rows fall into 8
// different 16-byte bank groups.  Scale bytes: [rows][CPR].
// Lane half h of MFMA sub-step j takes group h*CPR/2 + j; its CPR/2 scale
// bytes are contiguous and the instruction's op_sel picks byte j.
//
// Block order: consecutive block indices go to different XCDs (round
// robin), so the index is remapped so that the blocks resident on one XCD
// form compact groups of tiles (GROUP_M tile rows) that share A and B
// panels in that XCD's L2.

constexpr int kNumXcd = 8;

template <int BM, int BN, int BK, int SWZ = 0>
struct PipeLayout {
  static constexpr int kCPR = BK / 32;              // chunks (groups) per tile row
  static constexpr int kRowBytes = BK / 2;
  static constexpr int kRowsPerBankRow = 8 / kCPR;  // rows sharing one 128-byte bank row
  static constexpr int kA = 0;
  static constexpr int kB = BM * kRowBytes;
  static constexpr int kAs = (BM + BN) * kRowBytes;
  static constexpr int kBs = kAs + BM * kCPR;
  static constexpr int kStage = kBs + BN * kCPR;
  static constexpr int kCodeBlocks = (BM + BN) * kRowBytes / 1024;
  static constexpr int kScaleBlocks = (BM + BN) * kCPR / 256;
  __host__ __device__ static constexpr int swz(int r) { return ((r >> SWZ) / kRowsPerBankRow) & (kCPR - 1); }
};

// Tile coordinates of block `bid` among `ntiles` = tiles_m * tiles_n active
// tiles (XCD-aware order: the hardware deals consecutive block indices to the
// XCDs in turn, so XCD x receives blocks x, x+8, ...; those are given one
// contiguous range of logical tiles, which the group_m grouping turns into a
// compact block of tiles sharing A and B panels).
__device__ __forceinline__ void tile_of_block(int bid, int ntiles, int tiles_m, int tiles_n, int group_m,
                                              int* tm, int* tn) {
  const int x = bid % kNumXcd, q = ntiles / kNumXcd, rem = ntiles % kNumXcd;
  const int logical = x * q + (x < rem ? x : rem) + bid / kNumXcd;
  const int per_group = group_m * tiles_n;
  const int g = logical / per_group;
  const int first_m = g * group_m;
  const int gm = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
  const int in = logical - g * per_group;
  *tm = first_m + in % gm;
  *tn = in / gm;
}

// Inclusive prefix sum of v over the wave's 64 lanes.
__device__ __forceinline__ int wave_prefix_sum(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// Row tiles of BM rows per expert, from the device-side offsets, 64 experts
// per step (lane l takes expert e0 + l; every wave computes the same result):
// the total, and the expert, first row and end row of row tile `tm`.  Loads
// and prefix sums run across the lanes, so a block pays two rounds of
// parallel loads instead of 2E dependent ones.
template <int BM>
__device__ __forceinline__ int grouped_row_tiles(const int32_t* __restrict__ offsets, int E, int lane) {
  int total = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    const int t = e < E ? (int)(((int64_t)offsets[e + 1] - offsets[e] + BM - 1) / BM) : 0;
    total += __shfl(wave_prefix_sum(t, lane), 63, 64);
  }
  return total;
}
// Also the padded first row of the tile's expert minus its first row
// (*a_shift): in the expert-padded tiled activation layout, expert e's rows
// start at padded row P_e = sum over e' < e of ceil(rows_e' / 32) * 32.
template <int BM>
__device__ __forceinline__ bool grouped_tile(const int32_t* __restrict__ offsets, int E, int lane, int tm, int* e_out,
                                             int64_t* row_begin, int64_t* row_end, int64_t* a_shift) {
  int base = 0, pbase = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    int64_t b = 0, en = 0;
    if (e < E) {
      b = offsets[e];
      en = offsets[e + 1];
    }
    const int t = e < E ? (int)((en - b + BM - 1) / BM) : 0;
    const int pc = e < E ? (int)((en - b + 31) / 32 * 32) : 0;   // padded rows of expert e
    const int incl = base + wave_prefix_sum(t, lane), excl = incl - t;
    const int pincl = pbase + wave_prefix_sum(pc, lane), pexcl = pincl - pc;
    const unsigned long long hit = __ballot(t > 0 && tm >= excl && tm < incl);
    if (hit != 0ull) {
      const int l = __ffsll(hit) - 1;
      *e_out = e0 + l;
      const int64_t first = __shfl(b, l, 64);
      *row_begin = first + (int64_t)(tm - __shfl(excl, l, 64)) * BM;
      *row_end = __shfl(en, l, 64);
      *a_shift = (int64_t)__shfl(pexcl, l, 64) - first;
      return true;
    }
    base = __shfl(incl, 63, 64);
    pbase = __shfl(pincl, 63, 64);
  }
  return false;
}

// BT: W' in the tiled layout (see macaq_tile_weights): per expert, blocks of
// 32 rows x one 128-wide K-tile, 2 KiB of codes (each row's 16-byte chunks
// stored in the XOR-swizzled order the LDS tile uses) and 128 bytes of
// scales.  A copy instruction then reads 1 KiB of contiguous codes (and a
// scale copy 256 contiguous bytes) instead of 16 (64) rows' pieces
// (measured with 256-wide tiles: 56 against 33 B/clk per CU for such copies
// in isolation; the down-prefill layer's copies alone take 38 us of loop
// time tiled against 118 us row-major with 128-wide K-tiles).  AT: the
// activation codes and scales in the same tiled layout; for grouped layers
// every expert's rows start on a 32-row block (expert-padded), so that row
// tiles, which start at expert boundaries, start on blocks too.

// The MFMAs of one sub-step, J the sub-step (op_sel picks scale byte J).
template <int J, int FM, int FN>
__device__ __forceinline__ void mfma_substep_t(v16f (&acc)[FM][FN], const uint4 (&fa)[FM], const uint4 (&fb)[FN],
                                               const uint32_t (&sa)[FM], const uint32_t (&sb)[FN]) {
#pragma unroll
  for (int mi = 0; mi < FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < FN; ++ni)
      acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(as_operand(fa[mi]), as_operand(fb[ni]), acc[mi][ni],
                                                                     4, 4, J, (int)sa[mi], J, (int)sb[ni]);
}

// MFMAs LO .. HI-1 of one sub-step (index mi * FN + ni).
template <int J, int LO, int HI, int FM, int FN>
__device__ __forceinline__ void mfma_range_t(v16f (&acc)[FM][FN], const uint4 (&fa)[FM], const uint4 (&fb)[FN],
                                             const uint32_t (&sa)[FM], const uint32_t (&sb)[FN]) {
#pragma unroll
  for (int i = LO; i < HI; ++i) {
    const int mi = i / FN, ni = i % FN;
    acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(as_operand(fa[mi]), as_operand(fb[ni]), acc[mi][ni],
                                                                  4, 4, J, (int)sa[mi], J, (int)sb[ni]);
  }
}

// Calls f(std::integral_constant<int, I>) for I = 0 .. N-1 (compile-time
// indices for op_sel and register-set selection).
template <int N, typename F, int I = 0>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, F, I + 1>(static_cast<F&&>(f));
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int BK, int STAGES, int MINB = 1, int OUT = 0, bool BT = false,
          bool AT = false>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, MINB) void gemm_mxfp4_pipe_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, const int32_t* __restrict__ offsets, int E, int64_t M,
    int64_t N, int64_t K, void* __restrict__ Y, int tiles_m, int tiles_n, int group_m) {
  using T = GemmTile<BM, BN, WAVES_M, WAVES_N>;
  using L = PipeLayout<BM, BN, BK, 1>;
  constexpr int kWaves = WAVES_M * WAVES_N;
  constexpr int kCPR = L::kCPR;
  constexpr int NSUB = kCPR / 2;   // MFMA sub-steps per K-tile
  // Copies per wave per K-tile.  When a stage's blocks do not split evenly
  // over the waves, the last waves repeat blocks of the first ones (identical
  // bytes to the same LDS place), so every wave issues the same number of
  // copies and one vmcnt threshold fits all waves.
  constexpr int kCB = (L::kCodeBlocks + kWaves - 1) / kWaves;
  constexpr int kSB = (L::kScaleBlocks + kWaves - 1) / kWaves;
  constexpr int kLPT = kCB + kSB;
  static_assert((STAGES - 2) * kLPT < 64, "vmcnt range");
  static_assert(!(BT || AT) || BK == 128, "the tiled layouts have 128-wide K-tiles");
  static_assert(NSUB % 2 == 0, "an even number of sub-steps per K-tile");
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

  // ---- tile -> (expert, rows, columns).  Grouped: the active row tiles are
  // counted from the device-side offsets, so that the XCD-aware order spreads
  // only real tiles over the XCDs; surplus blocks exit.
  const int lane0 = (int)threadIdx.x & 63;
  const int active_m = offsets != nullptr ? grouped_row_tiles<BM>(offsets, E, lane0) : tiles_m;
  if ((int)blockIdx.x >= active_m * tiles_n) return;
  int tm, tn;
  tile_of_block((int)blockIdx.x, active_m * tiles_n, active_m, tiles_n, group_m, &tm, &tn);
  int e = 0;
  int64_t row_begin = 0, row_end = M, a_shift = 0;   // a_shift: tiled activation row = row + a_shift
  if (offsets != nullptr) {
    if (!grouped_tile<BM>(offsets, E, lane0, tm, &e, &row_begin, &row_end, &a_shift)) return;
  } else {
    row_begin = (int64_t)tm * BM;
    if (row_begin >= M) return;
  }
  const int64_t n0 = (int64_t)tn * BN;
  if (n0 >= N) return;
  const int64_t KB = K >> 1;
  const int64_t KG = K >> 5;
  const uint8_t* Bx = B + (int64_t)e * N * KB;
  const uint8_t* Bsx = Bs + (int64_t)e * N * KG;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  const int r32 = lane & 31;
  const int h = lane >> 5;
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;

  // ---- per-lane copy sources for K-tile 0 (advance by BK/2 code bytes and
  // CPR scale bytes per K-tile; tiled operands by 4 KiB and 256 bytes) and
  // wave-uniform LDS offsets within a stage.  Tiled rows sit at (row / 32,
  // K-tile, row % 32) with their chunks already in the LDS order, so the
  // lanes read them in memory order (tile rows start at multiples of 32, so a
  // row's swizzle in the LDS tile equals its swizzle in memory).
  const uint8_t* csrc[kCB];
  uint32_t ctile = 0, stile = 0;   // copies of tiled operands (wave-uniform bits)
#pragma unroll
  for (int i = 0; i < kCB; ++i) {
    const int blk = (wave * kCB + i) % L::kCodeBlocks;
    constexpr int rows_per_blk = 1024 / L::kRowBytes;
    const int row = blk * rows_per_blk + lane / kCPR;
    const int c = (lane % kCPR) ^ L::swz(row);
    if (row < BM) {
      int64_t gr = row_begin + row;
      if (gr >= row_end) gr = row_end - 1;
      if constexpr (AT) {
        const int64_t pr = gr + a_shift;
        csrc[i] = A + (pr >> 5) * (K >> 7) * 2048 + (pr & 31) * 64 + (lane % kCPR) * 16;
        ctile |= 1u << i;
      } else {
        csrc[i] = A + gr * KB + c * 16;
      }
    } else {
      int64_t gn = n0 + (row - BM);
      if (gn >= N) gn = N - 1;
      if constexpr (BT) {
        csrc[i] = Bx + (gn >> 5) * (K >> 7) * 2048 + (gn & 31) * 64 + (lane % kCPR) * 16;
        ctile |= 1u << i;
      } else {
        csrc[i] = Bx + gn * KB + c * 16;
      }
    }
  }
  const uint8_t* ssrc[kSB];
#pragma unroll
  for (int i = 0; i < kSB; ++i) {
    const int blk = (wave * kSB + i) % L::kScaleBlocks;
    const int d = blk * 64 + lane;            // dword of the [rows][CPR] scale tile
    const int row = d / (kCPR / 4), part = d % (kCPR / 4);
    if (row < BM) {
      int64_t gr = row_begin + row;
      if (gr >= row_end) gr = row_end - 1;
      if constexpr (AT) {
        const int64_t pr = gr + a_shift;
        ssrc[i] = As + (pr >> 5) * (K >> 7) * 128 + (pr & 31) * 4 + part * 4;
        stile |= 1u << i;
      } else {
        ssrc[i] = As + gr * KG + part * 4;
      }
    } else {
      int64_t gn = n0 + (row - BM);
      if (gn >= N) gn = N - 1;
      if constexpr (BT) {
        ssrc[i] = Bsx + (gn >> 5) * (K >> 7) * 128 + (gn & 31) * 4 + part * 4;
        stile |= 1u << i;
      } else {
        ssrc[i] = Bsx + gn * KG + part * 4;
      }
    }
  }

  // copies q0 <= q < q1 of K-tile kt into stage st (q < kCB: code copy q,
  // else scale copy q - kCB); the bounds are compile-time constants
  auto issue_q = [&](int kt, int st, auto q0c, auto q1c) {
    constexpr int q0 = decltype(q0c)::value, q1 = decltype(q1c)::value;
    const uint32_t base = lds_base + (uint32_t)(st * L::kStage);
    const int64_t cofs = (int64_t)kt * L::kRowBytes, cofs_t = (int64_t)kt * 2048;
    const int64_t sofs = (int64_t)kt * kCPR, sofs_t = (int64_t)kt * 128;
#pragma unroll
    for (int i = 0; i < kCB; ++i)
      if (i >= q0 && i < q1)
        dma16(csrc[i] + (((ctile >> i) & 1u) ? cofs_t : cofs),
              base + (uint32_t)(L::kA + ((wave * kCB + i) % L::kCodeBlocks) * 1024));
#pragma unroll
    for (int i = 0; i < kSB; ++i)
      if (kCB + i >= q0 && kCB + i < q1)
        dma4(ssrc[i] + (((stile >> i) & 1u) ? sofs_t : sofs),
             base + (uint32_t)(L::kAs + ((wave * kSB + i) % L::kScaleBlocks) * 256));
  };
  auto issue = [&](int kt, int st) { issue_q(kt, st, std::integral_constant<int, 0>{}, std::integral_constant<int, kLPT>{}); };
  // the refill of a stage is issued in two halves: the first right after the
  // barrier that frees the stage, the second at the start of the next K-tile
  // (the copies stay in K-tile order, so the vmcnt counts are unchanged)
  constexpr int kHalf = (kLPT + 1) / 2;

  v16f acc[T::kFM][T::kFN];
#pragma unroll
  for (int mi = 0; mi < T::kFM; ++mi)
#pragma unroll
    for (int ni = 0; ni < T::kFN; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  const int nk = (int)(K / BK);
  // prologue: every stage receives a tile (the last tile again where there
  // are fewer tiles than stages), so each stage is one counted group of copies
#pragma unroll
  for (int s = 0; s < STAGES; ++s) issue(s < nk ? s : nk - 1, s);

  int rowA[T::kFM], rowB[T::kFN];
#pragma unroll
  for (int mi = 0; mi < T::kFM; ++mi) rowA[mi] = wm * T::kTM + mi * 32 + r32;
#pragma unroll
  for (int ni = 0; ni < T::kFN; ++ni) rowB[ni] = wn * T::kTN + ni * 32 + r32;
  const int sw = L::swz(r32);
  const int sshift = (kCPR == 4) ? 16 * h : 0;   // scale bytes of lane half h
  const int sofs_h = (kCPR == 8) ? 4 * h : 0;

  uint32_t sa[2][T::kFM], sb[2][T::kFN];      // scales: this tile's [0], the next tile's [1]
  uint4 fa[2][T::kFM], fb[2][T::kFN];         // fragments: two sub-steps' sets
  auto load_scales = [&](int kt, int set) {
    const uint8_t* base = smem + (kt % STAGES) * L::kStage;
#pragma unroll
    for (int mi = 0; mi < T::kFM; ++mi)
      sa[set][mi] = *reinterpret_cast<const uint32_t*>(base + L::kAs + rowA[mi] * kCPR + sofs_h) >> sshift;
#pragma unroll
    for (int ni = 0; ni < T::kFN; ++ni)
      sb[set][ni] = *reinterpret_cast<const uint32_t*>(base + L::kBs + rowB[ni] * kCPR + sofs_h) >> sshift;
  };
  auto load_frags = [&](int kt, int j, int set) {
    const uint8_t* base = smem + (kt % STAGES) * L::kStage;
#pragma unroll
    for (int mi = 0; mi < T::kFM; ++mi)
      fa[set][mi] = *reinterpret_cast<const uint4*>(base + L::kA + rowA[mi] * L::kRowBytes +
                                                     (((h * (kCPR / 2) + j) ^ sw) << 4));
#pragma unroll
    for (int ni = 0; ni < T::kFN; ++ni)
      fb[set][ni] = *reinterpret_cast<const uint4*>(base + L::kB + rowB[ni] * L::kRowBytes +
                                                     (((h * (kCPR / 2) + j) ^ sw) << 4));
  };

  // tile 0 has landed once at most STAGES-1 later groups remain in flight
  if constexpr (STAGES == 2) wait_vmcnt<kLPT>();
  else if constexpr (STAGES == 3) wait_vmcnt<2 * kLPT>();
  else wait_vmcnt<3 * kLPT>();
  block_barrier();
  load_scales(0, 0);
  load_frags(0, 0, 0);

  constexpr int kMF = T::kFM * T::kFN;   // MFMAs per sub-step
  constexpr int kRD = T::kFM + T::kFN;   // fragment reads per sub-step
  constexpr int kPre = kMF >= 16 ? 4 : (kMF >= 8 ? 2 : 1);   // MFMAs ahead of a sub-step's copies and barrier
  constexpr int kSlots = kRD < kMF - kPre ? kRD : kMF - kPre;   // MFMAs that each carry some of the reads
  for (int kt = 0; kt < nk; ++kt) {
    static_for<NSUB>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      constexpr int cur = j & 1;
      // the first kPre MFMAs of each sub-step go ahead of its copies, waits
      // and barrier: they keep the SIMD's MFMA pipe busy while the wave
      // issues copies or waits
      mfma_range_t<j, 0, kPre>(acc, fa[cur], fb[cur], sa[0], sb[0]);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (j < NSUB - 1) {
        if constexpr (j == 0) {
          if (kt > 0) {
            const int pt = kt - 1 + STAGES;
            issue_q(pt < nk ? pt : nk - 1, (kt - 1) % STAGES, std::integral_constant<int, kHalf>{},
                    std::integral_constant<int, kLPT>{});
          }
        }
        load_frags(kt, j + 1, cur ^ 1);
      } else {
        // every wave holds this tile's last fragments: stage kt % STAGES is
        // free once all waves are here with their reads of it returned (the
        // barrier may be scheduled right after those reads are issued).
        // Tiles up to kt-1+STAGES are issued.
        wait_lgkmcnt0();
        wait_vmcnt<(STAGES - 2) * kLPT>();   // tile kt+1 has landed
        block_barrier();
        issue_q(kt + STAGES < nk ? kt + STAGES : nk - 1, kt % STAGES, std::integral_constant<int, 0>{},
                std::integral_constant<int, kHalf>{});
        load_scales(kt + 1, 1);              // past the last tile: unused, in-bounds LDS bytes
        load_frags(kt + 1, 0, cur ^ 1);
      }
      mfma_range_t<j, kPre, kMF>(acc, fa[cur], fb[cur], sa[0], sb[0]);
      // interleave: one MFMA, then that MFMA's share of the reads above
      constexpr int kReads = (j == NSUB - 1 ? 2 : 1) * kRD;
      constexpr int kPerSlot = (kReads + kSlots - 1) / kSlots;
#pragma unroll
      for (int q = 0; q < kSlots; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, kPerSlot, 0);
      }
      if constexpr (kMF - kPre - kSlots > 0) __builtin_amdgcn_sched_group_barrier(0x008, kMF - kPre - kSlots, 0);
    });
#pragma unroll
    for (int mi = 0; mi < T::kFM; ++mi) sa[0][mi] = sa[1][mi];
#pragma unroll
    for (int ni = 0; ni < T::kFN; ++ni) sb[0][ni] = sb[1][ni];
  }
  wait_vmcnt<0>();   // no copy into LDS outlives the loop (the stages are reused below)

  if constexpr (OUT == 0) {
    store_wave_tile_f32(acc, Y, row_begin + wm * T::kTM, row_end, n0 + wn * T::kTN, N, r32, h);
  } else {
    static_assert(STAGES * L::kStage >= kWaves * kEpiLdsBytes, "epilogue tiles must fit in the stages");
    __syncthreads();   // every wave is done reading the last K-tile
    store_wave_tile_lds<OUT>(acc, reinterpret_cast<float*>(smem + wave * kEpiLdsBytes), Y, row_begin + wm * T::kTM,
                             row_end, n0 + wn * T::kTN, N, lane);
  }
}

}  // namespace macaq

// Online activation transform + OCP MXFP4 quantization, and the offline
// weight preparation that runs the same pipeline with r = 1/s.
//
// Sources: "MACaQ Enables Streaming W4A4 Quantization with 32.5GB GPU
// Memory", section "Quantization mechanism" (scale + block Hadamard on the
// activation before the FP4 matmul, transformed weight prepared offline);
// "华为开源MACaQ:本地量化提速3倍", sections "量化不是单纯把模型“压小”" (OCP
// MXFP4: 32-element groups, E8M0 scale, E2M1 elements) and "MACaQ
// 真正解决的是跨层耦合" (32-element Hadamard blocks aligned to the groups).
//
// Work layout: one wave covers 512 consecutive columns (16 groups; lane l
// owns columns 8l .. 8l+7, a quad of lanes owns a group) of ROWS_PER_WAVE
// consecutive rows.  Each lane issues one 16-byte load per row (bf16) or two
// (fp32), so a wave's loads are fully coalesced 1 KiB (2 KiB) segments; all
// rows' loads are issued before the first row is transformed.  The 8 scale
// factors of the lane stay in registers across the rows (reloaded only when
// the expert changes).  Codes leave as one dword per lane per row (coalesced
// 256-byte segments); the scale byte is written by lane 0 of each quad.
//
// The kernel is HBM-bound: per element it reads 2 bytes (bf16) and writes
// 17/32 bytes.
#include "mx_common.h"

namespace macaq {

constexpr int kActRowsPerWave = 8;
constexpr int kActWavesPerBlock = 4;

// Element type tag of bf16 activations (raw 16-bit patterns).
struct Bf16Tag {};

template <typename XT>
struct RowLoad;

template <>
struct RowLoad<Bf16Tag> {
  uint4 v;
  __device__ __forceinline__ void load(const void* base, int64_t elem_off) {
    v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + elem_off);
  }
  __device__ __forceinline__ void widen(float (&t)[8]) const {
    t[0] = bf16_lo(v.x); t[1] = bf16_hi(v.x);
    t[2] = bf16_lo(v.y); t[3] = bf16_hi(v.y);
    t[4] = bf16_lo(v.z); t[5] = bf16_hi(v.z);
    t[6] = bf16_lo(v.w); t[7] = bf16_hi(v.w);
  }
};

template <>
struct RowLoad<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const void* base, int64_t elem_off) {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + elem_off);
    a = p[0];
    b = p[1];
  }
  __device__ __forceinline__ void widen(float (&t)[8]) const {
    t[0] = a.x; t[1] = a.y; t[2] = a.z; t[3] = a.w;
    t[4] = b.x; t[5] = b.y; t[6] = b.z; t[7] = b.w;
  }
};

// Expert of row r: rows_per_expert > 0 gives r / rows_per_expert (weights);
// otherwise the sorted offsets are scanned forward from `hint`.
__device__ __forceinline__ int expert_of(int64_t r, const int32_t* __restrict__ offsets, int E,
                                         int64_t rows_per_expert, int hint) {
  if (rows_per_expert > 0) return (int)(r / rows_per_expert);
  if (offsets == nullptr) return 0;
  int e = hint;
  while (e + 1 < E && r >= (int64_t)offsets[e + 1]) ++e;
  return e;
}

template <typename XT, bool RECIP>
__global__ __launch_bounds__(64 * kActWavesPerBlock) void act_quant_kernel(
    const void* __restrict__ x, const float* __restrict__ s, const int32_t* __restrict__ offsets,
    int E, int64_t rows_per_expert, int64_t M, int64_t K, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * kActWavesPerBlock + (threadIdx.x >> 6);
  const int64_t nchunk = ceil_div(K, 512);
  const int64_t chunk = wave % nchunk;
  const int64_t r0 = (wave / nchunk) * kActRowsPerWave;
  if (r0 >= M) return;
  const int64_t col = chunk * 512 + (int64_t)lane * 8;
  const bool active = col < K;  // K % 32 == 0: whole quads are in or out
  const uint32_t quad = (uint32_t)lane & 3u;
  const int nrows = (int)((M - r0) < kActRowsPerWave ? (M - r0) : kActRowsPerWave);

  RowLoad<XT> ld[kActRowsPerWave];
#pragma unroll
  for (int i = 0; i < kActRowsPerWave; ++i)
    if (active && i < nrows) ld[i].load(x, (r0 + i) * K + col);

  // Expert of the first row: the first e with offsets[e+1] > r0.
  int e = 0;
  if (rows_per_expert == 0 && offsets != nullptr) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)offsets[mid + 1] > r0) hi = mid; else lo = mid + 1;
    }
    e = lo;
  } else {
    e = expert_of(r0, offsets, E, rows_per_expert, 0);
  }
  int cur_e = -1;
  float sc[8];

#pragma unroll
  for (int i = 0; i < kActRowsPerWave; ++i) {
    if (i >= nrows) break;
    const int64_t r = r0 + i;
    e = expert_of(r, offsets, E, rows_per_expert, e);
    if (e != cur_e) {
      cur_e = e;
      if (active) {
        const float4* sp = reinterpret_cast<const float4*>(s + (int64_t)e * K + col);
        const float4 s0 = sp[0], s1 = sp[1];
        sc[0] = s0.x; sc[1] = s0.y; sc[2] = s0.z; sc[3] = s0.w;
        sc[4] = s1.x; sc[5] = s1.y; sc[6] = s1.z; sc[7] = s1.w;
        if (RECIP) {
#pragma unroll
          for (int j = 0; j < 8; ++j) sc[j] = 1.0f / sc[j];  // IEEE-correct fp32 division
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) sc[j] = 0.0f;
      }
    }
    float t[8];
    if (active) {
      ld[i].widen(t);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) t[j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = t[j] * sc[j];
    hadamard32_quad(t, quad);
    uint32_t b;
    const uint32_t packed = quantize_quad(t, &b);
    if (active) {
      *reinterpret_cast<uint32_t*>(codes + r * (K >> 1) + (col >> 1)) = packed;
      if (quad == 0) scales[r * (K >> 5) + (col >> 5)] = (uint8_t)b;
    }
  }
}

__global__ void encode_e2m1_kernel(const float* __restrict__ v, int64_t n, uint8_t* __restrict__ out) {
  const int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i0 >= n) return;
  float t[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) t[j] = (i0 + j < n) ? v[i0 + j] : 0.0f;
  const uint32_t p = e2m1_pack8(t);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (i0 + j < n) out[i0 + j] = (uint8_t)((p >> (4 * j)) & 0xFu);
}

// ---------------------------------------------------------------- launchers

hipError_t launch_act_quant(const void* x, bool x_f32, bool reciprocal, const float* s,
                            const int32_t* offsets, int E, int64_t rows_per_expert, int64_t M,
                            int64_t K, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  const int64_t waves = ceil_div(K, 512) * ceil_div(M, kActRowsPerWave);
  const int64_t blocks = ceil_div(waves, kActWavesPerBlock);
  const dim3 grid((unsigned)blocks), block(64 * kActWavesPerBlock);
  if (x_f32) {
    if (reciprocal)
      act_quant_kernel<float, true><<<grid, block, 0, stream>>>(x, s, offsets, E, rows_per_expert, M, K, codes, scales);
    else
      act_quant_kernel<float, false><<<grid, block, 0, stream>>>(x, s, offsets, E, rows_per_expert, M, K, codes, scales);
  } else {
    if (reciprocal)
      act_quant_kernel<Bf16Tag, true><<<grid, block, 0, stream>>>(x, s, offsets, E, rows_per_expert, M, K, codes, scales);
    else
      act_quant_kernel<Bf16Tag, false><<<grid, block, 0, stream>>>(x, s, offsets, E, rows_per_expert, M, K, codes, scales);
  }
  return hipGetLastError();
}

hipError_t launch_encode_e2m1(const float* v, int64_t n, uint8_t* codes, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t threads = ceil_div(n, 8);
  encode_e2m1_kernel<<<dim3((unsigned)ceil_div(threads, 256)), dim3(256), 0, stream>>>(v, n, codes);
  return hipGetLastError();
}

}  // namespace macaq

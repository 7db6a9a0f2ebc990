// Decode-sized layer (M <= 32 rows): MXFP4 GEMM that streams the prepared
// weight W' from HBM, with an optional fused activation transform.
//
// Sources: "MACaQ Enables Streaming W4A4 Quantization with 32.5GB GPU
// Memory", section "Deployment recommendations" (prefill and decode should be
// measured separately; the online activation transform weighs most on
// low-batch decode) and "华为开源MACaQ:本地量化提速3倍", section
// "推理最快达到 FP16 的 3.06 倍" (low-concurrency decode is bound by memory
// bandwidth).  The arithmetic is the layer's (include/macaq.h).
//
// At M <= 32 the layer is bound by reading W' (17/32 byte per weight).  The
// weight is the MFMA's A operand (32 weight rows per instruction) and the
// <= 32 activation rows are the B operand:
//   D[n][m] = sum_k w'(n,k) a(m,k),  v_mfma_scale_f32_32x32x64_f8f6f4.
// Operands go straight from global memory into registers; W' never passes
// through LDS.  K permutation (the same on both operands): in a 256-wide K
// chunk, lane half h of sub-step j takes group 2j + h, so for each weight
// row the two lanes of one instruction read 32 contiguous bytes and the four
// instructions of a chunk read the row's 128-byte line in order.  A lane's
// four scale bytes (groups h, 2+h, 4+h, 6+h) are gathered with one byte
// permute so that op_sel byte j is sub-step j's scale.
//
// Work split: a block owns 32 weight rows and the whole K range, which its
// WAVES waves split; each wave issues the loads of two chunks at a time and
// the waves' 32x32 partial sums are added in LDS in wave order
// (deterministic).  No cross-block
// reduction is needed, so the path needs no workspace.
//
// Fused variant: before the GEMM the block transforms and quantizes x[0:M,
// :] (the quad-per-group routine of the activation kernel) into LDS; the B
// fragments then come from LDS.  Every block repeats that transform, so the
// fused variant pays off only for very small M.
#include "mx_common.h"

namespace macaq {

typedef int v8i_d __attribute__((ext_vector_type(8)));
typedef float v16f_d __attribute__((ext_vector_type(16)));

constexpr int kDecRows = 32;               // weight rows per block
constexpr int kDecMaxM = 32;
constexpr size_t kDecLdsMax = 160 * 1024;   // LDS per workgroup on gfx950

__device__ __forceinline__ v8i_d dec_operand(const uint4& q) {
  v8i_d r;
  r[0] = (int)q.x; r[1] = (int)q.y; r[2] = (int)q.z; r[3] = (int)q.w;
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}

template <int J>
__device__ __forceinline__ void dec_mfma(v16f_d& acc, const uint4 (&wa)[4], const uint4 (&xb)[4], uint32_t ws,
                                         uint32_t xs) {
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(dec_operand(wa[J]), dec_operand(xb[J]), acc, 4, 4, J,
                                                        (int)ws, J, (int)xs);
}

// Scale bytes of groups h, 2+h, 4+h, 6+h of a chunk (8 bytes lo|hi) packed
// into bytes 0..3.
__device__ __forceinline__ uint32_t gather_scales(uint32_t lo, uint32_t hi, int h) {
  // v_perm_b32 selector bytes index {hi[3..0], lo[3..0]} as 7..0
  const uint32_t sel = h ? 0x07050301u : 0x06040200u;
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// One chunk of one operand row: lane (r, h) takes the 16-byte groups 2j + h.
__device__ __forceinline__ void load_chunk(const uint8_t* row, int64_t chunk, int h, uint4 (&v)[4]) {
  const uint4* p = reinterpret_cast<const uint4*>(row + chunk * 128) + h;
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = p[2 * j];
}
__device__ __forceinline__ uint32_t load_scales(const uint8_t* srow, int64_t chunk, int h) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(srow + chunk * 8);
  return gather_scales(p[0], p[1], h);
}

// Element type tag of bf16 activations for the fused prologue.
struct DecBf16 {};

template <typename XT>
__device__ __forceinline__ void dec_load8(const void* x, int64_t off, float (&t)[8]);
template <>
__device__ __forceinline__ void dec_load8<DecBf16>(const void* x, int64_t off, float (&t)[8]) {
  const uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + off);
  t[0] = bf16_lo(v.x); t[1] = bf16_hi(v.x); t[2] = bf16_lo(v.y); t[3] = bf16_hi(v.y);
  t[4] = bf16_lo(v.z); t[5] = bf16_hi(v.z); t[6] = bf16_lo(v.w); t[7] = bf16_hi(v.w);
}
template <>
__device__ __forceinline__ void dec_load8<float>(const void* x, int64_t off, float (&t)[8]) {
  const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + off);
  const float4 a = p[0], b = p[1];
  t[0] = a.x; t[1] = a.y; t[2] = a.z; t[3] = a.w; t[4] = b.x; t[5] = b.y; t[6] = b.z; t[7] = b.w;
}

// LDS row strides of the fused activation copy (padded against bank conflicts)
__host__ __device__ constexpr int64_t dec_xrow_bytes(int64_t K) { return K / 2 + 16; }
__host__ __device__ constexpr int64_t dec_xrow_groups(int64_t K) { return K / 32 + 8; }

template <int WAVES, bool FUSED, typename XT>
__global__ __launch_bounds__(64 * WAVES) void decode_gemm_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As,     // activation codes/scales (unfused)
    const void* __restrict__ x, const float* __restrict__ s,           // activations and scale (fused)
    const uint8_t* __restrict__ W, const uint8_t* __restrict__ Ws, int64_t M, int64_t N, int64_t K,
    float* __restrict__ Y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
  constexpr int kThreads = 64 * WAVES;
  const int64_t n0 = (int64_t)blockIdx.x * kDecRows;
  const int64_t KB = K >> 1, KG = K >> 5;
  const int kc = (int)(K >> 8);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r32 = lane & 31;
  const int h = lane >> 5;

  // LDS: [WAVES][32][32] fp32 partials, then (fused) the activation codes
  // [M][K/2 + 16] and scales [M][K/32 + 8].
  float* red = reinterpret_cast<float*>(dsm);
  const int64_t xrb = dec_xrow_bytes(K), xrg = dec_xrow_groups(K);
  uint8_t* xcodes = dsm + WAVES * 32 * 32 * 4;
  uint8_t* xscales = xcodes + M * xrb;

  if constexpr (FUSED) {
    const int groups_per_row = (int)KG;
    const int tasks = (int)M * groups_per_row;      // one quad of lanes per 32-element group
    const uint32_t quad = (uint32_t)lane & 3u;
    for (int t0 = tid >> 2; t0 < tasks; t0 += kThreads / 4) {
      const int m = t0 / groups_per_row, g = t0 % groups_per_row;
      const int64_t col = (int64_t)g * 32 + quad * 8;
      float t[8];
      dec_load8<XT>(x, m * K + col, t);
      const float4* sp = reinterpret_cast<const float4*>(s + col);
      const float4 s0 = sp[0], s1 = sp[1];
      t[0] = t[0] * s0.x; t[1] = t[1] * s0.y; t[2] = t[2] * s0.z; t[3] = t[3] * s0.w;
      t[4] = t[4] * s1.x; t[5] = t[5] * s1.y; t[6] = t[6] * s1.z; t[7] = t[7] * s1.w;
      hadamard32_quad(t, quad);
      uint32_t b;
      const uint32_t packed = quantize_quad(t, &b);
      *reinterpret_cast<uint32_t*>(xcodes + m * xrb + g * 16 + quad * 4) = packed;
      if (quad == 0) xscales[m * xrg + g] = (uint8_t)b;
    }
    __syncthreads();
  }

  // ---- this wave's chunks
  const int per_wave = (kc + WAVES - 1) / WAVES;
  const int c0 = wave * per_wave;
  const int c1 = (c0 + per_wave) < kc ? (c0 + per_wave) : kc;
  int64_t wn = n0 + r32;
  if (wn >= N) wn = N - 1;
  const int64_t am = r32 < M ? r32 : M - 1;
  const uint8_t* wrow = W + wn * KB;
  const uint8_t* wsrow = Ws + wn * KG;
  const uint8_t* arow = FUSED ? xcodes + am * xrb : A + am * KB;
  const uint8_t* asrow = FUSED ? xscales + am * xrg : As + am * KG;

  v16f_d acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

  // Two chunks per step: all their loads are issued before the first MFMA;
  // no registers carry over between steps (other waves of the CU cover the
  // load latency of this one).
  for (int c = c0; c < c1; c += 2) {
    const bool two = c + 1 < c1;
    uint4 wa0[4], xb0[4], wa1[4], xb1[4];
    load_chunk(wrow, c, h, wa0);
    load_chunk(arow, c, h, xb0);
    const uint32_t ws0 = load_scales(wsrow, c, h);
    const uint32_t xs0 = load_scales(asrow, c, h);
    uint32_t ws1 = 0, xs1 = 0;
    if (two) {
      load_chunk(wrow, c + 1, h, wa1);
      load_chunk(arow, c + 1, h, xb1);
      ws1 = load_scales(wsrow, c + 1, h);
      xs1 = load_scales(asrow, c + 1, h);
    }
    dec_mfma<0>(acc, wa0, xb0, ws0, xs0);
    dec_mfma<1>(acc, wa0, xb0, ws0, xs0);
    dec_mfma<2>(acc, wa0, xb0, ws0, xs0);
    dec_mfma<3>(acc, wa0, xb0, ws0, xs0);
    if (two) {
      dec_mfma<0>(acc, wa1, xb1, ws1, xs1);
      dec_mfma<1>(acc, wa1, xb1, ws1, xs1);
      dec_mfma<2>(acc, wa1, xb1, ws1, xs1);
      dec_mfma<3>(acc, wa1, xb1, ws1, xs1);
    }
  }

  // ---- add the waves' 32x32 tiles in wave order.  Lane (r32, h), register r
  // holds D[n = 8*(r/4) + 4*h + r%4][m = r32].
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int n = 8 * (r >> 2) + 4 * h + (r & 3);
    red[(wave * 32 + n) * 32 + r32] = acc[r];
  }
  __syncthreads();
  for (int idx = tid; idx < 32 * 32; idx += kThreads) {
    const int n = idx & 31, m = idx >> 5;   // consecutive threads: consecutive n of one row of y
    float v = red[n * 32 + m];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) v = v + red[(w * 32 + n) * 32 + m];
    if (m < M && n0 + n < N) Y[(int64_t)m * N + n0 + n] = v;
  }
}

// ---------------------------------------------------------------- host side

static int decode_waves(int64_t K) {
  const int64_t kc = K / 256;
  if (kc >= 64) return 16;
  if (kc >= 24) return 8;
  return 4;
}

static size_t decode_lds_bytes(int waves, int64_t M, int64_t K, bool fused) {
  size_t b = (size_t)waves * 32 * 32 * 4;
  if (fused) b += (size_t)M * (size_t)(dec_xrow_bytes(K) + dec_xrow_groups(K));
  return b;
}

bool decode_supported(int64_t M, int64_t N, int64_t K, int64_t E) {
  return E == 1 && M >= 1 && M <= kDecMaxM && N >= 1 && K % 256 == 0;
}

template <int WAVES, bool FUSED, typename XT>
static hipError_t launch_decode_w(const uint8_t* A, const uint8_t* As, const void* x, const float* s,
                                  const uint8_t* W, const uint8_t* Ws, int64_t M, int64_t N, int64_t K, float* Y,
                                  hipStream_t stream) {
  const size_t lds = decode_lds_bytes(WAVES, M, K, FUSED);
  if (FUSED) {
    static const hipError_t attr = hipFuncSetAttribute((const void*)decode_gemm_kernel<WAVES, FUSED, XT>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       (int)kDecLdsMax);
    if (attr != hipSuccess) return attr;
  }
  decode_gemm_kernel<WAVES, FUSED, XT><<<dim3((unsigned)ceil_div(N, kDecRows)), dim3(64 * WAVES), lds, stream>>>(
      A, As, x, s, W, Ws, M, N, K, Y);
  return hipGetLastError();
}

template <bool FUSED, typename XT>
static hipError_t launch_decode_impl(const uint8_t* A, const uint8_t* As, const void* x, const float* s,
                                     const uint8_t* W, const uint8_t* Ws, int64_t M, int64_t N, int64_t K,
                                     float* Y, hipStream_t stream) {
  switch (decode_waves(K)) {
    case 16: return launch_decode_w<16, FUSED, XT>(A, As, x, s, W, Ws, M, N, K, Y, stream);
    case 8: return launch_decode_w<8, FUSED, XT>(A, As, x, s, W, Ws, M, N, K, Y, stream);
    default: return launch_decode_w<4, FUSED, XT>(A, As, x, s, W, Ws, M, N, K, Y, stream);
  }
}

hipError_t launch_decode_gemm(const uint8_t* A, const uint8_t* As, const uint8_t* W, const uint8_t* Ws, int64_t M,
                              int64_t N, int64_t K, float* Y, hipStream_t stream) {
  return launch_decode_impl<false, DecBf16>(A, As, nullptr, nullptr, W, Ws, M, N, K, Y, stream);
}

// -------- fused transform + GEMM entry used by macaq_linear

bool linear_fused_supported(int64_t M, int64_t N, int64_t K, int64_t E) {
  return decode_supported(M, N, K, E) && decode_lds_bytes(decode_waves(K), M, K, true) <= kDecLdsMax;
}

hipError_t launch_linear_fused(const void* x, bool x_f32, const float* s, const uint8_t* B, const uint8_t* Bs,
                               int64_t M, int64_t N, int64_t K, float* Y, hipStream_t stream) {
  if (x_f32) return launch_decode_impl<true, float>(nullptr, nullptr, x, s, B, Bs, M, N, K, Y, stream);
  return launch_decode_impl<true, DecBf16>(nullptr, nullptr, x, s, B, Bs, M, N, K, Y, stream);
}

}  // namespace macaq

// Offline steps driven by the Hessian of the layer input: the Hessian itself,
// accumulated from calibration rows, and the Hessian exponent search that
// picks the E8M0 byte of every weight group.
//
// Sources: "MACaQ Enables Streaming W4A4 Quantization with 32.5GB GPU
// Memory", section "Flip-Refinement: optimizing FP4 codes with second-order
// information" (the loss of a quantized vector is one half of
// (x - q)^T H (x - q), H the Hessian of the layer input); "华为开源MACaQ:本地
// 量化提速3倍", section "Flip-Refinement:不重算,只改最值得改的 4-bit 数值" (the
// Hessian comes from calibration statistics; the ablation lists a Hessian
// exponent search above plain round-to-nearest).
//
// Readings (the pages give no rule):
// * H_e = X'^T X' over expert e's calibration rows, X' the fp32 activation
//   after the online transform (scale, 32-point butterfly, times C), i.e.
//   the Hessian in the basis the weights are quantized in.  Accumulated in
//   fp64 (every product of two fp32 values is exact there), stored as fp32.
// * Exponent search: per weight group the candidates are the plain byte b0
//   (exponent of max|x'| minus 2) and b0 + 1.  Each candidate's codes are the
//   usual round-to-nearest-even, saturating E2M1 codes; its error is
//   q = d^T H_gg d, d = x' - dequant (exact in fp64), H_gg the group's
//   diagonal 32x32 block.  q is summed in fp64 in a fixed order: u_i over
//   j = 0..31, then q over i = 0..31, no fused multiply-add (the library is
//   built with -ffp-contract=off).  b0 + 1 is kept only if its q is strictly
//   smaller.
#include "mx_common.h"

namespace macaq {

namespace {

constexpr int kHTile = 128;   // Hessian tile edge
constexpr int kHRows = 16;    // calibration rows staged per step

// 32 elements of one row group, widened to fp32.
template <int EB>
__device__ __forceinline__ void load_group(const void* base, int64_t elem, float (&t)[32]) {
  if constexpr (EB == 2) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = p[q];
      t[8 * q + 0] = bf16_lo(v.x); t[8 * q + 1] = bf16_hi(v.x);
      t[8 * q + 2] = bf16_lo(v.y); t[8 * q + 3] = bf16_hi(v.y);
      t[8 * q + 4] = bf16_lo(v.z); t[8 * q + 5] = bf16_hi(v.z);
      t[8 * q + 6] = bf16_lo(v.w); t[8 * q + 7] = bf16_hi(v.w);
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + elem);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint4 v = p[q];
      t[4 * q + 0] = __uint_as_float(v.x); t[4 * q + 1] = __uint_as_float(v.y);
      t[4 * q + 2] = __uint_as_float(v.z); t[4 * q + 3] = __uint_as_float(v.w);
    }
  }
}

// x' of one group in place: t = t * f (fp32), butterfly stages h = 1, 2, 4,
// 8, 16 (lower a + b, upper a - b), then times C.
__device__ __forceinline__ void transform_group(float (&t)[32], const float (&f)[32]) {
#pragma unroll
  for (int i = 0; i < 32; ++i) t[i] = t[i] * f[i];
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & h) == 0) {
        const float a = t[i], b = t[i + h];
        t[i] = a + b;
        t[i + h] = a - b;
      }
    }
  }
  const float c = hadamard_norm();
#pragma unroll
  for (int i = 0; i < 32; ++i) t[i] = t[i] * c;
}

}  // namespace

// ---------------------------------------------------------------------------
// Hessian: one 256-thread block per 128x128 tile (ti <= tj) of one expert's
// H.  Per step, 16 calibration rows are transformed (threads 0..127 each take
// one row-group of the two column ranges) into LDS as fp64; every thread
// then accumulates its 8x8 entries (rows ty + 16a, columns tx + 16c) with
// fp64 fused multiply-adds over the staged rows.  Off-diagonal tiles are also
// written transposed, so H comes out exactly symmetric.
template <int EB>
__global__ __launch_bounds__(256) void hessian_tile_kernel(const void* __restrict__ x, const float* __restrict__ s,
                                                           const int32_t* __restrict__ offsets, int64_t T,
                                                           int64_t K, float* __restrict__ H) {
  __shared__ double xa[kHRows][kHTile];
  __shared__ double xb[kHRows][kHTile];
  const int nt = (int)(K / kHTile);
  int rem = blockIdx.x, ti = 0;
  while (rem >= nt - ti) { rem -= nt - ti; ++ti; }
  const int tj = ti + rem;
  const int e = blockIdx.y;
  const int64_t r0 = offsets ? offsets[e] : 0;
  const int64_t r1 = offsets ? offsets[e + 1] : T;
  const float* se = s + (int64_t)e * K;
  float* He = H + (int64_t)e * K * K;
  const int tid = threadIdx.x;
  const bool diag = ti == tj;

  // transform task of this thread: row (tid >> 3) of the step, group (tid & 7):
  // groups 0..3 are the four 32-column groups of tile ti, 4..7 those of tj
  const int trow = tid >> 3, tgrp = tid & 7;
  const bool tasker = tid < 128 && (!diag || tgrp < 4);
  const int64_t tcol = (int64_t)(tgrp < 4 ? ti : tj) * kHTile + 32 * (tgrp & 3);
  double(*tdst)[kHTile] = tgrp < 4 ? xa : xb;
  float f[32];
  if (tasker) {
#pragma unroll
    for (int i = 0; i < 32; ++i) f[i] = se[tcol + i];
  }

  const int ty = tid >> 4, tx = tid & 15;
  double acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[a][c] = 0.0;

  for (int64_t base = r0; base < r1; base += kHRows) {
    if (tasker) {
      const int64_t row = base + trow;
      float t[32];
      if (row < r1) {
        load_group<EB>(x, row * K + tcol, t);
        transform_group(t, f);
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) t[i] = 0.0f;
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) tdst[trow][32 * (tgrp & 3) + i] = (double)t[i];
    }
    __syncthreads();
    const double(*ys)[kHTile] = diag ? xa : xb;
#pragma unroll 2
    for (int r = 0; r < kHRows; ++r) {
      double av[8], bv[8];
#pragma unroll
      for (int a = 0; a < 8; ++a) av[a] = xa[r][ty + 16 * a];
#pragma unroll
      for (int c = 0; c < 8; ++c) bv[c] = ys[r][tx + 16 * c];
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[a][c] = __builtin_fma(av[a], bv[c], acc[a][c]);
    }
    __syncthreads();
  }

  const int64_t i0 = (int64_t)ti * kHTile, j0 = (int64_t)tj * kHTile;
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float v = (float)acc[a][c];
      const int64_t i = i0 + ty + 16 * a, j = j0 + tx + 16 * c;
      He[i * K + j] = v;
      if (!diag) He[j * K + i] = v;
    }
}

// ---------------------------------------------------------------------------
// Exponent search: one 256-thread block per (256 weight rows, group g,
// expert e); one thread per row.  The group's Hessian block (fp64) and
// r = 1/s (fp32, IEEE division) are staged in LDS once per block.
template <int EB>
__global__ __launch_bounds__(256) void prep_hessian_kernel(const void* __restrict__ w, const float* __restrict__ s,
                                                           const float* __restrict__ H, int64_t N, int64_t K,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales) {
  __shared__ double hs[32][32];
  __shared__ float rs[32];
  const int g = blockIdx.y, e = blockIdx.z, tid = threadIdx.x;
  const int64_t col = 32 * (int64_t)g;
  const float* He = H + (int64_t)e * K * K;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int idx = tid + 256 * k;
    hs[idx >> 5][idx & 31] = (double)He[(col + (idx >> 5)) * K + col + (idx & 31)];
  }
  if (tid < 32) rs[tid] = 1.0f / s[(int64_t)e * K + col + tid];
  __syncthreads();
  const int64_t n = (int64_t)blockIdx.x * 256 + tid;
  if (n >= N) return;
  const int64_t row = (int64_t)e * N + n;

  float xp[32], f[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) f[i] = rs[i];
  load_group<EB>(w, row * K + col, xp);
  transform_group(xp, f);
  float m = fabsf(xp[0]);
#pragma unroll
  for (int i = 1; i < 32; ++i) m = fmaxf(m, fabsf(xp[i]));
  const uint32_t b0 = e8m0_from_amax(m);

  // codes and exact fp64 deltas of both candidates (b0 <= 252 for finite
  // input, so b0 + 1 still has a normal 2^(127-b) multiplier)
  uint32_t pk[2][4];
  double d[2][32];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t b = b0 + k;
    const float inv = inv_scale(b);
    const double sc = __longlong_as_double((long long)(b + 896u) << 52);  // 2^(b-127)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = xp[8 * q + i] * inv;
      const uint32_t p = e2m1_pack8(v);
      pk[k][q] = p;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t c = (p >> (4 * i)) & 0xFu, mi = c & 7u;
        // E2M1 magnitude of index mi: 0, 0.5 for mi < 2, else (1 + (mi & 1) / 2) * 2^((mi >> 1) - 1)
        const float mag = mi < 2u ? 0.5f * (float)mi : __uint_as_float((((mi >> 1) + 126u) << 23) | ((mi & 1u) << 22));
        const double deq = (double)((c & 8u) ? -mag : mag) * sc;
        d[k][8 * q + i] = (double)xp[8 * q + i] - deq;
      }
    }
  }

  double q0 = 0.0, q1 = 0.0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    double u0 = 0.0, u1 = 0.0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const double h = hs[i][j];
      u0 = u0 + h * d[0][j];
      u1 = u1 + h * d[1][j];
    }
    q0 = q0 + d[0][i] * u0;
    q1 = q1 + d[1][i] * u1;
  }
  const int k = q1 < q0 ? 1 : 0;
  reinterpret_cast<uint4*>(codes + row * (K / 2) + 16 * g)[0] =
      k ? make_uint4(pk[1][0], pk[1][1], pk[1][2], pk[1][3]) : make_uint4(pk[0][0], pk[0][1], pk[0][2], pk[0][3]);
  scales[row * (K / 32) + g] = (uint8_t)(b0 + k);
}

hipError_t launch_hessian(const void* x, bool x_f32, const float* s, const int32_t* offsets, int E, int64_t T,
                          int64_t K, float* H, hipStream_t stream) {
  const int64_t nt = K / kHTile;
  const dim3 grid((unsigned)(nt * (nt + 1) / 2), (unsigned)E);
  if (x_f32)
    hipLaunchKernelGGL(hessian_tile_kernel<4>, grid, dim3(256), 0, stream, x, s, offsets, T, K, H);
  else
    hipLaunchKernelGGL(hessian_tile_kernel<2>, grid, dim3(256), 0, stream, x, s, offsets, T, K, H);
  return hipGetLastError();
}

hipError_t launch_prep_hessian(const void* w, bool w_f32, const float* s, const float* H, int E, int64_t N,
                               int64_t K, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const dim3 grid((unsigned)ceil_div(N, 256), (unsigned)(K / 32), (unsigned)E);
  if (w_f32)
    hipLaunchKernelGGL(prep_hessian_kernel<4>, grid, dim3(256), 0, stream, w, s, H, N, K, codes, scales);
  else
    hipLaunchKernelGGL(prep_hessian_kernel<2>, grid, dim3(256), 0, stream, w, s, H, N, K, codes, scales);
  return hipGetLastError();
}

}  // namespace macaq

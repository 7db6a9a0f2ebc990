// Measurement aids (declared in include/macaq_probe.h): MFMA throughput from
// registers, and HBM streaming rates for a given read/write mix.  The
// kernels' roofline fractions are quoted against the datasheet figures
// (10.1 PFLOP/s, 8 TB/s); these kernels show what the chip sustains for the
// same instruction with no memory traffic, and for plain streams.
#include "mx_common.h"
#include "macaq_probe.h"

namespace macaq {

typedef int v8i_p __attribute__((ext_vector_type(8)));
typedef float v16f_p __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v8i_p probe_operand(const uint4& q) {
  v8i_p r;
  r[0] = (int)q.x; r[1] = (int)q.y; r[2] = (int)q.z; r[3] = (int)q.w;
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}

// FN accumulator columns: 4 x 4 tiles (256 accumulator registers) with one
// wave per SIMD, 4 x 2 with two (each wave then has at most 256 registers)
template <int WAVES, int FN>
__global__ __launch_bounds__(64 * WAVES) void mfma_probe_kernel(const uint4* __restrict__ src, int iters,
                                                                float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  uint4 fa[4], fb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    fa[i] = src[lane * 8 + i];
    fb[i] = src[lane * 8 + 4 + i];
  }
  constexpr int kScale = 0x7F7F7F7F;   // E8M0 127 = 1.0 in every byte
  v16f_p acc[4][FN];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < FN; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < FN; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(probe_operand(fa[mi]), probe_operand(fb[ni]),
                                                                      acc[mi][ni], 4, 4, 0, kScale, 0, kScale);
  }
  float sum = 0.0f;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < FN; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += acc[mi][ni][r];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

// Streaming probe: grid-stride over 16-byte chunks, non-temporal loads.
typedef unsigned int u32x4_p __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_probe_kernel(const u32x4_p* __restrict__ src, int64_t nr,
                                                           u32x4_p* __restrict__ dst, int64_t nw,
                                                           uint32_t* __restrict__ out) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  u32x4_p acc = {0u, 0u, 0u, 0u};
  if (nw == 0) {
    int64_t i = tid;
    for (; i + 3 * stride < nr; i += 4 * stride) {   // four loads in flight per lane
      const u32x4_p a = __builtin_nontemporal_load(&src[i]);
      const u32x4_p b = __builtin_nontemporal_load(&src[i + stride]);
      const u32x4_p c = __builtin_nontemporal_load(&src[i + 2 * stride]);
      const u32x4_p d = __builtin_nontemporal_load(&src[i + 3 * stride]);
      acc ^= a ^ b ^ c ^ d;
    }
    for (; i < nr; i += stride) acc ^= __builtin_nontemporal_load(&src[i]);
  } else if (nr == 0) {
    for (int64_t c = tid; c < nw; c += stride) {
      const uint32_t v = (uint32_t)c;
      const u32x4_p w = {v, v, v, v};
      dst[c] = w;
      acc ^= w;
    }
  } else {
    const int64_t R = nr / nw;
    for (int64_t c = tid; c < nw; c += stride) {
      u32x4_p v = {0u, 0u, 0u, 0u};
      for (int64_t k = 0; k < R; ++k) v ^= __builtin_nontemporal_load(&src[k * nw + c]);
      dst[c] = v;
      acc ^= v;
    }
  }
  out[tid] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

hipError_t launch_probe_stream(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes, int64_t blocks,
                               uint32_t* out, hipStream_t stream) {
  stream_probe_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
      static_cast<const u32x4_p*>(src), read_bytes / 16, static_cast<u32x4_p*>(dst), write_bytes / 16, out);
  return hipGetLastError();
}

hipError_t launch_probe_mfma(const void* src, int64_t blocks, int waves, int iters, float* out, hipStream_t stream) {
  if (waves == 8)
    mfma_probe_kernel<8, 2><<<dim3((unsigned)blocks), dim3(512), 0, stream>>>(static_cast<const uint4*>(src), iters,
                                                                              out);
  else
    mfma_probe_kernel<4, 4><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(static_cast<const uint4*>(src), iters,
                                                                              out);
  return hipGetLastError();
}

}  // namespace macaq

// Measurement aid: MFMA throughput from registers (declared in
// include/macaq_probe.h).  The GEMM kernels' roofline fraction is quoted
// against the 10.1 PFLOP/s datasheet figure; this kernel shows what the
// same block-scaled FP4 MFMA sustains on the chip with no memory traffic.
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

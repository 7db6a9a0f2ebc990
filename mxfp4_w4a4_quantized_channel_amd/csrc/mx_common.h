// Device building blocks shared by the quantizing kernels: bf16 widening,
// the 32-point Walsh-Hadamard butterfly laid out over a quad of lanes, the
// OCP MXFP4 group scale and the E2M1 encoder.  gfx950 only.
//
// Arithmetic contract (see include/macaq.h): per 32-element group along K,
// t = fp32(x) * s, butterfly stages h = 1, 2, 4, 8, 16 (lower a+b, upper
// a-b), x' = t * C, C = fp32 0x3E3504F3; scale byte from the exponent of
// max|x'| minus 2; E2M1 round-to-nearest-even with saturation.
//
// Lane layout: a group of 32 elements is held by 4 consecutive lanes (a
// "quad"), lane q of the quad holding elements 8q .. 8q+7.  Stages h = 1, 2,
// 4 pair registers of one lane; stages h = 8 and 16 pair lane q with lane
// q^1 and q^2, reached with DPP quad permutations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "macaq.h"

namespace macaq {

// Launcher override set by macaq_set_tuning (MACAQ_TUNE_*): 0 = automatic.
int tuning(int knob);

// 1/sqrt(32) rounded to fp32.
__device__ __forceinline__ float hadamard_norm() { return __uint_as_float(0x3E3504F3u); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Value of the lane q^1 (DPP quad_perm [1,0,3,2]) / q^2 ([2,3,0,1]).
__device__ __forceinline__ float quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}

// One in-register butterfly stage over 8 values: pairs (i, i+h) with (i&h)==0.
template <int H>
__device__ __forceinline__ void stage_local(float (&t)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if ((i & H) == 0) {
      const float a = t[i], b = t[i + H];
      t[i] = a + b;
      t[i + H] = a - b;
    }
  }
}

// Cross-lane stage: the lane whose quad bit is 0 holds the lower element a
// and gets a + b; the partner holds b and gets a - b.  Both are computed as
// partner + (+/- own): for the lower lane partner + own == own + partner, for
// the upper lane partner + (-own) == partner - own, bit for bit (IEEE
// subtraction is addition of the negation; addition commutes).
template <int QBIT>
__device__ __forceinline__ void stage_cross(float (&t)[8], uint32_t quad) {
  const uint32_t neg = ((quad >> QBIT) & 1u) << 31;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float own = t[i];
    const float partner = (QBIT == 0) ? quad_xor1(own) : quad_xor2(own);
    t[i] = partner + __uint_as_float(__float_as_uint(own) ^ neg);
  }
}

// Full 32-point butterfly + normalization of the quad's group; t in/out.
__device__ __forceinline__ void hadamard32_quad(float (&t)[8], uint32_t quad) {
  stage_local<1>(t);
  stage_local<2>(t);
  stage_local<4>(t);
  stage_cross<0>(t, quad);  // h = 8
  stage_cross<1>(t, quad);  // h = 16
  const float c = hadamard_norm();
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = t[i] * c;
}

// Group amax over the quad (every lane of the quad gets it).
__device__ __forceinline__ float quad_amax(const float (&t)[8]) {
  float m = fabsf(t[0]);
#pragma unroll
  for (int i = 1; i < 8; ++i) m = fmaxf(m, fabsf(t[i]));
  m = fmaxf(m, quad_xor1(m));
  m = fmaxf(m, quad_xor2(m));
  return m;
}

// E8M0 byte: exponent field of amax minus emax(E2M1) = 2, clamped at 0.
__device__ __forceinline__ uint32_t e8m0_from_amax(float amax) {
  const int ef = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  return (uint32_t)(ef > 2 ? ef - 2 : 0);
}

// 2^(127 - b) as fp32 (b <= 252, so the exponent field 254 - b is normal).
__device__ __forceinline__ float inv_scale(uint32_t b) { return __uint_as_float((254u - b) << 23); }

// Eight values already divided by the group scale -> eight E2M1 codes packed
// in one dword (element 2j in the low nibble of byte j).  The hardware
// conversion rounds to nearest even and saturates at 6; with scale 1.0 it
// applies no extra scaling.
__device__ __forceinline__ uint32_t e2m1_pack8(const float (&v)[8]) {
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[0], v[1], 1.0f, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[2], v[3], 1.0f, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[4], v[5], 1.0f, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[6], v[7], 1.0f, 3);
  return r;
}

// Quantize the quad's transformed group: returns 8 packed codes; *scale_out
// receives the group's E8M0 byte.
__device__ __forceinline__ uint32_t quantize_quad(float (&t)[8], uint32_t* scale_out) {
  const float amax = quad_amax(t);
  const uint32_t b = e8m0_from_amax(amax);
  const float m = inv_scale(b);
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = t[i] * m;  // exact: multiply by a power of two
  *scale_out = b;
  return e2m1_pack8(v);
}

// ---- direct global -> LDS copies and explicit wait counts
//
// global_load_lds_dword(x4): every lane copies 4 (16) bytes from its own
// global address to LDS at M0 + 4 (16) * lane.  The copies count in vmcnt
// like other vector loads and complete in issue order with them; the
// compiler does not see them, so code that overlaps them with compute waits
// for them explicitly with wait_vmcnt.  A compiler-visible vector load
// issued after such copies makes the compiler's own waits stricter (it does
// not count the copies), never weaker.

// The waitcnt and barrier builtins do not touch memory as far as the
// compiler's IR is concerned, so each is followed by an empty asm statement
// with a memory clobber: no load or store of LDS or global memory is moved
// across the wait (a read of a DMA-filled slot above the wait for its copy,
// or a copy into a slot above the wait for that slot's last reads).
template <int VM>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] at bits 3:0, vmcnt[5:4] at bits 15:14,
  // expcnt (7) and lgkmcnt (15) left at their maxima (no wait).
  __builtin_amdgcn_s_waitcnt((VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  asm volatile("" ::: "memory");
}

// Wait until every LDS (and scalar-memory) access of this wave completed;
// vmcnt and expcnt are left at their maxima.
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
  asm volatile("" ::: "memory");
}

// s_barrier with the same compiler ordering (no memory access moves across).
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void dma16(const uint8_t* g, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds_addr) : "memory");
}
// Non-temporal form, for bytes read exactly once (the streamed weights of
// the decode kernel, the activation rows): they do not evict lines that
// other blocks still read from L2.
__device__ __forceinline__ void dma16_nt(const uint8_t* g, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(g), "{m0}"(lds_addr) : "memory");
}
__device__ __forceinline__ void dma4(const uint8_t* g, uint32_t lds_addr) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(g), "{m0}"(lds_addr) : "memory");
}

// ---- GEMM output: fp32 or bf16, optionally SwiGLU over gate/up column pairs
//
// Output mode bits: kOutBf16 stores round-to-nearest-even bf16 instead of
// fp32; kOutSwiGLU stores, for each pair of accumulated columns (2j, 2j+1) =
// (gate, up), silu(gate) * up = gate / (1 + exp(-gate)) * up at column j of
// a [M][N/2] output.
constexpr int kOutBf16 = 1;
constexpr int kOutSwiGLU = 2;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);   // NaN stays NaN
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Two fp32 values rounded to the nearest bf16 (ties to even) and packed, lo in
// bits 0..15: one v_cvt_pk_bf16_f32.  For finite inputs this is bit-identical
// to f32_to_bf16_rne.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16_rne(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float silu_times(float g, float u) { return g / (1.0f + expf(-g)) * u; }

__device__ __forceinline__ void store_out(void* y, int64_t i, float v, int mode) {
  if (mode & kOutBf16) reinterpret_cast<uint16_t*>(y)[i] = f32_to_bf16_rne(v);
  else reinterpret_cast<float*>(y)[i] = v;
}

__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace macaq

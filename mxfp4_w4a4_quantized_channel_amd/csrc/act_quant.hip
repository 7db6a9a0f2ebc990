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
// One lane owns one 32-value group: a wave covers 64 groups at a time, a
// segment of 64, 32 or 16 groups in each of 1, 2 or 4 consecutive rows (see
// act_quant_lane_kernel below).  The kernel is HBM-bound: per element it
// reads 2 bytes (bf16) and writes 17/32 bytes.
#include "mx_common.h"

namespace macaq {

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

// ---------------------------------------------------------------------------
// One-lane-per-group kernel.  A wave's 64 groups are copied straight from
// global memory into a wave-private LDS ring (global_load_lds_dwordx4,
// coalesced: each copy instruction moves 1 KiB of consecutive bytes), and
// each lane then reads its own group from there.  Within a group the 16-byte
// chunks are XOR-swizzled so that the lanes' per-group reads hit every LDS
// bank once per phase.  All five butterfly stages run in the lane's
// registers.  The ring holds up to kDepth row blocks, so that many are in
// flight while one is transformed, without holding registers for them.
//
// Normalization folded into the quantization multiply: amax(x') equals
// RNE(max|u| * C) because rounding is monotone, and for scale bytes 3..250
// RNE(u * C * 2^(127-b)) equals RNE(u * C) * 2^(127-b) for every value that
// can reach a nonzero code (C * 2^(127-b) is an exact normal float; values
// whose x' would be subnormal land below 0.25 either way and keep their
// sign).  Lanes with other scale bytes take the two-multiply path.
template <int EB>  // bytes per input element (2 = bf16, 4 = fp32)
struct GroupIo {
  static constexpr int kGroupBytes = 32 * EB;
  static constexpr int kChunks = 2 * EB;                     // 16-byte chunks per group
  static constexpr int kBlockLds = 64 * kGroupBytes;         // one row block of a wave (4 or 8 KiB)
  static constexpr int kLoads = kBlockLds / 1024;            // 16-byte copies per lane per row block
  // LDS slot (16-byte unit) of chunk c of group g: chunk positions are
  // XOR-swizzled by the group's index within its 128-byte bank line, so
  // the 8 lanes of a read phase (8 consecutive groups, same c) cover 8
  // distinct 16-byte bank groups.  The XOR is its own inverse: position p
  // of group g holds chunk p ^ swz(g).
  static __device__ __forceinline__ int swz(int g) { return (g / (8 / kChunks)) & (kChunks - 1); }
  static __device__ __forceinline__ int slot(int g, int c) { return g * kChunks + (c ^ swz(g)); }
};

// Row blocks in flight per wave, and the block's LDS: each wave's ring, plus
// (SHARED) two staged slices of s, within the 64 KiB a block may take
// without an attribute: 48 KiB (bf16) or 64 KiB (fp32); with the staged
// factors one row block (measured on attn-proj: 7.2 us, against 8.4 with
// two, which allow fewer blocks per CU), 34 or 50 KiB.
template <int EB, bool SHARED>
constexpr int act_depth() { return SHARED ? 1 : (EB == 2 ? 3 : 2); }

template <int EB>
__device__ __forceinline__ void widen_group(const uint4 (&q)[EB * 2], float (&t)[32]) {
  if constexpr (EB == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      t[8 * i + 0] = bf16_lo(q[i].x); t[8 * i + 1] = bf16_hi(q[i].x);
      t[8 * i + 2] = bf16_lo(q[i].y); t[8 * i + 3] = bf16_hi(q[i].y);
      t[8 * i + 4] = bf16_lo(q[i].z); t[8 * i + 5] = bf16_hi(q[i].z);
      t[8 * i + 6] = bf16_lo(q[i].w); t[8 * i + 7] = bf16_hi(q[i].w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      t[4 * i + 0] = __uint_as_float(q[i].x); t[4 * i + 1] = __uint_as_float(q[i].y);
      t[4 * i + 2] = __uint_as_float(q[i].z); t[4 * i + 3] = __uint_as_float(q[i].w);
    }
  }
}

// Unnormalized butterfly, stages h = 1, 2, 4, 8, 16 (lower a+b, upper a-b).
__device__ __forceinline__ void fwht32_regs(float (&t)[32]) {
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
}

// Quantize the lane's group u (unnormalized butterfly output): 16 code bytes
// and the E8M0 byte.
__device__ __forceinline__ void quantize_group(const float (&u)[32], uint4* codes_out, uint32_t* b_out) {
  float m = fabsf(u[0]);
#pragma unroll
  for (int i = 1; i < 32; ++i) m = fmaxf(m, fabsf(u[i]));
  const float c = hadamard_norm();
  const uint32_t b = e8m0_from_amax(m * c);  // = amax of x' (monotone rounding)
  float v[32];
  if (b >= 3u && b <= 250u) {
    const float cs = __uint_as_float(__float_as_uint(c) + ((127u - b) << 23));  // C * 2^(127-b), exact
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = u[i] * cs;
  } else {
    const float inv = inv_scale(b);
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = (u[i] * c) * inv;
  }
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * q + 0], v[8 * q + 1], 1.0f, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * q + 2], v[8 * q + 3], 1.0f, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * q + 4], v[8 * q + 5], 1.0f, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * q + 6], v[8 * q + 7], 1.0f, 3);
    w[q] = r;
  }
  *codes_out = make_uint4(w[0], w[1], w[2], w[3]);
  *b_out = b;
}

// Plain OCP MXFP4 quantization of a group (no scale, no transform): the
// E8M0 byte comes from max|x| and the codes from x * 2^(127-b).
__device__ __forceinline__ void quantize_group_plain(const float (&u)[32], uint4* codes_out, uint32_t* b_out) {
  float m = fabsf(u[0]);
#pragma unroll
  for (int i = 1; i < 32; ++i) m = fmaxf(m, fabsf(u[i]));
  const uint32_t b = e8m0_from_amax(m);
  const float inv = inv_scale(b);
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = u[i] * inv;
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * q + 0], v[8 * q + 1], 1.0f, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * q + 2], v[8 * q + 3], 1.0f, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * q + 4], v[8 * q + 5], 1.0f, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * q + 6], v[8 * q + 7], 1.0f, 3);
    w[q] = r;
  }
  *codes_out = make_uint4(w[0], w[1], w[2], w[3]);
  *b_out = b;
}

// One wave processes a segment of GS consecutive groups (GS * 32 columns; GS
// = 64, 32 or 16, chosen so that the segments tile a row with the fewest idle
// lanes) of 64 / GS consecutive rows at a time, for `steps` such row blocks;
// lane l owns group (l % GS) of the segment in row l / GS of the row block.
// A row block's segments are loaded with coalesced 16-byte loads (load i
// covers bytes 1024 i + 16 l of the concatenated segments; a segment is at
// least 1 KiB, so no load straddles two rows).
//
// Two ways to lay the waves out and to get each lane's 32 factors of s:
// * per wave (SHARED false): consecutive waves take consecutive segments of
//   the same rows; a lane loads its group's factors once into registers
//   (128 bytes per lane, a different cache line for every lane) and reloads
//   them only when its row's expert changes.
// * per block (SHARED true, for waves of at most 2 row blocks, where that
//   load is a large share of a wave's work): a block's 4 waves take 4
//   consecutive row ranges of one segment, and the segment's slice of s
//   (GS x 32 factors, or their reciprocals when RECIP) is staged once per
//   block in LDS with coalesced loads, for the experts of the block's first
//   and last rows; each lane reads its factors from there every row block
//   (rows of a third expert read theirs from s).
//
// PLAIN: quantize the rows as they are (s = 1, H = I), the "pure MXFP4"
// baseline against which the online transform's cost is measured.
constexpr int kSStride = 36;                      // floats per staged group (144 B: conflict-free reads)
constexpr int kSLds = 64 * kSStride * 4;          // one staged slice of s, bytes
template <int EB, bool SHARED>
constexpr int act_lds_bytes() { return (SHARED ? 2 * kSLds : 0) + 4 * act_depth<EB, SHARED>() * GroupIo<EB>::kBlockLds; }

// Wait until at most `later` row blocks' copies of this wave are in flight.
template <int LOADS>
__device__ __forceinline__ void wait_row_blocks(int later) {
  if (later >= 2) wait_vmcnt<2 * LOADS>();
  else if (later == 1) wait_vmcnt<LOADS>();
  else wait_vmcnt<0>();
}

// TILED: codes and scales in the tiled layout the prefill GEMM copies with
// contiguous 1 KiB reads (macaq_tile_weights' layout, applied to the
// activation rows): per 32-row block and 128-wide K-tile, 2 KiB of codes
// (row r at 64 r, group chunk c at position c ^ ((r >> 2) & 3)) and 128
// bytes of scales (row r's 4 bytes at 4 r).  K % 128 == 0.
template <int EB, bool RECIP, bool PLAIN = false, bool SHARED = false, bool TILED = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(SHARED && EB == 2 && !RECIP ? 4 : (EB == 2 ? 3 : 2))))
void act_quant_lane_kernel(
    const void* __restrict__ x, const float* __restrict__ s, const int32_t* __restrict__ offsets, int E,
    int64_t rows_per_expert, int64_t M, int64_t K, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    int gs_log2, int steps) {
  static_assert(!(PLAIN && SHARED), "the plain quantizer has no factors to share");
  using IO = GroupIo<EB>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave_in_block = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (SGPR)
  const int64_t KG = K >> 5;
  const int gs = 1 << gs_log2;
  const int rw = 64 >> gs_log2;                      // rows per block step
  const int64_t nseg = ceil_div(KG, gs);
  const int64_t rows_per_wave = (int64_t)steps * rw;
  int64_t seg, rb, r0;
  if constexpr (SHARED) {
    seg = (int64_t)blockIdx.x % nseg;
    rb = ((int64_t)blockIdx.x / nseg) * 4 * rows_per_wave;   // the block's first row
    r0 = rb + wave_in_block * rows_per_wave;
  } else {
    const int64_t wave = (int64_t)blockIdx.x * 4 + wave_in_block;
    seg = wave % nseg;
    rb = r0 = (wave / nseg) * rows_per_wave;
    if (r0 >= M) return;
  }
  const int64_t r1 = (r0 + rows_per_wave) < M ? (r0 + rows_per_wave) : M;
  const int lr = lane >> gs_log2;                    // this lane's row within a block step
  const int lg = lane & (gs - 1);                    // this lane's group within the segment
  const int64_t g = seg * gs + lg;                   // this lane's group
  const bool g_ok = g < KG;
  const int seg_log2 = gs_log2 + 5 + (EB == 4 ? 2 : 1);   // log2 bytes of one row's segment
  const int64_t seg_groups = (KG - seg * gs < gs ? KG - seg * gs : gs);
  const int64_t seg_valid = seg_groups * IO::kGroupBytes;
  constexpr int kDepth = act_depth<EB, SHARED>();
  const uint32_t ring_off = (SHARED ? 2 * kSLds : 0) + (uint32_t)wave_in_block * kDepth * IO::kBlockLds;
  const uint32_t ring_lds = (uint32_t)(uintptr_t)lds + ring_off;
  const float* s_lds = reinterpret_cast<const float*>(lds);

  // expert of a row (rows sorted by expert)
  auto expert_of = [&](int64_t row) {
    if (rows_per_expert > 0) return (int)(row / rows_per_expert);
    if (offsets == nullptr) return 0;
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)offsets[mid + 1] > row) hi = mid; else lo = mid + 1;
    }
    return lo;
  };

  // Copy i of a row block: lane L fills slot 64 i + L, which is position
  // L % kChunks of concatenated group gp = (64 i + L) / kChunks and holds
  // that group's chunk position ^ swz(gp).  Concatenated group gp is group
  // gp % gs of the segment in row gp / gs of the block: the group of lane gp.
  int64_t src_off[IO::kLoads];
  int src_row[IO::kLoads];
#pragma unroll
  for (int i = 0; i < IO::kLoads; ++i) {
    const int p = 64 * i + lane, gp = p / IO::kChunks, c = (p % IO::kChunks) ^ IO::swz(gp);
    const int bpos = gp * IO::kGroupBytes + 16 * c;
    const int row_l = bpos >> seg_log2, o = bpos & ((1 << seg_log2) - 1);
    src_row[i] = o < seg_valid ? row_l : 64;      // 64: past every row block
    src_off[i] = (int64_t)row_l * K * EB + o;
  }
  auto issue_copies = [&](int64_t ra, int slot) {
    const uint8_t* base = reinterpret_cast<const uint8_t*>(x) + (ra * K + seg * gs * 32) * EB;
    const int64_t rows_left = r1 - ra;
#pragma unroll
    for (int i = 0; i < IO::kLoads; ++i) {
      // a chunk past the wave's rows or the row's last group belongs to a
      // lane that stores nothing: copy the block's first chunk in its place
      const uint8_t* src = src_row[i] < rows_left ? base + src_off[i] : base;
      dma16_nt(src, ring_lds + (uint32_t)(slot * IO::kBlockLds + 1024 * i));
    }
  };

  // experts: of this lane's first row, and (SHARED) of the block's first and
  // last rows; looked up before any x load, which the lookups would otherwise
  // wait for.  e_end is the end of the lane's expert (rows sorted by expert):
  // the expert walk in the loop loads an offset only when a row crosses it.
  int e = 0, e_a = 0, e_b = 0;
  int64_t e_end = 0;
  // TILED with experts: the lane's expert's first row (e_beg) and first
  // padded row (e_pad): expert e's rows start at padded row sum over
  // e' < e of ceil(rows_e' / 32) * 32, so that every expert starts a block
  int64_t e_beg = 0, e_pad = 0;
  // offsets[e_tbl + l] in lane l (the wave's first expert e_tbl and the 63
  // after it), so that walking over experts, runs of empty ones included,
  // reads a register of another lane instead of global memory (a load there
  // would wait for every copy in flight)
  int e_tbl = 0;
  int32_t tbl = 0;
  // advance every lane whose row r lies past its expert's end; the loop is
  // wave-uniform so that the lane shuffle sees every lane's table entry
  auto walk_experts = [&](int64_t r) {
    for (;;) {
      const bool adv = e + 1 < E && r >= e_end;
      if (!__any(adv)) break;
      const int k = e + 2 - e_tbl;                       // table index of the next expert's end
      const int32_t next_end = __shfl(tbl, k < 64 ? k : 0, 64);
      if (adv) {
        if constexpr (TILED) {
          e_pad += (e_end - e_beg + 31) / 32 * 32;
          e_beg = e_end;
        }
        ++e;
        e_end = k < 64 ? next_end : offsets[e + 1];
      }
    }
  };
  if constexpr (!PLAIN) {
    const int64_t rl = r0 + lr < M ? r0 + lr : M - 1;   // this lane's first row
    if (rows_per_expert > 0) {
      e = (int)(rl / rows_per_expert);
    } else if (offsets != nullptr) {
      // the wave's first row is wave-uniform: a binary search on scalar
      // loads; a lane whose first row lies past that expert walks on
      e = expert_of(r0 < M ? r0 : M - 1);
      e_end = offsets[e + 1];
      e_tbl = e;
      tbl = e_tbl + lane <= E ? offsets[e_tbl + lane] : 0;
      if constexpr (TILED) {
        e_beg = offsets[e];
        // padded rows of the experts before e, summed over the wave's lanes
        int64_t p = 0;
        for (int e0 = 0; e0 < e; e0 += 64) {
          const int ei = e0 + lane;
          if (ei < e) p += ((int64_t)offsets[ei + 1] - offsets[ei] + 31) / 32 * 32;
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) p += __shfl_xor(p, d, 64);
        e_pad = p;
      }
      walk_experts(rl);
    }
    if constexpr (SHARED) {
      const int64_t r_last = (rb + 4 * rows_per_wave < M ? rb + 4 * rows_per_wave : M) - 1;   // block's last row
      e_a = expert_of(rb < M ? rb : M - 1);
      e_b = expert_of(r_last);
    }
  }
  // per-wave layout: the lane's factors are loaded before the first copies
  // and waited for together with them
  int cur_e = -1;
  float sc[32];
  if constexpr (!PLAIN && !SHARED) {
    if (g_ok && r0 + lr < r1) {
      cur_e = e;
      const float4* sp = reinterpret_cast<const float4*>(s + (int64_t)e * K + g * 32);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 f = sp[i];
        sc[4 * i] = f.x; sc[4 * i + 1] = f.y; sc[4 * i + 2] = f.z; sc[4 * i + 3] = f.w;
      }
    }
  }
  const int nblk = r0 < M ? (int)ceil_div(r1 - r0, (int64_t)rw) : 0;   // row blocks of this wave
  for (int j = 0; j < kDepth && j < nblk; ++j) issue_copies(r0 + (int64_t)j * rw, j);
  if constexpr (!PLAIN && !SHARED) {
    wait_vmcnt<0>();
#pragma unroll
    for (int i = 0; i < 32; ++i) asm volatile("" : "+v"(sc[i]));   // no use of sc moves above the wait
    if (RECIP && cur_e >= 0) {
#pragma unroll
      for (int i = 0; i < 32; ++i) sc[i] = 1.0f / sc[i];  // IEEE-correct fp32 division
    }
  }
  if constexpr (SHARED) {
    // stage the segment's factors of experts e_a and e_b (when it differs)
    // while x is in flight: thread t copies bytes 16 t + 4096 p of a slice
    const int nslice = e_b != e_a ? 2 : 1;
    for (int sl = 0; sl < nslice; ++sl) {
      const uint8_t* src = reinterpret_cast<const uint8_t*>(s + (int64_t)(sl == 0 ? e_a : e_b) * K + seg * gs * 32);
      for (int64_t byte = 16 * (int64_t)threadIdx.x; byte < (int64_t)gs * 128; byte += 4096) {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (byte < seg_groups * 128) {
          v = *reinterpret_cast<const float4*>(src + byte);
          if (RECIP) {   // IEEE-correct fp32 division
            v.x = 1.0f / v.x; v.y = 1.0f / v.y; v.z = 1.0f / v.z; v.w = 1.0f / v.w;
          }
        }
        const int grp = (int)(byte >> 7), part = (int)(byte & 127);
        *reinterpret_cast<float4*>(lds + sl * kSLds + grp * (kSStride * 4) + part) = v;
      }
    }
    __syncthreads();
    if (r0 >= M) return;
  }

  for (int j = 0; j < nblk; ++j) {
    const int64_t ra = r0 + (int64_t)j * rw;
    const int slot = j % kDepth;
    wait_row_blocks<IO::kLoads>(kDepth - 1 < nblk - 1 - j ? kDepth - 1 : nblk - 1 - j);
    uint4 q[EB * 2];
#pragma unroll
    for (int c = 0; c < EB * 2; ++c)
      q[c] = *reinterpret_cast<const uint4*>(lds + ring_off + slot * IO::kBlockLds + 16 * IO::slot(lane, c));
    if (j + kDepth < nblk) {
      wait_lgkmcnt0();   // the slot's reads have landed before it is refilled
      issue_copies(ra + (int64_t)kDepth * rw, slot);
    }
    const int64_t r = ra + lr;                       // this lane's row
    const bool active = g_ok && r < r1;
    if constexpr (!PLAIN) {
      // expert of row r
      if (rows_per_expert > 0) e = (int)(r / rows_per_expert);
      else if (offsets != nullptr)
        walk_experts(r);
    }
    if constexpr (!PLAIN && !SHARED) {
      // this lane's factors, reloaded when its row's expert changes
      if (active && e != cur_e) {
        cur_e = e;
        const float4* sp = reinterpret_cast<const float4*>(s + (int64_t)e * K + g * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float4 q = sp[i];
          sc[4 * i] = q.x; sc[4 * i + 1] = q.y; sc[4 * i + 2] = q.z; sc[4 * i + 3] = q.w;
        }
        if (RECIP) {
#pragma unroll
          for (int i = 0; i < 32; ++i) sc[i] = 1.0f / sc[i];  // IEEE-correct fp32 division
        }
        // wait here, on the rare reload: left to the compiler, the wait for
        // these loads lands after the branch, where it would run on every row
        // block and drain the ring's copies each time
        wait_vmcnt<0>();
      }
    }
    float t[32];
    widen_group<EB>(q, t);
    uint4 cw;
    uint32_t b;
    if constexpr (PLAIN) {
      quantize_group_plain(t, &cw, &b);
    } else {
      if constexpr (SHARED) {
        if (e == e_a || e == e_b) {
          const float* sl = s_lds + (e == e_a ? 0 : kSLds / 4) + lg * kSStride;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float4 f = *reinterpret_cast<const float4*>(sl + 4 * i);
            t[4 * i] *= f.x; t[4 * i + 1] *= f.y; t[4 * i + 2] *= f.z; t[4 * i + 3] *= f.w;
          }
        } else if (active) {
          const float4* sp = reinterpret_cast<const float4*>(s + (int64_t)e * K + g * 32);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            float4 f = sp[i];
            if (RECIP) {
              f.x = 1.0f / f.x; f.y = 1.0f / f.y; f.z = 1.0f / f.z; f.w = 1.0f / f.w;
            }
            t[4 * i] *= f.x; t[4 * i + 1] *= f.y; t[4 * i + 2] *= f.z; t[4 * i + 3] *= f.w;
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) t[i] = t[i] * sc[i];
      }
      fwht32_regs(t);
      quantize_group(t, &cw, &b);
    }
    if (active) {
      if constexpr (TILED) {
        const int64_t pr = offsets != nullptr ? e_pad + (r - e_beg) : r;   // (padded) row
        const int64_t blk = (pr >> 5) * (K >> 7) + (g >> 2);
        const int rr = (int)(pr & 31), c = (int)(g & 3);
        *reinterpret_cast<uint4*>(codes + blk * 2048 + rr * 64 + ((c ^ ((rr >> 2) & 3)) << 4)) = cw;
        scales[blk * 128 + rr * 4 + c] = (uint8_t)b;
      } else {
        *reinterpret_cast<uint4*>(codes + r * (K >> 1) + g * 16) = cw;
        scales[r * KG + g] = (uint8_t)b;
      }
    }
  }
}

// ---------------------------------------------------------------- launchers

// Segment width (log2 of 64, 32 or 16 groups) that leaves the fewest idle
// lanes on a row of KG groups; ties go to the wider segment.
static int act_gs_log2(int64_t KG) {
  int best = 6;
  int64_t best_idle = ceil_div(KG, 64) * 64 - KG;
  for (int l = 5; l >= 4; --l) {
    const int64_t idle = ceil_div(KG, (int64_t)1 << l) * ((int64_t)1 << l) - KG;
    if (idle < best_idle) {
      best = l;
      best_idle = idle;
    }
  }
  return best;
}

struct ActLaunch {
  int gs_log2, steps;
  bool shared;
  dim3 grid;
};

// Row blocks per wave: units / 3072 rounded up, so that the grid is about
// one round of 3 blocks on each of the 256 CUs, clamped to 2..12, or 1 for
// grids of at most 4096 units (measured on MI355X with the copy ring:
// down-prefill 10 row blocks 32.0 us against 33.3 at 6 and 35.2 at 12; MoE
// 4 row blocks 19.0 us against 21.3 at 2 and 8; decode M32 1 row block
// 4.1 us against 5.2 at 2; attn-proj M2048 K4096 with tiled output, 4096
// units, 1 row block 6.4 us against 7.1 at 2).  Waves of at most 2 row blocks share s per block
// (measured: attn-proj activation 9.7 -> 8.5 us before the copy ring,
// 7.2 us with it); longer waves keep the per-wave layout, which reads x
// with better locality (down-prefill 37.9 vs 39.3 us, MoE per-token routing
// 19.8 vs 22.6 us).
static ActLaunch act_launch(int64_t M, int64_t K, bool plain, bool tiled = false) {
  ActLaunch a;
  a.gs_log2 = act_gs_log2(K / 32);
  // tiled output: four rows per step (16-group segments) where that tiles a
  // row as well as 32, so that a store instruction writes whole 128-byte
  // lines (rows r and r+1 of a 128-wide K-tile are adjacent 64-byte halves
  // of one line); measured on down-prefill M4096 K14336: 30.3 us against
  // 31.0 (32 groups) and 33.6 (64 groups)
  if (tiled && a.gs_log2 > 4) {
    const int64_t KG = K / 32;
    a.gs_log2 = (ceil_div(KG, 16) * 16 - KG <= ceil_div(KG, 32) * 32 - KG) ? 4 : 5;
  }
  if (const int force = tuning(MACAQ_TUNE_ACT_SEGMENT)) a.gs_log2 = force >= 64 ? 6 : (force >= 32 ? 5 : 4);
  const int64_t rw = 64 >> a.gs_log2;
  const int64_t nseg = ceil_div(K / 32, (int64_t)1 << a.gs_log2);
  const int64_t blocks = ceil_div(M, rw);
  const int64_t units = nseg * blocks;
  int64_t steps = ceil_div(units, (int64_t)3072);
  if (steps < 2) steps = 2;
  if (units <= 4096) steps = 1;
  if (steps > 12) steps = 12;
  if (steps > blocks) steps = blocks;
  if (const int force = tuning(MACAQ_TUNE_ACT_ROWS_PER_WAVE)) steps = force;
  a.steps = (int)steps;
  a.shared = !plain && steps <= 2;
  if (const int force = tuning(MACAQ_TUNE_ACT_SHARED_S)) a.shared = !plain && force == 2;
  const int64_t chunks = ceil_div(blocks, steps);   // row ranges of one wave
  a.grid = a.shared ? dim3((unsigned)(nseg * ceil_div(chunks, 4))) : dim3((unsigned)ceil_div(nseg * chunks, 4));
  return a;
}

template <int EB, bool RECIP, bool TILED = false>
static void launch_act_t(const ActLaunch& a, const void* x, const float* s, const int32_t* offsets, int E,
                         int64_t rows_per_expert, int64_t M, int64_t K, uint8_t* codes, uint8_t* scales,
                         hipStream_t stream) {
  if (a.shared)
    act_quant_lane_kernel<EB, RECIP, false, true, TILED><<<a.grid, dim3(256), act_lds_bytes<EB, true>(),
                                                           stream>>>(x, s, offsets, E, rows_per_expert, M, K, codes,
                                                                     scales, a.gs_log2, a.steps);
  else
    act_quant_lane_kernel<EB, RECIP, false, false, TILED><<<a.grid, dim3(256), act_lds_bytes<EB, false>(), stream>>>(
        x, s, offsets, E, rows_per_expert, M, K, codes, scales, a.gs_log2, a.steps);
}

hipError_t launch_act_quant(const void* x, bool x_f32, bool reciprocal, const float* s,
                            const int32_t* offsets, int E, int64_t rows_per_expert, int64_t M,
                            int64_t K, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  const ActLaunch a = act_launch(M, K, false);
  if (x_f32) {
    if (reciprocal) launch_act_t<4, true>(a, x, s, offsets, E, rows_per_expert, M, K, codes, scales, stream);
    else launch_act_t<4, false>(a, x, s, offsets, E, rows_per_expert, M, K, codes, scales, stream);
  } else {
    if (reciprocal) launch_act_t<2, true>(a, x, s, offsets, E, rows_per_expert, M, K, codes, scales, stream);
    else launch_act_t<2, false>(a, x, s, offsets, E, rows_per_expert, M, K, codes, scales, stream);
  }
  return hipGetLastError();
}

// The online transform with its output in the tiled layout of the prefill
// and grouped GEMMs (K % 128 == 0).  Dense: ceil(M / 32) * 32 rows; grouped
// (offsets != nullptr): expert e's rows start at padded row sum over e' < e
// of ceil(rows_e' / 32) * 32.  Padding rows are not written.
hipError_t launch_act_quant_tiled(const void* x, bool x_f32, const float* s, const int32_t* offsets, int E, int64_t M,
                                  int64_t K, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  const ActLaunch a = act_launch(M, K, false, true);
  if (x_f32) launch_act_t<4, false, true>(a, x, s, offsets, E, 0, M, K, codes, scales, stream);
  else launch_act_t<2, false, true>(a, x, s, offsets, E, 0, M, K, codes, scales, stream);
  return hipGetLastError();
}

hipError_t launch_quant_plain(const void* x, bool x_f32, int64_t M, int64_t K, uint8_t* codes, uint8_t* scales,
                              hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  const ActLaunch a = act_launch(M, K, true);
  if (x_f32)
    act_quant_lane_kernel<4, false, true><<<a.grid, dim3(256), act_lds_bytes<4, false>(), stream>>>(
        x, nullptr, nullptr, 1, 0, M, K, codes, scales, a.gs_log2, a.steps);
  else
    act_quant_lane_kernel<2, false, true><<<a.grid, dim3(256), act_lds_bytes<2, false>(), stream>>>(
        x, nullptr, nullptr, 1, 0, M, K, codes, scales, a.gs_log2, a.steps);
  return hipGetLastError();
}

hipError_t launch_encode_e2m1(const float* v, int64_t n, uint8_t* codes, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t threads = ceil_div(n, 8);
  encode_e2m1_kernel<<<dim3((unsigned)ceil_div(threads, 256)), dim3(256), 0, stream>>>(v, n, codes);
  return hipGetLastError();
}

}  // namespace macaq

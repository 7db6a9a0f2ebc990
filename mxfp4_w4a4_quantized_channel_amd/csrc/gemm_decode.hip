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
// K permutation (the same on both operands): in a 256-wide K chunk, lane
// half h of sub-step j takes group 2j + h.  A lane's four scale bytes
// (groups h, 2+h, 4+h, 6+h) are gathered with one byte permute so that
// op_sel byte j is sub-step j's scale.
//
// Memory path: a block owns 32 weight rows and the whole K range, which its
// waves split into contiguous chunk ranges.  Each wave copies its chunks
// from global memory straight into a private, double-buffered LDS stage with
// global_load_lds: one dwordx4 copy instruction reads 8 whole 128-byte rows
// of a chunk (whole cache lines; reading the MFMA's own lane layout from
// global memory instead touches 32 lines per instruction and streams about a
// third slower).  Slots are XOR-swizzled by row so the MFMA-layout reads
// from LDS spread over the banks.  The copy of chunk c + 1 is in flight
// while chunk c is multiplied.  In the unfused path the activation codes
// and scales of the chunk travel the same way, so that the loop holds no
// compiler-visible global load (whose compiler-inserted wait would also
// wait for the next chunk's copy).
//
// The waves' 32x32 partial sums are added in LDS in wave order
// (deterministic).  No cross-block reduction is needed, so the path needs no
// workspace.
//
// Fused variant: before the GEMM the block transforms and quantizes x[0:M,
// :] (the quad-per-group routine of the activation kernel) into LDS while the
// first weight chunk is in flight; the B fragments then come from LDS.
// Every block repeats that transform, so the fused variant pays off only for
// very small M.
#include <cstdlib>

#include "mx_common.h"

namespace macaq {

// W' is read exactly once per call: its copies carry the non-temporal hint
// (dma16_nt) so that the streamed weights do not evict the activation and
// scale lines the other blocks still read from L2.


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

template <typename XT>
constexpr int dec_eb = 2;          // bytes per activation element
template <>
constexpr int dec_eb<float> = 4;

// LDS row strides of the fused activation copy (padded against bank conflicts)
__host__ __device__ constexpr int64_t dec_xrow_bytes(int64_t K) { return K / 2 + 16; }
__host__ __device__ constexpr int64_t dec_xrow_groups(int64_t K) { return K / 32 + 8; }

// Layout of one staged 256-wide K chunk in a wave's LDS ring slot: W' codes
// of the block's 32 rows (4 x 1 KiB, row r at (r / 8) KiB + (r % 8) * 128
// with 16-byte slot p holding piece p ^ (r % 8)), then the activation's part
// of the chunk.  Activation kinds AK:
//   -1     streamed fused transform, M <= 2: the chunk's 256 values of s
//          (1 KiB, one dwordx4 instruction) and of x rows 0..1 (2 x 256 x EB
//          bytes, EB / 2 dwordx4 instructions); the wave transforms and
//          quantizes them after the chunk lands;
//   0      resident: the whole activation sits in LDS (fused transform by the
//          block before the loop);
//   1      M <= 2: codes of rows 0..1 (2 x 128 B, plain layout) copied by one
//          dword instruction;
//   8,16,32  M <= AK: codes of AK rows in the swizzled layout (AK / 8
//          dwordx4 instructions);
// and for AK > 0 the activation scales (32 rows x 8 bytes, one dword
// instruction; rows past M repeat row M - 1).
//
// W' scales do not travel per chunk (32 rows x 8 bytes would touch 32 cache
// lines per instruction, and with long rows those lines leave L1 before
// their next use).  They are staged per segment of SEG chunks into a slab of
// 32 rows x 8 SEG bytes, one dword copy instruction (64 / (2 SEG) rows x 8 SEG
// bytes) riding along with each chunk's copies and filling the slab of the
// next segment.  Three slabs rotate: the slab being filled was last read two
// segments ago.  SEG = 8, or 4 where 32 staged activation rows leave less
// LDS.
constexpr int kSlabs = 3;

template <int AK, int EB = 2, int RT = 1>
struct DecStage {
  static constexpr int kW = 0;                     // RT x 4 KiB of W' codes (RT 32-row tiles)
  static constexpr int kA = 4096 * RT;             // streamed: s chunk; else activation codes
  static constexpr int kX = kA + 1024;             // streamed: x chunk of rows 0..1
  static constexpr int kABytes = AK < 0 ? 1024 + 512 * EB : (AK == 0 ? 0 : (AK == 1 ? 256 : AK * 128));
  static constexpr int kAs = kA + kABytes;
  static constexpr int kBytes = kAs + (AK > 0 ? 256 : 0);
  static constexpr int kACopies = AK < 0 ? 1 + EB / 2 : (AK == 0 ? 0 : (AK == 1 ? 2 : AK / 8 + 1));
  // copy instructions per chunk: 4 RT codes, RT slab copies, the activation's
  static constexpr int kCopies = 5 * RT + kACopies;
};

// Per wave: STAGES ring slots, the scale slabs, and (streamed) the wave's
// quantized activation chunk: codes of rows 0..1 (2 x 128 B) and their 2 x 8
// scale bytes.
template <int STAGES, int AK, int EB = 2, int RT = 1>
struct DecWaveLds {
  static constexpr int kSeg = AK == 32 ? 4 : 8;          // chunks per scale segment
  static constexpr int kRowDwords = 2 * kSeg;            // slab row: 8 kSeg bytes
  static constexpr int kSlabBytes = 32 * RT * 8 * kSeg;
  static constexpr int kSlab0 = STAGES * DecStage<AK, EB, RT>::kBytes;
  static constexpr int kXq = kSlab0 + kSlabs * kSlabBytes;
  static constexpr int kXqBytes = AK < 0 ? 288 : 0;
  static constexpr int kBytes = kXq + kXqBytes;
};

__device__ __forceinline__ int dec_slot(int row, int piece) { return (row >> 3) * 1024 + (row & 7) * 128 + 16 * (piece ^ (row & 7)); }

// A block owns RT x 32 weight rows (RT MFMA row tiles sharing each
// activation chunk).
template <int WAVES, int STAGES, int AK, typename XT, int RT = 1>
__global__ __launch_bounds__(64 * WAVES) void decode_gemm_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As,     // activation codes/scales (unfused)
    const void* __restrict__ x, const float* __restrict__ s,           // activations and scale (fused)
    const uint8_t* __restrict__ W, const uint8_t* __restrict__ Ws, int64_t M, int64_t N, int64_t K,
    void* __restrict__ Y, int out_mode) {
  constexpr int EB = dec_eb<XT>;
  using S = DecStage<AK, EB, RT>;
  constexpr bool FUSED = AK == 0;     // resident activation, transformed before the loop
  constexpr bool STREAM = AK < 0;     // activation transformed chunk by chunk in the loop
  constexpr int AI = AK >= 8 ? AK / 8 : 1;
  extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
  constexpr int kThreads = 64 * WAVES;
  const int64_t n0 = (int64_t)blockIdx.x * kDecRows * RT;
  const int64_t KB = K >> 1, KG = K >> 5;
  const int kc = (int)(K >> 8);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31;
  const int h = lane >> 5;

  using WL = DecWaveLds<STAGES, AK, EB, RT>;
  // LDS: per wave STAGES ring slots and kSlabs scale slabs (all reused for
  // the [WAVES][32 RT][32] fp32 partial sums after the loop), then (fused)
  // the activation codes [M][K/2 + 16] and scales [M][K/32 + 8].
  uint8_t* ring = dsm + wave * WL::kBytes;
  const uint32_t ring_addr = (uint32_t)(uintptr_t)ring;
  const uint8_t* slabs = ring + WL::kSlab0;
  uint8_t* xq = ring + WL::kXq;   // streamed: this chunk's quantized activation
  float* red = reinterpret_cast<float*>(dsm);
  const int64_t xrb = dec_xrow_bytes(K), xrg = dec_xrow_groups(K);
  uint8_t* xcodes = dsm + WAVES * WL::kBytes;
  uint8_t* xscales = xcodes + M * xrb;

  // ---- this wave's chunks and the copy sources of chunk 0 (rows past N or
  // M repeat the last row; their results are not stored)
  const int per_wave = (kc + WAVES - 1) / WAVES;
  const int c0 = wave * per_wave;
  const int c1 = (c0 + per_wave) < kc ? (c0 + per_wave) : kc;
  const uint8_t* wsrc[4 * RT];
#pragma unroll
  for (int i = 0; i < 4 * RT; ++i) {
    const int row = 8 * i + (lane >> 3);
    const int64_t wn = n0 + row < N ? n0 + row : N - 1;
    wsrc[i] = W + wn * KB + 16 * ((lane & 7) ^ (row & 7));
  }
  // slab copy instruction t of a segment: lane l takes row
  // t * (64 / D) + l / D, dword l % D of the segment's D dwords (clamped
  // inside the row)
  constexpr int kSeg = WL::kSeg, kD = WL::kRowDwords;
  const int slab_lrow = lane / kD;
  const int64_t slab_lofs = 4 * (lane % kD);
  const uint8_t* asrc[AI];
  const uint8_t* assrc = As;
  if constexpr (AK == 1) {
    const int64_t am = (lane >> 5) < M ? (lane >> 5) : M - 1;
    asrc[0] = A + am * KB + 4 * (lane & 31);
  } else if constexpr (AK >= 8) {
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const int row = 8 * i + (lane >> 3);
      const int64_t am = row < M ? row : M - 1;
      asrc[i] = A + am * KB + 16 * ((lane & 7) ^ (row & 7));
    }
  }
  if constexpr (AK > 0) {
    const int64_t ams = (lane >> 1) < M ? (lane >> 1) : M - 1;
    assrc = As + ams * KG + 4 * (lane & 1);
  }
  // streamed: copy i of the x chunk covers bytes 1024 i + 16 l of the
  // [2 rows][256 EB bytes] area; rows past M repeat row M - 1
  const uint8_t* xsrc[STREAM ? EB / 2 : 1];
  if constexpr (STREAM) {
#pragma unroll
    for (int i = 0; i < EB / 2; ++i) {
      const int p = 1024 * i + 16 * lane;
      const int64_t row = p / (256 * EB) < M ? p / (256 * EB) : M - 1;
      xsrc[i] = reinterpret_cast<const uint8_t*>(x) + row * K * EB + p % (256 * EB);
    }
  }
  // copy t (of RT kSeg) of the W' scale slab of segment seg (relative to c0)
  auto issue_slab = [&](int seg, int t) {
    const int row = t * (64 / kD) + slab_lrow;
    const int64_t wn = n0 + row < N ? n0 + row : N - 1;
    int64_t ofs = (int64_t)(c0 + seg * kSeg) * 8 + slab_lofs;
    if (ofs > KG - 4) ofs = KG - 4;
    dma4(Ws + wn * KG + ofs, ring_addr + (uint32_t)(WL::kSlab0 + (seg % kSlabs) * WL::kSlabBytes + t * 256));
  };
  // chunk c's copies, plus RT slab copies for the segment after c's
  auto issue = [&](int c) {
    const uint32_t base = ring_addr + (uint32_t)(((c - c0) % STAGES) * S::kBytes);
    const int64_t co = (int64_t)c * 128, so = (int64_t)c * 8;
#pragma unroll
    for (int i = 0; i < 4 * RT; ++i) dma16_nt(wsrc[i] + co, base + S::kW + i * 1024);
#pragma unroll
    for (int i = 0; i < RT; ++i) issue_slab((c - c0) / kSeg + 1, ((c - c0) % kSeg) * RT + i);
    if constexpr (AK == 1) {
      dma4(asrc[0] + co, base + S::kA);
    } else if constexpr (AK >= 8) {
#pragma unroll
      for (int i = 0; i < AI; ++i) dma16(asrc[i] + co, base + S::kA + i * 1024);
    }
    if constexpr (AK > 0) dma4(assrc + so, base + S::kAs);
    if constexpr (STREAM) {
      dma16(reinterpret_cast<const uint8_t*>(s) + (int64_t)c * 1024 + 16 * lane, base + S::kA);
#pragma unroll
      for (int i = 0; i < EB / 2; ++i) dma16(xsrc[i] + (int64_t)c * 256 * EB, base + S::kX + i * 1024);
    }
  };
  // segment 0's slab, then fill the ring (before the fused transform, which
  // then overlaps the copies)
  if (c0 < c1) {
#pragma unroll
    for (int t = 0; t < kSeg * RT; ++t) issue_slab(0, t);
  }
#pragma unroll
  for (int q = 0; q < STAGES - 1; ++q)
    if (c0 + q < c1) issue(c0 + q);

  if constexpr (FUSED) {
    // one quad of lanes per 32-element group; each quad loads the inputs of
    // up to kBatch groups before transforming them, so their load latencies
    // overlap
    constexpr int kBatch = 4;
    constexpr int kQuads = kThreads / 4;
    const int groups_per_row = (int)KG;
    const int tasks = (int)M * groups_per_row;
    const uint32_t quad = (uint32_t)lane & 3u;
    for (int base = tid >> 2; base < tasks; base += kBatch * kQuads) {
      float t[kBatch][8];
      float4 sa[kBatch], sb[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int t0 = base + b * kQuads;   // the same for the quad's four lanes
        if (t0 < tasks) {
          const int m = t0 / groups_per_row, g = t0 % groups_per_row;
          const int64_t col = (int64_t)g * 32 + quad * 8;
          dec_load8<XT>(x, m * K + col, t[b]);
          const float4* sp = reinterpret_cast<const float4*>(s + col);
          sa[b] = sp[0];
          sb[b] = sp[1];
        }
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int t0 = base + b * kQuads;
        if (t0 < tasks) {
          const int m = t0 / groups_per_row, g = t0 % groups_per_row;
          float* v = t[b];
          v[0] = v[0] * sa[b].x; v[1] = v[1] * sa[b].y; v[2] = v[2] * sa[b].z; v[3] = v[3] * sa[b].w;
          v[4] = v[4] * sb[b].x; v[5] = v[5] * sb[b].y; v[6] = v[6] * sb[b].z; v[7] = v[7] * sb[b].w;
          hadamard32_quad(t[b], quad);
          uint32_t e;
          const uint32_t packed = quantize_quad(t[b], &e);
          *reinterpret_cast<uint32_t*>(xcodes + m * xrb + g * 16 + quad * 4) = packed;
          if (quad == 0) xscales[m * xrg + g] = (uint8_t)e;
        }
      }
    }
    __syncthreads();
  }

  const int ar = r32 < M ? r32 : (int)M - 1;   // activation row of this lane's B column
  const uint8_t* xrow = xcodes + ar * xrb;
  const uint8_t* xsrow = xscales + ar * xrg;

  v16f_d acc[RT];
#pragma unroll
  for (int tt = 0; tt < RT; ++tt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[tt][r] = 0.0f;

  for (int c = c0; c < c1; ++c) {
    // the slot about to be refilled was read (into registers) one chunk ago;
    // make sure those LDS reads have returned before the copy lands
    wait_lgkmcnt0();
    if (c + STAGES - 1 < c1) issue(c + STAGES - 1);
    // wait until chunk c has landed: the copies of the chunks after it may
    // stay in flight
    const int ahead = (c1 - 1 - c) < (STAGES - 1) ? (c1 - 1 - c) : (STAGES - 1);
    if (STAGES > 3 && ahead == 3) wait_vmcnt<(STAGES > 3 ? 3 : 0) * S::kCopies>();
    else if (STAGES > 2 && ahead == 2) wait_vmcnt<(STAGES > 2 ? 2 : 0) * S::kCopies>();
    else if (ahead == 1) wait_vmcnt<S::kCopies>();
    else wait_vmcnt<0>();
    const uint8_t* st = ring + ((c - c0) % STAGES) * S::kBytes;
    uint4 wa[RT][4], xb[4];
    uint32_t ws[RT];
    const int cs = c - c0;
#pragma unroll
    for (int tt = 0; tt < RT; ++tt) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        wa[tt][j] = *reinterpret_cast<const uint4*>(st + S::kW + dec_slot(32 * tt + r32, 2 * j + h));
      const uint2 wsv = *reinterpret_cast<const uint2*>(slabs + ((cs / kSeg) % kSlabs) * WL::kSlabBytes +
                                                        (32 * tt + r32) * (8 * kSeg) + (cs % kSeg) * 8);
      ws[tt] = gather_scales(wsv.x, wsv.y, h);
    }
    uint2 xsv;
    if constexpr (AK == 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) xb[j] = *reinterpret_cast<const uint4*>(st + S::kA + ar * 128 + 16 * (2 * j + h));
      xsv = *reinterpret_cast<const uint2*>(st + S::kAs + ar * 8);
    } else if constexpr (AK >= 8) {
#pragma unroll
      for (int j = 0; j < 4; ++j) xb[j] = *reinterpret_cast<const uint4*>(st + S::kA + dec_slot(ar, 2 * j + h));
      xsv = *reinterpret_cast<const uint2*>(st + S::kAs + ar * 8);
    } else if constexpr (STREAM) {
      // quad q of the wave: group q % 8 of row q / 8 (lanes 4q..4q+3, eight
      // values each), from the staged x and s; results to xq
      const int q = lane >> 2, m = q >> 3, g = q & 7;
      const uint32_t quad = (uint32_t)lane & 3u;
      if (m < M) {   // the same for the quad's four lanes
        float t[8];
        dec_load8<XT>(st + S::kX + m * 256 * EB, g * 32 + quad * 8, t);
        const float4* sp = reinterpret_cast<const float4*>(st + S::kA + (g * 32 + quad * 8) * 4);
        const float4 sa = sp[0], sb = sp[1];
        t[0] = t[0] * sa.x; t[1] = t[1] * sa.y; t[2] = t[2] * sa.z; t[3] = t[3] * sa.w;
        t[4] = t[4] * sb.x; t[5] = t[5] * sb.y; t[6] = t[6] * sb.z; t[7] = t[7] * sb.w;
        hadamard32_quad(t, quad);
        uint32_t e;
        const uint32_t packed = quantize_quad(t, &e);
        *reinterpret_cast<uint32_t*>(xq + m * 128 + g * 16 + quad * 4) = packed;
        if (quad == 0) xq[256 + m * 8 + g] = (uint8_t)e;
      }
      // the wave's LDS accesses complete in order: the reads below see the
      // writes above
#pragma unroll
      for (int j = 0; j < 4; ++j) xb[j] = *reinterpret_cast<const uint4*>(xq + ar * 128 + 16 * (2 * j + h));
      xsv = *reinterpret_cast<const uint2*>(xq + 256 + ar * 8);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) xb[j] = *reinterpret_cast<const uint4*>(xrow + (int64_t)c * 128 + 16 * (2 * j + h));
      xsv = *reinterpret_cast<const uint2*>(xsrow + (int64_t)c * 8);
    }
    const uint32_t xs = gather_scales(xsv.x, xsv.y, h);
#pragma unroll
    for (int tt = 0; tt < RT; ++tt) {
      dec_mfma<0>(acc[tt], wa[tt], xb, ws[tt], xs);
      dec_mfma<1>(acc[tt], wa[tt], xb, ws[tt], xs);
      dec_mfma<2>(acc[tt], wa[tt], xb, ws[tt], xs);
      dec_mfma<3>(acc[tt], wa[tt], xb, ws[tt], xs);
    }
  }

  // ---- add the waves' 32x32 tiles in wave order.  Lane (r32, h), register r
  // holds D[n = 8*(r/4) + 4*h + r%4][m = r32].  Every wave's copies have
  // landed (its last chunk waited for all of them), so after the barrier the
  // rings and slabs can hold the partial sums.
  constexpr int kRows = 32 * RT;
  __syncthreads();
#pragma unroll
  for (int tt = 0; tt < RT; ++tt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int n = 32 * tt + 8 * (r >> 2) + 4 * h + (r & 3);
      red[(wave * kRows + n) * 32 + r32] = acc[tt][r];
    }
  }
  __syncthreads();
  if (out_mode & kOutSwiGLU) {
    // columns (2j, 2j+1) = (gate, up) -> column n0/2 + j of the [M][N/2] output
    constexpr int kPairs = kRows / 2;
    for (int idx = tid; idx < kPairs * 32; idx += kThreads) {
      const int j = idx % kPairs, m = idx / kPairs;
      float g = red[(2 * j) * 32 + m], u = red[(2 * j + 1) * 32 + m];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) {
        g = g + red[(w * kRows + 2 * j) * 32 + m];
        u = u + red[(w * kRows + 2 * j + 1) * 32 + m];
      }
      if (m < M && n0 + 2 * j < N) store_out(Y, (int64_t)m * (N >> 1) + (n0 >> 1) + j, silu_times(g, u), out_mode);
    }
    return;
  }
  for (int idx = tid; idx < kRows * 32; idx += kThreads) {
    const int n = idx % kRows, m = idx / kRows;   // consecutive threads: consecutive n of one row of y
    float v = red[n * 32 + m];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) v = v + red[(w * kRows + n) * 32 + m];
    if (m < M && n0 + n < N) store_out(Y, (int64_t)m * N + n0 + n, v, out_mode);
  }
}

// ---------------------------------------------------------------- host side

// Activation kind: fused M <= 2 streams the transform through the loop;
// larger fused M transforms the whole activation into LDS first.
static int decode_ak(int64_t M, bool fused) {
  if (fused) return M <= 2 ? -1 : 0;
  return M <= 2 ? 1 : (M <= 8 ? 8 : (M <= 16 ? 16 : 32));
}

template <int RT>
static int stage_bytes_rt(int ak, int eb) {
  switch (ak) {
    case -1: return eb == 4 ? DecStage<-1, 4, RT>::kBytes : DecStage<-1, 2, RT>::kBytes;
    case 0: return DecStage<0, 2, RT>::kBytes;
    case 1: return DecStage<1, 2, RT>::kBytes;
    case 8: return DecStage<8, 2, RT>::kBytes;
    case 16: return DecStage<16, 2, RT>::kBytes;
    default: return DecStage<32, 2, RT>::kBytes;
  }
}

static size_t wave_lds_bytes(int stages, int ak, int eb, int rt) {
  const int stage = rt == 2 ? stage_bytes_rt<2>(ak, eb) : stage_bytes_rt<1>(ak, eb);
  return (size_t)stages * stage + kSlabs * 32 * rt * 8 * (ak == 32 ? 4 : 8) + (ak < 0 ? 288 : 0);
}

struct DecodeConfig {
  int waves, stages, ak, eb, rt;
};

static size_t decode_lds_bytes(const DecodeConfig& d, int64_t M, int64_t K) {
  size_t b = (size_t)d.waves * wave_lds_bytes(d.stages, d.ak, d.eb, d.rt);
  if (d.ak == 0) b += (size_t)M * (size_t)(dec_xrow_bytes(K) + dec_xrow_groups(K));
  return b;
}

// Block height: 64 weight rows (two MFMA row tiles sharing each activation
// chunk, which halves the activation's L2-to-LDS traffic) for more than 8
// staged activation rows when 32-row blocks would number more than two per
// CU; then 2 waves per block, so that two blocks stay resident per CU.
// Otherwise 32 rows and 4 or 8 waves (for small activations the extra waves
// keep more of W' in flight, which matters more).  Each wave keeps STAGES - 1 chunks in flight; the ring is made as
// deep as LDS allows (2 to 4 slots), within half of the CU's LDS when the
// grid has more blocks than CUs, within all of it otherwise.  8 waves drop
// to 4 where 2 slots do not fit, and, with more than 8 staged activation
// rows, where they would get only 2 slots: 4 waves with 4 slots keep 12
// chunks in flight per block instead of 8 (measured on down-proj M32
// N5120 K25600: 25.7 us against 29.7; the fused M1 down-proj keeps 8 waves
// of 2 slots, 18.3 us against 21.9 with 4 of 4).
static DecodeConfig decode_config(int64_t M, int64_t N, int64_t K, bool fused, int eb) {
  DecodeConfig d;
  d.ak = decode_ak(M, fused);
  d.eb = eb;
  d.rt = (d.ak > 8 && ceil_div(N, kDecRows) > 512) ? 2 : 1;
  if (const char* e = getenv("MACAQ_DECODE_ROWS")) d.rt = atoi(e) == 64 ? 2 : 1;   // tuning knob
  const int max_stages = d.rt == 2 ? 3 : 4;
  d.waves = d.rt == 2 ? 2 : (K / 256 >= 24 ? 8 : 4);
  const size_t budget = ceil_div(N, kDecRows * d.rt) > 256 ? kDecLdsMax / 2 : kDecLdsMax;
  d.stages = max_stages;
  while (d.stages > 2 && decode_lds_bytes(d, M, K) > budget) --d.stages;
  if (d.waves > 4 && ((d.ak > 8 && d.stages < 3) || decode_lds_bytes(d, M, K) > kDecLdsMax)) {
    d.waves = 4;
    d.stages = max_stages;
    while (d.stages > 2 && decode_lds_bytes(d, M, K) > budget) --d.stages;
  }
  if (d.rt == 1) {   // tuning knobs
    if (const char* e = getenv("MACAQ_DECODE_WAVES")) d.waves = atoi(e) == 8 ? 8 : 4;
    if (const char* e = getenv("MACAQ_DECODE_STAGES")) d.stages = atoi(e) >= 4 ? 4 : (atoi(e) == 3 ? 3 : 2);
  }
  return d;
}

bool decode_supported(int64_t M, int64_t N, int64_t K, int64_t E) {
  return E == 1 && M >= 1 && M <= kDecMaxM && N >= 1 && K % 256 == 0;
}

template <int WAVES, int STAGES, int AK, typename XT, int RT>
static hipError_t launch_decode_w(const uint8_t* A, const uint8_t* As, const void* x, const float* s,
                                  const uint8_t* W, const uint8_t* Ws, int64_t M, int64_t N, int64_t K, void* Y,
                                  int mode, size_t lds, hipStream_t stream) {
  static_assert(DecWaveLds<STAGES, AK, dec_eb<XT>, RT>::kBytes >= 32 * RT * 32 * 4,
                "partial sums must fit in the rings");
  static const hipError_t attr = hipFuncSetAttribute((const void*)decode_gemm_kernel<WAVES, STAGES, AK, XT, RT>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kDecLdsMax);
  if (attr != hipSuccess) return attr;
  decode_gemm_kernel<WAVES, STAGES, AK, XT, RT>
      <<<dim3((unsigned)ceil_div(N, kDecRows * RT)), dim3(64 * WAVES), lds, stream>>>(A, As, x, s, W, Ws, M, N, K, Y,
                                                                                      mode);
  return hipGetLastError();
}

template <int AK, typename XT>
static hipError_t launch_decode_impl(const DecodeConfig& d, const uint8_t* A, const uint8_t* As, const void* x,
                                     const float* s, const uint8_t* W, const uint8_t* Ws, int64_t M, int64_t N,
                                     int64_t K, void* Y, int mode, hipStream_t stream) {
  const size_t lds = decode_lds_bytes(d, M, K);
  if (lds > kDecLdsMax) return hipErrorInvalidValue;
  if (d.rt == 2) {
    if (d.stages >= 3) return launch_decode_w<2, 3, AK, XT, 2>(A, As, x, s, W, Ws, M, N, K, Y, mode, lds, stream);
    return launch_decode_w<2, 2, AK, XT, 2>(A, As, x, s, W, Ws, M, N, K, Y, mode, lds, stream);
  }
  if (d.waves == 8) {
    if (d.stages == 4) return launch_decode_w<8, 4, AK, XT, 1>(A, As, x, s, W, Ws, M, N, K, Y, mode, lds, stream);
    if (d.stages == 3) return launch_decode_w<8, 3, AK, XT, 1>(A, As, x, s, W, Ws, M, N, K, Y, mode, lds, stream);
    return launch_decode_w<8, 2, AK, XT, 1>(A, As, x, s, W, Ws, M, N, K, Y, mode, lds, stream);
  }
  if (d.stages == 4) return launch_decode_w<4, 4, AK, XT, 1>(A, As, x, s, W, Ws, M, N, K, Y, mode, lds, stream);
  if (d.stages == 3) return launch_decode_w<4, 3, AK, XT, 1>(A, As, x, s, W, Ws, M, N, K, Y, mode, lds, stream);
  return launch_decode_w<4, 2, AK, XT, 1>(A, As, x, s, W, Ws, M, N, K, Y, mode, lds, stream);
}

hipError_t launch_decode_gemm(const uint8_t* A, const uint8_t* As, const uint8_t* W, const uint8_t* Ws, int64_t M,
                              int64_t N, int64_t K, void* Y, int mode, hipStream_t stream) {
  const DecodeConfig d = decode_config(M, N, K, false, 2);
  switch (d.ak) {
    case 1: return launch_decode_impl<1, DecBf16>(d, A, As, nullptr, nullptr, W, Ws, M, N, K, Y, mode, stream);
    case 8: return launch_decode_impl<8, DecBf16>(d, A, As, nullptr, nullptr, W, Ws, M, N, K, Y, mode, stream);
    case 16: return launch_decode_impl<16, DecBf16>(d, A, As, nullptr, nullptr, W, Ws, M, N, K, Y, mode, stream);
    default: return launch_decode_impl<32, DecBf16>(d, A, As, nullptr, nullptr, W, Ws, M, N, K, Y, mode, stream);
  }
}

// -------- fused transform + GEMM entry used by macaq_linear

// Whether the fused path fits, for either activation dtype.
bool linear_fused_supported(int64_t M, int64_t N, int64_t K, int64_t E) {
  if (!decode_supported(M, N, K, E)) return false;
  for (int eb : {2, 4})
    if (decode_lds_bytes(decode_config(M, N, K, true, eb), M, K) > kDecLdsMax) return false;
  return true;
}

hipError_t launch_linear_fused(const void* x, bool x_f32, const float* s, const uint8_t* B, const uint8_t* Bs,
                               int64_t M, int64_t N, int64_t K, void* Y, int mode, hipStream_t stream) {
  const DecodeConfig d = decode_config(M, N, K, true, x_f32 ? 4 : 2);
  if (d.ak < 0) {
    if (x_f32) return launch_decode_impl<-1, float>(d, nullptr, nullptr, x, s, B, Bs, M, N, K, Y, mode, stream);
    return launch_decode_impl<-1, DecBf16>(d, nullptr, nullptr, x, s, B, Bs, M, N, K, Y, mode, stream);
  }
  if (x_f32) return launch_decode_impl<0, float>(d, nullptr, nullptr, x, s, B, Bs, M, N, K, Y, mode, stream);
  return launch_decode_impl<0, DecBf16>(d, nullptr, nullptr, x, s, B, Bs, M, N, K, Y, mode, stream);
}

}  // namespace macaq

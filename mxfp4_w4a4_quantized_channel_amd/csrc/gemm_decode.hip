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
#include <atomic>

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

// ---- one-launch layer (PUB): the first blocks of the grid transform the
// activation into the staging buffer, the rest wait for it.
//
// Synchronization words in the workspace (64-bit, device-coherent accesses,
// no read-modify-write among the publishers):
//   sync[0]       the blocks' finish count;
//   sync[16 + p]  publisher p's done word: the launch's epoch once its slice
//                 of the activation is stored (p < 64).
// Publisher 0 first sets the finish count to 0; each publisher stores its
// slice, waits for those stores, then stores its done word.  Wave 0 of every
// block polls all done words with one load (lane p reads word p) until each
// holds the epoch, so every block has seen publisher 0's reset before it adds
// to the finish count.  Once all of a block's waves are past that wait, the
// block adds 1 to the count; the block that completes it clears the done
// words and the count, so a graph replay of a captured launch (whose epoch
// is fixed) finds them clear.  The epoch is unique per launch in the
// process, so done words left by another call, or whatever bytes the
// workspace held, never read as done: the workspace needs no initial
// contents.
constexpr int kPubMax = 64;
constexpr int kPubSyncWords = 16 + kPubMax;

__device__ __forceinline__ void sync_store(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll the done words until all `pubs` hold this launch's epoch, about every
// two microseconds (s_sleep 64; polling eight times as often was slower, the
// polls themselves loading the memory path).  The publishing blocks are the
// lowest block indices, which the dispatcher places first, and they wait on
// nothing, so they are done within microseconds; the poll still gives up
// after `max_polls` polls (about a second by default) and returns false, and
// the block then writes NaN for every output it owns, so that a hand-over
// that never completed shows in y instead of passing for a result.  Called
// by a whole wave (the result is wave-uniform).
constexpr int kPubMaxPolls = 1 << 19;
__device__ __forceinline__ bool wait_published(unsigned long long* done, unsigned long long epoch, int pubs,
                                               int lane, int max_polls) {
  for (int i = 0; i < max_polls; ++i) {
    bool ok = true;
    if (lane < pubs) ok = __hip_atomic_load(done + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch;
    if (__builtin_amdgcn_ballot_w64(!ok) == 0) return true;
    __builtin_amdgcn_s_sleep(64);
  }
  return false;
}

// s_waitcnt vmcnt(n) for a wave-uniform n known only at run time.
__device__ __forceinline__ void wait_vmcnt_rt(int n) {
  switch (n) {
#define MACAQ_VM_CASE(k) case k: wait_vmcnt<k>(); break;
    MACAQ_VM_CASE(0) MACAQ_VM_CASE(1) MACAQ_VM_CASE(2) MACAQ_VM_CASE(3) MACAQ_VM_CASE(4) MACAQ_VM_CASE(5)
    MACAQ_VM_CASE(6) MACAQ_VM_CASE(7) MACAQ_VM_CASE(8) MACAQ_VM_CASE(9) MACAQ_VM_CASE(10) MACAQ_VM_CASE(11)
    MACAQ_VM_CASE(12) MACAQ_VM_CASE(13) MACAQ_VM_CASE(14) MACAQ_VM_CASE(15) MACAQ_VM_CASE(16) MACAQ_VM_CASE(17)
    MACAQ_VM_CASE(18) MACAQ_VM_CASE(19) MACAQ_VM_CASE(20) MACAQ_VM_CASE(21) MACAQ_VM_CASE(22) MACAQ_VM_CASE(23)
    MACAQ_VM_CASE(24) MACAQ_VM_CASE(25) MACAQ_VM_CASE(26) MACAQ_VM_CASE(27) MACAQ_VM_CASE(28) MACAQ_VM_CASE(29)
    MACAQ_VM_CASE(30) MACAQ_VM_CASE(31) MACAQ_VM_CASE(32) MACAQ_VM_CASE(33) MACAQ_VM_CASE(34) MACAQ_VM_CASE(35)
    MACAQ_VM_CASE(36) MACAQ_VM_CASE(37) MACAQ_VM_CASE(38) MACAQ_VM_CASE(39) MACAQ_VM_CASE(40) MACAQ_VM_CASE(41)
    MACAQ_VM_CASE(42) MACAQ_VM_CASE(43) MACAQ_VM_CASE(44) MACAQ_VM_CASE(45) MACAQ_VM_CASE(46) MACAQ_VM_CASE(47)
    MACAQ_VM_CASE(48) MACAQ_VM_CASE(49) MACAQ_VM_CASE(50) MACAQ_VM_CASE(51) MACAQ_VM_CASE(52) MACAQ_VM_CASE(53)
    MACAQ_VM_CASE(54) MACAQ_VM_CASE(55) MACAQ_VM_CASE(56) MACAQ_VM_CASE(57) MACAQ_VM_CASE(58) MACAQ_VM_CASE(59)
    MACAQ_VM_CASE(60) MACAQ_VM_CASE(61) MACAQ_VM_CASE(62)
#undef MACAQ_VM_CASE
    default: wait_vmcnt<63>();
  }
}

// Publisher block b of `pubs`: 32-element groups [b * per, (b + 1) * per) of
// the M x K/32 groups (row-major), one quad of lanes per group, batches of
// 4 groups per quad whose loads overlap; the same scale, transform and
// quantization as the activation kernel.  Codes [M][K/2] and scales
// [M][K/32] are stored device-coherent (sc1), so that blocks on other XCDs
// read them from memory once the count says they are there.
template <typename XT>
__device__ __forceinline__ void publish_slice(const void* x, const float* s, int64_t M, int64_t K, uint8_t* codes,
                                              uint8_t* scales, int b, int pubs, int tid, int threads) {
  constexpr int kBatch = 4;
  const int quads = threads / 4;
  const int64_t KG = K >> 5;
  const int64_t tasks = M * KG;
  const int64_t per = (tasks + pubs - 1) / pubs;
  const int64_t t_begin = (int64_t)b * per;
  const int64_t t_end = t_begin + per < tasks ? t_begin + per : tasks;
  const uint32_t quad = (uint32_t)tid & 3u;
  for (int64_t base = t_begin + (tid >> 2); base < t_end; base += (int64_t)kBatch * quads) {
    float t[kBatch][8];
    float4 sa[kBatch], sb[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int64_t t0 = base + (int64_t)j * quads;   // the same for the quad's four lanes
      if (t0 < t_end) {
        const int64_t m = t0 / KG, g = t0 % KG;
        const int64_t col = g * 32 + quad * 8;
        dec_load8<XT>(x, m * K + col, t[j]);
        const float4* sp = reinterpret_cast<const float4*>(s + col);
        sa[j] = sp[0];
        sb[j] = sp[1];
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int64_t t0 = base + (int64_t)j * quads;
      if (t0 < t_end) {
        const int64_t m = t0 / KG, g = t0 % KG;
        float* v = t[j];
        v[0] = v[0] * sa[j].x; v[1] = v[1] * sa[j].y; v[2] = v[2] * sa[j].z; v[3] = v[3] * sa[j].w;
        v[4] = v[4] * sb[j].x; v[5] = v[5] * sb[j].y; v[6] = v[6] * sb[j].z; v[7] = v[7] * sb[j].w;
        hadamard32_quad(t[j], quad);
        uint32_t e;
        const uint32_t packed = quantize_quad(t[j], &e);
        __hip_atomic_store(reinterpret_cast<uint32_t*>(codes + m * (K >> 1) + g * 16 + quad * 4), packed,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (quad == 0)
          __hip_atomic_store(scales + m * KG + g, (uint8_t)e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// A block owns RT x 32 weight rows (RT MFMA row tiles sharing each
// activation chunk).
template <int WAVES, int STAGES, int AK, typename XT, int RT = 1, bool PUB = false>
__global__ __launch_bounds__(64 * WAVES) void decode_gemm_kernel(
    const uint8_t* A, const uint8_t* As,                               // activation codes/scales (staged)
    const void* __restrict__ x, const float* __restrict__ s,           // activations and scale (fused)
    const uint8_t* __restrict__ W, const uint8_t* __restrict__ Ws, int64_t M, int64_t N, int64_t K,
    void* __restrict__ Y, int out_mode, float* __restrict__ part_ws, int ksplit,
    unsigned long long* sync, unsigned long long epoch, int pubs, int max_polls) {
  static_assert(!PUB || AK >= 8, "the one-launch layer stages 8, 16 or 32 activation rows");
  constexpr int EB = dec_eb<XT>;
  using S = DecStage<AK, EB, RT>;
  constexpr bool FUSED = AK == 0;     // resident activation, transformed before the loop
  constexpr bool STREAM = AK < 0;     // activation transformed chunk by chunk in the loop
  constexpr int AI = AK >= 8 ? AK / 8 : 1;
  extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
  constexpr int kThreads = 64 * WAVES;
  const int64_t n0 = (int64_t)blockIdx.x * kDecRows * RT;
  const int64_t KB = K >> 1, KG = K >> 5;
  bool pub_ok = true;   // one-launch layer: the activation's hand-over completed (wave 0)
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
  // K split over blockIdx.y (ksplit parts of the chunks), then over the waves
  const int part = (int)blockIdx.y;
  const int cb0 = (int)((int64_t)kc * part / ksplit), cb1 = (int)((int64_t)kc * (part + 1) / ksplit);
  const int per_wave = (cb1 - cb0 + WAVES - 1) / WAVES;
  const int c0 = cb0 + wave * per_wave;
  const int c1 = (c0 + per_wave) < cb1 ? (c0 + per_wave) : cb1;
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
  // chunk c's copies: the weight part (codes, plus RT slab copies for the
  // segment after c's), then the activation part
  auto issue_w = [&](int c) {
    const uint32_t base = ring_addr + (uint32_t)(((c - c0) % STAGES) * S::kBytes);
    const int64_t co = (int64_t)c * 128;
#pragma unroll
    for (int i = 0; i < 4 * RT; ++i) dma16_nt(wsrc[i] + co, base + S::kW + i * 1024);
#pragma unroll
    for (int i = 0; i < RT; ++i) issue_slab((c - c0) / kSeg + 1, ((c - c0) % kSeg) * RT + i);
  };
  auto issue_a = [&](int c) {
    const uint32_t base = ring_addr + (uint32_t)(((c - c0) % STAGES) * S::kBytes);
    const int64_t co = (int64_t)c * 128, so = (int64_t)c * 8;
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
  auto issue = [&](int c) {
    issue_w(c);
    issue_a(c);
  };
  // one-launch layer: a publishing block transforms its slice of x first
  // (its loads then wait for no copy), stores it device-coherent, waits for
  // the stores and adds to the count
  if constexpr (PUB) {
    const int flat = (int)(blockIdx.y * gridDim.x + blockIdx.x);
    if (flat < pubs) {
      if (flat == 0 && tid == 0) sync_store(sync, 0ull);
      publish_slice<XT>(x, s, M, K, const_cast<uint8_t*>(A), const_cast<uint8_t*>(As), flat, pubs, tid, kThreads);
      wait_vmcnt<0>();
      __syncthreads();
      if (tid == 0) sync_store(sync + 16 + flat, epoch);
    }
  }

  // segment 0's slab, then fill the ring (before the fused transform, which
  // then overlaps the copies).  One-launch layer: the weight copies of the
  // first chunks, the wait for the published activation, then its copies.
  if (c0 < c1) {
#pragma unroll
    for (int t = 0; t < kSeg * RT; ++t) issue_slab(0, t);
  }
  // weight chunks issued before the wait: the whole prologue (1 or none
  // measured no faster: the publishers' loads still queue behind the copies)
  constexpr int kPre = STAGES - 1;
  if constexpr (PUB) {
#pragma unroll
    for (int q = 0; q < kPre; ++q)
      if (c0 + q < c1) issue_w(c0 + q);
    if (wave == 0) pub_ok = wait_published(sync + 16, epoch, pubs, lane, max_polls);
    __syncthreads();   // (no wait for the copies in flight)
#pragma unroll
    for (int q = 0; q < kPre; ++q)
      if (c0 + q < c1) issue_a(c0 + q);
#pragma unroll
    for (int q = kPre; q < STAGES - 1; ++q)
      if (c0 + q < c1) issue(c0 + q);
  } else {
#pragma unroll
    for (int q = 0; q < STAGES - 1; ++q)
      if (c0 + q < c1) issue(c0 + q);
  }

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
    const int n_ch = c1 - c0, p0 = n_ch < STAGES - 1 ? n_ch : STAGES - 1;
    const int pre = kPre < p0 ? kPre : p0;
    if (PUB && c - c0 < pre) {
      // the first `pre` chunks' activation copies were issued after their
      // weight copies: after chunk c's come the activation copies of the
      // later ones, the prologue's whole chunks and the loop's so far
      const int loop_chunks = n_ch - STAGES >= 0 ? ((c - c0) < n_ch - STAGES ? (c - c0) : n_ch - STAGES) + 1 : 0;
      wait_vmcnt_rt((pre - 1 - (c - c0)) * S::kACopies + (p0 - pre + loop_chunks) * S::kCopies);
    } else if (STAGES > 3 && ahead == 3) wait_vmcnt<(STAGES > 3 ? 3 : 0) * S::kCopies>();
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
  // one-launch layer whose wait gave up: wave 0's tile, which every output
  // of the block (and every partial sum of a K split) adds, becomes NaN
  const bool poisoned = PUB && !pub_ok;
#pragma unroll
  for (int tt = 0; tt < RT; ++tt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int n = 32 * tt + 8 * (r >> 2) + 4 * h + (r & 3);
      red[(wave * kRows + n) * 32 + r32] = poisoned ? __builtin_nanf("") : acc[tt][r];
    }
  }
  __syncthreads();
  if constexpr (PUB) {
    // every wave of the block is past its wait for the activation: the last
    // block of the launch to get here clears the words
    if (tid < 64) {
      unsigned long long before = 0;
      if (tid == 0) before = __hip_atomic_fetch_add(sync, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      before = __shfl(before, 0);
      if (before == (unsigned long long)(gridDim.x * gridDim.y - 1)) {
        if (tid < pubs) sync_store(sync + 16 + tid, 0ull);
        if (tid == 0) sync_store(sync, 0ull);
      }
    }
  }
  if (ksplit > 1) {
    // this part's fp32 sums of the block's columns, [part][M][N]; the split
    // reduce kernel adds the parts in order and applies the output mode
    float* pw = part_ws + (int64_t)part * M * N;
    for (int idx = tid; idx < kRows * 32; idx += kThreads) {
      const int n = idx % kRows, m = idx / kRows;
      float v = red[n * 32 + m];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) v = v + red[(w * kRows + n) * 32 + m];
      if (m < M && n0 + n < N) pw[(int64_t)m * N + n0 + n] = v;
    }
    return;
  }
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

// Sum of the K-split parts of a decode GEMM, in part order, with the output
// mode: y[m][n] = p0[m][n] + p1[m][n] (+ ...), or for SwiGLU
// y[m][j] = silu(g) * u over the summed column pair (2j, 2j+1).
__global__ void decode_split_reduce_kernel(const float* __restrict__ part_ws, int ksplit, int64_t M, int64_t N,
                                           void* __restrict__ Y, int out_mode) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t MN = M * N;
  if (out_mode & kOutSwiGLU) {
    const int64_t half = N >> 1;
    if (i >= M * half) return;
    const int64_t m = i / half, j = i % half;
    float g = part_ws[m * N + 2 * j], u = part_ws[m * N + 2 * j + 1];
    for (int p = 1; p < ksplit; ++p) {
      g = g + part_ws[p * MN + m * N + 2 * j];
      u = u + part_ws[p * MN + m * N + 2 * j + 1];
    }
    store_out(Y, i, silu_times(g, u), out_mode);
    return;
  }
  if (i >= MN) return;
  float v = part_ws[i];
  for (int p = 1; p < ksplit; ++p) v = v + part_ws[p * MN + i];
  store_out(Y, i, v, out_mode);
}

// ---- decode GEMM for 3 to 32 activation rows, without a K split: waves
// split rows, and share each staged activation chunk.
//
// With 32 activation rows the activation's part of a chunk is as large as
// a 32-row tile's weights (with 8 rows a quarter); when every wave stages
// its own copy (waves splitting K, decode_gemm_kernel) that adds to the LDS
// fill per chunk and shortens the ring.  Here a block of WAVES waves owns 32 WAVES weight
// rows, wave w the 32 rows from n0 + 32 w, and all waves walk all chunks of
// K: the activation chunk (AK rows of codes and the 32 x 8 scale bytes) sits
// once per ring slot in LDS shared by the waves.  Each wave's weights and W'
// scale slabs are its own, as in decode_gemm_kernel.  Each wave issues its weight copies and a share of the
// activation copies (instruction i of the AK / 8 goes to wave i % WAVES,
// with waves past the last one repeating an instruction, and every wave
// copying the scale bytes: identical bytes to the same place), so every
// wave issues the same count per chunk.  One barrier per chunk: after each
// wave has waited for its own copies of chunk c and for its reads of chunk
// c - 1, the barrier makes the whole chunk visible and frees chunk c - 1's
// slot, which the copies of chunk c + STAGES - 1 then refill.
template <int WAVES, int STAGES, int AK>
struct DecRowsLds {
  static constexpr int kSeg = AK == 32 ? 4 : 8;                        // chunks per W' scale segment
  static constexpr int kSlabsR = (STAGES - 2 + kSeg) / kSeg + 2;       // ceil((STAGES - 1) / kSeg) + 2
  static constexpr int kSlabBytes = 32 * 8 * kSeg;
  static constexpr int kWave = STAGES * 4096 + kSlabsR * kSlabBytes;   // a wave's weight slots and slabs
  static constexpr int kAStage = AK * 128 + 256;                       // shared activation codes + scales
  static constexpr int kShared0 = WAVES * kWave;
  static constexpr int kBytes = kShared0 + STAGES * kAStage;
  static constexpr int kAI = AK / 8;                                   // activation code copies per chunk
  static constexpr int kAPerWave = (kAI + WAVES - 1) / WAVES;
  static constexpr int kCopies = 4 + 1 + kAPerWave + 1;                // per wave per chunk
};

template <int WAVES, int STAGES, int AK>
__global__ __launch_bounds__(64 * WAVES) void decode_rows_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ W,
    const uint8_t* __restrict__ Ws, int64_t M, int64_t N, int64_t K, void* __restrict__ Y, int out_mode) {
  static_assert(AK == 8 || AK == 16 || AK == 32, "8, 16 or 32 staged activation rows");
  using L = DecRowsLds<WAVES, STAGES, AK>;
  static_assert((STAGES - 2) * L::kCopies < 64, "vmcnt range");
  static_assert(L::kBytes >= 32 * WAVES * 32 * 4, "the output tile must fit in the rings");
  extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
  constexpr int kThreads = 64 * WAVES;
  constexpr int kRows = 32 * WAVES;
  constexpr int kSeg = L::kSeg, kD = 2 * kSeg;
  const int64_t KB = K >> 1, KG = K >> 5;
  const int kc = (int)(K >> 8);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31;
  const int h = lane >> 5;
  const int64_t n0 = (int64_t)blockIdx.x * kRows;
  const int64_t nw = n0 + 32 * wave;   // this wave's first weight row

  uint8_t* ring = dsm + wave * L::kWave;
  const uint32_t ring_addr = (uint32_t)(uintptr_t)ring;
  const uint8_t* slabs = ring + STAGES * 4096;
  const uint8_t* ash = dsm + L::kShared0;
  const uint32_t ash_addr = (uint32_t)(uintptr_t)ash;

  const int cb0 = 0, cb1 = kc;   // the block's chunks: the whole K range

  // copy sources (rows past N or M repeat the last row; their results are not stored)
  const uint8_t* wsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 8 * i + (lane >> 3);
    const int64_t wn = nw + row < N ? nw + row : N - 1;
    wsrc[i] = W + wn * KB + 16 * ((lane & 7) ^ (row & 7));
  }
  const int slab_lrow = lane / kD;
  const int64_t slab_lofs = 4 * (lane % kD);
  const uint8_t* asrc[L::kAPerWave];
  int adst[L::kAPerWave];
#pragma unroll
  for (int j = 0; j < L::kAPerWave; ++j) {
    const int i = (wave + j * WAVES) % L::kAI;   // activation copy instruction of this wave
    const int row = 8 * i + (lane >> 3);
    const int64_t am = row < M ? row : M - 1;
    asrc[j] = A + am * KB + 16 * ((lane & 7) ^ (row & 7));
    adst[j] = i * 1024;
  }
  const int64_t ams = (lane >> 1) < M ? (lane >> 1) : M - 1;
  const uint8_t* assrc = As + ams * KG + 4 * (lane & 1);

  auto issue_slab = [&](int seg, int t) {
    const int row = t * (64 / kD) + slab_lrow;
    const int64_t wn = nw + row < N ? nw + row : N - 1;
    int64_t ofs = (int64_t)(cb0 + seg * kSeg) * 8 + slab_lofs;
    if (ofs > KG - 4) ofs = KG - 4;
    dma4(Ws + wn * KG + ofs, ring_addr + (uint32_t)(STAGES * 4096 + (seg % L::kSlabsR) * L::kSlabBytes + t * 256));
  };
  auto issue = [&](int c) {
    const int slot = (c - cb0) % STAGES;
    const int64_t co = (int64_t)c * 128, so = (int64_t)c * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16_nt(wsrc[i] + co, ring_addr + (uint32_t)(slot * 4096 + i * 1024));
    issue_slab((c - cb0) / kSeg + 1, (c - cb0) % kSeg);
    const uint32_t abase = ash_addr + (uint32_t)(slot * L::kAStage);
#pragma unroll
    for (int j = 0; j < L::kAPerWave; ++j) dma16(asrc[j] + co, abase + (uint32_t)adst[j]);
    dma4(assrc + so, abase + (uint32_t)(AK * 128));
  };

  if (cb0 < cb1) {
#pragma unroll
    for (int t = 0; t < kSeg; ++t) issue_slab(0, t);
  }
#pragma unroll
  for (int q = 0; q < STAGES - 1; ++q)
    if (cb0 + q < cb1) issue(cb0 + q);

  const int ar = r32 < M ? r32 : (int)M - 1;   // activation row of this lane's B column
  v16f_d acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

  for (int c = cb0; c < cb1; ++c) {
    // this wave's copies of chunk c have landed when at most the chunks
    // after it (up to STAGES - 2, chunk c + STAGES - 1 not issued yet) are
    // in flight; its reads of chunk c - 1 have returned
    const int ahead = (cb1 - 1 - c) < (STAGES - 2) ? (cb1 - 1 - c) : (STAGES - 2);
    wait_vmcnt_rt(ahead * L::kCopies);
    wait_lgkmcnt0();
    block_barrier();   // chunk c complete in LDS; chunk c - 1's slot free
    if (c + STAGES - 1 < cb1) issue(c + STAGES - 1);
    const int cs = c - cb0;
    const uint8_t* st = ring + (cs % STAGES) * 4096;
    const uint8_t* sa = ash + (cs % STAGES) * L::kAStage;
    uint4 wa[4], xb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) wa[j] = *reinterpret_cast<const uint4*>(st + dec_slot(r32, 2 * j + h));
    const uint2 wsv = *reinterpret_cast<const uint2*>(slabs + ((cs / kSeg) % L::kSlabsR) * L::kSlabBytes +
                                                      r32 * (8 * kSeg) + (cs % kSeg) * 8);
    const uint32_t ws = gather_scales(wsv.x, wsv.y, h);
#pragma unroll
    for (int j = 0; j < 4; ++j) xb[j] = *reinterpret_cast<const uint4*>(sa + dec_slot(ar, 2 * j + h));
    const uint2 xsv = *reinterpret_cast<const uint2*>(sa + AK * 128 + ar * 8);
    const uint32_t xs = gather_scales(xsv.x, xsv.y, h);
    dec_mfma<0>(acc, wa, xb, ws, xs);
    dec_mfma<1>(acc, wa, xb, ws, xs);
    dec_mfma<2>(acc, wa, xb, ws, xs);
    dec_mfma<3>(acc, wa, xb, ws, xs);
  }

  // ---- output: lane (r32, h), register r holds D[n = 8*(r/4) + 4*h + r%4]
  // [m = r32] of this wave's 32 rows; through LDS ([block row n][m]) so that
  // consecutive threads store consecutive columns of y.  Every copy has
  // landed (the last chunk waited for all of them).
  float* red = reinterpret_cast<float*>(dsm);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int n = 32 * wave + 8 * (r >> 2) + 4 * h + (r & 3);
    red[n * 32 + r32] = acc[r];
  }
  __syncthreads();
  if (out_mode & kOutSwiGLU) {
    constexpr int kPairs = kRows / 2;
    for (int idx = tid; idx < kPairs * 32; idx += kThreads) {
      const int j = idx % kPairs, m = idx / kPairs;
      if (m < M && n0 + 2 * j < N)
        store_out(Y, (int64_t)m * (N >> 1) + (n0 >> 1) + j, silu_times(red[(2 * j) * 32 + m], red[(2 * j + 1) * 32 + m]),
                  out_mode);
    }
  } else {
    for (int idx = tid; idx < kRows * 32; idx += kThreads) {
      const int n = idx % kRows, m = idx / kRows;
      if (m < M && n0 + n < N) store_out(Y, (int64_t)m * N + n0 + n, red[n * 32 + m], out_mode);
    }
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
  int waves, stages, ak, eb, rt, ksplit;
};

// K split of the decode GEMM: with fewer row tiles than the 256 CUs, the K
// range of each row tile is cut into `ksplit` parts taken by as many blocks,
// so that every CU streams weights.  32-row blocks (4 waves) take the largest
// split up to 4 whose blocks fit two per CU and still leave each wave 8 or
// more 256-wide chunks; 64-row blocks (2 waves) the largest whose blocks fit
// one per CU.  The parts' fp32 partial sums go to the caller's workspace and
// a second kernel adds them in part order.  Measured on down-proj N5120
// K25600: fused M1 17.1 us against 18.4 unsplit (32-row blocks, 3 parts);
// M32 20.7 us with 64-row blocks in 3 parts (240 blocks), against 24.1 with
// 32-row blocks in 3 parts and 25.7 unsplit; M16 18.0 against 19.3 and 21.3.
// Grids just past one block per CU slot were slower than no split (32-row
// blocks in 2 parts: 30.5 us at M32; 64-row blocks in 4 parts: 29.1 us).
// macaq_set_tuning(MACAQ_TUNE_DECODE_SPLIT) forces the number of parts
// (1 = no split).
constexpr int kDecCUs = 256;
constexpr int kDecSplitWaves = 4;
static int decode_ksplit(int64_t N, int64_t K, int rt) {
  const int64_t tiles = ceil_div(N, kDecRows * rt);
  const int kc = (int)(K >> 8);
  int ks = 1;
  if (tiles < kDecCUs) {
    if (rt == 1) {
      while (ks < 4 && tiles * (ks + 1) <= 2 * kDecCUs && kc / ((ks + 1) * kDecSplitWaves) >= 8) ++ks;
    } else {
      while (ks < 4 && tiles * (ks + 1) <= kDecCUs && kc / ((ks + 1) * 2) >= 8) ++ks;
    }
  }
  if (const int force = tuning(MACAQ_TUNE_DECODE_SPLIT)) ks = force;
  return ks < kc ? ks : kc;   // at least one chunk per part
}

static size_t decode_lds_bytes(const DecodeConfig& d, int64_t M, int64_t K) {
  size_t b = (size_t)d.waves * wave_lds_bytes(d.stages, d.ak, d.eb, d.rt);
  if (d.ak == 0) b += (size_t)M * (size_t)(dec_xrow_bytes(K) + dec_xrow_groups(K));
  return b;
}

// Block height: 64 weight rows (two MFMA row tiles sharing each activation
// chunk, which halves the activation's L2-to-LDS traffic) for more than 8
// staged activation rows when 32-row blocks would number more than two per
// CU, or when they would number fewer than the CUs and the K split applies
// (the split then makes about one block per CU); 2 waves per block.
// Otherwise 32 rows and 4 or 8 waves (for small activations the extra waves
// keep more of W' in flight, which matters more).  Each wave keeps
// STAGES - 1 chunks in flight; the ring is made as deep as LDS allows (2 to
// 4 slots), within half of the CU's LDS when the grid has more blocks than
// CUs, within all of it otherwise.  8 waves drop to 4 where 2 slots do not
// fit, and, with more than 8 staged activation rows, where they would get
// only 2 slots: 4 waves with 4 slots keep 12 chunks in flight per block
// instead of 8 (measured on down-proj M32 N5120 K25600 without a split: 25.7
// us against 29.7).  Split 32-row blocks take 4 waves.
static DecodeConfig decode_config(int64_t M, int64_t N, int64_t K, bool fused, int eb) {
  DecodeConfig d;
  d.ak = decode_ak(M, fused);
  d.eb = eb;
  const int64_t t32 = ceil_div(N, kDecRows);
  d.rt = (d.ak > 8 && t32 > 512) ? 2 : 1;
  // narrow layers with more than 8 staged rows: 64-row blocks in K parts
  if (d.ak > 8 && t32 < kDecCUs && decode_ksplit(N, K, 2) > 1) d.rt = 2;
  if (const int force = tuning(MACAQ_TUNE_DECODE_ROWS)) d.rt = force == 64 ? 2 : 1;
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
  d.ksplit = decode_ksplit(N, K, d.rt);
  if (d.ksplit > 1 && d.rt == 1) {   // split blocks: 4 waves, two blocks per CU
    d.waves = kDecSplitWaves;
    const size_t split_budget = ceil_div(N, kDecRows) * d.ksplit > kDecCUs ? kDecLdsMax / 2 : kDecLdsMax;
    d.stages = max_stages;
    while (d.stages > 2 && decode_lds_bytes(d, M, K) > split_budget) --d.stages;
  }
  if (d.rt == 1) {   // forced ring shapes, kept only where they fit in LDS
    DecodeConfig f = d;
    if (const int force = tuning(MACAQ_TUNE_DECODE_WAVES)) f.waves = force == 8 ? 8 : 4;
    if (const int force = tuning(MACAQ_TUNE_DECODE_STAGES)) f.stages = force >= 4 ? 4 : (force == 3 ? 3 : 2);
    if (decode_lds_bytes(f, M, K) <= kDecLdsMax) d = f;
  }
  return d;
}

bool decode_supported(int64_t M, int64_t N, int64_t K, int64_t E) {
  return E == 1 && M >= 1 && M <= kDecMaxM && N >= 1 && K % 256 == 0;
}

// One-launch layer: counts word pair, epoch and number of publishing blocks.
struct PubLaunch {
  unsigned long long* sync = nullptr;
  unsigned long long epoch = 0;
  int pubs = 0;
  int max_polls = kPubMaxPolls;
};

// Epoch of a one-launch layer: a 40-bit value unique within the process
// (its start is arbitrary, away from the small integers that stale
// workspace bytes often hold).
static unsigned long long next_pub_epoch() {
  static std::atomic<unsigned long long> epoch{0x5f3a9c6e1ull};
  return epoch.fetch_add(1, std::memory_order_relaxed) & 0xffffffffffull;
}

template <int WAVES, int STAGES, int AK, typename XT, int RT, bool PUB>
static hipError_t launch_decode_w(const uint8_t* A, const uint8_t* As, const void* x, const float* s,
                                  const uint8_t* W, const uint8_t* Ws, int64_t M, int64_t N, int64_t K, void* Y,
                                  int mode, size_t lds, float* part_ws, int ksplit, const PubLaunch& pl,
                                  hipStream_t stream) {
  static_assert(DecWaveLds<STAGES, AK, dec_eb<XT>, RT>::kBytes >= 32 * RT * 32 * 4,
                "partial sums must fit in the rings");
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)decode_gemm_kernel<WAVES, STAGES, AK, XT, RT, PUB>, hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)kDecLdsMax);
  if (attr != hipSuccess) return attr;
  decode_gemm_kernel<WAVES, STAGES, AK, XT, RT, PUB>
      <<<dim3((unsigned)ceil_div(N, kDecRows * RT), (unsigned)ksplit), dim3(64 * WAVES), lds, stream>>>(
          A, As, x, s, W, Ws, M, N, K, Y, mode, part_ws, ksplit, pl.sync, pl.epoch, pl.pubs, pl.max_polls);
  if (ksplit > 1) {
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    const int64_t outs = (mode & kOutSwiGLU) ? M * (N >> 1) : M * N;
    decode_split_reduce_kernel<<<dim3((unsigned)ceil_div(outs, 256)), dim3(256), 0, stream>>>(part_ws, ksplit, M, N, Y,
                                                                                              mode);
  }
  return hipGetLastError();
}

template <int AK, typename XT, bool PUB = false>
static hipError_t launch_decode_impl(const DecodeConfig& d, const uint8_t* A, const uint8_t* As, const void* x,
                                     const float* s, const uint8_t* W, const uint8_t* Ws, int64_t M, int64_t N,
                                     int64_t K, void* Y, int mode, float* part_ws, hipStream_t stream,
                                     const PubLaunch& pl = PubLaunch()) {
  if (d.ksplit > 1 && part_ws == nullptr) return hipErrorInvalidValue;
  const size_t lds = decode_lds_bytes(d, M, K);
  if (lds > kDecLdsMax) return hipErrorInvalidValue;
#define MACAQ_DEC_LAUNCH(WV, ST, RTV) \
  launch_decode_w<WV, ST, AK, XT, RTV, PUB>(A, As, x, s, W, Ws, M, N, K, Y, mode, lds, part_ws, d.ksplit, pl, stream)
  if (d.rt == 2) {
    if (d.stages >= 3) return MACAQ_DEC_LAUNCH(2, 3, 2);
    return MACAQ_DEC_LAUNCH(2, 2, 2);
  }
  if (d.waves == 8) {
    if (d.stages == 4) return MACAQ_DEC_LAUNCH(8, 4, 1);
    if (d.stages == 3) return MACAQ_DEC_LAUNCH(8, 3, 1);
    return MACAQ_DEC_LAUNCH(8, 2, 1);
  }
  if (d.stages == 4) return MACAQ_DEC_LAUNCH(4, 4, 1);
  if (d.stages == 3) return MACAQ_DEC_LAUNCH(4, 3, 1);
  return MACAQ_DEC_LAUNCH(4, 2, 1);
#undef MACAQ_DEC_LAUNCH
}

// 3 to 32 rows (8, 16 or 32 staged activation rows) and no K split:
// decode_rows_kernel (64-row blocks of 2 waves sharing each activation
// chunk), unless a ring shape is forced (macaq_set_tuning DECODE_WAVES /
// DECODE_STAGES / DECODE_ROWS select decode_gemm_kernel's shapes).  Measured
// on one box against decode_gemm_kernel: gate/up M32 N25600 K5120 20.5 us
// against 22.2 (64-row blocks, each wave staging its own activation over
// half the K range; 5 slots 21.2, deeper rings slower), gate/up M8 16.0-16.2
// against 17.0-17.2 (32-row blocks of 4 waves); down-proj M32 N5120 K25600
// in 3 K parts 21.8-24.5 us (3 to 8 slots) against 20.9, so split layers
// keep decode_gemm_kernel.
constexpr int kRowsWaves = 2;
constexpr int kRowsMaxStages = 4;
static bool use_rows_kernel(int64_t M, int64_t N, int64_t K) {
  return decode_ak(M, false) >= 8 && !tuning(MACAQ_TUNE_DECODE_WAVES) && !tuning(MACAQ_TUNE_DECODE_STAGES) &&
         !tuning(MACAQ_TUNE_DECODE_ROWS) && decode_config(M, N, K, false, 2).ksplit == 1;
}

template <int AK>
static size_t rows_lds_bytes_ak(int stages) {
  switch (stages) {
    case 2: return DecRowsLds<kRowsWaves, 2, AK>::kBytes;
    case 3: return DecRowsLds<kRowsWaves, 3, AK>::kBytes;
    default: return DecRowsLds<kRowsWaves, 4, AK>::kBytes;
  }
}
static size_t rows_lds_bytes(int ak, int stages) {
  if (ak == 8) return rows_lds_bytes_ak<8>(stages);
  return ak == 16 ? rows_lds_bytes_ak<16>(stages) : rows_lds_bytes_ak<32>(stages);
}

// The deepest ring of up to kRowsMaxStages slots within the LDS budget
// (half of the CU's LDS when the blocks outnumber the CUs, so that two fit,
// else all of it).
struct DecRowsConfig {
  int ak, stages;
};
static DecRowsConfig rows_config(int64_t M, int64_t N) {
  DecRowsConfig r;
  r.ak = decode_ak(M, false);
  const int64_t blocks = ceil_div(N, 32 * kRowsWaves);
  const size_t budget = blocks > kDecCUs ? kDecLdsMax / 2 : kDecLdsMax;
  r.stages = kRowsMaxStages;
  while (r.stages > 2 && rows_lds_bytes(r.ak, r.stages) > budget) --r.stages;
  return r;
}

template <int STAGES, int AK>
static hipError_t launch_rows_s(const uint8_t* A, const uint8_t* As, const uint8_t* W, const uint8_t* Ws, int64_t M,
                                int64_t N, int64_t K, void* Y, int mode, hipStream_t stream) {
  using L = DecRowsLds<kRowsWaves, STAGES, AK>;
  static const hipError_t attr = hipFuncSetAttribute((const void*)decode_rows_kernel<kRowsWaves, STAGES, AK>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kDecLdsMax);
  if (attr != hipSuccess) return attr;
  decode_rows_kernel<kRowsWaves, STAGES, AK>
      <<<dim3((unsigned)ceil_div(N, 32 * kRowsWaves)), dim3(64 * kRowsWaves), L::kBytes, stream>>>(A, As, W, Ws, M, N,
                                                                                                 K, Y, mode);
  return hipGetLastError();
}

template <int AK>
static hipError_t launch_rows(const DecRowsConfig& r, const uint8_t* A, const uint8_t* As, const uint8_t* W,
                              const uint8_t* Ws, int64_t M, int64_t N, int64_t K, void* Y, int mode,
                              hipStream_t stream) {
  switch (r.stages) {
    case 2: return launch_rows_s<2, AK>(A, As, W, Ws, M, N, K, Y, mode, stream);
    case 3: return launch_rows_s<3, AK>(A, As, W, Ws, M, N, K, Y, mode, stream);
    default: return launch_rows_s<4, AK>(A, As, W, Ws, M, N, K, Y, mode, stream);
  }
}

hipError_t launch_decode_gemm(const uint8_t* A, const uint8_t* As, const uint8_t* W, const uint8_t* Ws, int64_t M,
                              int64_t N, int64_t K, void* Y, int mode, float* part_ws, hipStream_t stream) {
  if (use_rows_kernel(M, N, K)) {
    const DecRowsConfig r = rows_config(M, N);
    if (rows_lds_bytes(r.ak, r.stages) > kDecLdsMax) return hipErrorInvalidValue;
    if (r.ak == 8) return launch_rows<8>(r, A, As, W, Ws, M, N, K, Y, mode, stream);
    if (r.ak == 16) return launch_rows<16>(r, A, As, W, Ws, M, N, K, Y, mode, stream);
    return launch_rows<32>(r, A, As, W, Ws, M, N, K, Y, mode, stream);
  }
  const DecodeConfig d = decode_config(M, N, K, false, 2);
  switch (d.ak) {
    case 1: return launch_decode_impl<1, DecBf16>(d, A, As, nullptr, nullptr, W, Ws, M, N, K, Y, mode, part_ws, stream);
    case 8: return launch_decode_impl<8, DecBf16>(d, A, As, nullptr, nullptr, W, Ws, M, N, K, Y, mode, part_ws, stream);
    case 16: return launch_decode_impl<16, DecBf16>(d, A, As, nullptr, nullptr, W, Ws, M, N, K, Y, mode, part_ws, stream);
    default: return launch_decode_impl<32, DecBf16>(d, A, As, nullptr, nullptr, W, Ws, M, N, K, Y, mode, part_ws, stream);
  }
}

// Fused variant of a decode-sized layer: -1 the streamed transform (M <= 2),
// 0 the resident one (every block transforms the whole activation into its
// LDS: small layers, where ceil(N / 32) * M * K <= 2^20 and it fits), 1 the
// one-launch layer (the first blocks publish the transformed activation to
// the workspace, the others wait for it).
constexpr int64_t kDecResidentRepeat = int64_t(1) << 20;
static int fused_kind(int64_t M, int64_t N, int64_t K) {
  if (M <= 2) return -1;
  const int64_t repeat = ceil_div(N, kDecRows) * M * K;
  if (repeat <= kDecResidentRepeat) {
    bool fits = true;
    for (int eb : {2, 4})
      if (decode_lds_bytes(decode_config(M, N, K, true, eb), M, K) > kDecLdsMax) fits = false;
    if (fits) return 0;
  }
  return 1;
}

// One-launch workspace: activation codes [M][K/2] and scales [M][K/32] (each
// from a 256-byte boundary), the split's partial sums, then the
// synchronization words (two counts and eight ready-flag lines).
struct PubLayout {
  size_t scales, parts, sync, bytes;
};
static PubLayout pub_layout(int64_t M, int64_t N, int64_t K, const DecodeConfig& d) {
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  PubLayout l;
  l.scales = up((size_t)M * (size_t)K / 2);
  l.parts = l.scales + up((size_t)M * (size_t)K / 32);
  l.sync = l.parts + (d.ksplit > 1 ? up((size_t)d.ksplit * (size_t)M * (size_t)N * sizeof(float)) : 0);
  l.bytes = l.sync + kPubSyncWords * sizeof(unsigned long long);
  return l;
}

// Workspace the decode GEMM (fused: the fused layer) needs for this shape:
// the fp32 partial sums of a K split, and for the one-launch layer the
// staged activation and the counts; 0 when none.
size_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K, bool fused) {
  if (!decode_supported(M, N, K, 1)) return 0;
  if (fused && fused_kind(M, N, K) == 1) return pub_layout(M, N, K, decode_config(M, N, K, false, 2)).bytes;
  const DecodeConfig d = decode_config(M, N, K, fused, 2);
  return d.ksplit > 1 ? (size_t)d.ksplit * (size_t)M * (size_t)N * sizeof(float) : 0;
}

// -------- fused transform + GEMM entry used by macaq_linear

// Whether the fused path serves this shape (any decode-sized dense layer).
bool linear_fused_supported(int64_t M, int64_t N, int64_t K, int64_t E) { return decode_supported(M, N, K, E); }

// Whether the fused path of this shape is the one-launch layer.
bool linear_fused_one_launch(int64_t M, int64_t N, int64_t K) { return fused_kind(M, N, K) == 1; }

template <typename XT>
static hipError_t launch_one_launch(const void* x, const float* s, const uint8_t* B, const uint8_t* Bs, int64_t M,
                                    int64_t N, int64_t K, void* Y, int mode, uint8_t* ws, hipStream_t stream) {
  // the unfused path's ring shapes, with the activation staged in the workspace
  const DecodeConfig d = decode_config(M, N, K, false, 2);
  const PubLayout l = pub_layout(M, N, K, d);
  const int threads = 64 * (d.rt == 2 ? 2 : d.waves);
  const int64_t blocks = ceil_div(N, kDecRows * d.rt) * d.ksplit;
  const int64_t groups = M * (K / 32);
  int64_t pubs = ceil_div(groups, threads);   // one batch of 4 groups per quad of lanes
  if (pubs > kPubMax) pubs = kPubMax;
  if (pubs > blocks) pubs = blocks;
  PubLaunch pl;
  pl.sync = reinterpret_cast<unsigned long long*>(ws + l.sync);
  pl.epoch = next_pub_epoch();
  pl.pubs = (int)pubs;
  // a forced poll limit (tests of the give-up path): value v allows v - 1 polls
  if (const int force = tuning(MACAQ_TUNE_DECODE_POLLS)) pl.max_polls = force - 1;
  const uint8_t* A = ws;
  const uint8_t* As = ws + l.scales;
  float* part_ws = d.ksplit > 1 ? reinterpret_cast<float*>(ws + l.parts) : nullptr;
  switch (d.ak) {
    case 8: return launch_decode_impl<8, XT, true>(d, A, As, x, s, B, Bs, M, N, K, Y, mode, part_ws, stream, pl);
    case 16: return launch_decode_impl<16, XT, true>(d, A, As, x, s, B, Bs, M, N, K, Y, mode, part_ws, stream, pl);
    default: return launch_decode_impl<32, XT, true>(d, A, As, x, s, B, Bs, M, N, K, Y, mode, part_ws, stream, pl);
  }
}

hipError_t launch_linear_fused(const void* x, bool x_f32, const float* s, const uint8_t* B, const uint8_t* Bs,
                               int64_t M, int64_t N, int64_t K, void* Y, int mode, void* ws, hipStream_t stream) {
  const int kind = fused_kind(M, N, K);
  if (kind == 1) {
    if (ws == nullptr) return hipErrorInvalidValue;
    if (x_f32) return launch_one_launch<float>(x, s, B, Bs, M, N, K, Y, mode, static_cast<uint8_t*>(ws), stream);
    return launch_one_launch<DecBf16>(x, s, B, Bs, M, N, K, Y, mode, static_cast<uint8_t*>(ws), stream);
  }
  float* part_ws = static_cast<float*>(ws);
  const DecodeConfig d = decode_config(M, N, K, true, x_f32 ? 4 : 2);
  if (kind < 0) {
    if (x_f32) return launch_decode_impl<-1, float>(d, nullptr, nullptr, x, s, B, Bs, M, N, K, Y, mode, part_ws, stream);
    return launch_decode_impl<-1, DecBf16>(d, nullptr, nullptr, x, s, B, Bs, M, N, K, Y, mode, part_ws, stream);
  }
  if (x_f32) return launch_decode_impl<0, float>(d, nullptr, nullptr, x, s, B, Bs, M, N, K, Y, mode, part_ws, stream);
  return launch_decode_impl<0, DecBf16>(d, nullptr, nullptr, x, s, B, Bs, M, N, K, Y, mode, part_ws, stream);
}

}  // namespace macaq

// Flip-Refinement of prepared MXFP4 weight codes: per weight row, greedy
// single-code moves to the adjacent E2M1 level that lower the
// Hessian-weighted quantization loss, with an incrementally updated
// gradient.
//
// Sources: "MACaQ Enables Streaming W4A4 Quantization with 32.5GB GPU
// Memory", section "Flip-Refinement: optimizing FP4 codes with second-order
// information" (coordinate descent that moves single coordinates to adjacent
// representable values, judged by the loss one half of (x - q)^T H (x - q));
// "华为开源MACaQ:本地量化提速3倍", section "Flip-Refinement:不重算,只改最值得改的
// 4-bit 数值" (starts from round-to-nearest; each round takes only the most
// profitable adjustment of every output row; a row with no improving
// adjustment stops early; the gradient is updated incrementally instead of
// recomputing the matrix product).
//
// Readings: the loss of row n is 1/2 d^T H d, d = x' - dequant(codes), x'
// the fp32 transformed weight row and H the Hessian of the transformed input
// (K x K); scale bytes stay fixed.  A move takes one code to the adjacent
// level of the signed grid -6 .. -0.5, 0, 0.5 .. 6 (times the group scale);
// its gain is delta g_k - delta^2 H_kk / 2 with g = H^T d.  Ties go to the
// lowest coordinate, down before up; a move onto zero keeps the sign bit of
// the code it left.  All of it in fp64 in a fixed order: g_i = sum over j
// ascending of H_ji d_j (product and sum rounded separately: the library is
// built with -ffp-contract=off), then g -= delta H[k, :] per move (delta is a
// signed power of two, so each update is one rounding).
//
// Two kernels per chunk of rows: flip_grad_kernel forms g for the chunk (a
// tiled fp64 product with the transform of W and the dequantization fused
// into its operand loads) into the caller's workspace; flip_rounds_kernel
// then runs the rounds with one block per row, the row's g, codes and scale
// bytes held in registers and H_kk in LDS.
#include "mx_common.h"

namespace macaq {

namespace {

constexpr int kGTile = 128;   // rows x columns of a gradient tile

template <int EB>
__device__ __forceinline__ void load_w_group(const void* base, int64_t elem, float (&t)[32]) {
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

// E2M1 magnitude of index m (0, 0.5, 1, 1.5, 2, 3, 4, 6).
__device__ __forceinline__ float e2m1_mag(uint32_t m) {
  return m < 2u ? 0.5f * (float)m : __uint_as_float((((m >> 1) + 126u) << 23) | ((m & 1u) << 22));
}

// 2^(b - 127) as fp64 (b <= 254).
__device__ __forceinline__ double scale_f64(uint32_t b) { return __longlong_as_double((long long)(b + 896u) << 52); }

__device__ __forceinline__ int code_level(uint32_t c) {
  const int m = (int)(c & 7u);
  return (c & 8u) ? -m : m;
}

__device__ __forceinline__ uint32_t level_to_code(int L, uint32_t old_code) {
  if (L > 0) return (uint32_t)L;
  if (L < 0) return 8u | (uint32_t)(-L);
  return old_code & 8u;
}

}  // namespace

// ---------------------------------------------------------------------------
// g[n][i] = sum_j H[j][i] d[n][j] for a 128x128 tile (rows n of the chunk,
// columns i).  Per K-step of one 32-wide group: threads 0..127 each build one
// row's d for the group (widen W, times r = 1/s, butterfly, times C, minus
// the dequantized code) into LDS as fp64 [32][128]; all threads stage the
// matching 32 rows of H (fp32 -> fp64) as [32][128]; every thread then
// accumulates its 8x8 outputs (rows ty + 16a, columns tx + 16c) over the 32
// values in order, a multiply then an add (fused when that is exact).
template <int EB>
__global__ __launch_bounds__(256) void flip_grad_kernel(const void* __restrict__ w, const float* __restrict__ s,
                                                        const float* __restrict__ H, const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ scales, int64_t row0,
                                                        int64_t rows, int64_t N, int64_t K, double* __restrict__ G) {
  // expert blockIdx.z: its rows row0 .. row0 + rows - 1 of N, its gradient
  // rows at G + e * rows * K
  {
    const int64_t e = blockIdx.z;
    w = static_cast<const uint8_t*>(w) + e * N * K * EB;
    s += e * K;
    H += e * K * K;
    codes += e * N * (K / 2);
    scales += e * N * (K / 32);
    G += e * rows * K;
  }
  __shared__ double da[32][kGTile];
  __shared__ double hb[32][kGTile];
  __shared__ float rs[32];
  const int tid = threadIdx.x;
  const int64_t n0 = (int64_t)blockIdx.x * kGTile;   // within the chunk
  const int64_t i0 = (int64_t)blockIdx.y * kGTile;
  const int ty = tid >> 4, tx = tid & 15;
  const int64_t my_row = n0 + tid;                    // transform task (tid < 128)
  const bool tasker = tid < kGTile && my_row < rows;

  double acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[a][c] = 0.0;

  const int64_t G32 = K / 32;
  for (int64_t g = 0; g < G32; ++g) {
    const int64_t col = 32 * g;
    if (tid < 32) rs[tid] = 1.0f / s[col + tid];
    __syncthreads();
    int exact = 1;   // every d of this step has at most 29 significant bits
    if (tid < kGTile) {
      if (tasker) {
        const int64_t row = row0 + my_row;
        float t[32];
        load_w_group<EB>(w, row * K + col, t);
#pragma unroll
        for (int i = 0; i < 32; ++i) t[i] = t[i] * rs[i];
#pragma unroll
        for (int hh = 1; hh < 32; hh <<= 1) {
#pragma unroll
          for (int i = 0; i < 32; ++i) {
            if ((i & hh) == 0) {
              const float a = t[i], b = t[i + hh];
              t[i] = a + b;
              t[i + hh] = a - b;
            }
          }
        }
        const float cn = hadamard_norm();
        const uint4 cq = reinterpret_cast<const uint4*>(codes + row * (K / 2) + 16 * g)[0];
        const uint32_t cw[4] = {cq.x, cq.y, cq.z, cq.w};
        const double sc = scale_f64(scales[row * G32 + g]);
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const uint32_t c = (cw[i >> 3] >> (4 * (i & 7))) & 0xFu;
          const float m = e2m1_mag(c & 7u);
          const double deq = (double)((c & 8u) ? -m : m) * sc;
          const double d = (double)(t[i] * cn) - deq;
          exact &= (__double2loint(d) & 0xFFFFFF) == 0;
          da[i][tid] = d;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) da[i][tid] = 0.0;
      }
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int idx = tid + 256 * q;          // 32 x 128 entries
      hb[idx >> 7][idx & 127] = (double)H[(col + (idx >> 7)) * K + i0 + (idx & 127)];
    }
    // A d with at most 29 significant bits times an fp32 H entry (24 bits)
    // is exact in fp64, so a fused multiply-add rounds exactly like the
    // multiply-then-add of the stated order; round-to-nearest start codes
    // always qualify (d is a multiple of 2^(e-25) below 2^(e+3)).  Any other
    // step takes the separate multiply and add.
    if (__syncthreads_and(exact)) {
#pragma unroll 4
      for (int jj = 0; jj < 32; ++jj) {
        double av[8], bv[8];
#pragma unroll
        for (int a = 0; a < 8; ++a) av[a] = da[jj][ty + 16 * a];
#pragma unroll
        for (int c = 0; c < 8; ++c) bv[c] = hb[jj][tx + 16 * c];
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[a][c] = __builtin_fma(av[a], bv[c], acc[a][c]);
      }
    } else {
#pragma unroll 4
      for (int jj = 0; jj < 32; ++jj) {
        double av[8], bv[8];
#pragma unroll
        for (int a = 0; a < 8; ++a) av[a] = da[jj][ty + 16 * a];
#pragma unroll
        for (int c = 0; c < 8; ++c) bv[c] = hb[jj][tx + 16 * c];
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[a][c] = acc[a][c] + av[a] * bv[c];
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int64_t n = n0 + ty + 16 * a;
    if (n < rows) {
#pragma unroll
      for (int c = 0; c < 8; ++c) G[n * K + i0 + tx + 16 * c] = acc[a][c];
    }
  }
}

// ---------------------------------------------------------------------------
// Rounds: one block of NT threads per weight row; thread t owns coordinates
// k = t + NT*m (m < KPT).  Per round every thread scans its coordinates'
// down and up moves, the block reduces to the best (gain, candidate = 2k +
// up), and when that gain is positive every thread updates its g entries
// with row k of H while the owner of k moves its code.
struct Best {
  double gain;
  int cand;
};

__device__ __forceinline__ bool better(double g1, int c1, double g2, int c2) {
  return g1 > g2 || (g1 == g2 && c1 < c2);
}

// DPP lane moves (quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E; row_ror:4 =
// 0x124, row_ror:8 = 0x128) and lane reads, for the in-wave reductions.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const long long u = __double_as_longlong(v);
  const int lo = dpp_i<CTRL>((int)u), hi = dpp_i<CTRL>((int)(u >> 32));
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ double readlane_d(double v, int l) {
  const long long u = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)u, l), hi = __builtin_amdgcn_readlane((int)(u >> 32), l);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// Wave-uniform maximum of v (every lane gets it).
__device__ __forceinline__ double wave_max_d(double v) {
  v = fmax(v, dpp_d<0xB1>(v));
  v = fmax(v, dpp_d<0x4E>(v));
  v = fmax(v, dpp_d<0x124>(v));
  v = fmax(v, dpp_d<0x128>(v));   // every lane holds its 16-lane row's maximum
  return fmax(fmax(readlane_d(v, 0), readlane_d(v, 16)), fmax(readlane_d(v, 32), readlane_d(v, 48)));
}
__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, dpp_i<0xB1>(v));
  v = min(v, dpp_i<0x4E>(v));
  v = min(v, dpp_i<0x124>(v));
  v = min(v, dpp_i<0x128>(v));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Exponent (-1, 0 or 1) of the magnitude step from level L to L + 1 (0.5
// below 2, 1 from 2 to 4, 2 from 4 to 6).
__device__ __forceinline__ int step_exp(int L) {
  const int m = L >= 0 ? L : -L - 1;
  return (m >= 4) + (m >= 6) - 1;
}

// Waves per SIMD the register budget aims at: more resident rows hide more of
// each round's latency (about 6 VGPRs per coordinate plus 25).
template <int NT, int KPT>
constexpr int flip_waves() { return NT == 1024 || KPT <= 20 ? 4 : (KPT <= 28 ? 3 : 2); }

// A candidate move is keyed (k << 12) | (up << 11) | (p + 1024): k and the
// direction give the tie order (k ascending, down before up); p is the
// exponent of |delta| = 2^p (delta = +-step * 2^(b - 127), a power of two),
// carried so that every thread can rebuild delta from the winning key.  Every
// product with delta is then an exact ldexp: delta g_k = +-ldexp(g_k, p),
// delta^2 H_kk / 2 = ldexp(H_kk, 2p - 1), delta H[k, i] = +-ldexp(H[k, i], p).
//
// Per coordinate one word holds what the scan needs and what changes only
// when that coordinate moves: the code (bits 0-3), the down key's low bits
// p + 1024 (bits 4-15), the up key's low bits 2048 | (p + 1024) (bits
// 16-27), and whether a down / up move exists (bits 28 / 29; both clear past
// K).  A move that does not exist (past +-6, or past K) carries p = 700
// instead: with H_kk > 0, ldexp(H_kk, 1399) is +inf and its gain is -inf or
// NaN, which never compares greater, so the one-direction scan needs no test.
constexpr uint32_t kCanDown = 1u << 28, kCanUp = 1u << 29;
constexpr int kNoMove = 700;

__device__ __forceinline__ uint32_t coord_word(uint32_t code, int e0) {
  const int L = code_level(code);
  const int pd = L > -7 ? step_exp(L - 1) + e0 : kNoMove, pu = L < 7 ? step_exp(L) + e0 : kNoMove;
  return code | ((uint32_t)(pd + 1024) << 4) | ((uint32_t)(2048 | (pu + 1024)) << 16) |
         (L > -7 ? kCanDown : 0u) | (L < 7 ? kCanUp : 0u);
}
constexpr uint32_t kPastK = ((uint32_t)(kNoMove + 1024) << 4) | ((uint32_t)(2048 | (kNoMove + 1024)) << 16);

// Scale exponent b - 127 of a coordinate, from whichever of its moves exists.
__device__ __forceinline__ int coord_e0(uint32_t in) {
  const int L = code_level(in & 0xFu);
  return L > -7 ? (int)((in >> 4) & 2047u) - 1024 - step_exp(L - 1) : (int)((in >> 16) & 2047u) - 1024 - step_exp(L);
}
template <int NT, int KPT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(flip_waves<NT, KPT>())))
void flip_rounds_kernel(const float* __restrict__ H, int64_t row0, int64_t rows, int64_t N, int64_t K,
                        int max_rounds, const double* __restrict__ G, uint8_t* __restrict__ codes,
                        const uint8_t* __restrict__ scales, int32_t* __restrict__ moves_out) {
  {  // expert blockIdx.y, laid out as in flip_grad_kernel
    const int64_t e = blockIdx.y;
    H += e * K * K;
    G += e * rows * K;
    codes += e * N * (K / 2);
    scales += e * N * (K / 32);
    if (moves_out) moves_out += e * N;
  }
  constexpr int NW = NT / 64;
  __shared__ Best red[2][NW];
  __shared__ float diag[KPT][NT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t rl = blockIdx.x;               // row within the chunk
  const int64_t row = row0 + rl;
  const int64_t G32 = K / 32;
  const int Ki = (int)K;

  double g[KPT];
  uint32_t info[KPT];   // coord_word of each coordinate
#pragma unroll
  for (int m = 0; m < KPT; ++m) {
    const int64_t k = tid + (int64_t)NT * m;
    if (k < K) {
      g[m] = G[rl * K + k];
      diag[m][tid] = H[k * K + k];
      const uint32_t byte = codes[row * (K / 2) + (k >> 1)];
      info[m] = coord_word((byte >> (4 * (k & 1))) & 0xFu, (int)scales[row * G32 + (k >> 5)] - 127);
    } else {
      g[m] = 0.0;
      diag[m][tid] = 1.0f;   // positive, so that the no-move exponent gives -inf
      info[m] = kPastK;
    }
  }

  // With H_kk >= 0 a move can gain only in the direction of g_k (the other
  // gain is -|delta g_k| - delta^2 H_kk / 2 <= 0), and only positive gains
  // can win, so one candidate per coordinate suffices; the no-move exponent
  // needs H_kk > 0.  A row with some H_kk <= 0 scans both directions with
  // explicit tests.
  int neg_diag = 0;
#pragma unroll
  for (int m = 0; m < KPT; ++m) neg_diag |= !(diag[m][tid] > 0.0f);
  const bool both = __syncthreads_or(neg_diag) != 0;

  const double ninf = -__builtin_inf();
  int moves = 0;
  for (int r = 0; r < max_rounds; ++r) {
    // keep per-coordinate values derived from info out of the registers
    // between rounds: they are recomputed each round
#pragma unroll
    for (int m = 0; m < KPT; ++m) asm volatile("" : "+v"(info[m]));
    // likewise the coordinate indices (tid + NT * m): one register, rebuilt
    int t_r = tid;
    asm volatile("" : "+v"(t_r));
    // scan, without branches: candidates in the order k ascending (down
    // before up when both are scanned); a later candidate replaces the best
    // only if strictly better
    double bg = ninf;
    int bc = 0x7FFFFFFF;
    if (!both) {
#pragma unroll
      for (int m = 0; m < KPT; ++m) {
        const uint32_t in = info[m];
        const int f = (int)((in >> (g[m] > 0.0 ? 16 : 4)) & 4095u);   // the move toward g's sign
        const int p = (f & 2047) - 1024;
        const double hk = (double)diag[m][tid];
        // delta g_k = |delta| |g_k| in the chosen direction
        const double gn = ldexp(fabs(g[m]), p) - ldexp(hk, 2 * p - 1);
        const bool t = gn > bg;
        bg = t ? gn : bg; bc = t ? (((t_r + NT * m) << 12) | f) : bc;
      }
    } else {
#pragma unroll
      for (int m = 0; m < KPT; ++m) {
        const uint32_t in = info[m];
        const int fd = (int)((in >> 4) & 4095u), fu = (int)((in >> 16) & 4095u);
        const int pd = fd - 1024, pu = (fu & 2047) - 1024;
        const double hk = (double)diag[m][tid];
        double gd = -ldexp(g[m], pd) - ldexp(hk, 2 * pd - 1);
        double gu = ldexp(g[m], pu) - ldexp(hk, 2 * pu - 1);
        gd = (in & kCanDown) ? gd : ninf;
        gu = (in & kCanUp) ? gu : ninf;
        const int kk = (t_r + NT * m) << 12;
        const bool td = gd > bg;
        bg = td ? gd : bg; bc = td ? (kk | fd) : bc;
        const bool tu = gu > bg;
        bg = tu ? gu : bg; bc = tu ? (kk | fu) : bc;
      }
    }
    // wave: the largest gain, then the lowest key holding it
    const double wg = wave_max_d(bg);
    const int wc = wave_min_i(bg == wg ? bc : 0x7FFFFFFF);
    if (lane == 0) red[r & 1][wave] = Best{wg, wc};
    __syncthreads();
    bg = red[r & 1][0].gain; bc = red[r & 1][0].cand;
#pragma unroll
    for (int v = 1; v < NW; ++v) {
      const Best o = red[r & 1][v];
      if (better(o.gain, o.cand, bg, bc)) { bg = o.gain; bc = o.cand; }
    }
    if (!(bg > 0.0)) break;   // uniform: every thread holds the same best
    const int kb = bc >> 12;
    const bool up = (bc >> 11) & 1;
    const int p = (bc & 2047) - 1024;
    // g - delta H[k, :]: delta H[k, i] = -+2^p H[k, i] is exact, so one fused
    // multiply-add rounds the difference once, as the separate exact product
    // and subtraction do
    const double step = up ? -ldexp(1.0, p) : ldexp(1.0, p);
    // KPT is ceil(K / NT) rounded up to a multiple of 4, so only the last 4
    // slots can reach past K: the others take a uniform base per slot and one
    // 32-bit lane offset, those 4 clamp (entries past K are never read back)
    const float* hrow = H + (int64_t)kb * K;
    const char* hb = reinterpret_cast<const char*>(hrow);
    const unsigned off = (unsigned)t_r * 4u;
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
      float hv;
      if (m + 4 < KPT) {
        hv = *reinterpret_cast<const float*>(hb + (size_t)NT * 4 * m + off);
      } else {
        const int k = t_r + NT * m;
        hv = hrow[k < Ki ? k : Ki - 1];
      }
      g[m] = __builtin_fma((double)hv, step, g[m]);
    }
    const int mo = kb / NT;                                              // the owner's coordinate slot
    if (kb - mo * NT == t_r) {
#pragma unroll
      for (int m = 0; m < KPT; ++m) {
        if (m == mo) {
          const uint32_t old = info[m] & 0xFu;
          info[m] = coord_word(level_to_code(code_level(old) + (up ? 1 : -1), old), coord_e0(info[m]));
        }
      }
    }
    ++moves;
  }

  // codes back: coordinates k and k+1 sit in neighbouring lanes
#pragma unroll
  for (int m = 0; m < KPT; ++m) {
    const int64_t k = tid + (int64_t)NT * m;
    const uint32_t mine = info[m] & 0xFu;
    const uint32_t other = (uint32_t)__shfl_xor((int)mine, 1);
    if (k < K && (k & 1) == 0) codes[row * (K / 2) + (k >> 1)] = (uint8_t)(mine | (other << 4));
  }
  if (moves_out && tid == 0) moves_out[row] = moves;
}

// ---------------------------------------------------------------------------

// Both launches cover rows row0 .. row0 + rows - 1 of each of E experts (N
// rows each); G holds E * rows * K doubles.
hipError_t launch_flip_grad(const void* w, bool w_f32, const float* s, const float* H, const uint8_t* codes,
                            const uint8_t* scales, int E, int64_t row0, int64_t rows, int64_t N, int64_t K,
                            double* G, hipStream_t stream) {
  const dim3 grid((unsigned)ceil_div(rows, kGTile), (unsigned)(K / kGTile), (unsigned)E);
  if (w_f32)
    hipLaunchKernelGGL(flip_grad_kernel<4>, grid, dim3(256), 0, stream, w, s, H, codes, scales, row0, rows, N, K, G);
  else
    hipLaunchKernelGGL(flip_grad_kernel<2>, grid, dim3(256), 0, stream, w, s, H, codes, scales, row0, rows, N, K, G);
  return hipGetLastError();
}

namespace {
struct RoundsArgs {
  const float* H; int E; int64_t row0, rows, N, K; int max_rounds; const double* G;
  uint8_t* codes; const uint8_t* scales; int32_t* moves; hipStream_t stream;
};

template <int NT, int KPT>
void launch_rounds_t(const RoundsArgs& a) {
  hipLaunchKernelGGL((flip_rounds_kernel<NT, KPT>), dim3((unsigned)a.rows, (unsigned)a.E), dim3(NT), 0, a.stream,
                     a.H, a.row0, a.rows, a.N, a.K, a.max_rounds, a.G, a.codes, a.scales, a.moves);
}

template <int NT>
bool launch_rounds_nt(int kpt, const RoundsArgs& a) {
  switch (kpt) {
    case 4: launch_rounds_t<NT, 4>(a); return true;
    case 8: launch_rounds_t<NT, 8>(a); return true;
    case 12: launch_rounds_t<NT, 12>(a); return true;
    case 16: launch_rounds_t<NT, 16>(a); return true;
    case 20: launch_rounds_t<NT, 20>(a); return true;
    case 24: launch_rounds_t<NT, 24>(a); return true;
    case 28: launch_rounds_t<NT, 28>(a); return true;
    case 32: launch_rounds_t<NT, 32>(a); return true;
    default: return false;
  }
}
}  // namespace

// Rows per block thread layout: 256 threads up to K = 8192, 1024 threads up
// to K = 32768; each thread holds ceil(K / threads) coordinates (rounded up
// to a multiple of 4).
hipError_t launch_flip_rounds(const float* H, int E, int64_t row0, int64_t rows, int64_t N, int64_t K,
                              int max_rounds, const double* G, uint8_t* codes, const uint8_t* scales, int32_t* moves,
                              hipStream_t stream) {
  const int nt = K <= 8192 ? 256 : 1024;
  const int kpt = (int)((ceil_div(K, nt) + 3) / 4 * 4);
  const RoundsArgs a{H, E, row0, rows, N, K, max_rounds, G, codes, scales, moves, stream};
  const bool ok = nt == 256 ? launch_rounds_nt<256>(kpt, a) : launch_rounds_nt<1024>(kpt, a);
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace macaq

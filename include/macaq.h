/*
 * macaq.h — C ABI of the MXFP4 W4A4 linear layer with an online per-channel
 * scale and a 32-element block Hadamard transform, for AMD Instinct MI355X
 * (gfx950).
 *
 * What the layer computes (sources cited by page title and section):
 *
 *   y = x W^T                          "MACaQ Enables Streaming W4A4
 *                                       Quantization with 32.5GB GPU Memory",
 *                                       section "Quantization mechanism"
 *   y = (x diag(s) H)(W diag(1/s) H)^T  same section (its printed formula is
 *                                       garbled; this is the form that keeps
 *                                       y = x W^T), and the abstract of "MACaQ:
 *                                       Fast, Model Agnostic Calibrated
 *                                       Quantization for Low-Precision Weights
 *                                       and Activations": scale and block
 *                                       Hadamard online on the activations,
 *                                       inverses absorbed into the weights.
 *   H = block-diagonal of K/32 normalized Sylvester 32x32 Hadamards, the
 *       block equal to the MXFP4 scale group ("华为开源MACaQ:本地量化提速3倍",
 *       section "MACaQ 真正解决的是跨层耦合").
 *   Both operands are OCP MXFP4: 32-element groups, one E8M0 scale byte per
 *       group, E2M1 elements (same article, section "量化不是单纯把模型“压小”").
 *
 * Exact arithmetic contract (shared by every entry point that quantizes):
 *   per 32-element group along K, t = fp32(x) * s (fp32 multiply), then the
 *   unnormalized butterfly with stages h = 1,2,4,8,16 (lower index a+b, upper
 *   index a-b, fp32 round-to-nearest-even, no fused multiply-add), then
 *   x' = t * C with C = fp32 0x3E3504F3 (1/sqrt(32)).
 *   scale byte b = max(exponent_field(max|x'|) - 2, 0); element code =
 *   sign<<3 | RNE(|x'| * 2^(127-b)) onto {0,.5,1,1.5,2,3,4,6} (ties to even
 *   mantissa, saturating at 6, sign kept for zero).
 *   Packed codes: two per byte, even K index in the low nibble.
 *   Codes and scale bytes are bit-exact to that contract.
 *
 * Layouts (row-major, no padding):
 *   activations x      [M][K]    bf16 or fp32, rows sorted by expert
 *   per-channel s      [E][K]    fp32, finite and > 0
 *   expert_offsets     [E+1]     int32, offsets[0] = 0, non-decreasing,
 *                                offsets[E] = M (may be NULL when E == 1)
 *   weights W          [E][N][K] bf16 or fp32
 *   weight codes       [E][N][K/2]  uint8
 *   weight scales      [E][N][K/32] uint8
 *   activation codes   [M][K/2]     uint8
 *   activation scales  [M][K/32]    uint8
 *   output y           [M][N]    fp32
 *
 * Ownership and execution: every pointer argument except those documented
 * as host pointers is a device pointer owned by the caller; the library
 * never allocates device memory and keeps no per-call state.  Every call
 * enqueues work on `stream` (a hipStream_t passed as void*, NULL = the
 * default stream) and returns without synchronizing.  Outputs must not alias
 * inputs.  Arguments are validated on the host before anything is launched;
 * device-resident values (s > 0, sorted offsets, finite inputs) are
 * preconditions that are not checked.
 *
 * Graph capture: outside the debug mode below, a call launches kernels
 * only (no allocation, no memset, no synchronization), so it may be
 * captured into a HIP graph and replayed.  Make one call of each kind
 * before capturing: the first call sets a kernel attribute once.
 *
 * Debug mode: with the environment variable MACAQ_CHECK=1 (read at every
 * call), each entry point first waits for `stream` and checks the
 * device-resident preconditions it can read back cheaply: expert offsets
 * start at 0, never decrease and end at the row count; every factor of s is
 * finite and > 0 (MACAQ_ERR_INVALID_ARG otherwise, before any launch).  After
 * launching, it waits for `stream` again, so that a fault in one of its
 * kernels is reported as MACAQ_ERR_HIP by that call.  This is the only mode
 * in which the library synchronizes.
 *
 * Errors: a negative macaq_status.  macaq_last_error() returns a
 * thread-local description of the most recent failure on that thread.
 */
#ifndef MACAQ_H
#define MACAQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MACAQ_OK = 0,
  MACAQ_ERR_INVALID_ARG = -1, /* null pointer, bad size, misaligned pointer */
  MACAQ_ERR_UNSUPPORTED = -2, /* valid but not handled (dtype, K not a multiple of 128 for a GEMM) */
  MACAQ_ERR_NO_DEVICE = -3,   /* no HIP device visible */
  MACAQ_ERR_HIP = -4,         /* a HIP runtime call or a launch failed */
  MACAQ_ERR_WORKSPACE = -5    /* workspace missing or too small */
} macaq_status;

typedef enum { MACAQ_BF16 = 0, MACAQ_F32 = 1 } macaq_dtype;

/* flags of macaq_linear: which path computes the layer */
enum {
  MACAQ_PATH_AUTO = 0,    /* choose by M */
  MACAQ_PATH_FUSED = 1,   /* decode path: transform + quantization inside the GEMM kernel */
  MACAQ_PATH_UNFUSED = 2  /* macaq_quant_act into the workspace, then macaq_gemm */
};

/* epilogue of macaq_gemm_ex / macaq_linear_ex */
enum {
  MACAQ_EPI_NONE = 0,   /* y[m][n] = the layer output */
  MACAQ_EPI_SWIGLU = 1  /* weight rows are (gate, up) pairs: y[m][j] = silu(out[m][2j]) * out[m][2j+1] */
};

/* Layout bit: w_codes / w_scales are in the tiled layout made by
 * macaq_tile_weights.  OR'ed into the flags of macaq_linear / macaq_linear_ex
 * / macaq_linear_path / macaq_linear_workspace_bytes and into the epilogue
 * argument of macaq_gemm_ex. */
#define MACAQ_W_TILED 0x100u

/* Layout bit: a_codes / a_scales of macaq_gemm_ex are in the tiled,
 * expert-padded layout that macaq_quant_act_tiled writes (the layout of
 * macaq_tile_weights applied to the activation rows).  OR'ed into the
 * epilogue argument of macaq_gemm_ex together with MACAQ_W_TILED. */
#define MACAQ_A_TILED 0x200u

/* Knobs of macaq_set_tuning.  Value 0 of every knob is the library's own
 * choice; other values force one kernel variant:
 *   MACAQ_TUNE_GEMM_TILE          prefill / grouped GEMM block tile:
 *                                 1 = 256x256, 2 = 256x128, 3 = 128x128
 *   MACAQ_TUNE_GEMM_GROUP_M       tile rows per XCD group of the GEMM (1..64)
 *   MACAQ_TUNE_ACT_ROWS_PER_WAVE  row blocks per wave of the activation
 *                                 kernel (1..64)
 *   MACAQ_TUNE_ACT_SHARED_S       activation kernel's per-channel factors:
 *                                 1 = per lane in registers, 2 = staged per
 *                                 block in LDS
 *   MACAQ_TUNE_DECODE_WAVES       waves per decode block (4 or 8; 32-row blocks)
 *   MACAQ_TUNE_DECODE_STAGES      ring slots per decode wave (2..4; 32-row blocks)
 *   MACAQ_TUNE_DECODE_ROWS        weight rows per decode block (32 or 64)
 *   MACAQ_TUNE_ACT_SEGMENT        groups per row segment of a wave of the
 *                                 activation kernel (16, 32 or 64)
 *   MACAQ_TUNE_DECODE_SPLIT       K split of the decode GEMM: the number of
 *                                 blocks per row tile (1..16; 1 = no split)
 *   MACAQ_TUNE_DECODE_POLLS       polls of the one-launch fused layer's wait
 *                                 for the published activation before it
 *                                 gives up: v - 1 (1..64; 1 = give up at
 *                                 once).  For tests of the give-up path,
 *                                 which writes NaN to every output. */
enum {
  MACAQ_TUNE_GEMM_TILE = 0,
  MACAQ_TUNE_GEMM_GROUP_M = 1,
  MACAQ_TUNE_ACT_ROWS_PER_WAVE = 2,
  MACAQ_TUNE_ACT_SHARED_S = 3,
  MACAQ_TUNE_DECODE_WAVES = 4,
  MACAQ_TUNE_DECODE_STAGES = 5,
  MACAQ_TUNE_DECODE_ROWS = 6,
  MACAQ_TUNE_ACT_SEGMENT = 7,
  MACAQ_TUNE_DECODE_SPLIT = 8,
  MACAQ_TUNE_DECODE_POLLS = 9,
  MACAQ_TUNE_COUNT = 10
};

/* Library version as major*10000 + minor*100 + patch. */
int macaq_version(void);

/*
 * Process-wide override of one kernel choice, for tests and tuning sweeps
 * (the library reads no environment variable for these).  Every later call
 * on every thread uses it until it is set back to 0.  Codes and scale bytes
 * do not depend on any knob; the GEMM's fp32 summation order, and so the
 * last bits of y, can (tile shape, decode waves).  A forced choice that
 * cannot serve a shape is replaced by the automatic one.
 * Returns the previous value of the knob, or MACAQ_ERR_INVALID_ARG for an
 * unknown knob or a value outside the range listed above.
 */
int macaq_set_tuning(int knob, int value);

/* Static description of a status code (never NULL). */
const char* macaq_status_string(int status);

/* Thread-local description of the last failure on the calling thread ("" if none). */
const char* macaq_last_error(void);

/*
 * Offline weight preparation W' = quant(W diag(1/s) H) ("Quantization
 * mechanism": the transformed weight is prepared offline; abstract: the
 * inverse transforms are absorbed into the weights).
 * The per-channel factor is r = 1.0f / s[e][k] (IEEE fp32 division); the
 * rest follows the arithmetic contract above.
 *   w        [E][N][K] in w_dtype;  s [E][K] fp32
 *   w_codes  [E][N][K/2] out;       w_scales [E][N][K/32] out
 * Requires E >= 1, N >= 1, K >= 32, K % 32 == 0, w and w_codes 16-byte
 * aligned.
 */
int macaq_prepare_weights(const void* w, macaq_dtype w_dtype, const float* s,
                          int64_t E, int64_t N, int64_t K,
                          uint8_t* w_codes, uint8_t* w_scales, void* stream);

/*
 * Hessian of the layer input in the transformed basis, from calibration rows
 * ("MACaQ Enables Streaming W4A4 Quantization ...", section
 * "Flip-Refinement: optimizing FP4 codes with second-order information": the
 * quantization loss of a vector v is one half of v^T H v, H the Hessian of the
 * layer input; "华为开源MACaQ:本地量化提速3倍", section "Flip-Refinement:不重算,
 * 只改最值得改的 4-bit 数值": H comes from calibration statistics).
 *   h[e] = X'_e^T X'_e, X'_e the calibration rows of expert e after the online
 *   transform (the fp32 x' that macaq_quant_act quantizes, with s[e]).  The
 *   factor 2 of the second derivative and any division by the row count are
 *   left out.  Accumulated in fp64, stored as fp32 (round to nearest even);
 *   h[e] is exactly symmetric; an expert without rows gets h[e] = 0.
 *   x [T][K] in x_dtype, rows sorted by expert; s [E][K] fp32;
 *   expert_offsets [E+1] device int32 (NULL allowed when E == 1);
 *   h [E][K][K] fp32 out (every entry written).
 * Requires E >= 1, T >= 0, K % 128 == 0 (MACAQ_ERR_UNSUPPORTED otherwise),
 * x and s 16-byte aligned, h 4-byte aligned.  Work: 2*T*K*K flops (fp64).
 */
int macaq_hessian(const void* x, macaq_dtype x_dtype, const float* s, const int32_t* expert_offsets,
                  int64_t E, int64_t T, int64_t K, float* h, void* stream);

/*
 * Weight preparation with the Hessian exponent search ("华为开源MACaQ:本地量化
 * 提速3倍", section "Flip-Refinement:不重算,只改最值得改的 4-bit 数值": the
 * ablation's first step above round-to-nearest).  x' = W diag(1/s) H as in
 * macaq_prepare_weights; for each 32-element group the scale byte is b0 (the
 * plain rule) or b0 + 1, whichever gives the smaller q = d^T H_gg d, with
 * d = x' - dequant(codes at that byte) exact in fp64 and H_gg the group's
 * diagonal 32x32 block of h[e]; q is summed in fp64 with u_i = sum over
 * j = 0..31 of H_ij d_j, then q = sum over i = 0..31 of d_i u_i, each product
 * and sum rounded on its own; a tie keeps b0.  With h = 0 the result equals
 * macaq_prepare_weights.
 *   w [E][N][K] in w_dtype; s [E][K] fp32; h [E][K][K] fp32 (only the
 *   diagonal blocks are read), e.g. from macaq_hessian;
 *   w_codes [E][N][K/2] out; w_scales [E][N][K/32] out.
 * Requires E >= 1, N >= 1, K % 32 == 0, w, s and w_codes 16-byte aligned,
 * h 4-byte aligned.
 */
int macaq_prepare_weights_hessian(const void* w, macaq_dtype w_dtype, const float* s, const float* h,
                                  int64_t E, int64_t N, int64_t K,
                                  uint8_t* w_codes, uint8_t* w_scales, void* stream);

/*
 * Flip-Refinement of prepared weight codes ("MACaQ Enables Streaming W4A4
 * Quantization ...", section "Flip-Refinement: optimizing FP4 codes with
 * second-order information": coordinate descent moving single codes to
 * adjacent representable values under the loss one half of
 * (x - q)^T H (x - q); "华为开源MACaQ:本地量化提速3倍", section
 * "Flip-Refinement:不重算,只改最值得改的 4-bit 数值": start from round-to-nearest,
 * one best adjustment per output row and round, a row with no improving
 * adjustment stops, the gradient is updated incrementally).
 *   Per weight row: x' = W diag(1/s) H (as macaq_prepare_weights),
 *   d = x' - dequant(codes), g_i = sum over j = 0..K-1 of h[j][i] d_j (fp64,
 *   product and sum rounded separately).  Each round the row's candidate
 *   moves (one code to the adjacent level of the signed E2M1 grid, scale
 *   bytes fixed) are scored gain = delta g_k - delta^2 h[k][k] / 2 (fp64);
 *   the largest gain wins, ties to the lowest k, then to the downward move;
 *   if it is > 0 the code moves (a move onto zero keeps the sign bit of the
 *   code it left) and g -= delta h[k][:]; else the row stops.  At most
 *   max_rounds moves per row.
 *   w [E][N][K] in w_dtype; s [E][K] fp32; h [E][K][K] fp32 (e.g. from
 *   macaq_hessian); w_codes [E][N][K/2] in/out (normally the output of
 *   macaq_prepare_weights or macaq_prepare_weights_hessian); w_scales
 *   [E][N][K/32] in; moves [E][N] int32 out (moves made per row; may be
 *   NULL); workspace: device memory of at least
 *   macaq_flip_refine_workspace_bytes(128, K) bytes, 256-byte aligned, that
 *   holds the fp64 gradient: with room for E * N rows all experts run in one
 *   pair of launches, otherwise expert by expert in chunks of as many rows
 *   as fit.
 * Requires E >= 1, N >= 1, K % 128 == 0, K <= 32640, max_rounds >= 0;
 * w, s and w_codes 16-byte aligned, h 4-byte aligned.  Calls that share a
 * workspace must not overlap in time.
 */
int macaq_flip_refine(const void* w, macaq_dtype w_dtype, const float* s, const float* h,
                      int64_t E, int64_t N, int64_t K, int32_t max_rounds,
                      uint8_t* w_codes, const uint8_t* w_scales, int32_t* moves,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of macaq_flip_refine to process `rows` rows per chunk
 * (rows rounded up to 128): rows * K * 8. */
size_t macaq_flip_refine_workspace_bytes(int64_t rows, int64_t K);

/*
 * Online activation transform and MXFP4 quantization x' = (x diag(s_e) H),
 * codes/scales of x' ("Quantization mechanism": at inference the activation
 * is scaled and transformed before the FP4 matrix multiplication).
 *   x [M][K] in x_dtype, rows sorted by expert; s [E][K] fp32;
 *   expert_offsets [E+1] device int32 (NULL allowed when E == 1)
 *   a_codes [M][K/2] out; a_scales [M][K/32] out
 * Requires E >= 1, M >= 0, K >= 32, K % 32 == 0, x and a_codes 16-byte
 * aligned.  M == 0 is a no-op.
 */
int macaq_quant_act(const void* x, macaq_dtype x_dtype, const float* s,
                    const int32_t* expert_offsets, int64_t E, int64_t M, int64_t K,
                    uint8_t* a_codes, uint8_t* a_scales, void* stream);

/*
 * macaq_quant_act with the codes and scales in the tiled layout that the
 * prefill and grouped GEMMs copy with contiguous reads: per 32-row block b
 * and 128-wide K-tile t, 2048 bytes of codes at (b * K/128 + t) * 2048, row
 * r of the block at 64 r with its 16-byte chunk c (32 values) at position
 * c ^ ((r >> 2) & 3), and 128 bytes of scales at (b * K/128 + t) * 128, row
 * r's 4 bytes at 4 r.  Rows are padded per expert: expert e's rows start at
 * padded row P_e = sum over e' < e of ceil(rows_e' / 32) * 32 (P_0 = 0; for
 * E == 1 the padded rows are the rows), so every expert starts a block.
 * The same codes and scale bytes as macaq_quant_act, in other places.  The
 * macaq_linear unfused path of a layer with tiled weights stages its
 * activation this way.
 *   x [M][K] in x_dtype, rows sorted by expert; s [E][K] fp32;
 *   expert_offsets [E+1] device int32 (NULL allowed when E == 1);
 *   a_codes: macaq_quant_act_tiled_rows(M, E) * K/2 bytes out; a_scales:
 *   macaq_quant_act_tiled_rows(M, E) * K/32 bytes out (padding rows are not
 *   written).
 * Requires E >= 1, M >= 0, K % 128 == 0 (MACAQ_ERR_UNSUPPORTED otherwise),
 * x, s and a_codes 16-byte aligned.  M == 0 is a no-op.
 */
int macaq_quant_act_tiled(const void* x, macaq_dtype x_dtype, const float* s, const int32_t* expert_offsets,
                          int64_t E, int64_t M, int64_t K, uint8_t* a_codes, uint8_t* a_scales, void* stream);

/* Rows that macaq_quant_act_tiled's buffers hold for M rows over E experts:
 * ceil(M / 32) * 32 for E == 1, else ceil((M + 31 E) / 32) * 32 (an upper
 * bound of the padded rows for any split of the M rows). */
size_t macaq_quant_act_tiled_rows(int64_t M, int64_t E);

/*
 * MXFP4 x MXFP4 GEMM y = A' W'^T per expert ("Quantization mechanism": the
 * FP4 matrix multiplication; "华为开源MACaQ:本地量化提速3倍", section
 * "现在还不能把它当成通用量化工厂": dense and grouped W4A4 matmul).
 * y[m][n] = sum_k a(m,k) w(e(m),n,k) with exact FP4 x FP4 products scaled by
 * both E8M0 scales and accumulated in fp32 (the order of the fp32 sums is
 * the kernel's; results are deterministic run to run).
 *   a_codes [M][K/2], a_scales [M][K/32]; w_codes [E][N][K/2],
 *   w_scales [E][N][K/32]; expert_offsets [E+1] device (NULL when E == 1);
 *   y [M][N] fp32 out.
 * workspace: device scratch of macaq_gemm_workspace_bytes(M, N, K, E) bytes,
 * 256-byte aligned; NULL when that is 0.  The decode GEMM (M <= 32, E == 1,
 * row-major weights) splits K over up to 4 blocks per row tile when the row
 * tiles cannot fill the GPU; the parts' fp32 partial sums (parts * M * N * 4
 * bytes) go to the workspace and a second kernel adds them in part order.
 * Calls that share a workspace must not overlap in time.
 * Requires K % 128 == 0; K >= 128; all code pointers 16-byte aligned and
 * scale pointers 4-byte aligned.
 */
int macaq_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
               const int32_t* expert_offsets, int64_t E,
               const uint8_t* w_codes, const uint8_t* w_scales,
               int64_t M, int64_t N, int64_t K, float* y,
               void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes macaq_gemm needs for this shape (0: none). */
size_t macaq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t E);

/* Bytes of activation codes + scales for M rows of width K (M*K/2 + M*K/32),
 * each part rounded up to 256 bytes. */
size_t macaq_quant_act_bytes(int64_t M, int64_t K);

/*
 * Device workspace needed by macaq_linear for this shape and flags.  0 means
 * no workspace is needed (workspace may then be NULL).  The unfused path
 * keeps the activation codes and scales there between its two kernels, so
 * calls sharing one workspace must not overlap in time.
 */
size_t macaq_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t E, uint32_t flags);

/*
 * Path macaq_linear takes for this shape and flags: MACAQ_PATH_FUSED or
 * MACAQ_PATH_UNFUSED (a negative status for invalid flags).
 */
int macaq_linear_path(int64_t M, int64_t N, int64_t K, int64_t E, uint32_t flags);

/*
 * The whole online layer: y = quant(x diag(s_e) H) quant(W_e diag(1/s_e) H)^T
 * with weights already prepared by macaq_prepare_weights.
 *   x [M][K] (rows sorted by expert), s [E][K], expert_offsets [E+1] device
 *   (NULL when E == 1), w_codes/w_scales as produced by
 *   macaq_prepare_weights, y [M][N] fp32 out.
 * flags: MACAQ_PATH_AUTO / _FUSED / _UNFUSED.  Both paths produce the same
 * activation codes; y may differ between paths only by fp32 summation order.
 * The fused path serves E == 1, M <= 32 and K % 256 == 0, in one launch of
 * the decode GEMM kernel (two with a K split, whose partial sums a second
 * kernel adds).  For M <= 2 the kernel transforms each 256-wide chunk of the
 * activation as the weights stream past.  For larger M, in small layers
 * (ceil(N / 32) * M * K <= 2^20) where M * (K/2 + K/32 + 24) bytes fit beside
 * the weight staging in the 160 KiB of LDS, every block first transforms
 * the whole activation into its LDS.  Otherwise the first blocks of the
 * launch transform it into the workspace (the same codes and scales as
 * macaq_quant_act, stored device-coherent) and publish per-block done
 * words; the other blocks start streaming weights, wait for the words,
 * then run decode_gemm_kernel's ring over the staged codes (a block whose
 * wait gives up, after about a second, writes NaN to every output it owns
 * rather than a result of unpublished codes; such a launch may leave its
 * done words set, which a later call's fresh value ignores but a replay of
 * the same captured graph would not: clear the workspace before replaying
 * a graph whose launch gave up; the unfused
 * path of an unsplit layer uses another kernel, so y may differ from it by
 * fp32 summation order).  AUTO takes the fused path for M <= 2 and for the
 * small layers (one
 * launch beats two there); for the other decode shapes the two launches
 * measured faster than publishing within one.
 * Requires the argument rules of macaq_quant_act and macaq_gemm and a
 * workspace of macaq_linear_workspace_bytes(M, N, K, E, flags) bytes (the
 * unfused path's activation staging; on either decode path the partial
 * sums of a K split, as in macaq_gemm; on the fused path of the larger
 * layers also the staged activation and 640 bytes of done words and
 * counts).  The workspace needs no initial contents: done words hold a
 * value unique to each launch and are cleared by the launch's last block.
 */
int macaq_linear(const void* x, macaq_dtype x_dtype, const float* s,
                 const int32_t* expert_offsets, int64_t E,
                 const uint8_t* w_codes, const uint8_t* w_scales,
                 int64_t M, int64_t N, int64_t K, float* y,
                 void* workspace, size_t workspace_bytes, uint32_t flags, void* stream);

/* Size of the static scratch array of macaq_linear_noalloc: 32 MiB per
 * device, enough for the unfused path's activation codes and scales of
 * M * K <= 58.7 million values (e.g. M = 4096 rows of K = 14336). */
#define MACAQ_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * macaq_linear_ex without a workspace argument, for callers that cannot
 * allocate device memory or hand one in: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same arguments (minus
 * workspace and workspace_bytes), rules, kernels and results (bit for bit)
 * as macaq_linear_ex.  The staging that macaq_linear_ex keeps in the
 * caller's workspace (macaq_linear_workspace_bytes(M, N, K, E, flags) bytes:
 * the activation codes and scales on the unfused path, and the partial sums
 * of a decode K split on either decode path) lives instead in a static device array of
 * MACAQ_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs
 * on until the process ends; a shape that needs more returns
 * MACAQ_ERR_WORKSPACE before anything is launched.  The call never
 * allocates or frees memory; its first call on a device looks up that
 * device's copy of the array (make it before a graph capture).  Every call
 * on one device shares that device's array: calls that overlap in time on
 * one device (on different streams, or from different threads) race and
 * must be serialized by the caller.  Nothing in the array needs to start at
 * zero: the transform writes every byte the GEMM reads.
 */
int macaq_linear_noalloc(const void* x, macaq_dtype x_dtype, const float* s,
                         const int32_t* expert_offsets, int64_t E,
                         const uint8_t* w_codes, const uint8_t* w_scales,
                         int64_t M, int64_t N, int64_t K, void* y, macaq_dtype y_dtype, uint32_t epilogue,
                         uint32_t flags, void* stream);

/*
 * macaq_gemm and macaq_linear with a chosen output (the layer's consumer
 * step, after the pages' y = x W^T: a bf16 output and a SwiGLU over the
 * gate/up projection are what a decoder layer does with it).
 *   y_dtype MACAQ_F32: y as fp32; MACAQ_BF16: y rounded to bf16 (nearest,
 *   ties to even) from the same fp32 value.
 *   epilogue MACAQ_EPI_NONE: y [M][N].  MACAQ_EPI_SWIGLU: N must be even and
 *   weight row 2j is the gate and row 2j+1 the up projection of output
 *   column j; y [M][N/2] = silu(g) * u with g, u the fp32 results of those
 *   rows and silu(g) = g / (1 + exp(-g)) in fp32 (expf, IEEE division).
 * The epilogue argument of macaq_gemm_ex also carries the layout bits
 * MACAQ_W_TILED and MACAQ_A_TILED (the latter only with the former).
 * Other arguments, rules and errors as macaq_gemm / macaq_linear; y must be
 * aligned to its element size.  macaq_gemm and macaq_linear are these calls
 * with MACAQ_F32 and MACAQ_EPI_NONE.
 */
int macaq_gemm_ex(const uint8_t* a_codes, const uint8_t* a_scales,
                  const int32_t* expert_offsets, int64_t E,
                  const uint8_t* w_codes, const uint8_t* w_scales,
                  int64_t M, int64_t N, int64_t K, void* y, macaq_dtype y_dtype, uint32_t epilogue,
                  void* workspace, size_t workspace_bytes, void* stream);
int macaq_linear_ex(const void* x, macaq_dtype x_dtype, const float* s,
                    const int32_t* expert_offsets, int64_t E,
                    const uint8_t* w_codes, const uint8_t* w_scales,
                    int64_t M, int64_t N, int64_t K, void* y, macaq_dtype y_dtype, uint32_t epilogue,
                    void* workspace, size_t workspace_bytes, uint32_t flags, void* stream);

/*
 * Repack of prepared weights into the tiled layout that the prefill and
 * grouped GEMMs read with contiguous copies (an offline step beside
 * macaq_prepare_weights; the codes and scale bytes themselves are unchanged,
 * only their places).  Per expert, for 32-row group g and 128-wide K-tile t:
 * 2048 bytes of codes at (g * K/128 + t) * 2048, where row r of the group
 * has its 64 bytes at 64 r with its 16-byte chunk c (32 values) at
 * position c ^ ((r >> 2) & 3); and 128 bytes of scales at
 * (g * K/128 + t) * 128, row r's 4 bytes at 4 r.
 *   w_codes [E][N][K/2], w_scales [E][N][K/32] (macaq_prepare_weights'
 *   layout) in; t_codes, t_scales (same sizes) out; no aliasing.
 * Requires N % 32 == 0, K % 128 == 0, code pointers 16-byte and scale
 * pointers 4-byte aligned.  Layers with tiled weights (MACAQ_W_TILED) always
 * take the unfused path and the prefill / grouped GEMM, also for M <= 32.
 */
int macaq_tile_weights(const uint8_t* w_codes, const uint8_t* w_scales, int64_t E, int64_t N, int64_t K,
                       uint8_t* t_codes, uint8_t* t_scales, void* stream);

/*
 * Plain OCP MXFP4 quantization of rows, without the scale and the Hadamard
 * transform (s = 1, H = I): the "pure MXFP4" baseline the pages compare the
 * online transform against ("MACaQ: Fast, Model Agnostic Calibrated
 * Quantization ...", Abstract: the overhead is quoted over pure MXFP4).
 * Same E8M0 and E2M1 rules as above.  Applied to both x and W it gives the
 * operands of a transform-free W4A4 layer for the macaq_gemm call.
 *   x [M][K] in x_dtype; codes [M][K/2] out; scales [M][K/32] out.
 * Requires M >= 0, K % 32 == 0, x and codes 16-byte aligned.
 */
int macaq_quant_mxfp4(const void* x, macaq_dtype x_dtype, int64_t M, int64_t K, uint8_t* codes, uint8_t* scales,
                      void* stream);

/*
 * Element encoder alone, for exhaustive tests of the E2M1 rounding: codes[i]
 * = the 4-bit E2M1 code (sign<<3 | magnitude index) of v[i] with scale byte
 * 127 (no scaling), by the same hardware conversion
 * (v_cvt_scalef32_pk_fp4_f32, scale 1.0) the quantizing kernels use.
 *   v [n] fp32 device in, codes [n] uint8 device out (one code per byte).
 */
int macaq_encode_e2m1(const float* v, int64_t n, uint8_t* codes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MACAQ_H */

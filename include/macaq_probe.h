/*
 * Measurement aid of libmacaq (not part of the layer): a kernel that runs
 * nothing but the block-scaled FP4 MFMA of the GEMM kernels
 * (v_mfma_scale_f32_32x32x64_f8f6f4) from registers, so that a benchmark
 * can time the MFMA throughput the chip sustains for a given operand data
 * (the clock under MFMA load depends on how many operand bits toggle).
 *
 * macaq_probe_mfma: `blocks` blocks of 64 * waves_per_block threads
 * (waves_per_block 4 or 8, i.e. one or two waves per SIMD when a block sits
 * on each CU); every wave loads 128 bytes per lane of operand codes from
 * `src` (device, 8192 bytes, 16-byte aligned: lane l takes bytes
 * 128 l .. 128 l + 127, the same for every wave: bytes 0..63 feed the
 * first operand, 64..127 the second), then runs `iters` iterations of
 * independent MFMAs on a grid of 32x32 accumulator tiles (4 x 4 tiles, 16
 * MFMAs per iteration, with 4 waves per block; 4 x 2, 8 MFMAs, with 8;
 * scale byte 127 = 1.0 on both operands) and writes one float per thread,
 * the sum of its accumulators, to `out` (device, blocks * waves_per_block *
 * 64 floats).  FLOP per launch: blocks * waves_per_block * iters * m *
 * 131072 with m = 16 (4 waves per block) or 8 (8 waves per block).  Enqueued on `stream`;
 * returns MACAQ_OK or a negative status (invalid arguments are rejected on
 * the host before any launch).
 *
 * macaq_probe_stream: the HBM streaming rate for a given mix of reads and
 * writes, the practical ceiling of the bandwidth-bound kernels (the online
 * transform reads about 3.8 bytes per byte it writes).  `blocks` blocks of
 * 256 threads stream over `src` (device, read_bytes) and `dst` (device,
 * write_bytes), both 16-byte aligned with sizes multiples of 16, in 16-byte
 * chunks (non-temporal loads, grid-stride loops):
 *   write_bytes == 0: every chunk of src is read once;
 *   read_bytes == 0:  every chunk c of dst is written with four copies of
 *                     the 32-bit chunk index c;
 *   otherwise read_bytes must be R * write_bytes (R a whole number) and
 *                     chunk c of dst receives the XOR of src chunks
 *                     c, c + n, ..., c + (R-1) n  (n = write_bytes / 16).
 * Thread t of the grid writes to out[t] (device, blocks * 256 uint32) the
 * XOR, folded over the four 32-bit words, of every chunk it read (reads
 * only) or wrote (the other two forms).  Enqueued on `stream`; returns
 * MACAQ_OK or a negative status (arguments checked on the host first).
 */
#ifndef MACAQ_PROBE_H
#define MACAQ_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int macaq_probe_mfma(const void* src, int64_t blocks, int waves_per_block, int iters, float* out, void* stream);
int macaq_probe_stream(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes, int64_t blocks,
                       uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif

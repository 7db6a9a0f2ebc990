"""Tiled W' (macaq_tile_weights and MACAQ_W_TILED) on the GPU, through the C
ABI.  The repack is a permutation of bytes: it must equal a re-layout of
the row-major codes and scales written out here in numpy.  The GEMM reads
the same LDS tiles from either layout, so for a given tile shape its output
must be bitwise equal to the row-major GEMM's, and both are within the
oracle's bound."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import mxfp4_w4a4_quantized_channel_amd as mx

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
RTOL = 1e-5


def say(msg):
    print(f"[case] {msg}", flush=True)


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return workloads.bf16_bits(t)
    return t.numpy()


def tiled_reference(codes: np.ndarray, scales: np.ndarray):
    """The tiled layout as the header defines it: per expert, per 32-row group
    and 128-wide K-tile, 32 rows of 64 code bytes whose 16-byte chunk c sits
    at position c ^ ((r >> 2) & 3), then 32 rows of 4 scale bytes."""
    E, N, KH = codes.shape
    G, T = N // 32, KH // 64
    c = codes.reshape(E, G, 32, T, 4, 16).transpose(0, 1, 3, 2, 4, 5)    # [E, G, T, r, chunk, 16]
    r = np.arange(32)[:, None]
    p = np.arange(4)[None, :]
    src = p ^ ((r >> 2) & 3)                                             # chunk held at position p
    c = np.take_along_axis(c, np.broadcast_to(src[None, None, None, :, :, None], c.shape), axis=4)
    s = scales.reshape(E, G, 32, T, 4).transpose(0, 1, 3, 2, 4)          # [E, G, T, r, 4]
    return np.ascontiguousarray(c).reshape(E, N, KH), np.ascontiguousarray(s).reshape(E, N, KH // 16)


@pytest.mark.parametrize("E,N,K", [(1, 32, 128), (1, 32, 256), (2, 96, 768), (3, 128, 3072)])
def test_tile_weights_layout(E, N, K):
    say(f"tile_weights E{E} N{N} K{K}")
    rng = np.random.default_rng(E * 1000 + N + K)
    codes = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (E, N, K // 32), dtype=np.uint8)
    tc, ts = mx.tile_weights(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV))
    rc, rs = tiled_reference(codes, scales)
    assert np.array_equal(tc.cpu().numpy(), rc)
    assert np.array_equal(ts.cpu().numpy(), rs)


def _operands(M, N, K, E=1, seed=0, offsets=None):
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    w = torch.from_numpy((rng.standard_normal((E, N, K)) * 0.02).astype(np.float32)).to(torch.bfloat16).to(DEV)
    s = torch.from_numpy(rng.uniform(0.5, 2.0, (E, K)).astype(np.float32)).to(DEV)
    ac, asc = mx.quant_act(x, s, offsets)
    wc, wsc = mx.prepare_weights(w, s)
    return x, s, ac, asc, wc, wsc


TILED_SHAPES = [
    ("one 128 tile", (128, 128, 256)),
    ("ragged M, N tail of 32", (300, 224, 1024)),
    ("M=1", (1, 64, 512)),
    ("several 256 tiles", (520, 544, 2048)),
]


@pytest.mark.parametrize("tile", ["256x256", "256x128", "128x128"])
@pytest.mark.parametrize("name,shape", TILED_SHAPES, ids=[n for n, _ in TILED_SHAPES])
def test_tiled_gemm_equals_row_major(name, shape, tile, tune):
    """Each tile variant: the tiled GEMM's fp32 y equals the row-major GEMM's
    bit for bit, and is within the oracle's bound."""
    M, N, K = shape
    say(f"tiled gemm {name} M{M} N{N} K{K} tile {tile}")
    tune(mx.TUNE_GEMM_TILE, mx.GEMM_TILES[tile])
    x, s, ac, asc, wc, wsc = _operands(M, N, K, seed=M + N)
    tc, ts = mx.tile_weights(wc, wsc)
    y_t = mx.gemm(ac, asc, tc, ts, epilogue=mx.W_TILED)
    if M > 32:   # at M <= 32 the row-major call takes the decode kernel: compare with the oracle only
        y_r = mx.gemm(ac, asc, wc, wsc)
        torch.cuda.synchronize()
        assert torch.equal(y_t, y_r)
    y_ref, S = oracle.gemm(ac.cpu().numpy(), asc.cpu().numpy(), wc[0].cpu().numpy(), wsc[0].cpu().numpy())
    ok, worst, normwise = oracle.within_tolerance(y_t.cpu().numpy(), y_ref, S, RTOL)
    assert ok, f"worst {worst:.3g}"


def test_tiled_grouped_gemm_with_empty_experts():
    """Grouped layer with ragged and empty experts: tiled equals row-major."""
    say("tiled grouped gemm")
    E, N, K = 5, 160, 512
    counts = np.array([70, 0, 131, 1, 0])
    off = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).to(DEV)
    M = int(counts.sum())
    x, s, ac, asc, wc, wsc = _operands(M, N, K, E=E, seed=7, offsets=off)
    tc, ts = mx.tile_weights(wc, wsc)
    y_t = mx.gemm(ac, asc, tc, ts, off, epilogue=mx.W_TILED)
    y_r = mx.gemm(ac, asc, wc, wsc, off)
    torch.cuda.synchronize()
    assert torch.equal(y_t, y_r)


@pytest.mark.parametrize("epi,dt", [(mx.EPI_NONE, torch.float32), (mx.EPI_NONE, torch.bfloat16),
                                    (mx.EPI_SWIGLU, torch.bfloat16), (mx.EPI_SWIGLU, torch.float32)])
def test_tiled_linear_epilogues(epi, dt):
    """The whole layer with tiled weights (two launches) equals the row-major
    two-launch layer in every output form."""
    say(f"tiled linear epilogue {epi} {dt}")
    M, N, K = 200, 256, 1024
    x, s, ac, asc, wc, wsc = _operands(M, N, K, seed=11)
    tc, ts = mx.tile_weights(wc, wsc)
    y_t = mx.linear(x, s, tc, ts, flags=mx.PATH_AUTO | mx.W_TILED, out_dtype=dt, epilogue=epi)
    y_r = mx.linear(x, s, wc, wsc, flags=mx.PATH_UNFUSED, out_dtype=dt, epilogue=epi)
    torch.cuda.synchronize()
    assert torch.equal(y_t, y_r)


def test_tiled_linear_decode_rows():
    """M <= 32 with tiled weights takes the prefill GEMM (the decode kernel
    reads row-major weights): within the oracle's bound."""
    say("tiled linear M4")
    M, N, K = 4, 128, 1024
    x, s, ac, asc, wc, wsc = _operands(M, N, K, seed=3)
    tc, ts = mx.tile_weights(wc, wsc)
    y = mx.linear(x, s, tc, ts, flags=mx.W_TILED)
    y_ref, S = oracle.gemm(ac.cpu().numpy(), asc.cpu().numpy(), wc[0].cpu().numpy(), wsc[0].cpu().numpy())
    ok, worst, _ = oracle.within_tolerance(y.cpu().numpy(), y_ref, S, RTOL)
    assert ok, f"worst {worst:.3g}"


def test_tiled_full_size_attention_sampled():
    """attn-proj at full size (M2048 N4096 K4096) with tiled weights in the
    benchmark's default tile choice: bitwise equal to the row-major GEMM with
    the same tile, and sampled rows within the oracle's bound."""
    say("tiled full size attn-proj")
    wl = workloads.make(2)
    x, s = wl.x.to(DEV), wl.s.to(DEV)
    ac, asc = mx.quant_act(x, s)
    wc, wsc = mx.prepare_weights(wl.w.to(DEV), s)
    tc, ts = mx.tile_weights(wc, wsc)
    y_t = mx.gemm(ac, asc, tc, ts, epilogue=mx.W_TILED)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, wl.M - 1], np.random.default_rng(5).choice(wl.M, 14, replace=False)]))
    a_np, as_np = ac.cpu().numpy()[rows], asc.cpu().numpy()[rows]
    y_ref, S = oracle.gemm(a_np, as_np, wc[0].cpu().numpy(), wsc[0].cpu().numpy())
    ok, worst, _ = oracle.within_tolerance(y_t.cpu().numpy()[rows], y_ref, S, RTOL)
    assert ok, f"worst {worst:.3g}"


@pytest.mark.parametrize("E", [63, 64, 65, 130])
def test_grouped_gemm_many_experts(E):
    """The grouped GEMM finds each row tile's expert 64 experts at a time:
    expert counts on both sides of 64, with runs of empty experts, ragged
    counts and an expert past the first 64 that owns several row tiles.
    Each expert's rows are within the oracle's bound against that expert's
    weights, and the tiled layout equals the row-major one bit for bit."""
    say(f"grouped gemm E{E}")
    N, K = 64, 256
    rng = np.random.default_rng(E)
    counts = rng.integers(0, 40, E)
    counts[rng.random(E) < 0.4] = 0
    counts[E - 2] = 300
    counts[0] = 0
    off_np = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    off = torch.from_numpy(off_np).to(DEV)
    M = int(counts.sum())
    x, s, ac, asc, wc, wsc = _operands(M, N, K, E=E, seed=E + 1, offsets=off)
    y = mx.gemm(ac, asc, wc, wsc, off)
    tc, ts = mx.tile_weights(wc, wsc)
    y_t = mx.gemm(ac, asc, tc, ts, off, epilogue=mx.W_TILED)
    torch.cuda.synchronize()
    assert torch.equal(y, y_t)
    a_np, as_np, y_np = ac.cpu().numpy(), asc.cpu().numpy(), y.cpu().numpy()
    wc_np, ws_np = wc.cpu().numpy(), wsc.cpu().numpy()
    for e in np.nonzero(counts)[0]:
        r0, r1 = off_np[e], off_np[e + 1]
        y_ref, S = oracle.gemm(a_np[r0:r1], as_np[r0:r1], wc_np[e], ws_np[e])
        ok, worst, _ = oracle.within_tolerance(y_np[r0:r1], y_ref, S, RTOL)
        assert ok, f"expert {e}: worst {worst:.3g}"


def padded_rows(offsets, M: int):
    """Padded row of every row (expert e's rows start at the sum over e' < e
    of ceil(rows_e' / 32) * 32) and the buffer's row count, as the header
    defines them."""
    if offsets is None:
        return np.arange(M), (M + 31) // 32 * 32
    off = np.asarray(offsets, dtype=np.int64)
    E = len(off) - 1
    cnt = np.diff(off)
    pstart = np.concatenate([[0], np.cumsum((cnt + 31) // 32 * 32)])
    e_of = np.searchsorted(off, np.arange(M), side="right") - 1
    return pstart[e_of] + (np.arange(M) - off[e_of]), (M + 31 * E + 31) // 32 * 32


def tiled_rows_reference(codes: np.ndarray, scales: np.ndarray, M: int, offsets=None):
    """The activation rows in the tiled layout at their padded rows, and a
    mask of the bytes that belong to real rows (padding is not compared)."""
    prow, rows = padded_rows(offsets, M)
    pc = np.zeros((1, rows, codes.shape[1]), np.uint8)
    ps = np.zeros((1, rows, scales.shape[1]), np.uint8)
    pc[0, prow], ps[0, prow] = codes, scales
    real = np.zeros((1, rows, 1), bool)
    real[0, prow] = True
    rc, rs = tiled_reference(pc, ps)
    mc, ms = tiled_reference(np.broadcast_to(real, pc.shape).astype(np.uint8),
                             np.broadcast_to(real, ps.shape).astype(np.uint8))
    return rc.reshape(-1), rs.reshape(-1), mc.reshape(-1) == 1, ms.reshape(-1) == 1


@pytest.mark.parametrize("M,K,dt,counts", [(1, 256, torch.bfloat16, None), (37, 1152, torch.bfloat16, None),
                                           (64, 512, torch.float32, None), (300, 3072, torch.bfloat16, None),
                                           (33, 14336, torch.bfloat16, None),
                                           (300, 1024, torch.bfloat16, [3, 0, 130, 33, 0, 1, 133]),
                                           (96, 3072, torch.bfloat16, [0, 32, 0, 64, 0]),
                                           (16, 512, torch.bfloat16, [5] + [0] * 100 + [7] + [0] * 20 + [4]),
                                           (8192, 3072, torch.bfloat16, [0] * 6 + [8177, 3] + [0] * 12 + [12] + [0] * 43)])
def test_quant_act_tiled_bit_exact(M, K, dt, counts):
    """macaq_quant_act_tiled writes the oracle's codes and scale bytes in the
    tiled layout, each expert from its padded row on (padding rows are not
    compared)."""
    say(f"quant_act_tiled M{M} K{K} {dt} counts={counts}")
    rng = np.random.default_rng(M + K)
    E = 1 if counts is None else len(counts)
    off = None if counts is None else np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    xf = rng.standard_normal((M, K)) * np.where(rng.random(K) < 0.01, 50.0, 1.0)
    x = torch.from_numpy(xf).to(dt)
    s = torch.from_numpy(rng.uniform(0.25, 4.0, (E, K)).astype(np.float32))
    codes, scales = mx.quant_act_tiled(x.to(DEV), s.to(DEV), None if off is None else torch.from_numpy(off).to(DEV))
    rc, rs = oracle.quant_act(host(x), s.numpy(), off)
    tc, ts, mc, ms = tiled_rows_reference(rc, rs, M, off)
    assert np.array_equal(codes.cpu().numpy()[mc], tc[mc])
    assert np.array_equal(scales.cpu().numpy()[ms], ts[ms])


A_TILED_SHAPES = [
    ("one 128 tile", (128, 128, 256)),
    ("ragged M, N tail of 32", (300, 224, 1024)),
    ("M=1", (1, 64, 512)),
    ("several 256 tiles", (520, 544, 2048)),
    ("M not a multiple of 32, deep K", (100, 256, 7168)),
    ("K an odd number of 128-wide tiles", (96, 160, 1152)),
]


@pytest.mark.parametrize("out", ["f32", "bf16", "swiglu"])
@pytest.mark.parametrize("tile", ["256x256", "256x128", "128x128"])
@pytest.mark.parametrize("name,shape", A_TILED_SHAPES, ids=[n for n, _ in A_TILED_SHAPES])
def test_tiled_activation_gemm_equals_row_major(name, shape, tile, out, tune):
    """The GEMM reading tiled activations (MACAQ_A_TILED, as the dense
    linear path stages them) equals the same tile's GEMM on row-major
    activations bit for bit (the LDS tiles are the same), for each output
    form; the linear call with tiled weights equals both."""
    say(f"A-tiled gemm tile={tile} out={out} {name} {shape}")
    tune(mx.TUNE_GEMM_TILE, mx.GEMM_TILES[tile])
    M, N, K = shape
    x, s, ac, asc, wc, wsc = _operands(M, N, K, seed=M + N)
    tc, ts = mx.tile_weights(wc, wsc)
    atc, ats = mx.quant_act_tiled(x, s)
    odt = torch.float32 if out == "f32" else torch.bfloat16
    epi = mx.EPI_SWIGLU if out == "swiglu" else mx.EPI_NONE
    y_rm = mx.gemm(ac, asc, tc, ts, out_dtype=odt, epilogue=epi | mx.W_TILED)
    y_at = mx.gemm(atc, ats, tc, ts, out_dtype=odt, epilogue=epi | mx.W_TILED | mx.A_TILED, M=M)
    y_lin = mx.linear(x, s, tc, ts, flags=mx.W_TILED, out_dtype=odt, epilogue=epi)
    torch.cuda.synchronize()
    assert torch.equal(y_at, y_rm)
    assert torch.equal(y_lin, y_rm)
    if out == "f32":
        y_ref, S = oracle.gemm(ac.cpu().numpy(), asc.cpu().numpy(), wc[0].cpu().numpy(), wsc[0].cpu().numpy())
        ok, worst, nw = oracle.within_tolerance(y_at.cpu().numpy(), y_ref, S, RTOL)
        assert ok, f"worst {worst:.3g} normwise {nw:.3g}"


@pytest.mark.parametrize("counts", [[70, 0, 131, 1, 0], [0, 3, 0, 0, 300, 29, 64, 1], [8177, 12, 3]])
def test_grouped_tiled_activation_gemm(counts):
    """The grouped GEMM on expert-padded tiled activations equals the grouped
    GEMM on row-major activations (same tiled weights) bit for bit, the
    linear call with tiled weights equals both, and each expert's rows are
    within the oracle's bound."""
    say(f"grouped A-tiled gemm counts={counts}")
    E, N, K = len(counts), 96, 1024
    off_np = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    off = torch.from_numpy(off_np).to(DEV)
    M = int(off_np[-1])
    x, s, ac, asc, wc, wsc = _operands(M, N, K, E=E, seed=M + E, offsets=off)
    tc, ts = mx.tile_weights(wc, wsc)
    atc, ats = mx.quant_act_tiled(x, s, off)
    y_rm = mx.gemm(ac, asc, tc, ts, off, epilogue=mx.W_TILED)
    y_at = mx.gemm(atc, ats, tc, ts, off, epilogue=mx.W_TILED | mx.A_TILED, M=M)
    y_lin = mx.linear(x, s, tc, ts, off, flags=mx.W_TILED)
    torch.cuda.synchronize()
    assert torch.equal(y_at, y_rm)
    assert torch.equal(y_lin, y_rm)
    y_ref, S = oracle.gemm(ac.cpu().numpy(), asc.cpu().numpy(), wc.cpu().numpy(), wsc.cpu().numpy(), off_np)
    ok, worst, nw = oracle.within_tolerance(y_at.cpu().numpy(), y_ref, S, RTOL)
    assert ok, f"worst {worst:.3g} normwise {nw:.3g}"

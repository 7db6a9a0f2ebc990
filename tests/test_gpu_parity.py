"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Codes and scale bytes must be bit-exact.  GEMM / layer outputs must satisfy
|y - y_ref| <= 1e-5 * S elementwise, S = sum_k |a_k w_k| of the dequantized
operands (the componentwise bound of an fp32 dot product of exact FP4
products), and ||y - y_ref||_F <= 1e-5 ||y_ref||_F.

Small cases are compared element by element; full-size workloads on sampled
rows / outputs that the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import mxfp4_w4a4_quantized_channel_amd as mx

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
RTOL = 1e-5


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return workloads.bf16_bits(t)
    return t.numpy()


def say(msg):
    print(f"[case] {msg}", flush=True)


def assert_codes(got, want, values):
    bad = np.nonzero(got != want)[0]
    if bad.size:
        rows = [f"v={values[i]!r} bits=0x{np.float32(values[i]).view(np.uint32):08x} got={got[i]} want={want[i]}"
                for i in bad[:12]]
        raise AssertionError(f"{bad.size} mismatches:\n" + "\n".join(rows))


def gpu_prepare(wl):
    return mx.prepare_weights(wl.w.to(DEV), wl.s.to(DEV))


def oracle_prepare(wl, e, rows=None):
    w = host(wl.w[e])
    if rows is not None:
        w = w[rows]
    return oracle.prepare_weights(w, wl.s[e].numpy())


# ------------------------------------------------------------ element encoder

def test_encode_e2m1_exhaustive():
    """Every fp32 in [0.25, 8) and its negation, denormals, zeros, large values."""
    say("encode_e2m1 exhaustive [0.25, 8)")
    lo = int(np.float32(0.25).view(np.uint32))
    hi = int(np.float32(8.0).view(np.uint32))
    bits = np.arange(lo, hi, dtype=np.uint32)
    v = bits.view(np.float32)
    got = mx.encode_e2m1(torch.from_numpy(v).to(DEV)).cpu().numpy()
    want = oracle.e2m1_nearest(v)
    assert_codes(got, want, v)
    got_neg = mx.encode_e2m1(torch.from_numpy(-v).to(DEV)).cpu().numpy()
    assert_codes(got_neg, want | 8, -v)
    rng = np.random.default_rng(0)
    extra = np.concatenate([
        rng.integers(0, lo, 200000, dtype=np.uint32).view(np.float32),       # tiny incl. denormals
        np.array([0.0, -0.0, 8.0, 100.0, 6.0, 5.0, 7.0, 3.4e38], np.float32),
        -rng.integers(0, lo, 200000, dtype=np.uint32).view(np.float32),
    ]).astype(np.float32)
    got = mx.encode_e2m1(torch.from_numpy(extra).to(DEV)).cpu().numpy()
    want = oracle.e2m1_nearest(np.abs(extra)) | (np.signbit(extra).astype(np.uint8) << 3)
    assert_codes(got, want, extra)


# ------------------------------------------------------------ activation transform + quant

SMALL_ACT = [
    ("tiny fp32", dict(cfg=1)),
    ("cfg2-shaped ragged K", dict(cfg=2, shape=(37, 64, 1312))),
    ("cfg3-shaped t4", dict(cfg=3, shape=(19, 64, 2048))),
    ("cfg4-shaped M1", dict(cfg=4, shape=(1, 64, 5120))),
    ("cfg5 token routing", dict(cfg=5, shape=(300, 32, 256), routing="token_zipf")),
    ("cfg5 expert routing", dict(cfg=5, shape=(333, 32, 256))),
    ("literal scale rule", dict(cfg=2, shape=(9, 64, 512), scale_rule="literal")),
    ("cfg5 K3072 two rows per wave step", dict(cfg=5, shape=(500, 32, 3072))),
]


@pytest.mark.parametrize("name,kw", SMALL_ACT, ids=[n for n, _ in SMALL_ACT])
def test_quant_act_bit_exact(name, kw):
    say(f"quant_act {name}")
    wl = workloads.make(**kw)
    off = wl.offsets.to(DEV) if wl.E > 1 else None
    codes, scales = mx.quant_act(wl.x.to(DEV), wl.s.to(DEV), off)
    rc, rs = oracle.quant_act(host(wl.x), wl.s.numpy(), wl.offsets.numpy() if wl.E > 1 else None)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("steps", [1, 5])
def test_quant_act_rows_per_wave(steps, tune):
    """Waves of 1 and of 5 row steps (segments of 16 groups over 4 rows), with
    expert boundaries inside a step and inside a wave."""
    say(f"quant_act steps={steps}")
    tune(mx.TUNE_ACT_ROWS_PER_WAVE, steps)
    wl = workloads.make(cfg=5, shape=(333, 32, 256))
    codes, scales = mx.quant_act(wl.x.to(DEV), wl.s.to(DEV), wl.offsets.to(DEV))
    rc, rs = oracle.quant_act(host(wl.x), wl.s.numpy(), wl.offsets.numpy())
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


LAYOUT_ACT = [
    ("cfg2-shaped ragged K", dict(cfg=2, shape=(37, 64, 1312))),
    ("tiny fp32", dict(cfg=1)),
    ("cfg5 token routing", dict(cfg=5, shape=(300, 32, 256), routing="token_zipf")),
    ("cfg5 expert routing K3072", dict(cfg=5, shape=(500, 32, 3072))),
]


@pytest.mark.parametrize("steps", [None, 1, 3])
@pytest.mark.parametrize("shared", ["0", "1"])
@pytest.mark.parametrize("name,kw", LAYOUT_ACT, ids=[n for n, _ in LAYOUT_ACT])
def test_quant_act_both_layouts(name, kw, shared, steps, tune):
    """Both wave layouts of the activation kernel, forced: s per wave in
    registers, and s staged per block in LDS for the experts of the block's
    first and last rows (token routing puts many more experts in a block, so
    rows of other experts read s directly); also with 1 and 3 row blocks per
    wave."""
    say(f"quant_act {name} shared={shared} steps={steps}")
    tune(mx.TUNE_ACT_SHARED_S, 2 if shared == "1" else 1)
    if steps is not None:
        tune(mx.TUNE_ACT_ROWS_PER_WAVE, steps)
    wl = workloads.make(**kw)
    off = wl.offsets.to(DEV) if wl.E > 1 else None
    codes, scales = mx.quant_act(wl.x.to(DEV), wl.s.to(DEV), off)
    rc, rs = oracle.quant_act(host(wl.x), wl.s.numpy(), wl.offsets.numpy() if wl.E > 1 else None)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("steps", [None, 7])
@pytest.mark.parametrize("shared", ["0", "1"])
def test_quant_act_many_experts(shared, steps, tune):
    """130 experts with runs of empty ones and ragged counts: the wave's
    first expert comes from a binary search over the offsets, and lanes walk
    on across expert ends inside a row block, a wave and a block; 7 row
    blocks per wave refill each slot of the copy ring twice."""
    say(f"quant_act E130 shared={shared} steps={steps}")
    tune(mx.TUNE_ACT_SHARED_S, 2 if shared == "1" else 1)
    if steps is not None:
        tune(mx.TUNE_ACT_ROWS_PER_WAVE, steps)
    E, K = 130, 768
    rng = np.random.default_rng(130)
    counts = rng.integers(0, 9, E)
    counts[rng.random(E) < 0.4] = 0
    counts[[0, E - 1]] = [0, 5]
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(off[-1])
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    s = rng.uniform(0.25, 4.0, (E, K)).astype(np.float32)
    codes, scales = mx.quant_act(x.to(DEV), torch.from_numpy(s).to(DEV), torch.from_numpy(off).to(DEV))
    rc, rs = oracle.quant_act(host(x), s, off)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("shared", ["0", "1"])
@pytest.mark.parametrize("counts", [[5] + [0] * 100 + [7] + [0] * 20 + [4],
                                    [0] * 6 + [8177, 3] + [0] * 12 + [12] + [0] * 43],
                         ids=["runs of 100 and 20 empty experts in one wave", "expert-Zipf-like"])
def test_quant_act_long_runs_of_empty_experts(counts, shared, tune):
    """Rows of one wave separated by long runs of empty experts: the walk
    over experts reads the wave's table of 64 offsets, and past it global
    memory (the run of 100)."""
    say(f"quant_act long empty runs E{len(counts)} shared={shared}")
    tune(mx.TUNE_ACT_SHARED_S, 2 if shared == "1" else 1)
    E, K = len(counts), 3072
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(off[-1])
    rng = np.random.default_rng(M + E)
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    s = rng.uniform(0.25, 4.0, (E, K)).astype(np.float32)
    codes, scales = mx.quant_act(x.to(DEV), torch.from_numpy(s).to(DEV), torch.from_numpy(off).to(DEV))
    rc, rs = oracle.quant_act(host(x), s, off)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("shared", ["0", "1"])
@pytest.mark.parametrize("M,K", [(7, 32), (13, 96), (5, 160), (9, 2080)])
def test_quant_act_narrow_rows(M, K, shared, tune):
    """Rows of 1, 3, 5 and 65 groups: most lanes of a segment are past the
    row's last group, and their copies of the ring are stand-ins that no
    lane stores; M is not a multiple of the rows per block step."""
    say(f"quant_act narrow M{M} K{K} shared={shared}")
    tune(mx.TUNE_ACT_SHARED_S, 2 if shared == "1" else 1)
    rng = np.random.default_rng(M * K)
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    s = rng.uniform(0.25, 4.0, (1, K)).astype(np.float32)
    codes, scales = mx.quant_act(x.to(DEV), torch.from_numpy(s).to(DEV))
    rc, rs = oracle.quant_act(host(x), s, None)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("shared", ["0", "1"])
def test_prepare_weights_both_layouts(shared, tune):
    """Weight preparation (reciprocal factors, experts of N rows each) with
    either wave layout forced."""
    say(f"prepare_weights experts shared={shared}")
    tune(mx.TUNE_ACT_SHARED_S, 2 if shared == "1" else 1)
    wl = workloads.make(cfg=5, shape=(64, 48, 256))
    codes, scales = gpu_prepare(wl)
    for e in range(wl.E):
        rc, rs = oracle_prepare(wl, e)
        assert np.array_equal(scales[e].cpu().numpy(), rs), e
        assert np.array_equal(codes[e].cpu().numpy(), rc), e


def test_quant_act_empty_is_noop():
    say("quant_act M=0")
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    codes, scales = mx.quant_act(x, torch.ones(256, device=DEV))
    assert codes.shape == (0, 128) and scales.shape == (0, 8)


def test_quant_act_special_groups():
    """Spike, constant, zero, signed zero, saturation and tie groups."""
    say("quant_act special groups")
    K = 32 * 8
    x = np.zeros((4, K), np.float32)
    x[0, 0:32] = 0.0
    x[0, 32 + 5] = 6.0
    x[0, 64:96] = 0.25
    x[0, 96:128] = -0.0
    x[0, 128:160] = np.linspace(-3, 3, 32)
    x[0, 160:192] = 3.0e38 / 64
    x[0, 192:224] = 1e-40  # denormal inputs
    x[1] = np.random.default_rng(1).standard_normal(K) * 1e-30
    x[2] = np.random.default_rng(2).standard_normal(K) * 1e30
    x[3, ::7] = -1.0
    s = np.ones((1, K), np.float32)
    codes, scales = mx.quant_act(torch.from_numpy(x).to(DEV), torch.from_numpy(s).to(DEV))
    rc, rs = oracle.quant_act(x, s)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


# ------------------------------------------------------------ weight preparation

SMALL_W = [
    ("tiny fp32", dict(cfg=1)),
    ("cfg2-shaped", dict(cfg=2, shape=(8, 200, 1024))),
    ("cfg5 experts", dict(cfg=5, shape=(64, 48, 256))),
]


@pytest.mark.parametrize("name,kw", SMALL_W, ids=[n for n, _ in SMALL_W])
def test_prepare_weights_bit_exact(name, kw):
    say(f"prepare_weights {name}")
    wl = workloads.make(**kw)
    codes, scales = gpu_prepare(wl)
    for e in range(wl.E):
        rc, rs = oracle_prepare(wl, e)
        assert np.array_equal(scales[e].cpu().numpy(), rs), e
        assert np.array_equal(codes[e].cpu().numpy(), rc), e


# ------------------------------------------------------------ GEMM

def _check_y(y, y_ref, S):
    ok, worst, normwise = oracle.within_tolerance(y, y_ref, S, RTOL)
    assert ok, f"worst elementwise {worst:.3g}, normwise {normwise:.3g}"


SMALL_GEMM = [
    ("one tile", (128, 128, 256)),
    ("ragged M N, K tail 128", (200, 300, 640)),
    ("M=1", (1, 96, 384)),
    ("several tiles", (300, 260, 1024)),
]


@pytest.mark.parametrize("name,shape", SMALL_GEMM, ids=[n for n, _ in SMALL_GEMM])
def test_gemm_dense(name, shape):
    say(f"gemm {name} {shape}")
    M, N, K = shape
    rng = np.random.default_rng(M * 7 + N)
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    asc = rng.integers(110, 140, (M, K // 32), dtype=np.uint8)
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    wsc = rng.integers(110, 140, (N, K // 32), dtype=np.uint8)
    y = mx.gemm(*(torch.from_numpy(a).to(DEV) for a in (ac, asc, wc, wsc)))
    y_ref, S = oracle.gemm(ac, asc, wc, wsc)
    _check_y(y.cpu().numpy(), y_ref, S)


def test_gemm_exact_small_integers():
    """One group per row with unit scales: every product and sum is a small
    integer multiple of 2^-2, so fp32 accumulation is exact -> bit-exact."""
    say("gemm exact small integers")
    M, N, K = 64, 64, 128
    rng = np.random.default_rng(5)
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    asc = np.full((M, K // 32), 127, np.uint8)
    wsc = np.full((N, K // 32), 127, np.uint8)
    y = mx.gemm(*(torch.from_numpy(a).to(DEV) for a in (ac, asc, wc, wsc))).cpu().numpy()
    y_ref, _ = oracle.gemm(ac, asc, wc, wsc)
    assert np.array_equal(y.astype(np.float64), y_ref)


def test_gemm_grouped_ragged_with_empty_experts():
    say("gemm grouped ragged")
    E, N, K = 6, 160, 256
    counts = np.array([0, 130, 1, 0, 257, 3])
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(off[-1])
    rng = np.random.default_rng(6)
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    asc = rng.integers(110, 140, (M, K // 32), dtype=np.uint8)
    wc = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    wsc = rng.integers(110, 140, (E, N, K // 32), dtype=np.uint8)
    t = [torch.from_numpy(a).to(DEV) for a in (ac, asc, wc, wsc)]
    y = mx.gemm(*t, offsets=torch.from_numpy(off).to(DEV))
    y_ref, S = oracle.gemm(ac, asc, wc, wsc, off)
    _check_y(y.cpu().numpy(), y_ref, S)


# ------------------------------------------------------------ whole layer, small

SMALL_LINEAR = [
    ("tiny fp32", dict(cfg=1)),
    ("cfg2-shaped", dict(cfg=2, shape=(150, 200, 768))),
    ("cfg3-shaped", dict(cfg=3, shape=(64, 96, 2048))),
    ("cfg4-shaped M8", dict(cfg=4, shape=(8, 320, 1024))),
    ("cfg5 token routing", dict(cfg=5, shape=(512, 64, 256), routing="token_zipf")),
]


@pytest.mark.parametrize("flags", [mx.PATH_AUTO, mx.PATH_UNFUSED])
@pytest.mark.parametrize("name,kw", SMALL_LINEAR, ids=[n for n, _ in SMALL_LINEAR])
def test_linear_small(name, kw, flags):
    say(f"linear {name} flags={flags}")
    wl = workloads.make(**kw)
    off_np = wl.offsets.numpy() if wl.E > 1 else None
    wc, wsc = gpu_prepare(wl)
    y = mx.linear(wl.x.to(DEV), wl.s.to(DEV), wc, wsc,
                  wl.offsets.to(DEV) if wl.E > 1 else None, flags=flags).cpu().numpy()
    rwc, rws = zip(*(oracle_prepare(wl, e) for e in range(wl.E)))
    y_ref, S = oracle.linear(host(wl.x), wl.s.numpy(), np.stack(rwc), np.stack(rws), off_np)
    _check_y(y, y_ref, S)


def test_linear_deterministic():
    say("linear determinism")
    wl = workloads.make(2, shape=(256, 256, 1024))
    wc, wsc = gpu_prepare(wl)
    x, s = wl.x.to(DEV), wl.s.to(DEV)
    y1 = mx.linear(x, s, wc, wsc)
    y2 = mx.linear(x, s, wc, wsc)
    assert torch.equal(y1, y2)


# ------------------------------------------------------------ every GEMM kernel variant

TILES = ["256x256", "256x128", "128x128"]
TILE_SHAPES = [
    ("ragged M N", (300, 260, 1024)),
    ("K tail 128", (257, 129, 640)),
    ("single row tile", (5, 384, 256)),
]


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("name,shape", TILE_SHAPES, ids=[n for n, _ in TILE_SHAPES])
def test_gemm_each_tile_variant(tile, name, shape, tune):
    say(f"gemm tile={tile} {name} {shape}")
    tune(mx.TUNE_GEMM_TILE, mx.GEMM_TILES[tile])
    M, N, K = shape
    rng = np.random.default_rng(M + N + K)
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    asc = rng.integers(110, 140, (M, K // 32), dtype=np.uint8)
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    wsc = rng.integers(110, 140, (N, K // 32), dtype=np.uint8)
    y = mx.gemm(*(torch.from_numpy(a).to(DEV) for a in (ac, asc, wc, wsc)))
    y_ref, S = oracle.gemm(ac, asc, wc, wsc)
    _check_y(y.cpu().numpy(), y_ref, S)


@pytest.mark.parametrize("tile", TILES)
def test_gemm_grouped_each_tile_variant(tile, tune):
    say(f"gemm grouped tile={tile}")
    tune(mx.TUNE_GEMM_TILE, mx.GEMM_TILES[tile])
    E, N, K = 5, 200, 512
    counts = np.array([3, 0, 270, 1, 300])
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(off[-1])
    rng = np.random.default_rng(11)
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    asc = rng.integers(110, 140, (M, K // 32), dtype=np.uint8)
    wc = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    wsc = rng.integers(110, 140, (E, N, K // 32), dtype=np.uint8)
    t = [torch.from_numpy(a).to(DEV) for a in (ac, asc, wc, wsc)]
    y = mx.gemm(*t, offsets=torch.from_numpy(off).to(DEV))
    y_ref, S = oracle.gemm(ac, asc, wc, wsc, off)
    _check_y(y.cpu().numpy(), y_ref, S)


# ------------------------------------------------------------ decode-sized GEMM (M <= 32)

DECODE_SHAPES = [
    ("M1 8 chunks", (1, 200, 2048)),
    ("M3 4 chunks", (3, 5000, 1024)),
    ("M12 ragged N", (12, 1000, 2560)),
    ("M32 2 chunks", (32, 20000, 512)),
    ("M8 odd chunks", (8, 96, 256 * 7)),
    ("M5 16 waves", (5, 70, 256 * 65)),
    ("M32 25 chunks, 4 waves of 4 slots", (32, 64, 256 * 25)),
    ("M4 128 chunks, split 4", (4, 100, 256 * 128)),
]


def decode_parts(M, N, K, split):
    """Number of K parts the decode GEMM uses with row-major activation codes:
    with fewer row tiles than the 256 CUs, 32-row blocks (M <= 8) take the
    largest split up to 4 whose blocks fit two per CU with 8 or more 256-wide
    chunks for each of a block's 4 waves; above 8 rows, 64-row blocks of 2
    waves the largest that fits one per CU.  A forced value replaces it; at
    most one part per chunk."""
    kc = K // 256
    ks = 1
    t32, t64 = (N + 31) // 32, (N + 63) // 64
    if M <= 8 and t32 < 256:
        while ks < 4 and t32 * (ks + 1) <= 512 and kc // ((ks + 1) * 4) >= 8:
            ks += 1
    elif M > 8 and t32 < 256:
        while ks < 4 and t64 * (ks + 1) <= 256 and kc // ((ks + 1) * 2) >= 8:
            ks += 1
    if split:
        ks = split
    return min(ks, kc)



@pytest.mark.parametrize("waves,stages", [(8, 2), (4, 2), (4, 3)])
def test_gemm_decode_forced_rings(waves, stages, tune):
    """Decode rings forced on one M = 32 shape: 8 waves of 2 slots (no longer
    the default choice at M = 32) and 4 waves of 2 or 3 slots; each within
    the oracle's bound (the K split over the waves differs between them, so
    their fp32 sums are not compared bit for bit)."""
    say(f"gemm decode forced waves={waves} stages={stages}")
    tune(mx.TUNE_DECODE_WAVES, waves)
    tune(mx.TUNE_DECODE_STAGES, stages)
    M, N, K = 32, 96, 256 * 26
    rng = np.random.default_rng(2600 + waves)
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    asc = rng.integers(110, 140, (M, K // 32), dtype=np.uint8)
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    wsc = rng.integers(110, 140, (N, K // 32), dtype=np.uint8)
    y = mx.gemm(*[torch.from_numpy(a).to(DEV) for a in (ac, asc, wc, wsc)])
    y_ref, S = oracle.gemm(ac, asc, wc, wsc)
    _check_y(y.cpu().numpy(), y_ref, S)


@pytest.mark.parametrize("split", [0, 1, 3])
@pytest.mark.parametrize("name,shape", DECODE_SHAPES, ids=[n for n, _ in DECODE_SHAPES])
def test_gemm_decode(name, shape, split, tune):
    """Decode GEMM with its automatic K split (row tiles too few to fill the
    GPU, enough chunks per part), and with the split forced off and to 3
    parts (parts of a few chunks, waves with none): within the oracle's
    bound, and the same bits on a second call (the partial sums are added
    in a fixed order)."""
    say(f"gemm decode {name} {shape} split={split}")
    tune(mx.TUNE_DECODE_SPLIT, split)
    M, N, K = shape
    rng = np.random.default_rng(M * 131 + N)
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    asc = rng.integers(110, 140, (M, K // 32), dtype=np.uint8)
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    wsc = rng.integers(110, 140, (N, K // 32), dtype=np.uint8)
    t = [torch.from_numpy(a).to(DEV) for a in (ac, asc, wc, wsc)]
    parts = decode_parts(M, N, K, split)
    want = parts * M * N * 4 if parts > 1 else 0
    assert mx.lib().macaq_gemm_workspace_bytes(M, N, K, 1) == (want + 255) // 256 * 256
    y1 = mx.gemm(*t)
    y2 = mx.gemm(*t)
    y_ref, S = oracle.gemm(ac, asc, wc, wsc)
    _check_y(y1.cpu().numpy(), y_ref, S)
    assert torch.equal(y1, y2)


SPLIT_STALE = [
    ("M4 auto split 4", (4, 100, 256 * 128), 0, mx.EPI_NONE),
    ("M32 64-row tiles 3 parts", (32, 130, 256 * 24), 3, mx.EPI_NONE),
    ("M8 swiglu 2 parts", (8, 96, 256 * 16), 2, mx.EPI_SWIGLU),
]


@pytest.mark.parametrize("fill", ["ones", "random"])
@pytest.mark.parametrize("name,shape,split,epi", SPLIT_STALE, ids=[n for n, *_ in SPLIT_STALE])
def test_gemm_decode_split_stale_workspace(name, shape, split, epi, fill, tune):
    """A K-split decode GEMM on a workspace whose bytes are left over from
    something else (all 0xff, which reads as NaN, or random bytes): every
    partial sum the split reads is written first, so y is within the
    oracle's bound (SwiGLU: the bound carried through silu(g) u) and the
    same bits on a second call."""
    say(f"gemm decode split stale workspace {name} fill={fill}")
    tune(mx.TUNE_DECODE_SPLIT, split)
    M, N, K = shape
    assert decode_parts(M, N, K, split) > 1
    rng = np.random.default_rng(7100 + M + N)
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    asc = rng.integers(110, 140, (M, K // 32), dtype=np.uint8)
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    wsc = rng.integers(110, 140, (N, K // 32), dtype=np.uint8)
    t = [torch.from_numpy(a).to(DEV) for a in (ac, asc, wc, wsc)]
    need = int(mx.lib().macaq_gemm_workspace_bytes(M, N, K, 1))
    host_ws = np.full(need, 0xFF, dtype=np.uint8) if fill == "ones" else rng.integers(0, 256, need, dtype=np.uint8)
    ws = torch.from_numpy(host_ws).to(DEV)
    y1 = mx.gemm(*t, workspace=ws, epilogue=epi)
    y2 = mx.gemm(*t, workspace=ws, epilogue=epi)
    y_ref, S = oracle.gemm(ac, asc, wc, wsc)
    if epi == mx.EPI_SWIGLU:
        bound = oracle.swiglu_bound(y_ref, S, RTOL)
        err = np.abs(y1.cpu().numpy().astype(np.float64) - oracle.swiglu(y_ref))
        assert (err <= bound).all(), f"{(err > bound).sum()} outputs beyond the bound"
    else:
        _check_y(y1.cpu().numpy(), y_ref, S)
    assert torch.equal(y1, y2)


DECODE_LINEAR = [
    ("M1 fp32 tiny-shaped", dict(cfg=1, shape=(1, 96, 512))),
    ("M1", dict(cfg=4, shape=(1, 640, 2048))),
    ("M2 16 waves", dict(cfg=4, shape=(2, 300, 256 * 70))),
    ("M8", dict(cfg=4, shape=(8, 512, 1024))),
    ("M5 ragged N", dict(cfg=4, shape=(5, 300, 256 * 9))),
    ("M8 fp32 x", dict(cfg=1, shape=(8, 96, 512))),
    ("M3 K split", dict(cfg=4, shape=(3, 100, 256 * 128))),
    ("M32", dict(cfg=4, shape=(32, 256, 2560))),
]


@pytest.mark.parametrize("flags", [mx.PATH_FUSED, mx.PATH_UNFUSED, mx.PATH_AUTO])
@pytest.mark.parametrize("name,kw", DECODE_LINEAR, ids=[n for n, _ in DECODE_LINEAR])
def test_linear_decode_paths(name, kw, flags):
    say(f"linear decode {name} flags={flags}")
    wl = workloads.make(**kw)
    wc, wsc = gpu_prepare(wl)
    x, s = wl.x.to(DEV), wl.s.to(DEV)
    y = mx.linear(x, s, wc, wsc, flags=flags)
    y_again = mx.linear(x, s, wc, wsc, flags=flags)
    rwc, rws = oracle_prepare(wl, 0)
    y_ref, S = oracle.linear(host(wl.x), wl.s.numpy(), rwc, rws)
    _check_y(y.cpu().numpy(), y_ref, S)
    assert torch.equal(y, y_again)


ONE_LAUNCH = [
    ("M8", dict(cfg=4, shape=(8, 4160, 1024))),
    ("M3", dict(cfg=4, shape=(3, 4400, 2560))),
    ("M5 ragged N", dict(cfg=4, shape=(5, 3000, 2304))),
    ("M16", dict(cfg=4, shape=(16, 1000, 4096))),
    ("M32", dict(cfg=4, shape=(32, 640, 2560))),
    ("M8 K split 2", dict(cfg=4, shape=(8, 2048, 256 * 64))),
    ("M32 64-row tiles, K split 3", dict(cfg=4, shape=(32, 1024, 256 * 48))),
    ("M8 fp32 x", dict(cfg=1, shape=(8, 4160, 1024))),
]


@pytest.mark.parametrize("name,kw", ONE_LAUNCH, ids=[n for n, _ in ONE_LAUNCH])
def test_linear_one_launch(name, kw):
    """The fused path of a decode-sized layer too large for every block to
    transform the whole activation (ceil(N/32) M K > 2^20): the first blocks
    of the launch publish the transformed activation to the workspace and
    the others wait for it.  On a workspace of stale bytes (all 0xff) and
    again on the one the first call left: the staged codes and scales equal
    macaq_quant_act's bit for bit, y is the same bits on both calls, and
    sampled columns of y, and of the two-launch path's y (which may sum in
    another order), are within the oracle's bound."""
    say(f"linear one launch {name}")
    wl = workloads.make(**kw)
    M, N, K = wl.M, wl.N, wl.K
    assert mx.lib().macaq_linear_path(M, N, K, 1, mx.PATH_FUSED) == mx.PATH_FUSED
    wc, wsc = gpu_prepare(wl)
    x, s = wl.x.to(DEV), wl.s.to(DEV)
    need = mx.linear_workspace_bytes(M, N, K, 1, mx.PATH_FUSED)
    assert need >= (M * K // 2 + 255) // 256 * 256 + (M * K // 32 + 255) // 256 * 256 + 16
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    y1 = mx.linear(x, s, wc, wsc, flags=mx.PATH_FUSED, workspace=ws)
    torch.cuda.synchronize()
    codes, scales = mx.quant_act(x, s)
    sofs = (M * K // 2 + 255) // 256 * 256
    assert torch.equal(ws[: M * K // 2].view(M, K // 2), codes)
    assert torch.equal(ws[sofs: sofs + M * K // 32].view(M, K // 32), scales)
    y2 = mx.linear(x, s, wc, wsc, flags=mx.PATH_FUSED, workspace=ws)
    y_two = mx.linear(x, s, wc, wsc, flags=mx.PATH_UNFUSED)
    assert torch.equal(y1, y2)
    rows = np.unique(np.concatenate([np.arange(0, N, max(1, N // 48)), np.arange(max(0, N - 40), N)]))
    rwc, rws = oracle_prepare(wl, 0, rows)
    y_ref, S = oracle.linear(host(wl.x), wl.s.numpy(), rwc, rws)
    _check_y(y1.cpu().numpy()[:, rows], y_ref, S)
    _check_y(y_two.cpu().numpy()[:, rows], y_ref, S)


@pytest.mark.parametrize("name,kw", [ONE_LAUNCH[0], ONE_LAUNCH[5]], ids=[ONE_LAUNCH[0][0], ONE_LAUNCH[5][0]])
def test_linear_one_launch_gives_up_loudly(name, kw, tune):
    """The one-launch layer's wait for the published activation is bounded.
    Forced to give up at once (MACAQ_TUNE_DECODE_POLLS = 1: no poll), every
    block that waits writes NaN for each output it owns, so y is NaN
    everywhere (with and without a K split) instead of a result of
    unpublished codes; the launch still clears its done words, so the next
    call with the default limit gives the same y as a call that never gave
    up."""
    say(f"linear one launch gives up {name}")
    wl = workloads.make(**kw)
    M, N, K = wl.M, wl.N, wl.K
    wc, wsc = gpu_prepare(wl)
    x, s = wl.x.to(DEV), wl.s.to(DEV)
    ws = torch.zeros(mx.linear_workspace_bytes(M, N, K, 1, mx.PATH_FUSED), dtype=torch.uint8, device=DEV)
    y_ok = mx.linear(x, s, wc, wsc, flags=mx.PATH_FUSED, workspace=ws)
    tune(mx.TUNE_DECODE_POLLS, 1)
    y_nan = mx.linear(x, s, wc, wsc, flags=mx.PATH_FUSED, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isnan(y_nan).all()
    tune(mx.TUNE_DECODE_POLLS, 0)
    y_again = mx.linear(x, s, wc, wsc, flags=mx.PATH_FUSED, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y_again, y_ok)


ROWS_SHARED = [   # (M, N, K): 3 to 32 rows, no K split -> decode_rows_kernel
    (3, 2000, 2560),         # 8 staged rows (rows 3..7 repeat row 2)
    (8, 20000, 512),         # 8 staged rows, 313 blocks
    (9, 1000, 2560),         # 16 staged rows, ragged N (last 64-row block half full)
    (16, 20000, 512),        # 313 blocks: half-LDS budget, 2 chunks
    (17, 640, 256 * 30),     # 32 staged rows, W' scale slabs reused many times
    (31, 4096, 256 * 24),    # 64 blocks, whole LDS budget
    (32, 96, 256 * 3),       # 3 chunks: a ring longer than K
    (24, 300, 256 * 31),     # ragged N (last block 44 rows), odd chunk count
]


@pytest.mark.parametrize("M,N,K", ROWS_SHARED)
@pytest.mark.parametrize("epi", ["f32", "bf16", "swiglu"])
def test_gemm_decode_rows_kernel(M, N, K, epi):
    """The decode GEMM for 3 to 32 rows without a K split (2-wave 64-row
    blocks sharing each staged activation chunk): within the oracle's bound for fp32
    y, within that bound plus one bf16 rounding for bf16 y, and SwiGLU within
    the propagated bound; the same bits on a second call."""
    say(f"gemm decode rows kernel M{M} N{N} K{K} {epi}")
    assert decode_parts(M, N, K, 0) == 1
    rng = np.random.default_rng(9100 + M * 7 + N)
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    asc = rng.integers(110, 140, (M, K // 32), dtype=np.uint8)
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    wsc = rng.integers(110, 140, (N, K // 32), dtype=np.uint8)
    t = [torch.from_numpy(a).to(DEV) for a in (ac, asc, wc, wsc)]
    assert mx.lib().macaq_gemm_workspace_bytes(M, N, K, 1) == 0
    y_ref, S = oracle.gemm(ac, asc, wc, wsc)
    if epi == "f32":
        y1, y2 = mx.gemm(*t), mx.gemm(*t)
        _check_y(y1.cpu().numpy(), y_ref, S)
    elif epi == "bf16":
        y1, y2 = mx.gemm(*t, out_dtype=torch.bfloat16), mx.gemm(*t, out_dtype=torch.bfloat16)
        y = y1.float().cpu().numpy().astype(np.float64)
        tol = RTOL * S + 2.0 ** -8 * (np.abs(y_ref) + RTOL * S)
        assert (np.abs(y - y_ref) <= tol).all()
    else:
        y1, y2 = mx.gemm(*t, epilogue=mx.EPI_SWIGLU), mx.gemm(*t, epilogue=mx.EPI_SWIGLU)
        bound = oracle.swiglu_bound(y_ref, S, RTOL)
        err = np.abs(y1.cpu().numpy().astype(np.float64) - oracle.swiglu(y_ref))
        assert (err <= bound).all(), f"{(err > bound).sum()} outputs beyond the bound"
    assert torch.equal(y1, y2)


ROWS64_GEMM = [(1, 1000, 2560), (3, 200, 2048), (12, 70, 256 * 7), (32, 1000, 2560)]
ROWS64_LINEAR = [
    ("M1 fp32 tiny-shaped", dict(cfg=1, shape=(1, 96, 512))),
    ("M1", dict(cfg=4, shape=(1, 1000, 2560))),
    ("M2", dict(cfg=4, shape=(2, 300, 256 * 9))),
    ("M8", dict(cfg=4, shape=(8, 200, 1024))),
]


@pytest.mark.parametrize("shape", ROWS64_GEMM, ids=[f"M{m} N{n} K{k}" for m, n, k in ROWS64_GEMM])
def test_gemm_decode_64_row_blocks(shape, tune):
    """Blocks of 64 weight rows (two MFMA row tiles per activation chunk),
    ragged N included."""
    say(f"gemm decode 64-row blocks {shape}")
    tune(mx.TUNE_DECODE_ROWS, 64)
    M, N, K = shape
    rng = np.random.default_rng(M * 17 + N)
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    asc = rng.integers(110, 140, (M, K // 32), dtype=np.uint8)
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    wsc = rng.integers(110, 140, (N, K // 32), dtype=np.uint8)
    y = mx.gemm(*[torch.from_numpy(a).to(DEV) for a in (ac, asc, wc, wsc)])
    y_ref, S = oracle.gemm(ac, asc, wc, wsc)
    _check_y(y.cpu().numpy(), y_ref, S)


@pytest.mark.parametrize("flags", [mx.PATH_FUSED, mx.PATH_UNFUSED])
@pytest.mark.parametrize("name,kw", ROWS64_LINEAR, ids=[n for n, _ in ROWS64_LINEAR])
def test_linear_decode_64_row_blocks(name, kw, flags, tune):
    say(f"linear decode 64-row blocks {name} flags={flags}")
    tune(mx.TUNE_DECODE_ROWS, 64)
    wl = workloads.make(**kw)
    wc, wsc = gpu_prepare(wl)
    y = mx.linear(wl.x.to(DEV), wl.s.to(DEV), wc, wsc, flags=flags)
    rwc, rws = oracle_prepare(wl, 0)
    y_ref, S = oracle.linear(host(wl.x), wl.s.numpy(), rwc, rws)
    _check_y(y.cpu().numpy(), y_ref, S)


# ------------------------------------------------------------ pure MXFP4 (no transform)

@pytest.mark.parametrize("name,kw", SMALL_ACT[:4], ids=[n for n, _ in SMALL_ACT[:4]])
def test_quant_mxfp4_plain_bit_exact(name, kw):
    say(f"quant_mxfp4 plain {name}")
    wl = workloads.make(**kw)
    codes, scales = mx.quant_mxfp4(wl.x.to(DEV))
    rc, rs = oracle.quantize_mxfp4(oracle.as_f32(host(wl.x)))
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)

"""bf16 output and SwiGLU over a gate/up projection (macaq_gemm_ex /
macaq_linear_ex) against the oracle.

y (fp32) must satisfy the GEMM bound |y - y_ref| <= 1e-5 S; a bf16 output
adds at most half a bf16 spacing, 2^-8 |y|; a SwiGLU output is checked with
oracle.swiglu_bound (the same GEMM bound carried through silu(g) u).  The
bf16 output must also equal the round-to-nearest-even of the fp32 output of
the same call bit for bit (one fp32 value, two stores).
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


def say(msg):
    print(f"[case] {msg}", flush=True)


def host(t):
    t = t.detach().cpu().contiguous()
    return workloads.bf16_bits(t) if t.dtype == torch.bfloat16 else t.numpy()


def check_plain(y, y_ref, S, bf16):
    y = y.float().cpu().numpy().astype(np.float64)
    tol = RTOL * S + (2.0 ** -8 * (np.abs(y_ref) + RTOL * S) if bf16 else 0.0)
    bad = np.abs(y - y_ref) > tol
    assert not bad.any(), f"{bad.sum()} outputs beyond the bound; worst excess {np.max(np.abs(y - y_ref) - tol):.3g}"


def check_swiglu(y, y_ref, S, bf16):
    y = y.float().cpu().numpy().astype(np.float64)
    ref = oracle.swiglu(y_ref)
    tol = oracle.swiglu_bound(y_ref, S, RTOL)
    if bf16:
        tol = tol + 2.0 ** -8 * (np.abs(ref) + tol)
    bad = np.abs(y - ref) > tol
    assert not bad.any(), f"{bad.sum()} outputs beyond the bound; worst excess {np.max(np.abs(y - ref) - tol):.3g}"


def random_operands(M, N, K, E=1, seed=0):
    rng = np.random.default_rng(seed)
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    asc = rng.integers(118, 132, (M, K // 32), dtype=np.uint8)
    wc = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    wsc = rng.integers(118, 132, (E, N, K // 32), dtype=np.uint8)
    return ac, asc, wc, wsc


GEMM_SHAPES = [
    ("prefill 128x128 tiles, ragged", (300, 260, 1024), 1),
    ("prefill 256x128 tiles", (2048, 512, 512), 1),
    ("decode M5 ragged N", (5, 200, 1024), 1),
    ("decode M32 64-row blocks", (32, 20000, 512), 1),
    ("grouped 3 experts", (333, 256, 512), 3),
]


@pytest.mark.parametrize("name,shape,E", GEMM_SHAPES, ids=[n for n, _, _ in GEMM_SHAPES])
def test_gemm_bf16_and_swiglu(name, shape, E):
    say(f"gemm epilogues {name}")
    M, N, K = shape
    ac, asc, wc, wsc = random_operands(M, N, K, E, seed=M + N)
    off = None
    if E > 1:
        cuts = np.sort(np.random.default_rng(1).integers(0, M, E - 1))
        off_np = np.concatenate([[0], cuts, [M]]).astype(np.int32)
        off = torch.from_numpy(off_np).to(DEV)
    t = [torch.from_numpy(a).to(DEV) for a in (ac, asc, wc, wsc)]
    if E == 1:
        y_ref, S = oracle.gemm(ac, asc, wc[0], wsc[0])
    else:
        y_ref, S = oracle.gemm(ac, asc, wc, wsc, off_np)
    y32 = mx.gemm(*t, offsets=off)
    y16 = mx.gemm(*t, offsets=off, out_dtype=torch.bfloat16)
    check_plain(y32, y_ref, S, False)
    check_plain(y16, y_ref, S, True)
    assert torch.equal(y16, y32.to(torch.bfloat16))
    s32 = mx.gemm(*t, offsets=off, epilogue=mx.EPI_SWIGLU)
    s16 = mx.gemm(*t, offsets=off, epilogue=mx.EPI_SWIGLU, out_dtype=torch.bfloat16)
    assert s32.shape == (M, N // 2)
    check_swiglu(s32, y_ref, S, False)
    check_swiglu(s16, y_ref, S, True)
    assert torch.equal(s16, s32.to(torch.bfloat16))


@pytest.mark.parametrize("tile", ["256x256", "256x128", "128x128"])
def test_gemm_swiglu_each_tile_variant(tile, tune):
    say(f"gemm swiglu tile {tile}")
    tune(mx.TUNE_GEMM_TILE, mx.GEMM_TILES[tile])
    M, N, K = 300, 260, 512
    ac, asc, wc, wsc = random_operands(M, N, K, seed=7)
    t = [torch.from_numpy(a).to(DEV) for a in (ac, asc, wc, wsc)]
    y_ref, S = oracle.gemm(ac, asc, wc[0], wsc[0])
    check_swiglu(mx.gemm(*t, epilogue=mx.EPI_SWIGLU, out_dtype=torch.bfloat16), y_ref, S, True)
    check_plain(mx.gemm(*t, out_dtype=torch.bfloat16), y_ref, S, True)


LINEAR = [
    ("fused M1", dict(cfg=4, shape=(1, 640, 2048)), mx.PATH_FUSED),
    ("fused M2 fp32 x", dict(cfg=1, shape=(2, 96, 512)), mx.PATH_FUSED),
    ("fused M8 resident", dict(cfg=4, shape=(8, 256, 1024)), mx.PATH_FUSED),
    ("fused M16 resident", dict(cfg=4, shape=(16, 256, 1024)), mx.PATH_FUSED),
    ("unfused M64", dict(cfg=2, shape=(64, 256, 1024)), mx.PATH_UNFUSED),
    ("fused M1, K split in 2", dict(cfg=4, shape=(1, 128, 16384)), mx.PATH_FUSED),
    ("unfused M8, K split in 2", dict(cfg=4, shape=(8, 256, 16384)), mx.PATH_UNFUSED),
    ("unfused M16, 64-row blocks, K split in 3", dict(cfg=4, shape=(16, 256, 256 * 48)), mx.PATH_UNFUSED),
]


@pytest.mark.parametrize("name,kw,flags", LINEAR, ids=[n for n, _, _ in LINEAR])
def test_linear_bf16_and_swiglu(name, kw, flags):
    say(f"linear epilogues {name}")
    wl = workloads.make(**kw)
    wc, wsc = mx.prepare_weights(wl.w.to(DEV), wl.s.to(DEV))
    x, s = wl.x.to(DEV), wl.s.to(DEV)
    rwc, rws = oracle.prepare_weights(host(wl.w[0]), wl.s[0].numpy())
    y_ref, S = oracle.linear(host(wl.x), wl.s.numpy(), rwc, rws)
    for dt in (torch.float32, torch.bfloat16):
        y = mx.linear(x, s, wc, wsc, flags=flags, out_dtype=dt)
        check_plain(y, y_ref, S, dt == torch.bfloat16)
        z = mx.linear(x, s, wc, wsc, flags=flags, out_dtype=dt, epilogue=mx.EPI_SWIGLU)
        check_swiglu(z, y_ref, S, dt == torch.bfloat16)

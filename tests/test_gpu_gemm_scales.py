"""The MXFP4 GEMM over the whole E8M0 byte range (0..254 on either operand),
against the oracle, on every GEMM kernel: the prefill tiles (forced), the
grouped GEMM and the decode kernel.

* One nonzero product per output: the fp32 result must be the
  round-to-nearest-even value of the exact product, bit for bit, including
  fp32 subnormals, underflow to zero and overflow to infinity (R30).
* Random codes with extreme byte ranges (bytes 0..10 against 110..140,
  240..254 against 0..10, 0..10 on both sides) and all-zero activation
  groups meeting normal weights: within the GEMM bound plus the underflow
  term of R30, (K/32) * 2^-150.
"""
import numpy as np
import pytest
import torch

import oracle
import mxfp4_w4a4_quantized_channel_amd as mx

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

KERNELS = [   # (name, M, tile override): M <= 32 runs the decode kernel
    ("prefill 256x256", 300, "256x256"),
    ("prefill 256x128", 300, "256x128"),
    ("prefill 128x128", 300, "128x128"),
    ("decode M8", 8, None),
    ("decode M32", 32, None),
]


def gpu_gemm(ac, asc, wc, wsc, off=None):
    t = [torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (ac, asc, wc, wsc)]
    y = mx.gemm(*t, offsets=None if off is None else torch.from_numpy(off).to(DEV))
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("name,M,tile", KERNELS, ids=[k[0] for k in KERNELS])
def test_single_products_round_like_fp32(name, M, tile, tune):
    print(f"[case] single products {name}", flush=True)
    if tile is not None:
        tune(mx.TUNE_GEMM_TILE, mx.GEMM_TILES[tile])
    N, K = 256, 256
    rng = np.random.default_rng(M + 7)
    # row i: one nonzero value (random code) at a random element of group g;
    # weight row j: one nonzero value at the same element; bytes span 0..254
    ga = rng.integers(0, K // 32)
    el = rng.integers(0, 32)
    ac = np.zeros((M, K // 2), np.uint8)
    wc = np.zeros((N, K // 2), np.uint8)
    nonzero = np.array([c for c in range(16) if c & 7], np.uint8)     # no +-0 codes
    ca = rng.choice(nonzero, M)
    cw = rng.choice(nonzero, N)
    byte = ga * 16 + el // 2
    shift = 4 * (el % 2)
    ac[:, byte] = ca << shift
    wc[:, byte] = cw << shift
    asc = rng.integers(100, 150, (M, K // 32), dtype=np.uint8)   # groups of zero codes
    wsc = rng.integers(100, 150, (N, K // 32), dtype=np.uint8)
    asc[:, ga] = np.linspace(0, 254, M).astype(np.uint8)
    wsc[:, ga] = rng.permutation(np.linspace(0, 254, N).astype(np.uint8))
    y = gpu_gemm(ac, asc, wc, wsc)
    y_ref, _ = oracle.gemm(ac, asc, wc, wsc)
    with np.errstate(over="ignore"):
        want = y_ref.astype(np.float32)        # one rounding of the exact value
    # equal values: bit for bit, except that a product which underflows may
    # give either signed zero
    assert (y == want).all(), f"{int((y != want).sum())} outputs differ"
    # the sweep reaches every regime: subnormal, zero by underflow, infinity
    a = np.abs(want[want != 0])
    assert (a < 2.0 ** -126).any() and (want == 0).any() and np.isinf(want).any()


REGIMES = [   # (name, activation byte range, weight byte range)
    ("act 0..10, w 110..140 (subnormal products)", (0, 11), (110, 141)),
    ("act 110..140, w 0..10", (110, 141), (0, 11)),
    ("act 240..254, w 0..10", (240, 255), (0, 11)),
    ("act 0..10, w 240..254", (0, 11), (240, 255)),
    ("act 0..10, w 0..10 (everything underflows)", (0, 11), (0, 11)),
]


@pytest.mark.parametrize("rname,ar,wr", REGIMES, ids=[r[0] for r in REGIMES])
@pytest.mark.parametrize("name,M,tile", KERNELS, ids=[k[0] for k in KERNELS])
def test_random_codes_extreme_scale_bytes(name, M, tile, rname, ar, wr, tune):
    print(f"[case] extreme bytes {name} {rname}", flush=True)
    if tile is not None:
        tune(mx.TUNE_GEMM_TILE, mx.GEMM_TILES[tile])
    N, K = 160, 1024
    rng = np.random.default_rng(M * 31 + ar[0] + 7 * wr[0])
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    asc = rng.integers(*ar, (M, K // 32), dtype=np.uint8)
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    wsc = rng.integers(*wr, (N, K // 32), dtype=np.uint8)
    # all-zero activation groups (byte 0, codes 0 / -0) in some rows
    zr = rng.choice(M, max(1, M // 4), replace=False)
    for r in zr:
        g = rng.choice(K // 32, K // 64, replace=False)
        asc[r, g] = 0
        for gg in g:
            ac[r, gg * 16:(gg + 1) * 16] = rng.choice([0x00, 0x08, 0x80, 0x88], 16)
    y = gpu_gemm(ac, asc, wc, wsc)
    y_ref, S = oracle.gemm(ac, asc, wc, wsc)
    ok, worst, normwise = oracle.within_tolerance(y, y_ref, S, 1e-5, groups=K // 32)
    assert ok, f"worst {worst:.3g} normwise {normwise:.3g}"


def test_grouped_extreme_scale_bytes():
    """The grouped GEMM with experts whose weights sit at opposite ends of
    the byte range, and empty experts."""
    print("[case] grouped extreme bytes", flush=True)
    E, N, K = 4, 96, 512
    counts = np.array([70, 0, 130, 45])
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(off[-1])
    rng = np.random.default_rng(404)
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    asc = rng.integers(0, 255, (M, K // 32), dtype=np.uint8)
    wc = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    wsc = np.stack([rng.integers(lo, hi, (N, K // 32), dtype=np.uint8)
                    for lo, hi in ((0, 11), (110, 141), (240, 255), (60, 200))])
    asc = np.minimum(asc, 100)     # no product beyond fp32's range
    y = gpu_gemm(ac, asc, wc, wsc, off)
    y_ref, S = oracle.gemm(ac, asc, wc, wsc, off)
    ok, worst, normwise = oracle.within_tolerance(y, y_ref, S, 1e-5, groups=K // 32)
    assert ok, f"worst {worst:.3g} normwise {normwise:.3g}"

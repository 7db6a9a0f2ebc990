"""Pins of the CPU oracle to facts fixed outside it (closed forms, invariants,
brute force, hand-worked fixtures).  No GPU needed.

Each test names the plausible oracle mistake it would catch.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- Hadamard

def test_hadamard_closed_form_and_orthogonality():
    """Sylvester recursion == (-1)^popcount(i&j); H H^T = 32 I exactly;
    normalized H is orthogonal to 1e-15.  Catches a wrong sign/index in H."""
    h = oracle.sylvester_hadamard(32)
    closed = np.array([[(-1) ** bin(i & j).count("1") for j in range(32)] for i in range(32)])
    assert np.array_equal(h, closed)
    assert np.array_equal(h @ h.T, 32 * np.eye(32, dtype=np.int64))
    hn = h / np.sqrt(32.0)
    assert np.abs(hn @ hn.T - np.eye(32)).max() < 1e-15


def test_c_norm_bits():
    """C = RNE_f32(1/sqrt(32)) has the bit pattern 0x3E3504F3."""
    assert int(np.float32(oracle.C_NORM).view(np.uint32)) == 0x3E3504F3


def test_fwht_integer_inputs_equal_dense_product():
    """On small integers every fp32 add is exact, so the butterfly must equal
    t @ H32 exactly.  Catches a swapped a-b, a missing stage, a wrong pair."""
    rng = np.random.default_rng(1)
    t = rng.integers(-1000, 1000, size=(257, 32)).astype(np.float32)
    got = oracle.fwht32(t)
    want = t.astype(np.int64) @ oracle.sylvester_hadamard(32)
    assert np.array_equal(got.astype(np.int64), want)


def _fwht_recursive(t):
    """Butterfly from the doubling recursion H_2m = [[H,H],[H,-H]]: transform
    both halves, then combine (lower = a + b, upper = a - b), one fp32 rounding
    per operation.  Written independently of the oracle's loop."""
    n = t.shape[-1]
    if n == 1:
        return t.copy()
    a = _fwht_recursive(t[..., : n // 2])
    b = _fwht_recursive(t[..., n // 2:])
    return np.concatenate([(a + b).astype(np.float32), (a - b).astype(np.float32)], axis=-1)


def test_fwht_fp32_bits_equal_recursive_definition():
    """Bitwise equality with the recursive Sylvester definition on random fp32
    (rounding depends on operation order: catches a reversed stage order)."""
    rng = np.random.default_rng(2)
    t = (rng.standard_normal((4096, 32)) * np.exp(rng.uniform(-8, 8, (4096, 32)))).astype(np.float32)
    got = oracle.fwht32(t)
    want = _fwht_recursive(t)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # a descending-order butterfly gives different bits on such data
    rev = t.copy()
    for h in (16, 8, 4, 2, 1):
        lo = [i for i in range(32) if (i & h) == 0]
        hi = [i + h for i in lo]
        a, b = rev[:, lo], rev[:, hi]
        rev[:, lo], rev[:, hi] = a + b, a - b
    assert not np.array_equal(got.view(np.uint32), rev.view(np.uint32))


def test_transform_fp32_close_to_fp64_dense():
    """fp32 transform within the fp32 error bound of the fp64 dense product."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    s = np.exp(rng.uniform(-2, 2, 256)).astype(np.float32)
    got = oracle.transform(x, s).astype(np.float64)
    want = oracle.transform_dense_fp64(x, s)
    mag = np.abs(x.astype(np.float64) * s).reshape(64, 8, 32).sum(-1, keepdims=True)
    bound = 8 * 2.0 ** -24 * np.broadcast_to(mag, (64, 8, 32)).reshape(64, 256) / np.sqrt(32)
    assert np.all(np.abs(got - want) <= bound + 1e-30)


@pytest.mark.parametrize("cfg,shape", [(1, None), (2, (64, 96, 512)), (3, (32, 64, 1024)),
                                       (4, (8, 64, 1024)), (5, (256, 32, 256))])
def test_layer_equivalence_before_quantization(cfg, shape):
    """(x diag(s) H)(W diag(1/s) H)^T == x W^T in fp64 to 1e-12 (the absorbed
    inverse leaves the layer unchanged).  Catches H not orthogonal, s applied
    to the wrong operand, a transposed block."""
    wl = workloads.make(cfg, shape=shape) if shape else workloads.make(cfg)
    x = wl.x.to(dtype=__import__("torch").float64).numpy()
    off = wl.offsets.numpy()
    for e in range(wl.E):
        r0, r1 = off[e], off[e + 1]
        if r1 <= r0:
            continue
        W = wl.w[e].to(dtype=__import__("torch").float64).numpy()
        s = wl.s[e].numpy().astype(np.float64)
        xp = oracle.transform_dense_fp64(x[r0:r1], s)
        wp = oracle.transform_dense_fp64(W, 1.0 / s)
        y = xp @ wp.T
        ref = x[r0:r1] @ W.T
        comp = np.abs(x[r0:r1]) @ np.abs(W).T
        assert np.max(np.abs(y - ref) / comp) <= 1e-12
        assert np.linalg.norm(y - ref) / np.linalg.norm(ref) <= 1e-12


# ---------------------------------------------------------------- E8M0

def test_e8m0_bit_rule_and_invariant():
    """Shared exponent = floor(log2 amax) - 2, clamped; checked against the
    fp32 exponent field (an independent formula) and 4*2^e <= amax < 8*2^e.
    Catches an off-by-one emax or a wrong clamp."""
    rng = np.random.default_rng(4)
    bits = rng.integers(0, 0x7F800000, size=200000, dtype=np.uint32)
    specials = np.array([0, 1, 2, 0x007FFFFF, 0x00800000, 0x3F800000, 0x3F7FFFFF,
                         0x40800000, 0x407FFFFF, 0x7F7FFFFF, 0x01800000, 0x01FFFFFF], dtype=np.uint32)
    bits = np.concatenate([bits, specials])
    amax = bits.view(np.float32)
    got = oracle.e8m0_scale(amax).astype(np.int64)
    want = np.maximum(((bits >> 23) & 0xFF).astype(np.int64) - 2, 0)
    want = np.where(amax == 0, 0, want)
    assert np.array_equal(got, want)
    e = got - 127
    a = amax.astype(np.float64)
    ok = a >= 2.0 ** -125
    assert np.all(4 * 2.0 ** e[ok] <= a[ok]) and np.all(a[ok] < 8 * 2.0 ** e[ok])
    assert np.all(a[~ok] < 8 * 2.0 ** -127)


# ---------------------------------------------------------------- E2M1

def test_e2m1_table_from_bit_fields():
    """Magnitude table rebuilt from the E2M1 bit fields (bias 1, one
    subnormal) and compared with the golden OCP table."""
    gold = _load("e2m1_table.json")
    for code in range(16):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        val = (0.5 * m) if e == 0 else (2.0 ** (e - 1)) * (1 + m / 2)
        val = -val if s else val
        g = gold["codes"][hex(code)]
        assert val == g and np.signbit(val) == np.signbit(g)
        assert oracle.E2M1_VALUES[code & 7] == abs(g)
    assert gold["emax"] == oracle.E2M1_EMAX


def _round_by_quantum(v):
    """Independent RNE onto E2M1: the grid spacing is 0.5 below 2, 1 in [2,4)
    and 2 from 4; round v/spacing half-to-even; saturate at 6."""
    v = np.asarray(v, dtype=np.float64)
    q = np.where(v < 2, 0.5, np.where(v < 4, 1.0, 2.0))
    return np.minimum(np.round(v / q) * q, 6.0)


def test_e2m1_rounding_exhaustive():
    """Every fp32 value in [0.25, 8) (all values below round to 0) plus the
    tiny range sampled: nearest-code argmin == spacing-based RNE.  Catches a
    tie sent the wrong way or a missing saturation."""
    lo = int(np.float32(0.25).view(np.uint32))
    hi = int(np.float32(8.0).view(np.uint32))
    step = 1 << 22
    for b0 in range(lo, hi, step):
        bits = np.arange(b0, min(hi, b0 + step), dtype=np.uint32)
        v = bits.view(np.float32)
        idx = oracle.e2m1_nearest(v)
        assert np.array_equal(oracle.E2M1_VALUES[idx], _round_by_quantum(v)), hex(b0)
    rng = np.random.default_rng(5)
    small = rng.integers(0, lo, size=100000, dtype=np.uint32).view(np.float32)
    assert np.all(oracle.e2m1_nearest(small) == 0)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 100.0])
    assert list(oracle.E2M1_VALUES[oracle.e2m1_nearest(ties)]) == [0, 1, 1, 2, 2, 4, 4, 6, 6]
    # saturation holds for every finite magnitude up to the fp32 maximum
    big = np.array([8.0, 1e10, 2.0 ** 100, 3.4e38, np.finfo(np.float32).max], dtype=np.float32)
    assert np.all(oracle.e2m1_nearest(big) == 7)


def test_quantizer_round_trip_of_representable_groups():
    """Groups of exactly representable values val*2^e whose largest magnitude
    is 4 or 6 (so the shared exponent is e) come back unchanged."""
    rng = np.random.default_rng(6)
    R = 512
    codes = rng.integers(0, 16, size=(R, 32)).astype(np.uint8)
    top = np.where(rng.integers(0, 2, R) == 1, 7, 6).astype(np.uint8)
    codes[:, 0] = top | (codes[:, 0] & 8)
    codes[:, 1:] = np.minimum(codes[:, 1:] & 7, top[:, None]) | (codes[:, 1:] & 8)
    e = rng.integers(-120, 120, size=R)
    vals = np.where(codes & 8, -1.0, 1.0) * oracle.E2M1_VALUES[codes & 7] * np.ldexp(1.0, e)[:, None]
    packed, scales = oracle.quantize_mxfp4(vals.astype(np.float32))
    want = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    assert np.array_equal(scales[:, 0].astype(np.int64), e + 127)
    assert np.array_equal(packed, want)
    assert np.array_equal(oracle.dequantize_mxfp4(packed, scales), vals)


def test_worked_groups():
    """Hand-worked spike / constant / zero groups from the golden file."""
    gold = _load("worked_groups.json")
    for case in gold["cases"]:
        x = np.zeros((1, 32), dtype=np.float32)
        for k, v in case["x"].items():
            if k == "all":
                x[:] = v
            else:
                x[0, int(k)] = v
        packed, scales = oracle.quant_act(x, np.ones((1, 32), np.float32))
        assert int(scales[0, 0]) == case["scale"], case["name"]
        assert packed[0].tobytes().hex() == case["bytes"], case["name"]


def test_spike_closed_form_all_positions():
    """A spike c at position j gives 32 outputs of magnitude RNE(c*C) with
    signs (-1)^popcount(i&j); constant groups give one nonzero output."""
    rng = np.random.default_rng(7)
    for j in range(32):
        c = np.float32(rng.standard_normal() * 10)
        t = np.zeros((1, 32), np.float32)
        t[0, j] = c
        out = oracle.transform(t, np.ones(32, np.float32))[0]
        mag = np.float32(c * oracle.C_NORM)
        sign = np.array([(-1) ** bin(i & j).count("1") for i in range(32)], np.float32)
        assert np.array_equal(out.view(np.uint32), (sign * mag).astype(np.float32).view(np.uint32))
    c = np.float32(0.3)
    out = oracle.transform(np.full((1, 32), c, np.float32), np.ones(32, np.float32))[0]
    assert out[0] == np.float32(np.float32(32 * c) * oracle.C_NORM)
    assert np.all(out[1:] == 0) and not np.any(np.signbit(out[1:]))


def test_sign_of_zero_kept():
    """A negative value that rounds to 0 keeps the sign bit (code 0x8)."""
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 6.0
    packed, scales = oracle.quantize_mxfp4(x.copy())
    assert packed[0, 0] == 0x07
    x[0, 1] = -0.001
    packed, _ = oracle.quantize_mxfp4(x)
    assert packed[0, 0] == 0x87
    x[0, 1] = -0.0
    packed, _ = oracle.quantize_mxfp4(x)
    assert packed[0, 0] == 0x87


def test_storage_is_4p25_bits():
    """Bytes per row = K/2 codes + K/32 scales = 4.25 bit per element."""
    gold = _load("mxfp4_storage.json")
    K = 4096
    packed, scales = oracle.quantize_mxfp4(np.ones((3, K), np.float32))
    bits = 8 * (packed.shape[1] + scales.shape[1]) / K
    assert bits == gold["bits_per_element"]
    assert K // scales.shape[1] == gold["group_size"]


# ---------------------------------------------------------------- GEMM

def _brute_gemm(ac, asc, wc, wsc):
    """Triple loop over dequantized scalars (pure Python)."""
    M, N, K = ac.shape[0], wc.shape[0], 2 * ac.shape[1]

    def val(codes, scales, r, k):
        byte = int(codes[r, k // 2])
        c = (byte >> 4) if k % 2 else (byte & 0xF)
        mag = [0, 0.5, 1, 1.5, 2, 3, 4, 6][c & 7]
        return (-mag if c & 8 else mag) * 2.0 ** (int(scales[r, k // 32]) - 127)

    y = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            y[m, n] = sum(val(ac, asc, m, k) * val(wc, wsc, n, k) for k in range(K))
    return y


def test_gemm_brute_force_tiny():
    rng = np.random.default_rng(8)
    ac = rng.integers(0, 256, size=(3, 32), dtype=np.uint8)
    asc = rng.integers(100, 150, size=(3, 2), dtype=np.uint8)
    wc = rng.integers(0, 256, size=(5, 32), dtype=np.uint8)
    wsc = rng.integers(100, 150, size=(5, 2), dtype=np.uint8)
    y, S = oracle.gemm(ac, asc, wc, wsc)
    assert np.array_equal(y, _brute_gemm(ac, asc, wc, wsc))
    assert np.all(S >= np.abs(y))


def test_gemm_one_hot_selects_activation_values():
    """W' rows with a single code 2 (=1.0) at scale 127 select one dequantized
    activation value exactly."""
    rng = np.random.default_rng(9)
    K = 256
    ac = rng.integers(0, 256, size=(4, K // 2), dtype=np.uint8)
    asc = rng.integers(110, 140, size=(4, K // 32), dtype=np.uint8)
    wc = np.zeros((K, K // 2), np.uint8)
    for k in range(K):
        wc[k, k // 2] = 0x2 << (4 * (k % 2))
    wsc = np.full((K, K // 32), 127, np.uint8)
    y, _ = oracle.gemm(ac, asc, wc, wsc)
    assert np.array_equal(y, oracle.dequantize_mxfp4(ac, asc))


def test_gemm_grouped_uses_each_experts_weights():
    rng = np.random.default_rng(10)
    E, N, K, M = 3, 8, 64, 7
    ac = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    asc = rng.integers(120, 130, size=(M, K // 32), dtype=np.uint8)
    wc = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    wsc = rng.integers(120, 130, size=(E, N, K // 32), dtype=np.uint8)
    off = np.array([0, 3, 3, 7])
    y, _ = oracle.gemm(ac, asc, wc, wsc, off)
    for m in range(M):
        e = 0 if m < 3 else 2
        assert np.array_equal(y[m], _brute_gemm(ac[m:m + 1], asc[m:m + 1], wc[e], wsc[e])[0])


def test_quantized_layer_reduces_error_with_scale_and_rotation():
    """On the outlier-heavy tiny layer, the quantized layer's error drops when
    the block Hadamard and then the channel scale are added (the direction of
    the pages' ablation)."""
    wl = workloads.make(1)
    x = wl.x.numpy()
    W = wl.w[0].numpy()
    s = wl.s[0].numpy()
    ref = x.astype(np.float64) @ W.astype(np.float64).T

    def err(use_h, use_s):
        sx = s if use_s else np.ones_like(s)
        sw = oracle.weight_reciprocal(sx)
        if use_h:
            ax = oracle.transform(x, sx)
            aw = oracle.transform(W, sw)
        else:
            ax = (x * sx).astype(np.float32)
            aw = (W * sw).astype(np.float32)
        y, _ = oracle.gemm(*oracle.quantize_mxfp4(ax), *oracle.quantize_mxfp4(aw))
        return np.linalg.norm(y - ref) / np.linalg.norm(ref)

    plain, rot, both = err(False, False), err(True, False), err(True, True)
    assert both < rot < plain


def test_within_tolerance_rejects_planted_error():
    """The acceptance check flags a single perturbed output."""
    rng = np.random.default_rng(11)
    y = rng.standard_normal((16, 16))
    S = np.abs(y) + 1.0
    assert oracle.within_tolerance(y, y, S)[0]
    y2 = y.copy()
    y2[3, 4] += 1e-3
    assert not oracle.within_tolerance(y2, y, S)[0]


# ---------------------------------------------------------------- consumer step: bf16 output, SwiGLU

def test_gemm_single_product_closed_form_over_all_scale_bytes():
    """One nonzero value per row and K = 32: the dequantized fp64 GEMM equals
    (-1)^(sa^sw) val_a val_w 2^(ba + bw - 254) (E2M1 value by its bit
    fields, scale 2^(b - 127) per the OCP E8M0 definition) for every scale
    byte 0..254 on both sides, including products far outside fp32's range."""
    import math
    rng = np.random.default_rng(30)
    ba = np.arange(0, 255, dtype=np.uint8)
    bw = rng.permutation(ba)
    ca = rng.integers(0, 16, ba.size).astype(np.uint8)
    cw = rng.integers(0, 16, ba.size).astype(np.uint8)
    pa = np.zeros((ba.size, 16), np.uint8)
    pw = np.zeros((ba.size, 16), np.uint8)
    pa[:, 0], pw[:, 0] = ca, cw                     # element 0 in the low nibble
    y, S = oracle.gemm(pa, ba[:, None], pw, bw[:, None])

    def value(code):   # E2M1: sign bit 3, exponent bits 2:1 (bias 1), mantissa bit 0
        e, m = (int(code) >> 1) & 3, int(code) & 1
        mag = (m / 2.0) if e == 0 else (1 + m / 2.0) * 2.0 ** (e - 1)
        return -mag if code & 8 else mag
    for i in range(ba.size):
        for j in range(ba.size):
            want = math.ldexp(value(ca[i]) * value(cw[j]), int(ba[i]) + int(bw[j]) - 254)
            assert y[i, j] == want and S[i, j] == abs(want)


def test_within_tolerance_underflow_term():
    """R30: with groups = g the bound gains g * 2^-150 (absolute); without it
    a zero reference demands an exact zero, and anything beyond the bound is
    rejected."""
    zero = np.zeros((1, 1))
    tiny = np.array([[2.0 ** -150]])
    assert not oracle.within_tolerance(tiny, zero, zero, 1e-5)[0]
    assert oracle.within_tolerance(tiny, zero, zero, 1e-5, groups=1)[0]
    assert not oracle.within_tolerance(2 * tiny, zero, zero, 1e-5, groups=1)[0]
    assert oracle.within_tolerance(4 * tiny, zero, zero, 1e-5, groups=4)[0]
    ref, S = np.array([[1.0]]), np.array([[1.0]])
    assert oracle.within_tolerance(ref + 0.9e-5, ref, S, 1e-5, groups=8)[0]
    assert not oracle.within_tolerance(ref + 1.1e-5, ref, S, 1e-5, groups=8)[0]


def test_round_bf16_matches_torch_and_breaks_ties_to_even():
    import torch
    rng = np.random.default_rng(11)
    v = (rng.standard_normal(200000) * np.exp2(rng.integers(-30, 30, 200000))).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(oracle.round_bf16(v), ref)
    # exact halfway cases: 1 + 2^-8 lies between bf16 1 and 1 + 2^-7 -> even (1);
    # 1 + 3*2^-8 lies between 1 + 2^-7 and 1 + 2^-6 -> even (1 + 2^-6)
    half = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8)], dtype=np.float32)
    assert np.array_equal(oracle.round_bf16(half), np.array([1.0, 1 + 2.0 ** -6, -1.0], dtype=np.float32))


def test_swiglu_matches_logistic_and_closed_forms():
    from scipy.special import expit
    rng = np.random.default_rng(12)
    y = rng.standard_normal((7, 64)) * 4
    g, u = y[:, 0::2], y[:, 1::2]
    np.testing.assert_allclose(oracle.swiglu(y), g * expit(g) * u, rtol=1e-13, atol=1e-300)
    assert oracle.swiglu(np.array([[0.0, 5.0]]))[0, 0] == 0.0
    assert oracle.swiglu(np.array([[60.0, 2.0]]))[0, 0] == pytest.approx(120.0, rel=1e-12)
    assert abs(oracle.swiglu(np.array([[-60.0, 2.0]]))[0, 0]) < 1e-20
    # silu(1) = 1 / (1 + e^-1)
    assert oracle.swiglu(np.array([[1.0, 1.0]]))[0, 0] == pytest.approx(1 / (1 + np.exp(-1.0)), rel=1e-15)


def test_swiglu_bound_covers_perturbations_within_the_gemm_tolerance():
    rng = np.random.default_rng(13)
    y = rng.standard_normal((50, 40)) * 3
    S = np.abs(y) * 5 + 1
    y_pert = y + 1e-5 * S * rng.uniform(-1, 1, y.shape)
    d = np.abs(oracle.swiglu(y_pert) - oracle.swiglu(y))
    assert np.all(d <= oracle.swiglu_bound(y, S))
    # and the bound is not vacuous: a 10x larger perturbation breaks it somewhere
    y_far = y + 1e-4 * S
    assert np.any(np.abs(oracle.swiglu(y_far) - oracle.swiglu(y)) > oracle.swiglu_bound(y, S))

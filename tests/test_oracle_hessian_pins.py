"""Pins of the oracle's offline Hessian steps: the Hessian of the transformed
layer input and the Hessian exponent search for the weights' scale bytes.
No GPU needed.  Each test names the plausible oracle mistake it would catch.
"""
from fractions import Fraction

import numpy as np

import oracle

E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]


def _rng(*k):
    return np.random.default_rng(np.random.SeedSequence([7, *k]))


# ---------------------------------------------------------------- Hessian

def _block_hadamard(K):
    hn = oracle.sylvester_hadamard(32).astype(np.float64) / np.sqrt(32.0)
    return np.kron(np.eye(K // 32), hn)


def test_hessian_is_rotated_plain_hessian():
    """H' = B^T D (X^T X) D B with B the dense block Hadamard and D = diag(s):
    the Hessian in the transformed basis is the rotated Hessian of x * s.
    Catches a Hessian of the untransformed input, s applied inversely, or a
    transposed block."""
    T, K = 40, 128
    x = (_rng(1).standard_normal((T, K)) * 3).astype(np.float32)
    s = _rng(2).uniform(0.2, 4.0, K).astype(np.float32)
    h = oracle.hessian(x, s[None])[0]
    d = np.diag(s.astype(np.float64))
    b = _block_hadamard(K)
    xd = x.astype(np.float64)
    ref = b.T @ d @ (xd.T @ xd) @ d @ b
    xs = np.abs(oracle.transform_dense_fp64(x, s))
    bound = 1e-6 * (xs.T @ xs)
    assert np.all(np.abs(h - ref) <= bound)


def test_hessian_experts_and_empty_expert():
    """Each expert uses only its own rows and its own s; an expert without rows
    gets an all-zero Hessian.  Catches a shared s or rows of the wrong expert."""
    K = 64
    off = np.array([0, 10, 10, 25])
    x = _rng(3).standard_normal((25, K)).astype(np.float32)
    s = _rng(4).uniform(0.5, 2.0, (3, K)).astype(np.float32)
    h = oracle.hessian(x, s, off)
    assert h.shape == (3, K, K)
    assert not h[1].any()
    for e in (0, 2):
        r0, r1 = off[e], off[e + 1]
        assert np.array_equal(h[e], oracle.hessian(x[r0:r1], s[e][None])[0])
        assert not np.array_equal(h[e], oracle.hessian(x[r0:r1], s[2 - e][None])[0])


def test_hessian_symmetric_psd_trace():
    """H' is symmetric and positive semidefinite, and its trace equals
    sum ||x * s||^2 (the block Hadamard is orthogonal).  Catches a missing
    normalization C or a non-orthogonal butterfly."""
    T, K = 64, 96
    x = _rng(5).standard_normal((T, K)).astype(np.float32)
    s = _rng(6).uniform(0.5, 2.0, K).astype(np.float32)
    h = oracle.hessian(x, s[None])[0]
    assert np.array_equal(h, h.T)
    ev = np.linalg.eigvalsh(h)
    assert ev.min() >= -1e-9 * ev.max()
    tr = float(np.sum((x.astype(np.float64) * s) ** 2))
    assert abs(np.trace(h) - tr) <= 1e-6 * tr


# ---------------------------------------------------------------- exponent search

def _nearest_index(v: Fraction) -> int:
    """Brute-force nearest E2M1 magnitude; a tie goes to the even index."""
    best = min(range(8), key=lambda i: (abs(v - E2M1[i]), i % 2))
    return best


def _exact_group(xg, b, hb):
    """Exact codes and exact Hessian error of one fp32 group at scale byte b."""
    sc = Fraction(2) ** (int(b) - 127)
    codes, delta = [], []
    for v in xg:
        fv = Fraction(float(v))
        m = _nearest_index(abs(fv) / sc)
        neg = bool(np.signbit(v))
        codes.append((8 if neg else 0) | m)
        deq = (-1 if neg else 1) * E2M1[m] * sc
        delta.append(fv - deq)
    hf = [[Fraction(float(hb[i, j])) for j in range(32)] for i in range(32)]
    q = sum(delta[i] * sum(hf[i][j] * delta[j] for j in range(32)) for i in range(32))
    return codes, q


def _plain_b(xg):
    amax = max(abs(float(v)) for v in xg)
    if amax == 0:
        return 0
    e = int(np.floor(np.log2(amax))) - 2
    return max(min(e, 127), -127) + 127


def test_search_matches_exact_rational_bruteforce():
    """Exhaustive over the two candidates in exact rational arithmetic, with a
    brute-force nearest code: the oracle keeps b0 + 1 exactly when its exact
    Hessian-weighted error is smaller, and emits that candidate's codes.
    Catches a dropped cross term, a wrong sign in delta, the wrong candidate
    set, or a tie that moves the scale."""
    R, G = 6, 3
    rng = _rng(8)
    # heavy tails so that many groups saturate at the plain exponent
    xp = (rng.standard_t(2, (R, 32 * G)) * 2.0 ** rng.integers(-3, 4, (R, 1))).astype(np.float32)
    a = rng.standard_normal((G, 32, 40))
    hb = np.einsum("gik,gjk->gij", a, a).astype(np.float32)
    codes, scales = oracle.search_exponents(xp, hb)
    code = oracle.unpack_codes(codes).reshape(R, G, 32)
    ups = 0
    for r in range(R):
        for g in range(G):
            xg = xp[r, 32 * g:32 * (g + 1)]
            b0 = _plain_b(xg)
            c0, q0 = _exact_group(xg, b0, hb[g])
            c1, q1 = _exact_group(xg, b0 + 1, hb[g])
            if q0 != 0 and abs(q1 - q0) <= Fraction(1, 10 ** 9) * q0:
                continue   # near tie: decided by fp64 rounding, not pinned here
            up = q1 < q0
            ups += up
            assert scales[r, g] == (b0 + 1 if up else b0)
            assert list(code[r, g]) == (c1 if up else c0)
    assert 0 < ups < R * G   # both outcomes occur


def test_search_zero_hessian_is_plain_rule():
    """H = 0 makes both errors 0, and a tie keeps the plain scale: the search
    reduces to the OCP rule (prepare_weights).  Catches a tie rule that
    prefers b0 + 1."""
    rng = _rng(9)
    w = (rng.standard_normal((16, 128)) * 0.02).astype(np.float32)
    s = rng.uniform(0.3, 3.0, 128).astype(np.float32)
    got = oracle.prepare_weights_hessian(w, s, np.zeros((128, 128), np.float32))
    ref = oracle.prepare_weights(w, s)
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


def _group(vals):
    g = np.zeros(32, np.float32)
    g[:len(vals)] = vals
    return g


def test_search_worked_groups():
    """Hand-worked groups, H = I unless stated (values in units of 2^e):
    * [7.75, 0...]: b0 saturates to 6 (error 1.75^2); b0+1 rounds 3.875 up to
      4, i.e. 8 (error 0.25^2) -> b0 + 1, code 6 (= 4.0) at element 0.
    * [4, 1.5, -0.5, 3] * 8: exact at b0 (error 0) -> b0, exact codes.
    * [5.5, 1.25 x 31]: both candidates give the same deltas (-0.5, 0.25...)
      -> tie -> b0.
    * [7, 0.6] with H = [[1, -0.5], [-0.5, 1]]: b0 gives deltas (1, 0.1), error
      0.91; b0+1 (codes 4 and 0.5, i.e. 8 and 1) gives (-1, -0.4), error 0.76
      -> b0 + 1.  With H = I the same
      group keeps b0 (1.01 < 1.16): the cross term decides."""
    eye = np.eye(32, dtype=np.float32)
    cases = []
    cases.append((_group([7.75]), eye, 128, [6] + [0] * 31))
    cases.append((_group([32.0, 12.0, -4.0, 24.0]), eye, 130, [6, 3, 9, 5] + [0] * 28))
    cases.append((_group([5.5] + [1.25] * 31), eye, 127, [7] + [2] * 31))
    hc = eye.copy()
    hc[0, 1] = hc[1, 0] = -0.5
    cases.append((_group([7.0, 0.6]), hc, 128, [6, 1] + [0] * 30))
    cases.append((_group([7.0, 0.6]), eye, 127, [7, 1] + [0] * 30))
    for xg, h, b, code in cases:
        c, sc = oracle.search_exponents(xg[None], h[None])
        assert int(sc[0, 0]) == b
        assert list(oracle.unpack_codes(c)[0]) == code


def test_search_power_of_two_invariance():
    """Scaling x' by 2^k shifts every chosen scale byte by k and keeps the
    codes; scaling H by 4 changes nothing (the errors scale exactly).
    Catches rounding in the error that depends on magnitude, or a decision
    taken on a relative threshold."""
    rng = _rng(10)
    xp = (rng.standard_t(3, (8, 128))).astype(np.float32)
    a = rng.standard_normal((4, 32, 32))
    hb = np.einsum("gik,gjk->gij", a, a).astype(np.float32)
    c0, s0 = oracle.search_exponents(xp, hb)
    for k in (-5, 3):
        c1, s1 = oracle.search_exponents((xp * np.float32(2.0 ** k)).astype(np.float32), hb)
        assert np.array_equal(c0, c1) and np.array_equal(s1.astype(int), s0.astype(int) + k)
    c2, s2 = oracle.search_exponents(xp, (hb * 4).astype(np.float32))
    assert np.array_equal(c0, c2) and np.array_equal(s0, s2)

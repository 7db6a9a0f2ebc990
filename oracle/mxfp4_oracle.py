"""CPU oracle for the MXFP4 W4A4 linear layer with an online per-channel
scale and a 32-element block Hadamard transform.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only
the test suite, the smoke check and the benchmark's CPU-baseline leg use it.
It is a plain, slow, step-by-step restatement of what the layer computes,
written from these sources (cited by page title and section):

* [abstract]  "MACaQ: Fast, Model Agnostic Calibrated Quantization for
  Low-Precision Weights and Activations" (Hugging Face Daily Papers mirror),
  Abstract: a per-channel scale and a block-Hadamard transform are applied
  online to each layer's activations; the inverse transforms are absorbed
  into the weights.
* [mechanism] "MACaQ Enables Streaming W4A4 Quantization with 32.5GB GPU
  Memory" (zicq.com, English), section "Quantization mechanism: absorbing
  online transforms into weights": the layer is y = x W^T; the transformed
  weight is prepared offline; at inference the activation is scaled and
  transformed, then goes through the FP4 matrix multiplication.
* [mxfp4-def] "华为开源MACaQ:本地量化提速3倍" (openai-hub.com news),
  section "量化不是单纯把模型“压小”": OCP MXFP4 splits data into groups of 32
  elements sharing one E8M0 scale; each element is E2M1.
* [block-32]  same article, section "MACaQ 真正解决的是跨层耦合": the
  Hadamard rotation is an orthogonal add/subtract transform restricted to
  32-element blocks that coincide with the MXFP4 scale groups; the inverse is
  absorbed into the weights so the layer's external basis is unchanged.
* [rtn]       "MACaQ Enables Streaming ..." section "Flip-Refinement":
  round-to-nearest maps a value to the numerically closest FP4 code.
* [flip]      same page, section "Flip-Refinement: optimizing FP4 codes with
  second-order information": the quantization loss of a vector is taken as
  one half of (x - q)^T H (x - q), H the Hessian of the layer input from
  calibration data.
* [ablation]  "华为开源MACaQ:本地量化提速3倍", section "Flip-Refinement:不重算,
  只改最值得改的 4-bit 数值": the Llama-3-8B ablation lists a Hessian exponent
  search as the first step above plain round-to-nearest; the Hessian comes
  from calibration statistics of the layer input.

Readings taken where the pages are silent (each is also listed in the
design notes):

* R1  y = (x diag(s) H)(W diag(1/s) H)^T with H the block-diagonal of K/32
      normalized 32x32 Hadamards; the garbled printed form "y=(Hs)(HW^T)^T"
      is read this way because it is the only form that keeps y = x W^T
      while absorbing the inverses into W.
* R2  H32 is the Sylvester Hadamard, H32[i][j] = (-1)^popcount(i & j),
      natural order, no random signs; normalized by C = RNE_f32(1/sqrt(32)).
* R3  order: t = fp32(x) * s (one fp32 rounding); then the unnormalized
      butterfly with stages h = 1, 2, 4, 8, 16, lower index gets a + b and
      upper index gets a - b (fp32, round-to-nearest-even, no fused
      multiply-add); then x' = t * C (one rounding).
* R7  E8M0 exponent: e = floor(log2(amax)) - 2 (2 = largest exponent of
      E2M1), clamped to [-127, 127]; the stored byte is e + 127.  An all-zero
      group stores 0.
* R8  element rounding: nearest E2M1 value of |x'| / 2^e, ties to the value
      with an even mantissa bit; R9: values above 6 saturate to 6;
      R10: the sign bit is kept, also for values that round to zero.
* R14 code = sign << 3 | magnitude index (0..7 -> 0, .5, 1, 1.5, 2, 3, 4, 6);
      two codes per byte, the even element in the low nibble.
* R15 row-major layouts: codes [rows][K/2], scales [rows][K/32].
* R5  weights use r = fp32(1 / s) (IEEE division) in place of s.
* R23 the Hessian is that of the layer output error with respect to a
      transformed weight row: H_e = X'^T X' over expert e's calibration rows,
      X' the fp32 x' of the online transform.  The factor 2 and any division
      by the token count are left out (a positive factor changes no choice).
* R24 Hessian exponent search (the pages name it, give no rule): per weight
      group the candidates are the plain byte b0 (R7) and b0 + 1, which stops
      the saturation of values above 6 * 2^e at the cost of resolution.  Each
      candidate's codes follow R8-R10; its error is q = d^T H_gg d with
      d = x' - dequant(codes) and H_gg the group's 32x32 diagonal block of H
      (a group's scale only moves that group's codes; cross-group terms are
      left out so that every group is decided on its own).  b0 + 1 is kept
      only when its q is strictly smaller.
* R25 q is computed in fp64 in a fixed order (inner sums over j ascending,
      then the outer sum over i ascending, no fused multiply-add), so that
      the choice is reproducible; d is exact in fp64 (at most 28 significant
      bits) and so is every product H_ij d_j.
* R26 Flip-Refinement loss of a weight row: 1/2 d^T H d, d = x' - dequant
      (x' the fp32 transformed weight row, H the Hessian of R23, full K x K);
      scale bytes stay fixed and only codes move.
* R27 a move takes one code to the adjacent value of the signed E2M1 grid
      (-6 .. -0.5, 0, 0.5 .. 6, times the group's scale); no move past +-6.
      Each round a row applies its one best move if that lowers its loss,
      else it stops; at most max_rounds moves (a caller's bound: the pages
      give none).
* R28 ties between equal gains go to the lowest coordinate, then to the
      downward move; a move onto zero keeps the sign bit of the code it left.
* R29 the gradient g = H^T d (= H d for the symmetric Hessian) is formed
      once in fp64 (j ascending, products and sums rounded separately) and
      then only updated, g -= delta H[k, :] (delta a signed power of two, so
      each update is one rounding), as the pages describe; every gain is
      delta g_k - delta^2 H_kk / 2 in fp64.
* R30 GEMM results at the edges of the fp32 range: y is fp32 with IEEE
      gradual underflow and overflow.  The acceptance bound of a result adds
      (K/32) * 2^-150 (one rounding into the subnormal range per 32-value
      group, half the subnormal spacing each) where results can fall below
      2^-126; beyond the largest fp32 value a result is +-inf, which is the
      round-to-nearest value of the exact one.

Floating-point arithmetic that decides a code (the transform) is done in
fp32 exactly as stated above, because the codes must be bit-exact; the GEMM
is the dequantized product in fp64.

The offline sections (Hessian, exponent search, Flip-Refinement) follow
[flip] and [ablation] with readings R23-R29; its decisions are pinned by exact rational
arithmetic in the tests.  The last section (bf16 output, SwiGLU over a
gate/up projection) restates a consumer step after the layer; it is not from
the pages.
"""
from __future__ import annotations

import numpy as np

GROUP = 32

# E2M1 magnitudes by 3-bit index (OCP MX v1.0 E2M1: bias 1, one subnormal).
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_EMAX = 2  # floor(log2(6))

# Normalization of the 32-point Hadamard: 1/sqrt(32) rounded to fp32.
C_NORM = np.float32(1.0 / np.sqrt(32.0))


# --------------------------------------------------------------------------
# transform  ([abstract], [mechanism], [block-32]; readings R1-R3)
# --------------------------------------------------------------------------

def sylvester_hadamard(n: int = GROUP) -> np.ndarray:
    """Integer Sylvester Hadamard matrix of order n (a power of two), built by
    the doubling recursion H_{2m} = [[H_m, H_m], [H_m, -H_m]]."""
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def fwht32(t: np.ndarray) -> np.ndarray:
    """Unnormalized 32-point Walsh-Hadamard butterfly on the last axis (fp32).

    Stages h = 1, 2, 4, 8, 16 in that order; in each stage every index i with
    (i & h) == 0 is paired with i + h and the pair (a, b) becomes
    (a + b, a - b).  Each add/subtract is one fp32 operation rounded to
    nearest even.
    """
    assert t.dtype == np.float32 and t.shape[-1] == GROUP
    t = t.copy()
    for h in (1, 2, 4, 8, 16):
        lo = [i for i in range(GROUP) if (i & h) == 0]
        hi = [i + h for i in lo]
        a = t[..., lo]
        b = t[..., hi]
        t[..., lo] = a + b
        t[..., hi] = a - b
    return t


def transform(x_f32: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """x' = ((x * scale) H32) * C per 32-element group, in fp32 (R3).

    x_f32: [R, K] float32 activations (or weights); scale: [R, K] or [K]
    float32 per-channel factors (s for activations, fp32(1/s) for weights).
    """
    R, K = x_f32.shape
    assert K % GROUP == 0
    t = (x_f32 * scale).astype(np.float32)                 # one fp32 multiply
    u = fwht32(t.reshape(R, K // GROUP, GROUP))
    return (u * C_NORM).astype(np.float32).reshape(R, K)    # one fp32 multiply


def transform_dense_fp64(x: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """The same transform in fp64 as a dense product with the block-diagonal
    normalized Hadamard (R1, R2); independent of the butterfly."""
    x = np.asarray(x, dtype=np.float64) * np.asarray(scale, dtype=np.float64)
    R, K = x.shape
    h = sylvester_hadamard(GROUP).astype(np.float64) / np.sqrt(float(GROUP))
    return (x.reshape(R, K // GROUP, GROUP) @ h).reshape(R, K)


# --------------------------------------------------------------------------
# OCP MXFP4 quantization ([mxfp4-def], [rtn]; readings R7-R14)
# --------------------------------------------------------------------------

def e8m0_scale(amax: np.ndarray) -> np.ndarray:
    """Shared-exponent byte of each group: floor(log2(amax)) - 2 + 127,
    clamped to [0, 254]; 0 for an all-zero group (R7, R11, R12)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)               # amax = m * 2^ex, m in [0.5, 1)
    e = ex.astype(np.int64) - 1 - E2M1_EMAX
    e = np.clip(e, -127, 127)
    return np.where(amax > 0, e + 127, 0).astype(np.uint8)


def e2m1_nearest(v: np.ndarray) -> np.ndarray:
    """Index (0..7) of the E2M1 magnitude nearest to v >= 0; a tie goes to
    the even index (even mantissa bit); values above 6 land on 6 (R8, R9)."""
    # Every v >= 5 has 6 as its nearest value; clamping at 8 keeps that and
    # keeps the fp64 distances below exact (no absorption for huge v).
    v = np.minimum(np.asarray(v, dtype=np.float64), 8.0)[..., None]
    dist = np.abs(v - E2M1_VALUES)
    best = dist == dist.min(axis=-1, keepdims=True)
    even = (np.arange(8) % 2 == 0)
    preference = best * np.where(even, 2, 1)
    return preference.argmax(axis=-1).astype(np.uint8)


def quantize_mxfp4(xp: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Quantize fp32 rows x' [R, K] to packed E2M1 codes [R, K/2] and E8M0
    scale bytes [R, K/32] (R7-R15)."""
    assert xp.dtype == np.float32
    R, K = xp.shape
    g = xp.reshape(R, K // GROUP, GROUP)
    amax = np.abs(g).max(axis=-1)
    scales = e8m0_scale(amax)
    return pack_codes(encode_groups(g, scales)), scales


def encode_groups(g: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """4-bit codes of fp32 groups g [..., 32] at given scale bytes [...]:
    sign << 3 | nearest E2M1 index of |x'| / 2^(b-127) (R8-R10, R14)."""
    # |x'| / 2^(b-127), computed as a multiply by an exact power of two in fp32
    inv = np.ldexp(np.float32(1.0), 127 - scales.astype(np.int32)).astype(np.float32)
    v = (np.abs(g) * inv[..., None]).astype(np.float32)
    mag = e2m1_nearest(v)
    return (np.signbit(g).astype(np.uint8) << 3) | mag


def pack_codes(code: np.ndarray) -> np.ndarray:
    """Codes [R, G, 32] -> bytes [R, 16 G], the even element in the low nibble."""
    code = code.reshape(code.shape[0], -1)
    return (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """[R, K/2] bytes -> [R, K] 4-bit codes (even element in the low nibble)."""
    R, H = packed.shape
    out = np.empty((R, 2 * H), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def dequantize_mxfp4(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact fp64 values of MXFP4 rows: (-1)^s * E2M1 * 2^(b - 127)."""
    code = unpack_codes(packed)
    R, K = code.shape
    mag = E2M1_VALUES[code & 7]
    sign = np.where(code & 8, -1.0, 1.0)
    scale = np.ldexp(1.0, scales.astype(np.int64) - 127)
    return (sign * mag).reshape(R, K // GROUP, GROUP).__mul__(scale[..., None]).reshape(R, K)


# --------------------------------------------------------------------------
# layer entry points ([mechanism], [abstract])
# --------------------------------------------------------------------------

def as_f32(x) -> np.ndarray:
    """Activations/weights to fp32: bfloat16 bit patterns (uint16) are widened
    exactly (bits << 16); float32 arrays pass through."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32)
    assert x.dtype == np.float32, x.dtype
    return x


def expert_of_rows(offsets: np.ndarray, M: int) -> np.ndarray:
    """Expert index of every row, from sorted row offsets [E+1]."""
    offsets = np.asarray(offsets, dtype=np.int64)
    rows = np.arange(M)
    return np.searchsorted(offsets, rows, side="right") - 1


def quant_act(x, s: np.ndarray, offsets=None) -> tuple[np.ndarray, np.ndarray]:
    """Online activation path: x' = (x * s_e) H_blk, then MXFP4.

    x: [M, K] bf16 bits (uint16) or float32; s: [E, K] float32;
    offsets: [E+1] row offsets (rows sorted by expert), None for E = 1.
    """
    xf = as_f32(x)
    s = np.asarray(s, dtype=np.float32).reshape(-1, xf.shape[1])
    if offsets is None:
        assert s.shape[0] == 1
        row_scale = np.broadcast_to(s[0], xf.shape)
    else:
        row_scale = s[expert_of_rows(offsets, xf.shape[0])]
    return quantize_mxfp4(transform(xf, row_scale))


def weight_reciprocal(s: np.ndarray) -> np.ndarray:
    """r = 1 / s as an IEEE fp32 division."""
    s = np.asarray(s, dtype=np.float32)
    return (np.float32(1.0) / s).astype(np.float32)


def prepare_weights(w, s: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Offline weights W' = quant(W diag(1/s) H_blk) for one expert.

    w: [N, K] bf16 bits or float32; s: [K] float32.
    Returns codes [N, K/2] and scales [N, K/32].
    """
    wf = as_f32(w)
    r = weight_reciprocal(np.asarray(s).reshape(-1))
    return quantize_mxfp4(transform(wf, np.broadcast_to(r, wf.shape)))


def gemm(a_codes, a_scales, w_codes, w_scales, offsets=None):
    """Dequantized fp64 product y = A' W'^T per expert.

    a_*: [M, ...] activation codes/scales; w_*: [E, N, ...] or [N, ...].
    Returns (y, S) with S = |A'| |W'|^T, the componentwise magnitude used to
    bound floating-point accumulation error.
    """
    a = dequantize_mxfp4(a_codes, a_scales)
    w_codes = np.asarray(w_codes)
    w_scales = np.asarray(w_scales)
    if w_codes.ndim == 2:
        w_codes, w_scales = w_codes[None], w_scales[None]
    E, N = w_codes.shape[:2]
    M = a.shape[0]
    if offsets is None:
        offsets = np.array([0, M])
    offsets = np.asarray(offsets, dtype=np.int64)
    y = np.zeros((M, N), dtype=np.float64)
    S = np.zeros((M, N), dtype=np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 <= r0:
            continue
        we = dequantize_mxfp4(w_codes[e], w_scales[e])
        y[r0:r1] = a[r0:r1] @ we.T
        S[r0:r1] = np.abs(a[r0:r1]) @ np.abs(we).T
    return y, S


def linear(x, s, w_codes, w_scales, offsets=None):
    """Whole online layer: quant_act, then the MXFP4 GEMM."""
    ac, asc = quant_act(x, s, offsets)
    return gemm(ac, asc, w_codes, w_scales, offsets)


def within_tolerance(y: np.ndarray, y_ref: np.ndarray, S: np.ndarray, rtol: float = 1e-5, groups: int = 0):
    """GEMM acceptance: |y - y_ref| <= rtol * S + groups * 2^-150 elementwise
    (S = 0 and groups = 0 demand an exact 0) and ||y - y_ref||_F <= rtol *
    ||y_ref||_F + sqrt(#elements) * groups * 2^-150.  Returns (ok, worst
    elementwise ratio |y - y_ref| / bound, normwise relative error).

    groups > 0 admits IEEE fp32 gradual underflow (reading R30): a value
    rounded into the subnormal range carries an absolute error of at most
    half the subnormal spacing, 2^-150, and each 32-value group's scaled sum
    enters the fp32 result through at most one such rounding.  Pass
    groups = K / 32 only where results can fall below fp32's normal range."""
    y = np.asarray(y, dtype=np.float64)
    d = np.abs(y - y_ref)
    atol = float(groups) * 2.0 ** -150
    bound = rtol * S + atol
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, d / np.where(bound > 0, bound, 1.0), np.where(d > 0, np.inf, 0.0)) * rtol
    worst = float(ratio.max()) if ratio.size else 0.0
    nref = float(np.linalg.norm(y_ref))
    nd = float(np.linalg.norm(y - y_ref))
    normwise = nd / nref if nref > 0 else nd
    norm_ok = nd <= rtol * nref + np.sqrt(max(d.size, 1)) * atol
    return (worst <= rtol and norm_ok), worst, normwise


# --------------------------------------------------------------------------
# offline: Hessian of the layer input and the Hessian exponent search for the
# weights' E8M0 bytes ([flip], [ablation]; readings R23-R25)
# --------------------------------------------------------------------------

def hessian(xcal, s, offsets=None) -> np.ndarray:
    """H_e = X'_e^T X'_e over the calibration rows of expert e, in fp64 (R23).

    xcal: [T, K] bf16 bits (uint16) or float32, rows sorted by expert;
    s: [E, K] float32; offsets: [E+1] row offsets (None for E = 1).  X' is
    the fp32 activation after the online transform (the x' that the online
    path quantizes).  Returns [E, K, K] float64; an expert without rows gets 0.
    """
    xf = as_f32(xcal)
    T, K = xf.shape
    s = np.asarray(s, dtype=np.float32).reshape(-1, K)
    E = s.shape[0]
    if offsets is None:
        assert E == 1
        offsets = np.array([0, T])
    offsets = np.asarray(offsets, dtype=np.int64)
    H = np.zeros((E, K, K))
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            xp = transform(xf[r0:r1], s[e]).astype(np.float64)
            H[e] = xp.T @ xp
    return H


def diagonal_blocks(h: np.ndarray) -> np.ndarray:
    """[K, K] -> the K/32 diagonal 32x32 blocks [K/32, 32, 32]."""
    K = h.shape[-1]
    G = K // GROUP
    return np.stack([h[GROUP * g:GROUP * (g + 1), GROUP * g:GROUP * (g + 1)] for g in range(G)])


def dequantize_groups(code: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact fp64 values of codes [..., 32] at scale bytes [...]."""
    mag = E2M1_VALUES[code & 7]
    sign = np.where(code & 8, -1.0, 1.0)
    return sign * mag * np.ldexp(1.0, scales.astype(np.int64) - 127)[..., None]


def hessian_error(delta: np.ndarray, hb: np.ndarray) -> np.ndarray:
    """q = delta^T Hb delta per group, fp64, in the fixed order of R25:
    u_i = sum_j Hb[i, j] delta_j (j = 0, 1, ..., 31), then q = sum_i delta_i
    u_i (i = 0, 1, ..., 31), every product and sum rounded on its own.

    delta: [..., G, 32] float64; hb: [G, 32, 32] (cast to float64).
    """
    hb = np.asarray(hb, dtype=np.float64)
    q = np.zeros(delta.shape[:-1])
    for i in range(GROUP):
        u = np.zeros(delta.shape[:-1])
        for j in range(GROUP):
            u = u + hb[:, i, j] * delta[..., j]
        q = q + delta[..., i] * u
    return q


def search_exponents(xp: np.ndarray, hb: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Hessian exponent search over fp32 rows x' [R, K] with the diagonal
    blocks hb [K/32, 32, 32] (R24): each group tries the plain scale byte b0
    (R7) and b0 + 1 and keeps b0 + 1 only when its Hessian-weighted error is
    strictly smaller.  Returns packed codes [R, K/2] and scale bytes [R, K/32].
    """
    assert xp.dtype == np.float32
    R, K = xp.shape
    g = xp.reshape(R, K // GROUP, GROUP)
    b0 = e8m0_scale(np.abs(g).max(axis=-1)).astype(np.int64)
    xd = g.astype(np.float64)
    errs, codes = [], []
    for b in (b0, b0 + 1):
        c = encode_groups(g, b)
        codes.append(c)
        errs.append(hessian_error(xd - dequantize_groups(c, b), hb))
    up = errs[1] < errs[0]
    scales = np.where(up, b0 + 1, b0).astype(np.uint8)
    code = np.where(up[..., None], codes[1], codes[0])
    return pack_codes(code), scales


def prepare_weights_hessian(w, s: np.ndarray, h: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """W' of one expert with Hessian-searched scale bytes: x' = W diag(1/s)
    H_blk as in prepare_weights, then search_exponents with the diagonal
    blocks of h [K, K] (the Hessian of the expert's transformed input)."""
    wf = as_f32(w)
    r = weight_reciprocal(np.asarray(s).reshape(-1))
    xp = transform(wf, np.broadcast_to(r, wf.shape))
    return search_exponents(xp, diagonal_blocks(np.asarray(h)))


# --------------------------------------------------------------------------
# offline: Flip-Refinement of the weight codes ([flip], [ablation];
# readings R26-R29)
# --------------------------------------------------------------------------

# Signed E2M1 levels -7..7 (level L has value sign(L) * E2M1_VALUES[|L|]).
E2M1_LEVELS = np.concatenate([-E2M1_VALUES[:0:-1], E2M1_VALUES])


def code_levels(code: np.ndarray) -> np.ndarray:
    """4-bit codes -> signed levels -7..7 (both zero codes give level 0)."""
    mag = (code & 7).astype(np.int64)
    return np.where(code & 8, -mag, mag)


def level_code(level: np.ndarray, old_code: np.ndarray) -> np.ndarray:
    """Signed level -> 4-bit code; level 0 keeps the sign bit of old_code (a
    move onto zero keeps the sign of the code it came from) (R28)."""
    mag = np.abs(level).astype(np.uint8)
    sign = np.where(level < 0, 8, np.where(level > 0, 0, old_code & 8)).astype(np.uint8)
    return sign | mag


def flip_refine(xp: np.ndarray, codes: np.ndarray, scales: np.ndarray, h: np.ndarray,
                max_rounds: int) -> tuple[np.ndarray, np.ndarray]:
    """Flip-Refinement of MXFP4 rows (R26-R29).

    xp: [R, K] fp32 x' of the weight rows; codes [R, K/2] packed start codes
    (normally round-to-nearest); scales [R, K/32] kept fixed; h [K, K] the
    Hessian of the transformed input.  For every row the loss is
    L = 1/2 d^T H d with d = x' - dequant(codes).  The gradient g = H^T d is
    formed once (fp64, g_i = sum over j ascending of h[j, i] d_j, multiply and
    add rounded separately), then each round every active row takes its best
    single move of one code to the adjacent signed E2M1 level: the gain of
    moving coordinate k by delta is delta g_k - delta^2 h[k, k] / 2; the best
    candidate (the first in the order k ascending, down before up, among the
    largest gains) is applied when its gain is > 0, and the gradient is
    updated by g -= delta h[k, :]; otherwise the row stops.  Returns the
    refined packed codes and the number of moves of each row.
    """
    R, K = xp.shape
    G = K // GROUP
    hd = np.asarray(h, dtype=np.float64)
    code = unpack_codes(codes).astype(np.uint8)
    level = code_levels(code)
    sc = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), GROUP, axis=1)   # [R, K]
    d = xp.astype(np.float64) - E2M1_LEVELS[level + 7] * sc
    g = np.zeros((R, K))
    for j in range(K):
        g = g + hd[j][None, :] * d[:, j:j + 1]
    diag = np.diagonal(hd).copy()
    moves = np.zeros(R, dtype=np.int64)
    active = np.ones(R, dtype=bool)
    rows = np.arange(R)
    for _ in range(max_rounds):
        if not active.any():
            break
        dn = np.where(level > -7, (E2M1_LEVELS[np.maximum(level - 1, -7) + 7] - E2M1_LEVELS[level + 7]) * sc, 0.0)
        up = np.where(level < 7, (E2M1_LEVELS[np.minimum(level + 1, 7) + 7] - E2M1_LEVELS[level + 7]) * sc, 0.0)
        gain = np.empty((R, 2 * K))
        gain[:, 0::2] = np.where(level > -7, dn * g - 0.5 * dn * dn * diag, -np.inf)
        gain[:, 1::2] = np.where(level < 7, up * g - 0.5 * up * up * diag, -np.inf)
        best = np.argmax(gain, axis=1)
        take = active & (gain[rows, best] > 0)
        active = take
        for r in np.nonzero(take)[0]:
            k, is_up = divmod(int(best[r]), 2)
            delta = up[r, k] if is_up else dn[r, k]
            new_level = level[r, k] + (1 if is_up else -1)
            code[r, k] = level_code(np.array(new_level), code[r, k])
            level[r, k] = new_level
            g[r] = g[r] - delta * hd[k]
            moves[r] += 1
    return pack_codes(code.reshape(R, G, GROUP)), moves


def layer_loss(xp: np.ndarray, codes: np.ndarray, scales: np.ndarray, h: np.ndarray) -> np.ndarray:
    """1/2 d^T H d per row with d = x' - dequant(codes), fp64 (library matmul)."""
    d = xp.astype(np.float64) - dequantize_mxfp4(codes, scales)
    return 0.5 * np.einsum("ri,ij,rj->r", d, np.asarray(h, dtype=np.float64), d)


# --------------------------------------------------------------------------
# consumer step after the layer (not part of the pages' method: what a
# decoder layer does next with y -- store it as bf16, or combine a gate/up
# projection with SwiGLU).  Readings: R21 bf16 is round-to-nearest-even of
# the fp32 result; R22 weight rows (2j, 2j+1) are (gate, up) of output
# column j, out = silu(g) * u with silu(g) = g / (1 + exp(-g)).
# --------------------------------------------------------------------------

def round_bf16(v) -> np.ndarray:
    """fp32 values -> the nearest bf16 value (ties to even mantissa), as
    float32 (finite inputs)."""
    b = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def swiglu(y) -> np.ndarray:
    """out[:, j] = silu(y[:, 2j]) * y[:, 2j+1], in fp64."""
    y = np.asarray(y, dtype=np.float64)
    g, u = y[:, 0::2], y[:, 1::2]
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def swiglu_bound(y_ref: np.ndarray, S: np.ndarray, rtol: float = 1e-5) -> np.ndarray:
    """Elementwise bound on |swiglu(y) - swiglu(y_ref)| when each GEMM output
    is within rtol * S of y_ref, plus fp32 rounding of the epilogue: silu has
    |silu'| <= 1.1, so |d(silu(g) u)| <= 1.1 dg (|u| + du) + |silu(g)| du, and
    the fp32 exp, add, divide and multiply add at most 8 units of 2^-24 of
    the result (relative)."""
    g, u = y_ref[:, 0::2], y_ref[:, 1::2]
    dg, du = rtol * S[:, 0::2], rtol * S[:, 1::2]
    with np.errstate(over="ignore"):   # exp(-g) = inf for very negative g gives silu = -0
        sg = g / (1.0 + np.exp(-g))
    return 1.1 * dg * (np.abs(u) + du) + np.abs(sg) * du + 8 * 2.0 ** -24 * np.abs(sg * u) + 1e-30

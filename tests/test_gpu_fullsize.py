"""Parity at the full workload sizes, in the launch configuration the
benchmark times (tiled W' for the prefill and grouped layers, as bench.py
runs them, and the row-major layout beside it): every activation and weight
code and scale byte bit-exact against the oracle, and layer outputs within
the GEMM tolerance — all outputs of the decode and tiny layers, whole rows
of outputs for a row sample of the prefill and grouped layers.  The oracle
runs in row chunks on a thread pool (tests/oracle_rows.py); weights and
references shared by several cases are computed once."""
import numpy as np
import pytest
import torch

import oracle
import oracle_rows
import workloads
import mxfp4_w4a4_quantized_channel_amd as mx

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def host(t):
    t = t.detach().cpu().contiguous()
    return workloads.bf16_bits(t) if t.dtype == torch.bfloat16 else t.numpy()


FULL = [
    ("tiny M16 N128 K256 fp32", dict(cfg=1), "rowmajor"),
    ("attn-proj M2048 N4096 K4096 tiled", dict(cfg=2), "tiled"),
    ("attn-proj M2048 N4096 K4096 row-major", dict(cfg=2), "rowmajor"),
    ("attn-proj literal s=sigma tiled", dict(cfg=2, scale_rule="literal"), "tiled"),
    ("down-prefill M4096 N4096 K14336 tiled", dict(cfg=3), "tiled"),
    ("down-prefill M4096 N4096 K14336 row-major", dict(cfg=3), "rowmajor"),
    ("decode gate/up M1", dict(cfg=4, variant=0, M=1), "rowmajor"),
    ("decode gate/up M8", dict(cfg=4, variant=0, M=8), "rowmajor"),
    ("decode gate/up M32", dict(cfg=4, variant=0, M=32), "rowmajor"),
    ("decode down M1", dict(cfg=4, variant=1, M=1), "rowmajor"),
    ("decode down M8", dict(cfg=4, variant=1, M=8), "rowmajor"),
    ("decode down M32", dict(cfg=4, variant=1, M=32), "rowmajor"),
    ("MoE E64 expert-Zipf tiled", dict(cfg=5), "tiled"),
    ("MoE E64 expert-Zipf row-major", dict(cfg=5), "rowmajor"),
    ("MoE E64 token-Zipf tiled", dict(cfg=5, routing="token_zipf"), "tiled"),
    ("MoE E64 token-Zipf row-major", dict(cfg=5, routing="token_zipf"), "rowmajor"),
]

_WL, _W, _A, _Y = {}, {}, {}, {}


def _key(kw, *drop):
    return tuple(sorted((k, v) for k, v in kw.items() if k not in drop))


def workload(kw):
    k = _key(kw)
    if k not in _WL:
        _WL[k] = workloads.make(**kw)
    return _WL[k]


def oracle_weights(kw, wl):
    """Oracle W' of every expert; shared by the cases with the same weights
    (decode M and MoE routing do not change them)."""
    k = _key(kw, "M", "routing")
    if k not in _W:
        _W[k] = [oracle_rows.prepare_weights(host(wl.w[e]), wl.s[e].numpy()) for e in range(wl.E)]
    return _W[k]


def oracle_acts(kw, wl):
    k = _key(kw)
    if k not in _A:
        _A[k] = oracle_rows.quant_act(host(wl.x), wl.s.numpy(), wl.offsets.numpy() if wl.E > 1 else None)
    return _A[k]


def sample_rows(wl):
    """Rows whose outputs are compared: all of a decode or tiny layer; else
    32 random rows plus the first and last row of every non-empty expert."""
    M = wl.M
    if M <= 32:
        return np.arange(M)
    rng = np.random.default_rng(1234)
    off = wl.offsets.numpy().astype(np.int64)
    edges = [r for e in range(wl.E) if off[e + 1] > off[e] for r in (off[e], off[e + 1] - 1)]
    return np.unique(np.concatenate([rng.choice(M, 32, replace=False), edges]))


def oracle_outputs(kw, wl, rows, rac, ras, rw):
    """fp64 reference y and S for whole output rows `rows`, per expert."""
    k = _key(kw)
    if k not in _Y:
        e_rows = oracle.expert_of_rows(wl.offsets.numpy(), wl.M)[rows] if wl.E > 1 else np.zeros(len(rows), int)
        y_ref = np.empty((len(rows), wl.N))
        S = np.empty_like(y_ref)
        for e in np.unique(e_rows):
            sel = np.nonzero(e_rows == e)[0]
            y_ref[sel], S[sel] = oracle.gemm(rac[rows[sel]], ras[rows[sel]], *rw[e])
        _Y[k] = (y_ref, S)
    return _Y[k]


@pytest.mark.parametrize("name,kw,layout", FULL, ids=[n for n, _, _ in FULL])
def test_full_size(name, kw, layout):
    print(f"[case] full size {name}", flush=True)
    wl = workload(kw)
    M, N, K, E = wl.M, wl.N, wl.K, wl.E
    off = wl.offsets.to(DEV) if E > 1 else None
    x, s = wl.x.to(DEV), wl.s.to(DEV)
    wc, wsc = mx.prepare_weights(wl.w.to(DEV), s)
    ac, asc = mx.quant_act(x, s, off)
    flags = mx.PATH_AUTO
    if layout == "tiled":
        assert M > 32 and N % 32 == 0 and K % 256 == 0   # the benchmark's rule for tiled W'
        tc, ts = mx.tile_weights(wc, wsc)
        y = mx.linear(x, s, tc, ts, off, flags=flags | mx.W_TILED)
    else:
        y = mx.linear(x, s, wc, wsc, off, flags=flags)
    torch.cuda.synchronize()

    # every code and scale byte of the activation and of every expert's W'
    rac, ras = oracle_acts(kw, wl)
    assert np.array_equal(asc.cpu().numpy(), ras)
    assert np.array_equal(ac.cpu().numpy(), rac)
    rw = oracle_weights(kw, wl)
    wc_h, wsc_h = wc.cpu().numpy(), wsc.cpu().numpy()
    for e in range(E):
        assert np.array_equal(wsc_h[e], rw[e][1]), f"expert {e} weight scales"
        assert np.array_equal(wc_h[e], rw[e][0]), f"expert {e} weight codes"

    # whole output rows within the GEMM tolerance
    rows = sample_rows(wl)
    y_ref, S = oracle_outputs(kw, wl, rows, rac, ras, rw)
    ok, worst, normwise = oracle.within_tolerance(y.cpu().numpy()[rows], y_ref, S, 1e-5)
    assert ok, f"{len(rows)} rows: worst {worst:.3g} normwise {normwise:.3g}"


FULL_EPI = [
    ("attn-proj bf16", dict(cfg=2), mx.EPI_NONE),
    ("attn-proj SwiGLU", dict(cfg=2), mx.EPI_SWIGLU),
    ("decode gate/up M1 SwiGLU", dict(cfg=4, variant=0, M=1), mx.EPI_SWIGLU),
    ("decode gate/up M32 SwiGLU", dict(cfg=4, variant=0, M=32), mx.EPI_SWIGLU),
    ("MoE E64 expert-Zipf SwiGLU", dict(cfg=5), mx.EPI_SWIGLU),
]


@pytest.mark.parametrize("name,kw,epi", FULL_EPI, ids=[n for n, _, _ in FULL_EPI])
def test_full_size_epilogues(name, kw, epi):
    """Full-size layers with a bf16 output and/or the SwiGLU epilogue, in the
    benchmark's launch configuration (tiled W' above 32 rows): the bf16
    output equals round-to-nearest-even of the same path's fp32 output
    everywhere, and sampled fp32 outputs are within the oracle's bound (GEMM
    bound carried through silu(g) * u)."""
    print(f"[case] full size epilogue {name}", flush=True)
    wl = workload(kw)
    M, N, K, E = wl.M, wl.N, wl.K, wl.E
    off = wl.offsets.to(DEV) if E > 1 else None
    x, s = wl.x.to(DEV), wl.s.to(DEV)
    wc, wsc = mx.prepare_weights(wl.w.to(DEV), s)
    flags = mx.PATH_AUTO
    if M > 32:
        wc, wsc = mx.tile_weights(wc, wsc)
        flags |= mx.W_TILED
    y32 = mx.linear(x, s, wc, wsc, off, flags=flags, out_dtype=torch.float32, epilogue=epi)
    y16 = mx.linear(x, s, wc, wsc, off, flags=flags, out_dtype=torch.bfloat16, epilogue=epi)
    torch.cuda.synchronize()
    y32 = y32.cpu().numpy()
    assert np.array_equal(workloads.bf16_bits(y16.cpu()), (oracle.round_bf16(y32).view(np.uint32) >> 16).astype(np.uint16))

    rng = np.random.default_rng(4321)
    offs = wl.offsets.numpy()
    rows = np.unique(np.concatenate([rng.choice(M, min(M, 16), replace=False), [0, M - 1]]))
    e_rows = oracle.expert_of_rows(offs, M)[rows] if E > 1 else np.zeros(len(rows), int)
    width = N // 2 if epi == mx.EPI_SWIGLU else N
    outs = np.unique(np.concatenate([rng.choice(width, min(width, 16), replace=False), [0, width - 1]]))
    wrows = np.stack([2 * outs, 2 * outs + 1], axis=1).reshape(-1) if epi == mx.EPI_SWIGLU else outs
    xs = host(wl.x)[rows]
    for e in np.unique(e_rows):
        sel = np.nonzero(e_rows == e)[0]
        rac, ras = oracle.quant_act(xs[sel], wl.s[e:e + 1].numpy())
        rwc, rws = oracle.prepare_weights(host(wl.w[e])[wrows], wl.s[e].numpy())
        y_ref, S = oracle.gemm(rac, ras, rwc, rws)
        got = y32[np.ix_(rows[sel], outs)].astype(np.float64)
        if epi == mx.EPI_SWIGLU:
            ref, tol = oracle.swiglu(y_ref), oracle.swiglu_bound(y_ref, S, 1e-5)
        else:
            ref, tol = y_ref, 1e-5 * S
        bad = np.abs(got - ref) > tol
        assert not bad.any(), f"expert {e}: {bad.sum()} outputs beyond the bound"

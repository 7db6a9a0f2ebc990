"""Parity at the full workload sizes, in the launch configuration the
benchmark times: codes of sampled rows bit-exact, sampled outputs of the
whole layer within the GEMM tolerance.  The oracle quantizes only the
sampled activation rows and weight rows."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import mxfp4_w4a4_quantized_channel_amd as mx

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def host(t):
    t = t.detach().cpu().contiguous()
    return workloads.bf16_bits(t) if t.dtype == torch.bfloat16 else t.numpy()


FULL = [
    ("attn-proj M2048 N4096 K4096", dict(cfg=2)),
    ("down-prefill M4096 N4096 K14336", dict(cfg=3)),
    ("decode gate/up M1", dict(cfg=4, variant=0, M=1)),
    ("decode gate/up M8", dict(cfg=4, variant=0, M=8)),
    ("decode gate/up M32", dict(cfg=4, variant=0, M=32)),
    ("decode down M1", dict(cfg=4, variant=1, M=1)),
    ("decode down M32", dict(cfg=4, variant=1, M=32)),
    ("MoE E64 expert-Zipf", dict(cfg=5)),
    ("MoE E64 token-Zipf", dict(cfg=5, routing="token_zipf")),
]


@pytest.mark.parametrize("name,kw", FULL, ids=[n for n, _ in FULL])
def test_full_size(name, kw):
    print(f"[case] full size {name}", flush=True)
    wl = workloads.make(**kw)
    M, N, K, E = wl.M, wl.N, wl.K, wl.E
    off = wl.offsets.to(DEV) if E > 1 else None
    x, s = wl.x.to(DEV), wl.s.to(DEV)
    wc, wsc = mx.prepare_weights(wl.w.to(DEV), s)
    ac, asc = mx.quant_act(x, s, off)
    y = mx.linear(x, s, wc, wsc, off)
    torch.cuda.synchronize()

    rng = np.random.default_rng(1234)
    offs = wl.offsets.numpy()
    rows = np.unique(np.concatenate([rng.choice(M, min(M, 24), replace=False), [0, M - 1]]))
    xs = host(wl.x)[rows]
    e_rows = oracle.expert_of_rows(offs, M)[rows] if E > 1 else np.zeros(len(rows), int)
    # activation codes of the sampled rows
    rac = np.empty((len(rows), K // 2), np.uint8)
    ras = np.empty((len(rows), K // 32), np.uint8)
    for i, (r, e) in enumerate(zip(rows, e_rows)):
        c, sc = oracle.quant_act(xs[i:i + 1], wl.s[e:e + 1].numpy())
        rac[i], ras[i] = c[0], sc[0]
    assert np.array_equal(ac[rows].cpu().numpy(), rac)
    assert np.array_equal(asc[rows].cpu().numpy(), ras)
    # sampled outputs: weight rows of each sampled row's expert
    cols = np.unique(np.concatenate([rng.choice(N, min(N, 24), replace=False), [0, N - 1]]))
    y_np = y.cpu().numpy()
    for e in np.unique(e_rows):
        sel = np.nonzero(e_rows == e)[0]
        rwc, rws = oracle.prepare_weights(host(wl.w[e])[cols], wl.s[e].numpy())
        assert np.array_equal(wc[e][cols].cpu().numpy(), rwc)
        assert np.array_equal(wsc[e][cols].cpu().numpy(), rws)
        y_ref, S = oracle.gemm(rac[sel], ras[sel], rwc, rws)
        got = y_np[np.ix_(rows[sel], cols)]
        ok, worst, normwise = oracle.within_tolerance(got, y_ref, S, 1e-5)
        assert ok, f"expert {e}: worst {worst:.3g} normwise {normwise:.3g}"


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
    benchmark's launch configuration: the bf16 output equals round-to-nearest-
    even of the same path's fp32 output everywhere, and sampled fp32 outputs
    are within the oracle's bound (GEMM bound carried through silu(g) * u)."""
    print(f"[case] full size epilogue {name}", flush=True)
    wl = workloads.make(**kw)
    M, N, K, E = wl.M, wl.N, wl.K, wl.E
    off = wl.offsets.to(DEV) if E > 1 else None
    x, s = wl.x.to(DEV), wl.s.to(DEV)
    wc, wsc = mx.prepare_weights(wl.w.to(DEV), s)
    y32 = mx.linear(x, s, wc, wsc, off, out_dtype=torch.float32, epilogue=epi)
    y16 = mx.linear(x, s, wc, wsc, off, out_dtype=torch.bfloat16, epilogue=epi)
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

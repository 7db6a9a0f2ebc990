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

"""Byte offsets past 2^31 and 2^32: a layer of M = 139264 rows of K = 32768
bf16 values (9.1 GB of activation, 2.3 GB of codes), N = 64.  Rows from
32768 on start past 2^31 bytes of x, rows from 131072 on past 2^31 bytes of
codes (and past 2^32 bytes of x).  For sampled rows on both sides of those
boundaries, the activation codes and scale bytes (row-major path) are
bit-exact against the oracle, and the layer's outputs (tiled weights and
tiled activation staging, the benchmark's launch configuration) are within
the GEMM bound."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import mxfp4_w4a4_quantized_channel_amd as mx

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
M, N, K = 139264, 64, 32768
ROWS = [0, 1, 32767, 32768, 65535, 65536, 131071, 131072, 131073, M - 2, M - 1]


def test_offsets_past_2_31_and_2_32():
    print(f"[case] large offsets M{M} N{N} K{K}", flush=True)
    gen = torch.Generator(device=DEV).manual_seed(31)
    x = torch.randn((M, K), generator=gen, device=DEV, dtype=torch.bfloat16)
    rng = np.random.default_rng(32)
    s_h = rng.uniform(0.5, 2.0, (1, K)).astype(np.float32)
    w_h = torch.from_numpy(rng.standard_normal((1, N, K)).astype(np.float32) * 0.02).to(torch.bfloat16)
    s = torch.from_numpy(s_h).to(DEV)
    rows = np.array(ROWS)
    xs = workloads.bf16_bits(x[torch.from_numpy(rows).to(DEV)].cpu())
    rac, ras = oracle.quant_act(xs, s_h)
    rwc, rws = oracle.prepare_weights(workloads.bf16_bits(w_h[0]), s_h[0])

    ac, asc = mx.quant_act(x, s)
    torch.cuda.synchronize()
    idx = torch.from_numpy(rows).to(DEV)
    assert np.array_equal(asc[idx].cpu().numpy(), ras)
    assert np.array_equal(ac[idx].cpu().numpy(), rac)
    del ac, asc

    wc, wsc = mx.prepare_weights(w_h.to(DEV), s)
    tc, ts = mx.tile_weights(wc, wsc)
    y = mx.linear(x, s, tc, ts, flags=mx.PATH_AUTO | mx.W_TILED)
    torch.cuda.synchronize()
    y_ref, S = oracle.gemm(rac, ras, rwc, rws)
    ok, worst, normwise = oracle.within_tolerance(y[idx].cpu().numpy(), y_ref, S, 1e-5)
    assert ok, f"worst {worst:.3g} normwise {normwise:.3g}"
    del x, y, tc, ts, wc, wsc
    torch.cuda.empty_cache()

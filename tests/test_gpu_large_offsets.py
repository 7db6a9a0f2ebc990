"""Byte offsets past 2^31 and 2^32.  A layer of M = 139264 rows of K = 32768
bf16 values (9.1 GB of activation, 2.3 GB of codes), N = 64.  Rows from
32768 on start past 2^31 bytes of x, rows from 131072 on past 2^31 bytes of
codes (and past 2^32 bytes of x).  For sampled rows on both sides of those
boundaries, the activation codes and scale bytes (row-major path) are
bit-exact against the oracle, and the layer's outputs (tiled weights and
tiled activation staging, the benchmark's launch configuration) are within
the GEMM bound.  Decode layers and a grouped layer whose weight codes span
more than 2^31 bytes are checked on sampled outputs the same way."""
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


@pytest.mark.parametrize("M,flags", [(1, mx.PATH_FUSED), (8, mx.PATH_UNFUSED)])
def test_decode_weights_past_2_31(M, flags):
    """Decode layers whose W' codes span 2.3 GB (N = 139264, K = 32768):
    sampled output columns on both sides of 2^31 bytes of W' codes."""
    N2, K2 = 139264, 32768
    print(f"[case] large decode weights M{M} N{N2} K{K2} flags={flags}", flush=True)
    gen = torch.Generator(device=DEV).manual_seed(33)
    w = torch.randn((1, N2, K2), generator=gen, device=DEV, dtype=torch.bfloat16) * 0.02
    rng = np.random.default_rng(34)
    s_h = rng.uniform(0.5, 2.0, (1, K2)).astype(np.float32)
    x_h = torch.from_numpy(rng.standard_normal((M, K2)).astype(np.float32)).to(torch.bfloat16)
    s = torch.from_numpy(s_h).to(DEV)
    cols = np.array([0, 1, 65535, 65536, 131071, 131072, N2 - 1])
    wc, wsc = mx.prepare_weights(w, s)
    w_rows = workloads.bf16_bits(w[0, torch.from_numpy(cols).to(DEV)].cpu())
    del w
    y = mx.linear(x_h.to(DEV), s, wc, wsc, flags=flags)
    torch.cuda.synchronize()
    rwc, rws = oracle.prepare_weights(w_rows, s_h[0])
    idx = torch.from_numpy(cols).to(DEV)
    assert np.array_equal(wc[0, idx].cpu().numpy(), rwc) and np.array_equal(wsc[0, idx].cpu().numpy(), rws)
    rac, ras = oracle.quant_act(workloads.bf16_bits(x_h), s_h)
    y_ref, S = oracle.gemm(rac, ras, rwc, rws)
    ok, worst, normwise = oracle.within_tolerance(y[:, idx].cpu().numpy(), y_ref, S, 1e-5)
    assert ok, f"worst {worst:.3g} normwise {normwise:.3g}"
    del wc, wsc, y
    torch.cuda.empty_cache()


def test_grouped_weights_past_2_31():
    """A grouped layer whose experts' W' span 2.1 GB (E = 64, N = 2048,
    K = 32768; the last experts start past 2^31 bytes): tiled W' and tiled
    activation staging, sampled rows of the first and last experts."""
    E, N2, K2 = 64, 2048, 32768
    counts = np.zeros(E, np.int64)
    counts[[0, 1, 31, 62, 63]] = [40, 3, 70, 33, 90]
    off_h = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M2 = int(off_h[-1])
    print(f"[case] large grouped weights E{E} N{N2} K{K2} M{M2}", flush=True)
    gen = torch.Generator(device=DEV).manual_seed(35)
    w = torch.randn((E, N2, K2), generator=gen, device=DEV, dtype=torch.bfloat16) * 0.02
    rng = np.random.default_rng(36)
    s_h = rng.uniform(0.5, 2.0, (E, K2)).astype(np.float32)
    x_h = torch.from_numpy(rng.standard_normal((M2, K2)).astype(np.float32)).to(torch.bfloat16)
    s = torch.from_numpy(s_h).to(DEV)
    off = torch.from_numpy(off_h).to(DEV)
    cols = np.array([0, 1, 1023, N2 - 1])
    wc, wsc = mx.prepare_weights(w, s)
    tc, ts = mx.tile_weights(wc, wsc)
    del wc, wsc
    rows = np.array([0, 39, 40, 113, 114, 146, M2 - 90, M2 - 1])
    e_rows = oracle.expert_of_rows(off_h, M2)[rows]
    w_rows = {e: workloads.bf16_bits(w[e, torch.from_numpy(cols).to(DEV)].cpu()) for e in np.unique(e_rows)}
    del w
    y = mx.linear(x_h.to(DEV), s, tc, ts, off, flags=mx.PATH_AUTO | mx.W_TILED)
    torch.cuda.synchronize()
    y_h = y.cpu().numpy()
    xb = workloads.bf16_bits(x_h)
    for e in np.unique(e_rows):
        sel = rows[e_rows == e]
        rac, ras = oracle.quant_act(xb[sel], s_h[e:e + 1])
        rwc, rws = oracle.prepare_weights(w_rows[e], s_h[e])
        y_ref, S = oracle.gemm(rac, ras, rwc, rws)
        ok, worst, normwise = oracle.within_tolerance(y_h[np.ix_(sel, cols)], y_ref, S, 1e-5)
        assert ok, f"expert {e}: worst {worst:.3g} normwise {normwise:.3g}"
    del tc, ts, y
    torch.cuda.empty_cache()

"""The layer under HIP graph capture, through the C ABI: the kernels
allocate nothing, clear nothing with memset nodes and never synchronize, so
a captured call replays correctly.  Each case captures one macaq_linear
call (static input, output and workspace), then replays the graph three
times with new input written by eager work in between, and checks every
replay bit for bit against an eager call on the same input."""
import numpy as np
import pytest
import torch

import workloads
import mxfp4_w4a4_quantized_channel_amd as mx

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"[case] {msg}", flush=True)


CASES = [
    ("prefill, tiled W'", dict(cfg=2, shape=(200, 256, 1024)), mx.PATH_AUTO, True),
    ("decode M1, fused", dict(cfg=4, shape=(1, 512, 2048)), mx.PATH_AUTO, False),
    ("decode M8, two launches", dict(cfg=4, shape=(8, 512, 2048)), mx.PATH_UNFUSED, False),
    ("decode M32, K split in 3 with its reduce", dict(cfg=4, shape=(32, 256, 256 * 48)), mx.PATH_UNFUSED, False),
    ("decode M8, one launch (published activation)", dict(cfg=4, shape=(8, 4160, 1024)), mx.PATH_FUSED, False),
    ("decode M32, one launch with a K split in 3", dict(cfg=4, shape=(32, 1024, 256 * 48)), mx.PATH_FUSED, False),
    ("MoE, grouped", dict(cfg=5, shape=(300, 64, 512), routing="token_zipf"), mx.PATH_AUTO, True),
]


@pytest.mark.parametrize("name,kw,flags,tiled", CASES, ids=[c[0] for c in CASES])
def test_linear_replays_in_hip_graph(name, kw, flags, tiled):
    say(f"graph {name}")
    wl = workloads.make(**kw)
    s = wl.s.to(DEV)
    off = wl.offsets.to(DEV) if wl.E > 1 else None
    wc, wsc = mx.prepare_weights(wl.w.to(DEV), s)
    if tiled:
        wc, wsc = mx.tile_weights(wc, wsc)
        flags |= mx.W_TILED
    x = wl.x.to(DEV).clone()
    y0 = mx.linear(x, s, wc, wsc, off, flags=flags)       # eager, also the first-call set-up
    need = mx.linear_workspace_bytes(wl.M, wl.N, wl.K, wl.E, flags)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=DEV) if need > 0 else None
    out = torch.empty_like(y0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mx.linear(x, s, wc, wsc, off, flags=flags, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mx.linear(x, s, wc, wsc, off, flags=flags, out=out, workspace=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(len(name))
    for rep in range(3):
        fresh = torch.from_numpy(rng.standard_normal(tuple(x.shape)).astype(np.float32)).to(x.dtype)
        x.copy_(fresh.to(DEV))
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        ref = mx.linear(x, s, wc, wsc, off, flags=flags)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep}"

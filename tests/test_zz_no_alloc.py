"""macaq_linear_noalloc (the entry point with no workspace argument, whose
staging lives in the library's static device array) against macaq_linear_ex
with a caller workspace: bit for bit on consecutive calls of different sizes
(the array keeps the previous call's bytes), on the unfused prefill, grouped
and decode paths and the fused decode paths (streamed, and one launch with
the published activation and its counts in the array), with and without the
decode K split (whose partial sums also live in the array)."""
import numpy as np
import pytest
import torch

import workloads
import mxfp4_w4a4_quantized_channel_amd as mx

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [   # consecutive calls: each smaller than the one before
    ("attn-proj M2048 N4096 K4096, tiled W'", dict(cfg=2), True, mx.PATH_AUTO),
    ("MoE-shaped M300 N64 K1024", dict(cfg=5, shape=(300, 64, 1024)), False, mx.PATH_AUTO),
    ("decode-shaped M32 N1024 K12288 one launch, K split in 3", dict(cfg=4, shape=(32, 1024, 256 * 48)), False,
     mx.PATH_FUSED),
    ("decode-shaped M8 N256 K16384, K split in 2", dict(cfg=4, shape=(8, 256, 16384)), False, mx.PATH_AUTO),
    ("decode-shaped M8 N512 K2048", dict(cfg=4, shape=(8, 512, 2048)), False, mx.PATH_AUTO),
    ("decode-shaped M8 N4160 K1024 one launch", dict(cfg=4, shape=(8, 4160, 1024)), False, mx.PATH_FUSED),
    ("decode-shaped M1 N128 K16384 fused, K split in 2", dict(cfg=4, shape=(1, 128, 16384)), False, mx.PATH_FUSED),
    ("decode-shaped M2 N256 K1024 fused", dict(cfg=4, shape=(2, 256, 1024)), False, mx.PATH_FUSED),
]


def _layer(kw, tiled):
    wl = workloads.make(**kw)
    off = wl.offsets.to(DEV) if wl.E > 1 else None
    x, s = wl.x.to(DEV), wl.s.to(DEV)
    wc, wsc = mx.prepare_weights(wl.w.to(DEV), s)
    if tiled:
        wc, wsc = mx.tile_weights(wc, wsc)
    return x, s, wc, wsc, off


def test_noalloc_equals_workspace_entry_point():
    for name, kw, tiled, path in CASES:
        print(f"[case] noalloc {name}", flush=True)
        x, s, wc, wsc, off = _layer(kw, tiled)
        flags = path | (mx.W_TILED if tiled else 0)
        for out_dtype in (torch.float32, torch.bfloat16):
            ref = mx.linear(x, s, wc, wsc, off, flags=flags, out_dtype=out_dtype)
            got = mx.linear_noalloc(x, s, wc, wsc, off, flags=flags, out_dtype=out_dtype)
            torch.cuda.synchronize()
            assert torch.equal(got, ref), f"{name} {out_dtype}"
        # a second call of the same shape on other activations reuses the array
        x2 = x.flip(0).contiguous() if off is None else x
        ref = mx.linear(x2, s, wc, wsc, off, flags=flags)
        got = mx.linear_noalloc(x2, s, wc, wsc, off, flags=flags)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"{name} second call"


def test_noalloc_refuses_oversize_shape():
    """A shape whose staging exceeds the static array is refused before any
    launch; the library stays usable."""
    M, N, K = 8192, 64, 16384    # 71 MB of activation codes and scales
    need = mx.linear_workspace_bytes(M, N, K, 1, mx.PATH_UNFUSED)
    assert need > mx.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    s = torch.ones((1, K), dtype=torch.float32, device=DEV)
    wc = torch.zeros((1, N, K // 2), dtype=torch.uint8, device=DEV)
    wsc = torch.zeros((1, N, K // 32), dtype=torch.uint8, device=DEV)
    with pytest.raises(mx.MacaqError, match="static scratch"):
        mx.linear_noalloc(x, s, wc, wsc, flags=mx.PATH_UNFUSED)
    x, s, wc, wsc, off = _layer(CASES[2][1], False)
    assert torch.equal(mx.linear_noalloc(x, s, wc, wsc), mx.linear(x, s, wc, wsc))

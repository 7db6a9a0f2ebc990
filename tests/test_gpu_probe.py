"""The measurement aids of include/macaq_probe.h run through the C ABI.
MFMA probe: zero operands leave every accumulator at zero; random operand
bytes (all E2M1 codes are finite) give finite sums.  Streaming probe: each
form moves exactly the bytes it states (the written chunks and the per-thread
XOR checksums are recomputed here with numpy)."""
import ctypes

import numpy as np
import pytest
import torch

import mxfp4_w4a4_quantized_channel_amd as mx

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("waves", [4, 8])
def test_probe_runs(waves):
    print(f"[case] mfma probe waves={waves}", flush=True)
    L = mx.lib()
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for data in ("zero", "random"):
        src = (torch.randint(0, 256, (8192,), dtype=torch.uint8) if data == "random"
               else torch.zeros(8192, dtype=torch.uint8)).to(DEV)
        out = torch.full((8 * waves * 64,), float("nan"), dtype=torch.float32, device=DEV)
        assert L.macaq_probe_mfma(ctypes.c_void_p(src.data_ptr()), 8, waves, 3,
                                  ctypes.c_void_p(out.data_ptr()), sp) == 0
        torch.cuda.synchronize()
        if data == "zero":
            assert torch.equal(out, torch.zeros_like(out))
        else:
            assert torch.isfinite(out).all()


def _xor_fold(a: np.ndarray) -> np.uint32:
    """XOR over every 32-bit word of a uint32 array."""
    return np.bitwise_xor.reduce(a.reshape(-1), dtype=np.uint32) if a.size else np.uint32(0)


@pytest.mark.parametrize("nr,nw,blocks", [(4096, 0, 3), (0, 1000, 2), (4096, 1024, 5), (12288, 3072, 1), (64, 64, 7)])
def test_stream_probe(nr, nw, blocks):
    """nr / nw: 16-byte chunks read / written; the grid is smaller and larger
    than the chunk count (grid-stride loops, idle threads write 0)."""
    print(f"[case] stream probe chunks read {nr} written {nw} blocks {blocks}", flush=True)
    L = mx.lib()
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rng = np.random.default_rng(nr + nw + blocks)
    src_np = rng.integers(0, 2 ** 32, (max(nr, 1), 4), dtype=np.uint32)[:nr]
    src = torch.from_numpy(src_np.view(np.int32).copy()).to(DEV)
    dst = torch.full((max(nw, 1), 4), -1, dtype=torch.int32, device=DEV)
    out = torch.full((blocks * 256,), -1, dtype=torch.int32, device=DEV)
    assert L.macaq_probe_stream(ctypes.c_void_p(src.data_ptr() if nr else 0), 16 * nr,
                                ctypes.c_void_p(dst.data_ptr() if nw else 0), 16 * nw, blocks,
                                ctypes.c_void_p(out.data_ptr()), sp) == 0
    torch.cuda.synchronize()
    got_out = out.cpu().numpy().view(np.uint32)
    if nw == 0:
        want = src_np
    elif nr == 0:
        want = np.repeat(np.arange(nw, dtype=np.uint32)[:, None], 4, axis=1)
    else:
        want = np.bitwise_xor.reduce(src_np.reshape(nr // nw, nw, 4), axis=0)
    if nw:
        assert np.array_equal(dst.cpu().numpy().view(np.uint32)[:nw], want)
    threads = blocks * 256
    for t in range(threads):   # thread t handled chunks t, t + threads, ...
        assert got_out[t] == _xor_fold(want[t::threads]), t

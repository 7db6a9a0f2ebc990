"""The MFMA probe (a measurement aid, include/macaq_probe.h) runs through the
C ABI: zero operands leave every accumulator at zero; random operand bytes
(all E2M1 codes are finite) give finite sums."""
import ctypes

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

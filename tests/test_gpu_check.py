"""The MACAQ_CHECK=1 debug mode of the C ABI on the GPU: valid calls give
the same results as without it (it only adds waits and read-backs), and
device-resident inputs that break the preconditions (expert offsets that
do not start at 0, decrease or do not end at the row count; factors of s
that are zero, negative or not finite) are refused with
MACAQ_ERR_INVALID_ARG before anything is launched.  The broken inputs are
only ever passed with the check on: without it they would be read by the
kernels."""
import numpy as np
import pytest
import torch

import workloads
import mxfp4_w4a4_quantized_channel_amd as mx

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture
def check_on(monkeypatch):
    monkeypatch.setenv("MACAQ_CHECK", "1")


def _moe_case():
    wl = workloads.make(cfg=5, shape=(300, 64, 256), routing="token_zipf")
    return wl, wl.x.to(DEV), wl.s.to(DEV), wl.offsets.to(DEV)


def test_check_mode_same_results(monkeypatch):
    """quant_act over experts, the grouped GEMM, the dense linear layer and
    weight preparation, with and without the check."""
    say("MACAQ_CHECK valid calls")
    wl, x, s, off = _moe_case()
    wc, wsc = mx.prepare_weights(wl.w.to(DEV), s)
    dense = workloads.make(cfg=2, shape=(40, 96, 512))
    dx, ds = dense.x.to(DEV), dense.s.to(DEV)
    dwc, dwsc = mx.prepare_weights(dense.w.to(DEV), ds)

    def run():
        ac, asc = mx.quant_act(x, s, off)
        y = mx.gemm(ac, asc, wc, wsc, off)
        yl = mx.linear(dx, ds, dwc, dwsc)
        pc, ps = mx.prepare_weights(dense.w.to(DEV), ds)
        torch.cuda.synchronize()
        return [t.cpu() for t in (ac, asc, y, yl, pc, ps)]

    monkeypatch.delenv("MACAQ_CHECK", raising=False)
    ref = run()
    monkeypatch.setenv("MACAQ_CHECK", "1")
    got = run()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


@pytest.mark.parametrize("kind", ["end past M", "end short of M", "decreasing", "not from 0"])
def test_check_mode_refuses_bad_offsets(kind, check_on):
    say(f"MACAQ_CHECK offsets {kind}")
    wl, x, s, off = _moe_case()
    o = wl.offsets.clone()
    if kind == "end past M":
        o[-1] = o[-1] + 5
    elif kind == "end short of M":
        o[-1] = o[-1] - 1
    elif kind == "decreasing":
        i = int(np.argmax(np.diff(o.numpy()) > 0))   # an expert with rows: move its end below its start
        o[i + 1] = o[i] - 1
    else:
        o[0] = 1
    bad = o.to(DEV)
    with pytest.raises(mx.MacaqError) as ei:
        mx.quant_act(x, s, bad)
    assert ei.value.status == -1 and "MACAQ_CHECK" in str(ei.value)
    wc, wsc = mx.prepare_weights(wl.w.to(DEV), s)
    ac, asc = mx.quant_act(x, s, off)
    with pytest.raises(mx.MacaqError) as ei:
        mx.gemm(ac, asc, wc, wsc, bad)
    assert ei.value.status == -1
    with pytest.raises(mx.MacaqError) as ei:
        mx.linear(x, s, wc, wsc, bad)
    assert ei.value.status == -1
    torch.cuda.synchronize()


@pytest.mark.parametrize("value", [0.0, -1.0, float("nan"), float("inf")])
def test_check_mode_refuses_bad_factors(value, check_on):
    say(f"MACAQ_CHECK s = {value}")
    dense = workloads.make(cfg=2, shape=(16, 64, 256))
    s = dense.s.clone()
    s.view(-1)[37] = value
    s = s.to(DEV)
    with pytest.raises(mx.MacaqError) as ei:
        mx.quant_act(dense.x.to(DEV), s)
    assert ei.value.status == -1 and "s[37]" in str(ei.value)
    with pytest.raises(mx.MacaqError):
        mx.prepare_weights(dense.w.to(DEV), s)
    good_wc, good_wsc = mx.prepare_weights(dense.w.to(DEV), dense.s.to(DEV))
    with pytest.raises(mx.MacaqError):
        mx.linear(dense.x.to(DEV), s, good_wc, good_wsc)
    torch.cuda.synchronize()

"""The C ABI library loads, exports every function include/*.h declares,
and validates arguments on the host (no GPU needed: nothing is launched)."""
import ctypes
import os
import re

import pytest

import mxfp4_w4a4_quantized_channel_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "macaq.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))

OK, INVALID, UNSUPPORTED, NO_DEVICE, HIPERR, WORKSPACE = 0, -1, -2, -3, -4, -5
A16 = 0x10000  # a fake, 256-byte aligned, non-null "device pointer" (never dereferenced)


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(macaq_[a-z0-9_]+)\s*\(", text)))


def test_probe_validation():
    """The MFMA probe (a measurement aid) rejects bad arguments on the host."""
    mx.lib()
    assert mx.macaq_probe_mfma(None, 256, 4, 1, A16, None) == INVALID
    assert mx.macaq_probe_mfma(A16 + 4, 256, 4, 1, A16, None) == INVALID
    assert mx.macaq_probe_mfma(A16, 0, 4, 1, A16, None) == INVALID
    assert mx.macaq_probe_mfma(A16, 256, 6, 1, A16, None) == INVALID
    assert mx.macaq_probe_mfma(A16, 256, 4, 0, A16, None) == INVALID
    assert mx.macaq_probe_mfma(A16, 256, 8, 10, A16, None) == NO_DEVICE


def test_stream_probe_validation():
    """The streaming probe (a measurement aid) rejects bad arguments on the
    host: sizes not multiples of 16, nothing to stream, missing or misaligned
    buffers, a read size that is not a whole multiple of the write size, a
    block count out of range, a null out."""
    mx.lib()
    assert mx.macaq_probe_stream(A16, 100, A16, 16, 8, A16, None) == INVALID
    assert mx.macaq_probe_stream(A16, 0, A16, 0, 8, A16, None) == INVALID
    assert mx.macaq_probe_stream(None, 4096, None, 0, 8, A16, None) == INVALID
    assert mx.macaq_probe_stream(A16 + 4, 4096, None, 0, 8, A16, None) == INVALID
    assert mx.macaq_probe_stream(A16, 4096, A16 + 8, 1024, 8, A16, None) == INVALID
    assert mx.macaq_probe_stream(A16, 4096, A16, 1536, 8, A16, None) == INVALID
    assert mx.macaq_probe_stream(A16, 4096, A16, 1024, 0, A16, None) == INVALID
    assert mx.macaq_probe_stream(A16, 4096, A16, 1024, 8, None, None) == INVALID
    assert mx.macaq_probe_stream(A16, 4096, A16, 1024, 8, A16, None) == NO_DEVICE
    assert mx.macaq_probe_stream(None, 0, A16, 1024, 8, A16, None) == NO_DEVICE


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["macaq_prepare_weights", "macaq_quant_act", "macaq_linear", "macaq_gemm",
              "macaq_linear_workspace_bytes", "macaq_status_string", "macaq_last_error", "macaq_version"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    L = mx.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    out = os.popen(f"nm -D --defined-only {mx.library_path}").read()
    for n in declared_functions():
        assert re.search(rf"\bT {n}\b", out), n


def test_version_and_status_strings():
    assert mx.version() == 10000
    L = mx.lib()
    for code in (OK, INVALID, UNSUPPORTED, NO_DEVICE, HIPERR, WORKSPACE, 12345):
        assert isinstance(L.macaq_status_string(code), bytes)
    assert L.macaq_status_string(WORKSPACE) == b"workspace too small"


def qa(x=A16, dt=0, s=A16, off=None, E=1, M=4, K=64, c=A16, sc=A16):
    return mx.macaq_quant_act(x, dt, s, off, E, M, K, c, sc, None)


def test_quant_act_validation():
    mx.lib()
    assert qa(K=48) == INVALID           # K % 32 != 0
    assert qa(K=0) == INVALID
    assert qa(E=0) == INVALID
    assert qa(M=-1) == INVALID
    assert qa(E=2, off=None) == INVALID  # offsets needed for E > 1
    assert qa(x=None) == INVALID
    assert qa(x=A16 + 2) == INVALID      # misaligned
    assert qa(dt=7) == UNSUPPORTED
    assert qa(M=0) == OK                 # no-op, no device touched
    assert b"K must be" in (mx.lib().macaq_quant_act(A16, 0, A16, None, 1, 4, 40, A16, A16, None) and
                            mx.macaq_last_error())


def gm(a=A16, asc=A16, off=None, E=1, w=A16, ws=A16, M=4, N=8, K=256, y=A16):
    return mx.macaq_gemm(a, asc, off, E, w, ws, M, N, K, y, None, 0, None)


def test_gemm_validation():
    mx.lib()
    assert gm(K=96) == UNSUPPORTED       # multiple of 32 but not of 128
    assert gm(K=100) == INVALID
    assert gm(N=0) == INVALID
    assert gm(w=None) == INVALID
    assert gm(a=A16 + 8) == INVALID
    assert gm(asc=A16 + 1) == INVALID
    assert gm(E=3) == INVALID            # no offsets
    assert gm(M=0) == OK


def test_linear_validation_and_workspace():
    L = mx.lib()
    need = L.macaq_linear_workspace_bytes(64, 128, 256, 1, mx.PATH_UNFUSED)
    assert need == L.macaq_quant_act_bytes(64, 256) > 0
    assert L.macaq_quant_act_bytes(64, 256) >= 64 * 256 * 17 // 32
    r = mx.macaq_linear(A16, 0, A16, None, 1, A16, A16, 64, 128, 256, A16, A16, need - 1,
                        mx.PATH_UNFUSED, None)
    assert r == WORKSPACE
    r = mx.macaq_linear(A16, 0, A16, None, 1, A16, A16, 64, 128, 256, A16, None, 0,
                        mx.PATH_UNFUSED, None)
    assert r == WORKSPACE
    r = mx.macaq_linear(A16, 0, A16, None, 1, A16, A16, 64, 128, 256, A16, A16, need, 9, None)
    assert r == INVALID


def test_prepare_weights_validation():
    mx.lib()
    pw = mx.macaq_prepare_weights
    assert pw(A16, 0, A16, 1, 8, 33, A16, A16, None) == INVALID
    assert pw(A16, 0, A16, 0, 8, 64, A16, A16, None) == INVALID
    assert pw(None, 0, A16, 1, 8, 64, A16, A16, None) == INVALID
    assert pw(A16, 3, A16, 1, 8, 64, A16, A16, None) == UNSUPPORTED


def test_hessian_validation():
    mx.lib()
    hs = mx.macaq_hessian
    # x, dtype, s, offsets, E, T, K, h
    assert hs(A16, 0, A16, None, 1, 16, 96, A16, None) == UNSUPPORTED    # K % 128 != 0
    assert hs(A16, 0, A16, None, 1, 16, 100, A16, None) == INVALID       # K % 32 != 0
    assert hs(A16, 0, A16, None, 0, 16, 128, A16, None) == INVALID       # E < 1
    assert hs(A16, 0, A16, None, 1, -1, 128, A16, None) == INVALID       # T < 0
    assert hs(A16, 0, A16, None, 2, 16, 128, A16, None) == INVALID       # offsets needed
    assert hs(None, 0, A16, None, 1, 16, 128, A16, None) == INVALID
    assert hs(A16, 0, A16, None, 1, 16, 128, None, None) == INVALID
    assert hs(A16 + 4, 0, A16, None, 1, 16, 128, A16, None) == INVALID   # x misaligned
    assert hs(A16, 0, A16, None, 1, 16, 128, A16 + 2, None) == INVALID   # h misaligned
    assert hs(A16, 5, A16, None, 1, 16, 128, A16, None) == UNSUPPORTED


def test_prepare_weights_hessian_validation():
    mx.lib()
    ph = mx.macaq_prepare_weights_hessian
    # w, dtype, s, h, E, N, K, codes, scales
    assert ph(A16, 0, A16, A16, 1, 8, 48, A16, A16, None) == INVALID
    assert ph(A16, 0, A16, A16, 1, 0, 64, A16, A16, None) == INVALID
    assert ph(A16, 0, A16, None, 1, 8, 64, A16, A16, None) == INVALID
    assert ph(A16, 0, A16, A16 + 1, 1, 8, 64, A16, A16, None) == INVALID
    assert ph(A16, 0, A16 + 4, A16, 1, 8, 64, A16, A16, None) == INVALID
    assert ph(A16, 9, A16, A16, 1, 8, 64, A16, A16, None) == UNSUPPORTED


def test_flip_refine_validation_and_workspace():
    mx.lib()
    fr = mx.macaq_flip_refine
    need = mx.flip_refine_workspace_bytes(128, 256)
    assert need == 128 * 256 * 8
    assert mx.flip_refine_workspace_bytes(1, 256) == need          # rounded up to 128 rows
    assert mx.flip_refine_workspace_bytes(0, 256) == 0
    # w, dtype, s, h, E, N, K, max_rounds, codes, scales, moves, ws, ws_bytes
    assert fr(A16, 0, A16, A16, 1, 8, 96, 4, A16, A16, None, A16, need, None) == UNSUPPORTED   # K % 128
    assert fr(A16, 0, A16, A16, 1, 8, 32768, 4, A16, A16, None, A16, 1 << 40, None) == UNSUPPORTED
    assert fr(A16, 0, A16, A16, 1, 8, 100, 4, A16, A16, None, A16, need, None) == INVALID
    assert fr(A16, 0, A16, A16, 1, 0, 256, 4, A16, A16, None, A16, need, None) == INVALID
    assert fr(A16, 0, A16, A16, 1, 8, 256, -1, A16, A16, None, A16, need, None) == INVALID
    assert fr(A16, 0, A16, None, 1, 8, 256, 4, A16, A16, None, A16, need, None) == INVALID
    assert fr(A16, 0, A16, A16, 1, 8, 256, 4, A16 + 8, A16, None, A16, need, None) == INVALID
    assert fr(A16, 0, A16, A16, 1, 8, 256, 4, A16, A16, None, A16, need - 1, None) == WORKSPACE
    assert fr(A16, 0, A16, A16, 1, 8, 256, 4, A16, A16, None, None, need, None) == WORKSPACE
    assert fr(A16, 0, A16, A16, 1, 8, 256, 4, A16, A16, None, A16 + 64, need, None) == INVALID   # ws alignment
    assert fr(A16, 2, A16, A16, 1, 8, 256, 4, A16, A16, None, A16, need, None) == UNSUPPORTED


def test_valid_calls_without_a_device_report_no_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    assert qa() == NO_DEVICE
    assert gm() == NO_DEVICE
    assert mx.macaq_hessian(A16, 0, A16, None, 1, 16, 128, A16, None) == NO_DEVICE
    assert mx.macaq_prepare_weights_hessian(A16, 0, A16, A16, 1, 8, 64, A16, A16, None) == NO_DEVICE
    assert mx.macaq_flip_refine(A16, 0, A16, A16, 1, 8, 256, 4, A16, A16, None, A16, 1 << 20, None) == NO_DEVICE
    assert mx.macaq_tile_weights(A16, A16, 1, 64, 512, A16 * 16, A16 * 16, None) == NO_DEVICE
    assert b"no HIP device" in mx.lib().macaq_last_error()


def test_linear_path_choice_and_workspace():
    """AUTO takes the one-launch fused path for M <= 2 on a dense layer with
    K % 256 == 0, and for small layers (ceil(N/32) * M * K <= 2^20), the
    two-launch path otherwise; only the latter needs a workspace for the
    activation codes and scales."""
    L = mx.lib()
    P = L.macaq_linear_path
    assert P(1, 25600, 5120, 1, mx.PATH_AUTO) == mx.PATH_FUSED
    assert P(2, 5120, 25600, 1, mx.PATH_AUTO) == mx.PATH_FUSED
    assert P(3, 5120, 25600, 1, mx.PATH_AUTO) == mx.PATH_UNFUSED
    assert P(16, 128, 256, 1, mx.PATH_AUTO) == mx.PATH_FUSED            # tiny: 4 * 16 * 256 repeated values
    assert P(32, 1024, 1024, 1, mx.PATH_AUTO) == mx.PATH_FUSED          # exactly 2^20
    assert P(32, 1056, 1024, 1, mx.PATH_AUTO) == mx.PATH_UNFUSED        # one 32-row block more
    assert P(1, 4096, 4096 + 128, 1, mx.PATH_AUTO) == mx.PATH_UNFUSED   # K % 256 != 0
    assert P(1, 1024, 3072, 64, mx.PATH_AUTO) == mx.PATH_UNFUSED        # grouped
    assert P(2048, 4096, 4096, 1, mx.PATH_AUTO) == mx.PATH_UNFUSED
    assert P(8, 128, 256, 1, mx.PATH_FUSED) == mx.PATH_FUSED
    assert P(8, 128, 256, 1, mx.PATH_UNFUSED) == mx.PATH_UNFUSED
    assert P(8, 128, 256, 1, 7) == INVALID
    assert L.macaq_linear_workspace_bytes(1, 25600, 5120, 1, mx.PATH_AUTO) == 0
    assert L.macaq_linear_workspace_bytes(8, 25600, 5120, 1, mx.PATH_AUTO) == L.macaq_quant_act_bytes(8, 5120)
    assert L.macaq_linear_workspace_bytes(1, 25600, 5120, 1, mx.PATH_UNFUSED) == L.macaq_quant_act_bytes(1, 5120)


def test_forced_fused_path_refuses_what_it_cannot_serve():
    L = mx.lib()
    lin = mx.macaq_linear
    # 32 rows of a 25600-wide activation: the one-launch fused layer, which
    # stages the activation (and its counts) in the workspace
    need = L.macaq_linear_workspace_bytes(32, 5120, 25600, 1, mx.PATH_FUSED)
    assert need >= 32 * 25600 // 2 + 32 * 25600 // 32 + 16
    assert lin(A16, 0, A16, None, 1, A16, A16, 32, 5120, 25600, A16, None, 0, mx.PATH_FUSED, None) == WORKSPACE
    # grouped layers and K % 256 != 0 take the two-launch path only
    assert lin(A16, 0, A16, A16, 2, A16, A16, 1, 512, 1024, A16, None, 0, mx.PATH_FUSED, None) == UNSUPPORTED
    assert lin(A16, 0, A16, None, 1, A16, A16, 1, 512, 384, A16, None, 0, mx.PATH_FUSED, None) == UNSUPPORTED
    # M > 32 is not a decode shape
    assert lin(A16, 0, A16, None, 1, A16, A16, 33, 512, 1024, A16, None, 0, mx.PATH_FUSED, None) == UNSUPPORTED


def test_output_dtype_and_epilogue_validation():
    mx.lib()
    ge = mx.macaq_gemm_ex
    # unknown y dtype, unknown epilogue, SwiGLU with odd N, misaligned bf16/fp32 y
    assert ge(A16, A16, None, 1, A16, A16, 4, 8, 256, A16, 7, 0, None, 0, None) == UNSUPPORTED
    assert ge(A16, A16, None, 1, A16, A16, 4, 8, 256, A16, 1, 5, None, 0, None) == INVALID
    assert ge(A16, A16, None, 1, A16, A16, 4, 9, 256, A16, 1, 1, None, 0, None) == INVALID
    assert ge(A16, A16, None, 1, A16, A16, 4, 8, 256, A16 + 1, 0, 0, None, 0, None) == INVALID
    assert ge(A16, A16, None, 1, A16, A16, 4, 8, 256, A16 + 2, 1, 0, None, 0, None) == INVALID
    assert ge(A16, A16, None, 1, A16, A16, 0, 8, 256, A16 + 2, 0, 1, None, 0, None) == OK   # M == 0: no-op
    le = mx.macaq_linear_ex
    assert le(A16, 0, A16, None, 1, A16, A16, 4, 9, 256, A16, 0, 1, None, 0, 0, None) == INVALID


def test_tiled_weights_validation():
    """macaq_tile_weights and the MACAQ_W_TILED layout bit: shape rule
    (N % 32 == 0, K % 128 == 0), pointers, aliasing; layers with tiled
    weights take the two-launch path and refuse the fused decode path."""
    mx.lib()
    tw = mx.macaq_tile_weights
    A2 = A16 * 16
    assert tw(A16, A16, 1, 48, 512, A2, A2, None) == UNSUPPORTED      # N % 32 != 0
    assert tw(A16, A16, 1, 64, 416, A2, A2, None) == UNSUPPORTED      # K % 128 != 0
    assert tw(A16, A16, 1, 64, 48, A2, A2, None) == INVALID           # K % 32 != 0
    assert tw(A16, A16, 0, 64, 512, A2, A2, None) == INVALID
    assert tw(None, A16, 1, 64, 512, A2, A2, None) == INVALID
    assert tw(A16 + 4, A16, 1, 64, 512, A2, A2, None) == INVALID      # misaligned codes
    assert tw(A16, A16 + 2, 1, 64, 512, A2, A2, None) == INVALID      # misaligned scales
    assert tw(A16, A16, 1, 64, 512, A16 + 256, A2, None) == INVALID   # output overlaps input
    T = mx.W_TILED
    ge = mx.macaq_gemm_ex
    assert ge(A16, A16, None, 1, A16, A16, 4, 48, 256, A16, 0, T, None, 0, None) == UNSUPPORTED
    assert ge(A16, A16, None, 1, A16, A16, 4, 64, 416, A16, 0, T, None, 0, None) == UNSUPPORTED   # K % 128 != 0
    assert ge(A16, A16, None, 1, A16, A16, 4, 64, 256, A16, 0, T | 4, None, 0, None) == INVALID   # unknown epilogue
    assert ge(A16, A16, None, 1, A16, A16, 0, 64, 256, A16, 0, T, None, 0, None) == OK           # M == 0
    le = mx.macaq_linear_ex
    assert le(A16, 0, A16, None, 1, A16, A16, 1, 64, 256, A16, 0, 0, None, 0, mx.PATH_FUSED | T, None) == UNSUPPORTED
    assert le(A16, 0, A16, None, 1, A16, A16, 1, 64, 256, A16, 0, 0, None, 0, 8 | T, None) == INVALID
    L = mx.lib()
    assert L.macaq_linear_path(1, 25600, 5120, 1, mx.PATH_AUTO | T) == mx.PATH_UNFUSED
    # a dense layer with tiled weights stages its activation tiled: whole 32-row blocks
    assert L.macaq_linear_workspace_bytes(1, 25600, 5120, 1, mx.PATH_AUTO | T) == L.macaq_quant_act_bytes(32, 5120)
    assert L.macaq_linear_workspace_bytes(33, 4096, 4096, 1, T) == L.macaq_quant_act_bytes(64, 4096)
    # grouped: every expert starts a 32-row block, at most ceil((M + 31 E) / 32) * 32 rows
    assert L.macaq_quant_act_tiled_rows(33, 4) == 160
    assert L.macaq_linear_workspace_bytes(33, 1024, 3072, 4, T) == L.macaq_quant_act_bytes(160, 3072)


def test_set_tuning_validation_and_restore():
    """macaq_set_tuning: unknown knobs and out-of-range values are refused;
    a valid value returns the previous one, and 0 restores the automatic
    choice."""
    mx.lib()
    assert mx.macaq_set_tuning(-1, 0) == INVALID
    assert mx.macaq_set_tuning(10, 0) == INVALID
    assert mx.macaq_set_tuning(mx.TUNE_DECODE_POLLS, 65) == INVALID
    assert mx.macaq_set_tuning(mx.TUNE_GEMM_TILE, 4) == INVALID
    assert mx.macaq_set_tuning(mx.TUNE_ACT_SHARED_S, -1) == INVALID
    assert mx.set_tuning(mx.TUNE_GEMM_TILE, 3) == 0
    assert mx.set_tuning(mx.TUNE_GEMM_TILE, 1) == 3
    assert mx.set_tuning(mx.TUNE_GEMM_TILE, 0) == 1
    assert mx.set_tuning(mx.TUNE_DECODE_ROWS, 64) == 0
    assert mx.set_tuning(mx.TUNE_DECODE_ROWS, 0) == 64
    with pytest.raises(mx.MacaqError):
        mx.set_tuning(mx.TUNE_DECODE_WAVES, 9)


def test_no_tuning_environment_on_the_launch_path():
    """The kernel choices read no environment variable (only the MACAQ_CHECK
    debug switch is read by the entry points)."""
    csrc = os.path.join(ROOT, "mxfp4_w4a4_quantized_channel_amd", "csrc")
    for f in os.listdir(csrc):
        text = open(os.path.join(csrc, f)).read()
        for m in re.finditer(r"getenv\(\s*\"([A-Z_]+)\"", text):
            assert m.group(1) == "MACAQ_CHECK", (f, m.group(1))


def test_noalloc_validation_before_any_device_call():
    """macaq_linear_noalloc checks its arguments and refuses a shape whose
    staging exceeds the static scratch array before touching a device."""
    mx.lib()
    la = lambda M=4, N=8, K=256, E=1, flags=0, x=A16: mx.macaq_linear_noalloc(
        x, 0, A16, None, E, A16, A16, M, N, K, A16, 1, 0, flags, None)
    assert la(K=100) == INVALID
    assert la(flags=7) == INVALID
    assert la(x=None) == INVALID
    assert la(M=0) == OK
    assert la(M=8192, K=16384, flags=2) == WORKSPACE
    assert b"static scratch" in mx.macaq_last_error()

"""Python binding of libmacaq.so, the MI355X (gfx950) MXFP4 W4A4 linear layer
with an online per-channel scale and a 32-element block Hadamard transform.

The binding only marshals arguments: it checks tensor dtypes, devices,
shapes and contiguity, allocates outputs with torch, and passes raw device
pointers and torch's current HIP stream to the C ABI declared in
include/macaq.h.  Every step of the layer runs in the library's HIP kernels;
there is no fallback.  If the library is missing or fails to load, every
call raises.

Raw C entry points are available under their C names (``macaq_linear`` ...);
the tensor-level functions below carry the same names without the prefix.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "lib", "MacaqError", "BF16", "F32", "PATH_AUTO", "PATH_FUSED", "PATH_UNFUSED",
    "prepare_weights", "quant_act", "gemm", "linear", "linear_workspace_bytes",
    "encode_e2m1", "quant_mxfp4", "version", "library_path", "EPI_NONE", "EPI_SWIGLU",
    "hessian", "prepare_weights_hessian", "flip_refine", "flip_refine_workspace_bytes",
    "set_tuning", "linear_noalloc", "quant_act_tiled", "A_TILED", "W_TILED", "NOALLOC_SCRATCH_BYTES", "TUNE_GEMM_TILE", "TUNE_GEMM_GROUP_M",
    "TUNE_ACT_ROWS_PER_WAVE", "TUNE_ACT_SHARED_S",
    "TUNE_DECODE_WAVES", "TUNE_DECODE_STAGES", "TUNE_DECODE_ROWS", "TUNE_ACT_SEGMENT", "TUNE_DECODE_SPLIT",
    "TUNE_DECODE_POLLS", "GEMM_TILES",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libmacaq.so")

BF16, F32 = 0, 1
PATH_AUTO, PATH_FUSED, PATH_UNFUSED = 0, 1, 2
EPI_NONE, EPI_SWIGLU = 0, 1
NOALLOC_SCRATCH_BYTES = 32 << 20   # static staging of macaq_linear_noalloc, per device
A_TILED = 0x200   # activation codes in the tiled layout (gemm's epilogue argument, with W_TILED, E == 1)
W_TILED = 0x100   # weights in macaq_tile_weights' layout (OR into linear's flags / gemm's epilogue)
# knobs of macaq_set_tuning (0 = the library's own choice)
(TUNE_GEMM_TILE, TUNE_GEMM_GROUP_M, TUNE_ACT_ROWS_PER_WAVE, TUNE_ACT_SHARED_S, TUNE_DECODE_WAVES,
 TUNE_DECODE_STAGES, TUNE_DECODE_ROWS, TUNE_ACT_SEGMENT, TUNE_DECODE_SPLIT, TUNE_DECODE_POLLS) = range(10)
GEMM_TILES = {"256x256": 1, "256x128": 2, "128x128": 3}   # values of TUNE_GEMM_TILE
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported", -3: "no device", -4: "HIP error",
          -5: "workspace too small"}


class MacaqError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({detail})")


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise ImportError(f"{library_path} is missing: build it with "
                          f"`python -c 'import __graft_entry__ as g; g.build()'` "
                          f"or `python {os.path.join(_HERE, 'build.py')}`")
    L = ctypes.CDLL(library_path)
    vp, i64, u32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
    ci = ctypes.c_int
    sig = {
        "macaq_version": (ci, []),
        "macaq_set_tuning": (ci, [ci, ci]),
        "macaq_status_string": (ctypes.c_char_p, [ci]),
        "macaq_last_error": (ctypes.c_char_p, []),
        "macaq_prepare_weights": (ci, [vp, ci, vp, i64, i64, i64, vp, vp, vp]),
        "macaq_quant_act": (ci, [vp, ci, vp, vp, i64, i64, i64, vp, vp, vp]),
        "macaq_gemm": (ci, [vp, vp, vp, i64, vp, vp, i64, i64, i64, vp, vp, sz, vp]),
        "macaq_quant_act_bytes": (sz, [i64, i64]),
        "macaq_quant_act_tiled": (ci, [vp, ci, vp, vp, i64, i64, i64, vp, vp, vp]),
        "macaq_quant_act_tiled_rows": (sz, [i64, i64]),
        "macaq_gemm_workspace_bytes": (sz, [i64, i64, i64, i64]),
        "macaq_linear_workspace_bytes": (sz, [i64, i64, i64, i64, u32]),
        "macaq_linear_path": (ci, [i64, i64, i64, i64, u32]),
        "macaq_linear": (ci, [vp, ci, vp, vp, i64, vp, vp, i64, i64, i64, vp, vp, sz, u32, vp]),
        "macaq_gemm_ex": (ci, [vp, vp, vp, i64, vp, vp, i64, i64, i64, vp, ci, u32, vp, sz, vp]),
        "macaq_linear_ex": (ci, [vp, ci, vp, vp, i64, vp, vp, i64, i64, i64, vp, ci, u32, vp, sz, u32, vp]),
        "macaq_linear_noalloc": (ci, [vp, ci, vp, vp, i64, vp, vp, i64, i64, i64, vp, ci, u32, u32, vp]),
        "macaq_encode_e2m1": (ci, [vp, i64, vp, vp]),
        "macaq_quant_mxfp4": (ci, [vp, ci, i64, i64, vp, vp, vp]),
        "macaq_hessian": (ci, [vp, ci, vp, vp, i64, i64, i64, vp, vp]),
        "macaq_prepare_weights_hessian": (ci, [vp, ci, vp, vp, i64, i64, i64, vp, vp, vp]),
        "macaq_flip_refine": (ci, [vp, ci, vp, vp, i64, i64, i64, ctypes.c_int32, vp, vp, vp, vp, sz, vp]),
        "macaq_flip_refine_workspace_bytes": (sz, [i64, i64]),
        "macaq_tile_weights": (ci, [vp, vp, i64, i64, i64, vp, vp, vp]),
        "macaq_probe_mfma": (ci, [vp, i64, ci, ci, vp, vp]),
        "macaq_probe_stream": (ci, [vp, i64, vp, i64, i64, vp, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
        globals()[name] = f
    _lib = L
    return L


def lib():
    """The loaded ctypes library (raises ImportError if it is not built)."""
    return _load()


def version() -> int:
    return _load().macaq_version()


def set_tuning(knob: int, value: int) -> int:
    """Force one kernel choice process-wide (0 restores the automatic one);
    returns the knob's previous value."""
    prev = _load().macaq_set_tuning(int(knob), int(value))
    if prev < 0:
        _check(prev, "macaq_set_tuning")
    return prev


def _check(status: int, where: str):
    if status != 0:
        detail = _load().macaq_last_error().decode(errors="replace")
        raise MacaqError(status, where, detail)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"activations/weights must be bfloat16 or float32, got {t.dtype}")


def _need(t: torch.Tensor, name: str, dtype=None, dim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, got {t.dim()}")


def prepare_weights(w: torch.Tensor, s: torch.Tensor):
    """W' = quant(W diag(1/s) H) -> (codes [E,N,K/2] uint8, scales [E,N,K/32] uint8).

    w: [N, K] or [E, N, K] bf16/fp32; s: [K] or [E, K] fp32.
    """
    _load()
    if w.dim() == 2:
        w = w[None]
    if s.dim() == 1:
        s = s[None]
    _need(w, "w", dim=3)
    _need(s, "s", torch.float32, 2)
    E, N, K = w.shape
    if tuple(s.shape) != (E, K):
        raise ValueError(f"s must be [{E}, {K}], got {tuple(s.shape)}")
    codes = torch.empty((E, N, K // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((E, N, K // 32), dtype=torch.uint8, device=w.device)
    _check(macaq_prepare_weights(_ptr(w), _dtype_code(w), _ptr(s), E, N, K, _ptr(codes), _ptr(scales),
                                 _stream(w.device)), "macaq_prepare_weights")
    return codes, scales


def hessian(x: torch.Tensor, s: torch.Tensor, offsets: torch.Tensor | None = None, out=None):
    """Hessian of the transformed layer input from calibration rows:
    [E, K, K] fp32, h[e] = X'_e^T X'_e.

    x: [T, K] bf16/fp32 (rows sorted by expert); s: [K] or [E, K] fp32;
    offsets: [E+1] int32 GPU tensor (None when E == 1).
    """
    _load()
    if s.dim() == 1:
        s = s[None]
    _need(x, "x", dim=2)
    _need(s, "s", torch.float32, 2)
    T, K = x.shape
    E = s.shape[0]
    if offsets is not None:
        _need(offsets, "offsets", torch.int32, 1)
        if offsets.numel() != E + 1:
            raise ValueError("offsets must have E+1 entries")
    if out is None:
        out = torch.empty((E, K, K), dtype=torch.float32, device=x.device)
    else:
        _need(out, "out", torch.float32, 3)
        if tuple(out.shape) != (E, K, K):
            raise ValueError(f"out must be [{E}, {K}, {K}], got {tuple(out.shape)}")
    _check(macaq_hessian(_ptr(x), _dtype_code(x), _ptr(s), _ptr(offsets), E, T, K, _ptr(out),
                         _stream(x.device)), "macaq_hessian")
    return out


def prepare_weights_hessian(w: torch.Tensor, s: torch.Tensor, h: torch.Tensor):
    """W' with Hessian-searched scale bytes -> (codes [E,N,K/2], scales [E,N,K/32]).

    w: [N, K] or [E, N, K] bf16/fp32; s: [K] or [E, K] fp32; h: [K, K] or
    [E, K, K] fp32 (only the diagonal 32x32 blocks are read).
    """
    _load()
    if w.dim() == 2:
        w = w[None]
    if s.dim() == 1:
        s = s[None]
    if h.dim() == 2:
        h = h[None]
    _need(w, "w", dim=3)
    _need(s, "s", torch.float32, 2)
    _need(h, "h", torch.float32, 3)
    E, N, K = w.shape
    if tuple(s.shape) != (E, K):
        raise ValueError(f"s must be [{E}, {K}], got {tuple(s.shape)}")
    if tuple(h.shape) != (E, K, K):
        raise ValueError(f"h must be [{E}, {K}, {K}], got {tuple(h.shape)}")
    codes = torch.empty((E, N, K // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((E, N, K // 32), dtype=torch.uint8, device=w.device)
    _check(macaq_prepare_weights_hessian(_ptr(w), _dtype_code(w), _ptr(s), _ptr(h), E, N, K, _ptr(codes),
                                         _ptr(scales), _stream(w.device)), "macaq_prepare_weights_hessian")
    return codes, scales


def flip_refine_workspace_bytes(rows: int, K: int) -> int:
    return int(_load().macaq_flip_refine_workspace_bytes(rows, K))


def flip_refine(w: torch.Tensor, s: torch.Tensor, h: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                max_rounds: int, workspace: torch.Tensor | None = None, chunk_rows: int | None = None):
    """Flip-Refinement of prepared codes, in place -> moves per row [E, N] int32.

    w: [N, K] or [E, N, K] bf16/fp32; s: [K] or [E, K]; h: [K, K] or
    [E, K, K] fp32; codes [E, N, K/2] uint8 (refined in place); scales
    [E, N, K/32] uint8.  The workspace (allocated here if not given) holds
    the fp64 gradient of chunk_rows rows at a time (default: all E * N rows,
    one pair of launches for all experts).
    """
    _load()
    if w.dim() == 2:
        w = w[None]
    if s.dim() == 1:
        s = s[None]
    if h.dim() == 2:
        h = h[None]
    if codes.dim() == 2:
        codes, scales = codes[None], scales[None]
    _need(w, "w", dim=3)
    _need(s, "s", torch.float32, 2)
    _need(h, "h", torch.float32, 3)
    _need(codes, "codes", torch.uint8, 3)
    _need(scales, "scales", torch.uint8, 3)
    E, N, K = w.shape
    if tuple(s.shape) != (E, K) or tuple(h.shape) != (E, K, K):
        raise ValueError("s must be [E, K] and h [E, K, K]")
    if tuple(codes.shape) != (E, N, K // 2) or tuple(scales.shape) != (E, N, K // 32):
        raise ValueError("codes must be [E, N, K/2] and scales [E, N, K/32]")
    if workspace is None:
        workspace = torch.empty(flip_refine_workspace_bytes(chunk_rows or E * N, K), dtype=torch.uint8,
                                device=w.device)
    moves = torch.empty((E, N), dtype=torch.int32, device=w.device)
    _check(macaq_flip_refine(_ptr(w), _dtype_code(w), _ptr(s), _ptr(h), E, N, K, int(max_rounds), _ptr(codes),
                             _ptr(scales), _ptr(moves), _ptr(workspace), workspace.numel(), _stream(w.device)),
           "macaq_flip_refine")
    return moves


def quant_act(x: torch.Tensor, s: torch.Tensor, offsets: torch.Tensor | None = None):
    """Online transform + MXFP4 of activations -> (codes [M,K/2], scales [M,K/32]).

    x: [M, K] bf16/fp32 (rows sorted by expert); s: [K] or [E, K] fp32;
    offsets: [E+1] int32 GPU tensor (None when E == 1).
    """
    _load()
    if s.dim() == 1:
        s = s[None]
    _need(x, "x", dim=2)
    _need(s, "s", torch.float32, 2)
    M, K = x.shape
    E = s.shape[0]
    if offsets is not None:
        _need(offsets, "offsets", torch.int32, 1)
        if offsets.numel() != E + 1:
            raise ValueError("offsets must have E+1 entries")
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
    _check(macaq_quant_act(_ptr(x), _dtype_code(x), _ptr(s), _ptr(offsets), E, M, K, _ptr(codes),
                           _ptr(scales), _stream(x.device)), "macaq_quant_act")
    return codes, scales


def quant_act_tiled(x: torch.Tensor, s: torch.Tensor, offsets: torch.Tensor | None = None):
    """quant_act in the tiled, expert-padded layout the prefill and grouped
    GEMMs read -> (codes [rows*K/2] uint8, scales [rows*K/32] uint8), flat,
    rows = macaq_quant_act_tiled_rows(M, E).  Use with
    gemm(..., epilogue=W_TILED | A_TILED, M=M)."""
    _load()
    if s.dim() == 1:
        s = s[None]
    _need(x, "x", dim=2)
    _need(s, "s", torch.float32, 2)
    M, K = x.shape
    E = s.shape[0]
    if offsets is not None:
        _need(offsets, "offsets", torch.int32, 1)
    rows = int(_load().macaq_quant_act_tiled_rows(M, E))
    codes = torch.empty(rows * K // 2, dtype=torch.uint8, device=x.device)
    scales = torch.empty(rows * K // 32, dtype=torch.uint8, device=x.device)
    _check(macaq_quant_act_tiled(_ptr(x), _dtype_code(x), _ptr(s), _ptr(offsets), E, M, K, _ptr(codes), _ptr(scales),
                                 _stream(x.device)), "macaq_quant_act_tiled")
    return codes, scales


def _w_shape(w_codes, w_scales):
    if w_codes.dim() == 2:
        w_codes, w_scales = w_codes[None], w_scales[None]
    _need(w_codes, "w_codes", torch.uint8, 3)
    _need(w_scales, "w_scales", torch.uint8, 3)
    return w_codes, w_scales


def _out(M, N, out_dtype, epilogue, device, out):
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"out_dtype must be float32 or bfloat16, got {out_dtype}")
    width = N // 2 if (epilogue & ~(W_TILED | A_TILED)) == EPI_SWIGLU else N
    if out is None:
        return torch.empty((M, width), dtype=out_dtype, device=device)
    _need(out, "out", out_dtype, 2)
    if tuple(out.shape) != (M, width):
        raise ValueError(f"out must be [{M}, {width}], got {tuple(out.shape)}")
    return out


def gemm(a_codes, a_scales, w_codes, w_scales, offsets=None, out=None, workspace=None,
         out_dtype=torch.float32, epilogue=EPI_NONE, M=None):
    """y = A' W'^T from MXFP4 operands: [M, N] (or [M, N/2] with EPI_SWIGLU)
    in out_dtype (float32 or bfloat16).  A workspace, when one is needed (the
    partial sums of a decode K split), is allocated here unless the caller
    passes one; its contents need no initialization.  With A_TILED
    in the epilogue argument, a_codes / a_scales are quant_act_tiled's flat
    buffers and M must be given."""
    _load()
    w_codes, w_scales = _w_shape(w_codes, w_scales)
    E, N, KH = w_codes.shape
    K = 2 * KH
    if epilogue & A_TILED:
        _need(a_codes, "a_codes", torch.uint8, 1)
        _need(a_scales, "a_scales", torch.uint8, 1)
        if M is None:
            raise ValueError("M is needed with tiled activation codes")
        rows = int(_load().macaq_quant_act_tiled_rows(M, E))
        if a_codes.numel() < rows * K // 2 or a_scales.numel() < rows * K // 32:
            raise ValueError("tiled activation buffers too small")
    else:
        _need(a_codes, "a_codes", torch.uint8, 2)
        _need(a_scales, "a_scales", torch.uint8, 2)
        M = a_codes.shape[0]
    y = _out(M, N, out_dtype, epilogue, a_codes.device, out)
    need = int(_load().macaq_gemm_workspace_bytes(M, N, K, E))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=a_codes.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ydt = F32 if out_dtype == torch.float32 else BF16
    _check(macaq_gemm_ex(_ptr(a_codes), _ptr(a_scales), _ptr(offsets), E, _ptr(w_codes), _ptr(w_scales),
                         M, N, K, _ptr(y), ydt, epilogue, _ptr(workspace), ws_bytes, _stream(a_codes.device)),
           "macaq_gemm")
    return y


def linear_workspace_bytes(M, N, K, E=1, flags=PATH_AUTO) -> int:
    return int(_load().macaq_linear_workspace_bytes(M, N, K, E, flags))


def linear(x, s, w_codes, w_scales, offsets=None, flags=PATH_AUTO, out=None, workspace=None,
           out_dtype=torch.float32, epilogue=EPI_NONE):
    """The whole online layer y = quant(x diag(s) H) W'^T: [M, N] (or
    [M, N/2] with EPI_SWIGLU) in out_dtype (float32 or bfloat16)."""
    _load()
    if s.dim() == 1:
        s = s[None]
    w_codes, w_scales = _w_shape(w_codes, w_scales)
    _need(x, "x", dim=2)
    _need(s, "s", torch.float32, 2)
    M, K = x.shape
    E, N, _ = w_codes.shape
    need = linear_workspace_bytes(M, N, K, E, flags)
    if workspace is None and need > 0:   # (its contents need no initialization)
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    y = _out(M, N, out_dtype, epilogue, x.device, out)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ydt = F32 if out_dtype == torch.float32 else BF16
    _check(macaq_linear_ex(_ptr(x), _dtype_code(x), _ptr(s), _ptr(offsets), E, _ptr(w_codes), _ptr(w_scales),
                           M, N, K, _ptr(y), ydt, epilogue, _ptr(workspace), ws_bytes, flags, _stream(x.device)),
           "macaq_linear")
    return y


def linear_noalloc(x, s, w_codes, w_scales, offsets=None, flags=PATH_AUTO, out=None,
                   out_dtype=torch.float32, epilogue=EPI_NONE):
    """linear() through macaq_linear_noalloc: no workspace; the unfused
    path's staging lives in the library's static device array."""
    _load()
    if s.dim() == 1:
        s = s[None]
    w_codes, w_scales = _w_shape(w_codes, w_scales)
    _need(x, "x", dim=2)
    _need(s, "s", torch.float32, 2)
    M, K = x.shape
    E, N, _ = w_codes.shape
    y = _out(M, N, out_dtype, epilogue, x.device, out)
    ydt = F32 if out_dtype == torch.float32 else BF16
    _check(macaq_linear_noalloc(_ptr(x), _dtype_code(x), _ptr(s), _ptr(offsets), E, _ptr(w_codes), _ptr(w_scales),
                                M, N, K, _ptr(y), ydt, epilogue, flags, _stream(x.device)),
           "macaq_linear_noalloc")
    return y


def tile_weights(w_codes, w_scales):
    """Prepared weights (row-major codes [E, N, K/2], scales [E, N, K/32])
    repacked into the tiled layout the prefill and grouped GEMMs read with
    contiguous copies; same shapes and bytes, other places.  Use the result
    with W_TILED in linear's flags or gemm's epilogue.  N % 32 == 0 and
    K % 128 == 0."""
    _load()
    w_codes, w_scales = _w_shape(w_codes, w_scales)
    E, N, KH = w_codes.shape
    tc, ts = torch.empty_like(w_codes), torch.empty_like(w_scales)
    _check(macaq_tile_weights(_ptr(w_codes), _ptr(w_scales), E, N, 2 * KH, _ptr(tc), _ptr(ts),
                              _stream(w_codes.device)), "macaq_tile_weights")
    return tc, ts


def quant_mxfp4(x: torch.Tensor):
    """Plain OCP MXFP4 of rows (no scale, no transform) -> (codes [M,K/2], scales [M,K/32])."""
    _load()
    _need(x, "x", dim=2)
    M, K = x.shape
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
    _check(macaq_quant_mxfp4(_ptr(x), _dtype_code(x), M, K, _ptr(codes), _ptr(scales), _stream(x.device)),
           "macaq_quant_mxfp4")
    return codes, scales


def encode_e2m1(v: torch.Tensor) -> torch.Tensor:
    """E2M1 code (one per byte) of each fp32 value, by the library's encoder."""
    _load()
    _need(v, "v", torch.float32)
    out = torch.empty(v.shape, dtype=torch.uint8, device=v.device)
    _check(macaq_encode_e2m1(_ptr(v), v.numel(), _ptr(out), _stream(v.device)), "macaq_encode_e2m1")
    return out

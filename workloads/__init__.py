"""Seeded synthetic inputs for the MXFP4 W4A4 linear layer.

This module only draws random tensors and routes tokens; it holds none of
the layer's arithmetic (no transform, no quantization, no GEMM).  Both the
CPU oracle's tests and the HIP path's tests and benchmark take their inputs
from here, so that the two sides see identical bits.

The pages measure on Llama-3-8B / Qwen3-32B layers and on WikiText-2 / C4,
none of which is available offline.  The tensors below only take the
*shapes* of those models' linear layers (attention projection, MLP
down-projection, decode gate/up/down, MoE experts) with synthetic values:
Gaussian or Student-t activations with a few seeded outlier channels and
Gaussian weights.

Every draw uses ``np.random.default_rng(SeedSequence([seed, cfg, variant,
stream]))`` with streams 0 = outlier channels, 1 = calibration activations,
2 = measured activations, 3 = weights, 4 = routing.  Values are drawn in
float64, outlier channels are multiplied, and the result is cast with
round-to-nearest-even (torch's CPU cast) to bfloat16, or kept in float32
for the tiny layer.

The per-channel scale comes from the smoothing factor
``sigma_k = sqrt(max_t |Xcal[t,k]| / max_n |W[n,k]|)`` over a calibration
draw that shares the outlier channels with the measured activations
(computed in float64 on the cast tensors).  The layer multiplies x by s and
W by 1/s; by default ``s = 1 / sigma`` (``scale_rule="smooth"``), which
shrinks outlier channels of x.  ``scale_rule="literal"`` gives ``s = sigma``,
which multiplies outlier channels up instead.  Either is rounded to float32;
the layer is exact in both cases before quantization.  Mixture-of-experts
layers have one ``s`` and one weight matrix per expert.
"""
from __future__ import annotations

import dataclasses
import numpy as np
import torch

__all__ = ["Workload", "make", "CONFIG_NAMES", "bf16_bits", "zipf_expert_counts"]

STREAM_OUTLIERS, STREAM_CALIB, STREAM_X, STREAM_W, STREAM_ROUTE = 0, 1, 2, 3, 4


@dataclasses.dataclass
class Workload:
    """One synthetic linear layer.

    x:        [M, K] activations (torch bfloat16, or float32 for the tiny layer),
              rows sorted by expert for mixture-of-experts layers
    w:        [E, N, K] weights, same dtype family as x
    s:        [E, K] float32 per-channel scales (> 0)
    offsets:  [E+1] int32 row offsets of each expert in x (offsets[E] == M)
    xcal:     [T, K] calibration activations s was derived from, rows sorted
              by expert (only with make(..., keep_calib=True), else None)
    cal_offsets: [E+1] int32 row offsets of each expert in xcal (or None)
    """
    name: str
    x: torch.Tensor
    w: torch.Tensor
    s: torch.Tensor
    offsets: torch.Tensor
    outlier_channels: np.ndarray
    xcal: torch.Tensor | None = None
    cal_offsets: torch.Tensor | None = None

    @property
    def M(self) -> int:
        return int(self.x.shape[0])

    @property
    def K(self) -> int:
        return int(self.x.shape[1])

    @property
    def N(self) -> int:
        return int(self.w.shape[1])

    @property
    def E(self) -> int:
        return int(self.w.shape[0])


def _rng(seed: int, cfg: int, variant: int, stream: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, cfg, variant, stream, *extra]))


def _cast(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(dtype)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw 16-bit patterns of a bfloat16 tensor as a numpy uint16 array."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _draw_acts(rng, rows, K, dist, outliers, factor, chunk=1024):
    out = np.empty((rows, K), dtype=np.float64)
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        if dist == "normal":
            blk = rng.standard_normal((r1 - r0, K))
        elif dist == "t4":
            blk = rng.standard_t(4.0, size=(r1 - r0, K))
        else:
            raise ValueError(dist)
        blk[:, outliers] *= factor
        out[r0:r1] = blk
    return out


def _colmax_abs(t: torch.Tensor) -> np.ndarray:
    return t.abs().to(torch.float64).amax(dim=0).numpy()


def _scale(calib: torch.Tensor, w: torch.Tensor, rule: str) -> np.ndarray:
    """sigma_k = sqrt(max|calib[:,k]| / max|w[:,k]|) in float64; returns
    s = 1/sigma ("smooth") or s = sigma ("literal"), rounded to float32."""
    ax = _colmax_abs(calib)
    aw = _colmax_abs(w)
    aw = np.where(aw > 0, aw, 1.0)
    ax = np.where(ax > 0, ax, 1.0)
    if rule == "smooth":
        return np.sqrt(aw / ax).astype(np.float32)
    if rule == "literal":
        return np.sqrt(ax / aw).astype(np.float32)
    raise ValueError(rule)


def zipf_expert_counts(rng: np.random.Generator, n_experts: int, tokens: int, a: float) -> np.ndarray:
    """Split ``tokens`` over experts in proportion to iid Zipf(a) weights.

    Each expert draws one Zipf(a) weight; counts are floor(tokens * z / sum z)
    plus the leftover tokens handed out by largest fractional part (stable).
    With a = 1.1 the weights have infinite mean, so a few experts take almost
    every token and many are empty.
    """
    z = rng.zipf(a, size=n_experts).astype(np.float64)
    share = tokens * z / z.sum()
    base = np.floor(share).astype(np.int64)
    left = tokens - int(base.sum())
    frac = share - base
    order = np.argsort(-frac, kind="stable")
    base[order[:left]] += 1
    return base


def _token_zipf_counts(rng, n_experts, tokens, a):
    """Per-token routing: each token picks an expert from a Zipf(a) law truncated to n_experts ranks."""
    ranks = np.arange(1, n_experts + 1, dtype=np.float64)
    p = ranks ** (-a)
    p /= p.sum()
    choice = rng.choice(n_experts, size=tokens, p=p)
    return np.bincount(choice, minlength=n_experts).astype(np.int64)


CONFIG_NAMES = {
    1: "tiny M16 N128 K256 fp32",
    2: "attn-proj M2048 N4096 K4096 bf16",
    3: "down-prefill M4096 N4096 K14336 bf16",
    4: "decode gate/up M{1,8,32} N25600 K5120 / down N5120 K25600 bf16",
    5: "MoE E64 T8192 N1024 K3072 bf16",
}


def make(cfg: int, *, variant: int = 0, M: int | None = None, seed: int = 0,
         shape: tuple[int, int, int] | None = None, routing: str = "expert_zipf",
         scale_rule: str = "smooth", keep_calib: bool = False) -> Workload:
    """Build the synthetic layer of config ``cfg`` (1..5).

    variant: config 4 only, 0 = gate/up (K5120 N25600), 1 = down (K25600 N5120).
    M:       config 4 only, number of decode rows (first M rows of a 32-row draw).
    shape:   optional (M, N, K) override that keeps the config's value
             distributions; used for small parity cases.
    routing: config 5 only, "expert_zipf" (iid Zipf(1.1) weight per expert,
             largest-remainder split; many experts empty) or "token_zipf"
             (each token draws a rank from Zipf(1.1) truncated to 64 experts).
    scale_rule: "smooth" (s = 1/sigma, default) or "literal" (s = sigma).
    keep_calib: also return the calibration draw (xcal, cal_offsets).
    """
    if cfg == 1:
        Mx, N, K = shape or (16, 128, 256)
        dist, frac, factor, w_std, n_cal, dtype = "normal", None, 40.0, 0.02, 64, torch.float32
        outl = np.array([c for c in (3, 97) if c < K], dtype=np.int64)
        E = 1
    elif cfg == 2:
        Mx, N, K = shape or (2048, 4096, 4096)
        dist, frac, factor, w_std, n_cal, dtype, E = "normal", 0.01, 50.0, 0.02, 4096, torch.bfloat16, 1
    elif cfg == 3:
        Mx, N, K = shape or (4096, 4096, 14336)
        dist, frac, factor, w_std, n_cal, dtype, E = "t4", 0.005, 100.0, 0.015, 4096, torch.bfloat16, 1
    elif cfg == 4:
        if shape is None:
            N, K = (25600, 5120) if variant == 0 else (5120, 25600)
            Mx = 32
        else:
            Mx, N, K = shape
        dist, frac, factor, w_std, n_cal, dtype, E = "normal", 0.01, 50.0, 0.02, 4096, torch.bfloat16, 1
    elif cfg == 5:
        Mx, N, K = shape or (8192, 1024, 3072)
        dist, frac, factor, w_std, n_cal, dtype, E = "normal", 0.01, 50.0, 0.02, 512, torch.bfloat16, 64
    else:
        raise ValueError(f"unknown config {cfg}")

    if cfg != 1:
        n_out = int(round(frac * K))
        outl = np.sort(_rng(seed, cfg, variant, STREAM_OUTLIERS).choice(K, n_out, replace=False))

    if cfg == 5:
        rr = _rng(seed, cfg, variant, STREAM_ROUTE)
        if routing == "expert_zipf":
            counts = zipf_expert_counts(rr, E, Mx, 1.1)
        elif routing == "token_zipf":
            counts = _token_zipf_counts(rr, E, Mx, 1.1)
        else:
            raise ValueError(routing)
        x = _cast(_draw_acts(_rng(seed, cfg, variant, STREAM_X), Mx, K, dist, outl, factor), dtype)
        ws, ss, cals = [], [], []
        for e in range(E):
            w_e = _cast(_rng(seed, cfg, variant, STREAM_W, e).standard_normal((N, K)) * w_std, dtype)
            cal = _cast(_draw_acts(_rng(seed, cfg, variant, STREAM_CALIB, e), n_cal, K, dist, outl, factor), dtype)
            ss.append(_scale(cal, w_e, scale_rule))
            ws.append(w_e)
            if keep_calib:
                cals.append(cal)
        w = torch.stack(ws)
        s = torch.from_numpy(np.stack(ss))
        offsets = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32))
        name = f"{CONFIG_NAMES[5]} routing={routing}"
        if not keep_calib:
            return Workload(name, x, w, s, offsets, outl)
        cal_off = torch.arange(E + 1, dtype=torch.int32) * n_cal
        return Workload(name, x, w, s, offsets, outl, torch.cat(cals), cal_off)

    x_all = _draw_acts(_rng(seed, cfg, variant, STREAM_X), Mx, K, dist, outl, factor)
    if cfg == 4 and M is not None:
        x_all = x_all[:M]
    x = _cast(x_all, dtype)
    w = _cast(_rng(seed, cfg, variant, STREAM_W).standard_normal((N, K)) * w_std, dtype)
    cal = _cast(_draw_acts(_rng(seed, cfg, variant, STREAM_CALIB), n_cal, K, dist, outl, factor), dtype)
    s = torch.from_numpy(_scale(cal, w, scale_rule))[None, :].contiguous()
    offsets = torch.tensor([0, x.shape[0]], dtype=torch.int32)
    name = CONFIG_NAMES[cfg] if shape is None else f"cfg{cfg}-shaped M{x.shape[0]} N{N} K{K}"
    if not keep_calib:
        return Workload(name, x, w[None].contiguous(), s, offsets, outl)
    cal_off = torch.tensor([0, cal.shape[0]], dtype=torch.int32)
    return Workload(name, x, w[None].contiguous(), s, offsets, outl, cal, cal_off)

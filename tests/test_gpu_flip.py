"""Flip-Refinement on the GPU (macaq_flip_refine, through the C ABI) against
the CPU oracle: refined codes and the number of moves per row bit-exact,
from the same start codes, scale bytes and fp32 Hessian on both sides (the
decisions are fp64 comparisons made in the same operation order)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import mxfp4_w4a4_quantized_channel_amd as mx

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return workloads.bf16_bits(t)
    return t.numpy()


def say(msg):
    print(f"[case] {msg}", flush=True)


def xprime_w(w_bits, s):
    wf = oracle.as_f32(w_bits)
    return oracle.transform(wf, np.broadcast_to(oracle.weight_reciprocal(s), wf.shape))


def run_both(w, s, h, start, max_rounds, rows=None, chunk_rows=None):
    """w torch [E,N,K]; s numpy [E,K]; h numpy fp32 [E,K,K]; start = (codes,
    scales) numpy [E,...].  Returns GPU and oracle (codes, moves) per expert."""
    c0, s0 = start
    codes = torch.from_numpy(c0.copy()).to(DEV)
    scales = torch.from_numpy(s0).to(DEV)
    moves = mx.flip_refine(w.to(DEV), torch.from_numpy(s).to(DEV), torch.from_numpy(h).to(DEV), codes, scales,
                           max_rounds, chunk_rows=chunk_rows)
    torch.cuda.synchronize()
    gc, gm = codes.cpu().numpy(), moves.cpu().numpy()
    out = []
    for e in range(w.shape[0]):
        wb = host(w[e])
        sel = np.arange(wb.shape[0]) if rows is None else rows
        xp = xprime_w(wb[sel], s[e])
        rc, rm = oracle.flip_refine(xp, c0[e][sel], s0[e][sel], h[e], max_rounds)
        out.append((gc[e][sel], gm[e][sel], rc, rm))
    return out


def check(out, what):
    total = 0
    for e, (gc, gm, rc, rm) in enumerate(out):
        bad = np.nonzero((gc != rc).any(axis=1) | (gm != rm))[0]
        assert bad.size == 0, f"{what} expert {e}: rows {bad[:8].tolist()} differ (moves gpu {gm[bad[:4]]}, oracle {rm[bad[:4]]})"
        total += int(rm.sum())
    return total


def calib_case(cfg, N, K):
    wl = workloads.make(cfg, shape=(16, N, K), keep_calib=True)
    h = oracle.hessian(host(wl.xcal), wl.s.numpy()).astype(np.float32)
    return wl, h


@pytest.mark.parametrize("cfg,rounds", [(2, 0), (2, 7), (2, 10000), (1, 10000), (3, 40)])
def test_flip_small_calibration_hessian(cfg, rounds):
    """Dense layer, calibration Hessian, round-to-nearest start codes: fp32
    weights (cfg 1) and bf16; no rounds, a few rounds, and to convergence."""
    wl, h = calib_case(cfg, 96, 256)
    say(f"flip cfg{cfg} N96 K256 rounds {rounds}")
    s = wl.s.numpy()
    start = tuple(np.stack(a) for a in zip(*[oracle.prepare_weights(host(wl.w[e]), s[e]) for e in range(wl.E)]))
    total = check(run_both(wl.w, s, h, start, rounds), f"cfg{cfg} rounds {rounds}")
    print(f"moves: {total}")
    if rounds:
        assert total > 0


def test_flip_from_hessian_searched_bytes():
    """Start from the Hessian exponent search's codes and bytes."""
    wl, h = calib_case(2, 64, 512)
    say("flip from searched bytes N64 K512")
    s = wl.s.numpy()
    start = oracle.prepare_weights_hessian(host(wl.w[0]), s[0], h[0])
    start = (start[0][None], start[1][None])
    assert check(run_both(wl.w, s, h, start, 10000), "searched start") > 0


def test_flip_experts_random_coupled_hessians_and_chunks():
    """Three experts with their own s and strongly coupled random PSD
    Hessians, heavy-tailed weights, a ragged row count (300) processed in
    chunks of 128 rows: same result as one chunk, and as the oracle."""
    E, N, K = 3, 300, 384
    rng = np.random.default_rng(np.random.SeedSequence([17, 1]))
    w = torch.from_numpy((rng.standard_t(3, (E, N, K)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    s = rng.uniform(0.5, 2.0, (E, K)).astype(np.float32)
    h = np.empty((E, K, K), np.float32)
    for e in range(E):
        a = rng.standard_normal((K, K // 3))
        h[e] = (a @ a.T + 0.1 * np.eye(K)).astype(np.float32)
    start = tuple(np.stack(a) for a in zip(*[oracle.prepare_weights(host(w[e]), s[e]) for e in range(E)]))
    say(f"flip experts E{E} N{N} K{K} chunks of 128")
    out = run_both(w, s, h, start, 60, chunk_rows=128)
    assert check(out, "chunked") > 0
    codes = torch.from_numpy(start[0].copy()).to(DEV)
    moves = mx.flip_refine(w.to(DEV), torch.from_numpy(s).to(DEV), torch.from_numpy(h).to(DEV), codes,
                           torch.from_numpy(start[1]).to(DEV), 60)
    torch.cuda.synchronize()
    for e in range(E):
        assert np.array_equal(codes[e].cpu().numpy(), out[e][0])
        assert np.array_equal(moves[e].cpu().numpy(), out[e][1])


def test_flip_arbitrary_start_codes():
    """Start codes that are not round-to-nearest (random codes in some
    groups): their residuals carry more than 29 significant bits, so the
    gradient kernel takes the separate multiply and add for those column
    steps; codes and moves stay bit-exact."""
    wl, h = calib_case(2, 64, 512)
    say("flip from arbitrary start codes N64 K512")
    s = wl.s.numpy()
    c0, s0 = oracle.prepare_weights(host(wl.w[0]), s[0])
    rng = np.random.default_rng(np.random.SeedSequence([17, 3]))
    c0 = c0.copy()
    cols = np.concatenate([np.arange(16 * g, 16 * g + 16) for g in (1, 2, 9)])   # groups 1, 2 and 9
    c0[:, cols] = rng.integers(0, 256, (c0.shape[0], cols.size), dtype=np.uint8)
    assert check(run_both(wl.w, s, h, (c0[None], s0[None]), 10000), "arbitrary start") > 0


def test_flip_negative_diagonal_scans_both_directions():
    """A symmetric but indefinite H with some negative diagonal entries: a
    move against the sign of g_k can then gain, so the kernel scans both
    directions for such rows; codes and moves stay bit-exact."""
    N, K = 48, 256
    rng = np.random.default_rng(np.random.SeedSequence([17, 4]))
    w = torch.from_numpy((rng.standard_normal((1, N, K)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    s = rng.uniform(0.5, 2.0, (1, K)).astype(np.float32)
    a = rng.standard_normal((K, 64))
    h = a @ a.T
    neg = rng.choice(K, 12, replace=False)
    h[neg, neg] = -rng.uniform(1.0, 30.0, 12)
    h = h.astype(np.float32)[None]
    start = oracle.prepare_weights(host(w[0]), s[0])
    say(f"flip negative diagonal N{N} K{K}")
    assert check(run_both(w, s, h, (start[0][None], start[1][None]), 300), "negative diagonal") > 0


def test_flip_wide_rows_1024_threads():
    """K = 8320 (above 8192: 1024 threads per row, 12 coordinates each, the
    last ones past K masked)."""
    N, K = 4, 8320
    rng = np.random.default_rng(np.random.SeedSequence([17, 2]))
    w = torch.from_numpy((rng.standard_normal((1, N, K)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    s = rng.uniform(0.5, 2.0, (1, K)).astype(np.float32)
    a = rng.standard_normal((K, 48))
    h = (a @ a.T + 0.05 * np.eye(K)).astype(np.float32)[None]
    start = oracle.prepare_weights(host(w[0]), s[0])
    say(f"flip wide rows N{N} K{K}")
    assert check(run_both(w, s, h, (start[0][None], start[1][None]), 150), "wide") > 0


def test_flip_fullsize_sampled_rows():
    """Decode gate/up weights at full size (N25600 K5120) with the full
    calibration Hessian, 48 rounds: 48 sampled rows (first and last
    included) against the oracle."""
    wl = workloads.make(4, variant=0, M=1, keep_calib=True)
    N, K = wl.N, wl.K
    say(f"flip full size N{N} K{K} rounds 48")
    s = wl.s.numpy()
    h = oracle.hessian(host(wl.xcal), s).astype(np.float32)
    start = oracle.prepare_weights(host(wl.w[0]), s[0])
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(3).choice(N, 46, replace=False)]))
    out = run_both(wl.w, s, h, (start[0][None], start[1][None]), 48, rows=rows)
    assert check(out, "full size") > 0

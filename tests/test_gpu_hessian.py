"""Parity of the offline Hessian steps on the GPU (through the C ABI) with
the CPU oracle.

* macaq_hessian: the GPU accumulates exact fp32 x products in fp64 and
  rounds once to fp32, so every entry must satisfy
  |h - h_ref| <= 2^-24 |h_ref| + 1e-11 S (h_ref the oracle's fp64 Hessian,
  S = |X'|^T |X'|), and h must be exactly symmetric.
* macaq_prepare_weights_hessian: codes and scale bytes bit-exact against the
  oracle when both take the same fp32 Hessian (the oracle's, rounded).
* The whole offline chain (GPU Hessian, then GPU search) against the
  oracle's chain: the chosen bytes agree except where the oracle's two
  candidate errors are a near tie (relative gap below 1e-6), where either
  choice is correct.
"""
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


def xprime(x_bits, s_row):
    """Oracle x' (fp64 copy) of calibration rows, for magnitude bounds."""
    return oracle.transform(oracle.as_f32(x_bits), s_row).astype(np.float64)


def check_hessian(h_gpu: np.ndarray, h_ref: np.ndarray, S: np.ndarray, what: str):
    bound = 2.0 ** -24 * np.abs(h_ref) + 1e-11 * S
    bad = np.abs(h_gpu.astype(np.float64) - h_ref) > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} entries outside the bound, e.g. {np.argwhere(bad)[:4].tolist()}"


# ------------------------------------------------------------------ Hessian

@pytest.mark.parametrize("cfg,T", [(1, 64), (2, 4096), (2, 77), (3, 1000)])
def test_hessian_small(cfg, T):
    """Whole Hessian, dense layer: fp32 (cfg 1) and bf16 calibration rows,
    a ragged row count (77 = 4 steps of 16 + 13), K = 256 (two 128 tiles,
    one off-diagonal)."""
    say(f"hessian cfg{cfg} T{T} K256")
    wl = workloads.make(cfg, shape=(16, 64, 256), keep_calib=True)
    xc = wl.xcal[:T].contiguous()
    h = mx.hessian(xc.to(DEV), wl.s.to(DEV))
    torch.cuda.synchronize()
    h = h.cpu().numpy()
    assert h.shape == (1, 256, 256)
    assert np.array_equal(h[0], h[0].T)
    href = oracle.hessian(host(xc), wl.s.numpy())
    xp = np.abs(xprime(host(xc), wl.s[0].numpy()))
    check_hessian(h[0], href[0], xp.T @ xp, f"cfg{cfg} T{T}")


def test_hessian_experts_ragged_and_empty():
    """Several experts with their own s, ragged and empty row ranges, and an
    expert with all of its rows in the last partial step."""
    K = 384
    wl = workloads.make(5, shape=(64, 32, K), keep_calib=True)
    off = np.array([0, 100, 100, 612, 613, 613, 1024], dtype=np.int32)
    E = len(off) - 1
    xc = wl.xcal[:off[-1]].contiguous()
    s = wl.s[:E].contiguous()
    say(f"hessian experts E{E} K{K} offsets {off.tolist()}")
    h = mx.hessian(xc.to(DEV), s.to(DEV), torch.from_numpy(off).to(DEV))
    torch.cuda.synchronize()
    h = h.cpu().numpy()
    href = oracle.hessian(host(xc), s.numpy(), off)
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        if r1 == r0:
            assert not h[e].any()
            continue
        xp = np.abs(xprime(host(xc[r0:r1]), s[e].numpy()))
        check_hessian(h[e], href[e], xp.T @ xp, f"expert {e}")
        assert np.array_equal(h[e], h[e].T)


def test_hessian_no_rows_writes_zeros():
    """T = 0: the output is fully written with zeros (no stale memory)."""
    say("hessian T0 K128")
    s = torch.ones((1, 128), dtype=torch.float32, device=DEV)
    x = torch.empty((0, 128), dtype=torch.bfloat16, device=DEV)
    out = torch.full((1, 128, 128), 7.0, dtype=torch.float32, device=DEV)
    mx.hessian(x, s, out=out)
    torch.cuda.synchronize()
    assert not out.cpu().numpy().any()


@pytest.mark.parametrize("which", ["gateup", "moe"])
def test_hessian_fullsize_sampled_tiles(which):
    """Full-size Hessians (decode gate/up K5120 from 4096 calibration rows;
    MoE K3072 from 512 rows for each of the 64 experts), checked on sampled
    128x128 tiles that the oracle computes from the tile's columns alone (a
    column group's x' depends only on that group's inputs)."""
    if which == "gateup":
        wl = workloads.make(4, variant=0, M=1, keep_calib=True)
        tiles = [(0, 0), (3, 29), (39, 39), (17, 20)]
        experts = [0]
    else:
        wl = workloads.make(5, keep_calib=True)
        tiles = [(0, 0), (5, 21), (23, 23)]
        experts = [0, 6, 63]
    K = wl.K
    say(f"hessian full size {which} T{wl.xcal.shape[0]} K{K} E{wl.E}")
    off = None if wl.E == 1 else wl.cal_offsets.to(DEV)
    h = mx.hessian(wl.xcal.to(DEV), wl.s.to(DEV), off)
    torch.cuda.synchronize()
    xbits = host(wl.xcal)
    co = wl.cal_offsets.numpy()
    for e in experts:
        he = h[e].cpu().numpy()
        for ti, tj in tiles:
            cols = np.concatenate([np.arange(128 * ti, 128 * ti + 128), np.arange(128 * tj, 128 * tj + 128)])
            if ti == tj:
                cols = cols[:128]
            xs = xbits[co[e]:co[e + 1]][:, cols]
            sc = wl.s[e].numpy()[cols]
            href = oracle.hessian(xs, sc[None])[0]
            xp = np.abs(xprime(xs, sc))
            got = he[cols][:, cols]
            check_hessian(got, href, xp.T @ xp, f"{which} expert {e} tile ({ti},{tj})")


# ------------------------------------------------------------------ exponent search

def oracle_h32(xcal_bits, s, off=None):
    """The oracle's Hessian rounded to fp32: the common input of both sides."""
    return oracle.hessian(xcal_bits, s, off).astype(np.float32)


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_prep_hessian_small_bitexact(cfg):
    """Calibration Hessian, dense layer (fp32 weights for cfg 1, bf16
    otherwise): codes and scale bytes bit-exact, and the search does move
    some groups off the plain byte."""
    wl = workloads.make(cfg, shape=(16, 96, 256), keep_calib=True)
    say(f"prep_hessian cfg{cfg} N96 K256")
    h = oracle_h32(host(wl.xcal), wl.s.numpy())
    c, sc = mx.prepare_weights_hessian(wl.w.to(DEV), wl.s.to(DEV), torch.from_numpy(h).to(DEV))
    torch.cuda.synchronize()
    rc, rs = oracle.prepare_weights_hessian(host(wl.w[0]), wl.s[0].numpy(), h[0])
    assert np.array_equal(sc[0].cpu().numpy(), rs)
    assert np.array_equal(c[0].cpu().numpy(), rc)
    moved = int((rs != oracle.prepare_weights(host(wl.w[0]), wl.s[0].numpy())[1]).sum())
    print(f"groups moved to b0+1: {moved} of {rs.size}")
    assert moved > 0


def test_prep_hessian_random_psd_heavy_tails_experts():
    """Three experts with their own s and random PSD Hessians, Student-t(2)
    weights (many saturating groups); the off-diagonal blocks of h hold NaN
    and must not be read."""
    E, N, K = 3, 72, 512
    rng = np.random.default_rng(np.random.SeedSequence([11, 3]))
    w = torch.from_numpy((rng.standard_t(2, (E, N, K)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    s = rng.uniform(0.25, 4.0, (E, K)).astype(np.float32)
    h = np.full((E, K, K), np.nan, dtype=np.float32)
    for e in range(E):
        for g in range(K // 32):
            a = rng.standard_normal((32, 48))
            h[e, 32 * g:32 * g + 32, 32 * g:32 * g + 32] = (a @ a.T).astype(np.float32)
    say(f"prep_hessian random PSD E{E} N{N} K{K}")
    c, sc = mx.prepare_weights_hessian(w.to(DEV), torch.from_numpy(s).to(DEV), torch.from_numpy(h).to(DEV))
    torch.cuda.synchronize()
    moved = 0
    for e in range(E):
        rc, rs = oracle.prepare_weights_hessian(host(w[e]), s[e], h[e])
        assert np.array_equal(sc[e].cpu().numpy(), rs), f"expert {e} scales"
        assert np.array_equal(c[e].cpu().numpy(), rc), f"expert {e} codes"
        moved += int((rs != oracle.prepare_weights(host(w[e]), s[e])[1]).sum())
    assert moved > 0


def test_prep_hessian_zero_hessian_is_plain_prepare():
    """h = 0: every tie keeps the plain byte, so the output equals
    macaq_prepare_weights bit for bit (and the oracle's plain W')."""
    wl = workloads.make(2, shape=(16, 200, 384))
    say("prep_hessian h=0 N200 K384")
    h = torch.zeros((1, 384, 384), dtype=torch.float32, device=DEV)
    c, sc = mx.prepare_weights_hessian(wl.w.to(DEV), wl.s.to(DEV), h)
    pc, ps = mx.prepare_weights(wl.w.to(DEV), wl.s.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(c, pc) and torch.equal(sc, ps)
    rc, rs = oracle.prepare_weights(host(wl.w[0]), wl.s[0].numpy())
    assert np.array_equal(c[0].cpu().numpy(), rc) and np.array_equal(sc[0].cpu().numpy(), rs)


def test_prep_hessian_fullsize_sampled_rows():
    """Decode gate/up weights at full size (N25600 K5120) with the
    calibration Hessian's diagonal blocks (the rest NaN): 256 sampled rows
    bit-exact against the oracle, including the first and the last row."""
    wl = workloads.make(4, variant=0, M=1, keep_calib=True)
    N, K = wl.N, wl.K
    say(f"prep_hessian full size N{N} K{K}")
    xbits = host(wl.xcal)
    s0 = wl.s[0].numpy()
    h = np.full((K, K), np.nan, dtype=np.float32)
    for g in range(K // 32):
        cols = slice(32 * g, 32 * g + 32)
        h[cols, cols] = oracle.hessian(xbits[:, cols], s0[cols][None])[0].astype(np.float32)
    c, sc = mx.prepare_weights_hessian(wl.w.to(DEV), wl.s.to(DEV), torch.from_numpy(h)[None].to(DEV))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(5).choice(N, 254, replace=False)]))
    rc, rs = oracle.prepare_weights_hessian(host(wl.w[0])[rows], s0, h)
    assert np.array_equal(sc[0].cpu().numpy()[rows], rs)
    assert np.array_equal(c[0].cpu().numpy()[rows], rc)


def test_offline_chain_gpu_hessian_then_search():
    """GPU Hessian -> GPU search against oracle Hessian -> oracle search.  The
    fp32 Hessians may differ in the last bit, so a group may only disagree
    where the oracle's candidate errors are a near tie."""
    wl = workloads.make(2, shape=(16, 128, 512), keep_calib=True)
    say("offline chain cfg2-shaped N128 K512")
    hg = mx.hessian(wl.xcal.to(DEV), wl.s.to(DEV))
    c, sc = mx.prepare_weights_hessian(wl.w.to(DEV), wl.s.to(DEV), hg)
    torch.cuda.synchronize()
    h = oracle_h32(host(wl.xcal), wl.s.numpy())[0]
    rc, rs = oracle.prepare_weights_hessian(host(wl.w[0]), wl.s[0].numpy(), h)
    gs = sc[0].cpu().numpy()
    diff = np.argwhere(gs != rs)
    if diff.size:
        xp = oracle.transform(oracle.as_f32(host(wl.w[0])),
                              np.broadcast_to(oracle.weight_reciprocal(wl.s[0].numpy()), (128, 512)))
        g = xp.reshape(128, 16, 32)
        b0 = oracle.e8m0_scale(np.abs(g).max(axis=-1)).astype(np.int64)
        hb = oracle.diagonal_blocks(h)
        q = [oracle.hessian_error(g.astype(np.float64) - oracle.dequantize_groups(oracle.encode_groups(g, b), b), hb)
             for b in (b0, b0 + 1)]
        for r, gi in diff:
            gap = abs(q[1][r, gi] - q[0][r, gi]) / max(q[0][r, gi], 1e-300)
            assert gap < 1e-6, f"row {r} group {gi}: gap {gap}"
    same = np.all(gs == rs, axis=1)
    cg = c[0].cpu().numpy()
    assert np.array_equal(cg[same], rc[same])
    print(f"groups differing (near ties): {len(diff)}")

"""Pins of the oracle's Flip-Refinement (per-row greedy moves of single codes
to adjacent E2M1 levels under the Hessian-weighted loss).  No GPU needed.
Each test names the plausible oracle mistake it would catch.
"""
import numpy as np

import oracle


def _rng(*k):
    return np.random.default_rng(np.random.SeedSequence([13, *k]))


def _coupled_h(rng, K, rank=None, scale=1.0):
    """A PSD Hessian with strong off-diagonal coupling (fp32)."""
    a = rng.standard_normal((K, rank or K // 2))
    return (scale * (a @ a.T) + 0.05 * np.eye(K)).astype(np.float32)


def _case(seed, R, K, tail=3):
    rng = _rng(seed)
    xp = rng.standard_t(tail, (R, K)).astype(np.float32)
    codes, scales = oracle.quantize_mxfp4(xp)
    return rng, xp, codes, scales


def _single_moves(code_row, scales_row):
    """Every state one adjacent-level move away from code_row (unpacked)."""
    K = code_row.size
    lev = oracle.code_levels(code_row)
    out = []
    for k in range(K):
        for step in (-1, 1):
            nl = lev[k] + step
            if -7 <= nl <= 7:
                c = code_row.copy()
                c[k] = oracle.level_code(np.array(nl), c[k])
                out.append((k, step, c))
    return out


def _loss_row(xp_row, code_row, scales_row, h):
    packed = oracle.pack_codes(code_row.reshape(1, -1, 32))
    return float(oracle.layer_loss(xp_row[None], packed, scales_row[None], h)[0])


def test_flip_each_move_is_the_best_single_move():
    """Replaying the refinement one round at a time, every applied move is the
    single adjacent move with the largest loss decrease when the loss is
    recomputed densely from scratch (not from the incremental gradient), and
    the final state has no improving single move.  Catches a wrong gradient
    (sign, transposed update, stale entry), a wrong gain formula or a wrong
    level step."""
    rng, xp, codes, scales = _case(1, 4, 64)
    h = _coupled_h(rng, 64)
    prev = oracle.unpack_codes(codes)
    total = 0
    for t in range(1, 40):
        c_t, moves = oracle.flip_refine(xp, codes, scales, h, t)
        cur = oracle.unpack_codes(c_t)
        for r in range(xp.shape[0]):
            if (cur[r] == prev[r]).all():
                continue
            base = _loss_row(xp[r], prev[r], scales[r], h)
            cands = [(base - _loss_row(xp[r], c, scales[r], h), k, st) for k, st, c in _single_moves(prev[r], scales[r])]
            best = max(g for g, _, _ in cands)
            got = base - _loss_row(xp[r], cur[r], scales[r], h)
            assert best > 0 and got >= best - 1e-9 * max(base, 1e-30), (t, r, got, best)
            assert int((cur[r] != prev[r]).sum()) == 1
            total += 1
        prev = cur
    assert total > 10
    final, moves = oracle.flip_refine(xp, codes, scales, h, 1000)
    fin = oracle.unpack_codes(final)
    for r in range(xp.shape[0]):
        base = _loss_row(xp[r], fin[r], scales[r], h)
        for _, _, c in _single_moves(fin[r], scales[r]):
            assert _loss_row(xp[r], c, scales[r], h) >= base - 1e-9 * max(base, 1e-30)


def test_flip_loss_strictly_decreases():
    """The Hessian-weighted loss never increases and falls with every move;
    refining from Hessian-searched scale bytes behaves the same.  Catches a
    move applied with a non-positive gain."""
    rng, xp, codes, scales = _case(2, 8, 128)
    h = _coupled_h(rng, 128)
    hb = oracle.diagonal_blocks(h)
    for start in ((codes, scales), oracle.search_exponents(xp, hb)):
        c0, s0 = start
        last = oracle.layer_loss(xp, c0, s0, h)
        last_moves = np.zeros(xp.shape[0], dtype=np.int64)
        for t in (1, 2, 4, 8, 16, 32):
            c, moves = oracle.flip_refine(xp, c0, s0, h, t)
            loss = oracle.layer_loss(xp, c, s0, h)
            moved = moves > last_moves
            assert np.all(loss[moved] < last[moved])
            assert np.all(loss[~moved] == last[~moved])
            last, last_moves = loss, moves
        assert last_moves.sum() > 0


def test_flip_diagonal_hessian_keeps_round_to_nearest():
    """With a diagonal Hessian every coordinate is on its own and the
    round-to-nearest code is already the best: nothing moves (a tie has gain
    0 and is not taken).  Catches gains that ignore H_kk or a move taken on a
    zero gain."""
    rng, xp, codes, scales = _case(3, 6, 96)
    h = np.diag(rng.uniform(0.1, 5.0, 96)).astype(np.float32)
    c, moves = oracle.flip_refine(xp, codes, scales, h, 50)
    assert np.array_equal(c, codes) and not moves.any()


def test_flip_zero_hessian_or_zero_rounds_is_identity():
    rng, xp, codes, scales = _case(4, 3, 64)
    c, m = oracle.flip_refine(xp, codes, scales, np.zeros((64, 64), np.float32), 10)
    assert np.array_equal(c, codes) and not m.any()
    c, m = oracle.flip_refine(xp, codes, scales, _coupled_h(rng, 64), 0)
    assert np.array_equal(c, codes) and not m.any()


def _pair_case(x0, x1, h01):
    """Two coupled coordinates; a third, uncoupled value 4.0 (exactly
    representable) sets the group's scale to 2^0."""
    xp = np.zeros((1, 32), np.float32)
    xp[0, :3] = [x0, x1, 4.0]
    codes, scales = oracle.quantize_mxfp4(xp)
    h = np.eye(32, dtype=np.float32)
    h[0, 1] = h[1, 0] = h01
    return xp, codes, scales, h


def test_flip_worked_pair():
    """x' = (0.7, 0.7) at scale 1 rounds to (0.5, 0.5), d = (0.2, 0.2).  With
    H = [[1, .9], [.9, 1]] the loss is 0.076; moving either coordinate up to
    1.0 gives 0.011 (gain 0.065, a tie broken to coordinate 0); after it no
    move helps.  Result: codes (2, 1) = (1.0, 0.5), one move."""
    xp, codes, scales, h = _pair_case(0.7, 0.7, 0.9)
    assert int(scales[0, 0]) == 127
    c, m = oracle.flip_refine(xp, codes, scales, h, 10)
    u = oracle.unpack_codes(c)[0]
    assert list(u[:3]) == [2, 1, 6] and not u[3:].any() and m[0] == 1


def test_flip_move_onto_zero_keeps_sign_and_tie_order():
    """x' = (-0.3, 0.3), H = [[1, -.95], [-.95, 1]]: round-to-nearest gives
    (-0.5, 0.5); moving coordinate 0 up to zero and coordinate 1 down to zero
    have exactly equal gains, and the tie goes to the lower coordinate.  The
    zero keeps the sign bit of -0.5: codes (0x8, 0x1), one move."""
    xp, codes, scales, h = _pair_case(-0.3, 0.3, -0.95)
    u0 = oracle.unpack_codes(codes)[0]
    assert int(scales[0, 0]) == 127 and list(u0[:3]) == [9, 1, 6]
    c, m = oracle.flip_refine(xp, codes, scales, h, 10)
    u = oracle.unpack_codes(c)[0]
    assert list(u[:2]) == [8, 1] and m[0] == 1


def test_flip_rows_are_independent_and_saturation_respected():
    """Refining a subset of rows gives the same rows as refining all rows
    (no state shared between rows), and no code moves past +-6.  Catches a
    gradient shared between rows."""
    rng, xp, codes, scales = _case(5, 10, 64, tail=1.5)
    h = _coupled_h(rng, 64)
    c_all, m_all = oracle.flip_refine(xp, codes, scales, h, 25)
    sel = np.array([7, 2, 9])
    c_sub, m_sub = oracle.flip_refine(xp[sel], codes[sel], scales[sel], h, 25)
    assert np.array_equal(c_all[sel], c_sub) and np.array_equal(m_all[sel], m_sub)
    lev = oracle.code_levels(oracle.unpack_codes(c_all))
    assert lev.min() >= -7 and lev.max() <= 7

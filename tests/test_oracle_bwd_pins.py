"""Pins for the oracle's backward of the grouped matmul and of the gated expert MLP
(the custom VJP the pages describe: an input-gradient grouped GEMM against the
transposed weights and a ragged-contracting weight-gradient GEMM).  Each test
checks the oracle against something other than its own formulas: library
matmuls on blocks, finite differences of the forward oracle (pinned on its own
elsewhere), adjoint identities, and zero cases."""
import numpy as np
import pytest

from oracle import oracle as O


def grid_values(rng, shape, scale=1.0):
    """float32 values that are multiples of 2^-12 in [-scale, scale]: a step of
    2^-5 up or down stays exactly representable."""
    q = rng.integers(-4096, 4097, size=shape) / 4096.0 * scale
    return q.astype(np.float32)


def f64(a):
    return a.astype(np.float64) if a.dtype == np.float32 else O.bf16_to_f64(a)


# --------------------------------------------------- grouped matmul VJP --

def test_single_group_is_plain_matmul():
    rng = np.random.default_rng(0)
    R, N, K = 9, 7, 5
    dZ = grid_values(rng, (R, N))
    X = grid_values(rng, (R, K))
    W = grid_values(rng, (1, N, K))
    off = np.array([0, R], np.int32)
    np.testing.assert_allclose(O.ragged_dlhs(dZ, W, off), f64(dZ) @ f64(W[0]), rtol=1e-14,
                               atol=1e-14)
    np.testing.assert_allclose(O.ragged_drhs(X, dZ, off)[0], f64(dZ).T @ f64(X), rtol=1e-14,
                               atol=1e-14)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_groups_are_independent_blocks(dt):
    rng = np.random.default_rng(1)
    sizes = [3, 0, 5, 2]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    R_phys, N, K, E = 13, 6, 4, len(sizes)
    dZ = grid_values(rng, (R_phys, N))
    X = grid_values(rng, (R_phys, K))
    W = grid_values(rng, (E, N, K))
    if dt == "bf16":
        dZ, X, W = (O.to_bf16(a.astype(np.float64)) for a in (dZ, X, W))
    dX = O.ragged_dlhs(dZ, W, off)
    dW = O.ragged_drhs(X, dZ, off)
    for e in range(E):
        rows = slice(off[e], off[e + 1])
        np.testing.assert_allclose(dX[rows], f64(dZ)[rows] @ f64(W[e]), rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(dW[e], f64(dZ)[rows].T @ f64(X)[rows], rtol=1e-13, atol=1e-13)
    assert np.all(dW[1] == 0.0)                      # empty group
    assert np.all(np.isnan(dX[off[-1]:]))            # rows past the groups are not written


def test_adjoint_identity_ties_both_gradients_to_the_forward():
    # For the bilinear Z[r] = W[e(r)] X[r]:  <dZ, Z> = <dX, X> = sum_e <dW[e], W[e]>.
    # A transposed operand or a row of the wrong group breaks one of the equalities.
    rng = np.random.default_rng(2)
    sizes = [4, 1, 6]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    R, N, K, E = 11, 5, 8, 3
    dZ, X, W = grid_values(rng, (R, N)), grid_values(rng, (R, K)), grid_values(rng, (E, N, K))
    Z = np.zeros((R, N))
    for e in range(E):
        for r in range(off[e], off[e + 1]):
            for n in range(N):                        # the forward by its definition
                Z[r, n] = sum(float(W[e, n, k]) * float(X[r, k]) for k in range(K))
    lhs = float(np.sum(f64(dZ) * Z))
    dX = O.ragged_dlhs(dZ, W, off)
    dW = O.ragged_drhs(X, dZ, off)
    assert lhs == pytest.approx(float(np.sum(dX * f64(X))), rel=1e-12, abs=1e-12)
    assert lhs == pytest.approx(float(np.sum(dW * f64(W))), rel=1e-12, abs=1e-12)


# ------------------------------------------------ gated expert MLP VJP --

def _loss(X, off, W_gu, W_d, dY, H):
    """Lambda = sum over grouped rows of <Y[r], dY[r]>, Y from the forward oracle."""
    E = off.size - 1
    ex = np.full(X.shape[0], -1, np.int32)
    for e in range(E):
        ex[off[e]:off[e + 1]] = e
    Y = O.expert_rows(X, ex, list(W_gu), list(W_d), H)
    return float(np.sum(Y * dY.astype(np.float64)))


def _fd(f, a, idx, eps):
    """Four-point central difference of f along element idx of a (fourth order)."""
    base = a[idx]
    vals = []
    for s in (2, 1, -1, -2):
        a[idx] = np.float32(float(base) + s * eps)
        vals.append(f())
    a[idx] = base
    return (-vals[0] + 8 * vals[1] - 8 * vals[2] + vals[3]) / (12 * eps)


def test_expert_backward_matches_finite_differences_of_the_forward():
    rng = np.random.default_rng(3)
    E, d, H = 2, 8, 4
    off = np.array([0, 3, 5], np.int32)
    R = 6                                             # one spare row past the groups
    X = grid_values(rng, (R, d))
    W_gu = grid_values(rng, (E, 2 * H, d), 0.5)
    W_d = grid_values(rng, (E, d, H), 0.5)
    dY = grid_values(rng, (R, d))
    dX, dWgu, dWd = O.expert_rows_bwd(X, dY, off, W_gu, W_d)
    eps = 2.0 ** -6
    f = lambda: _loss(X, off, W_gu, W_d, dY, H)
    for r in range(off[-1]):
        for c in range(d):
            assert dX[r, c] == pytest.approx(_fd(f, X, (r, c), eps), abs=2e-4), ("dX", r, c)
    for e in range(E):
        for i in range(2 * H):
            for c in range(d):
                assert dWgu[e, i, c] == pytest.approx(_fd(f, W_gu, (e, i, c), eps), abs=2e-4), \
                    ("dW_gu", e, i, c)
        for o in range(d):
            for i in range(H):
                assert dWd[e, o, i] == pytest.approx(_fd(f, W_d, (e, o, i), eps), abs=2e-4), \
                    ("dW_d", e, o, i)
    assert np.all(np.isnan(dX[off[-1]:]))


def test_down_weight_gradient_uses_the_stored_hidden():
    # bf16: dW_d[e] = dY[group]^T h[group] with h exactly as the forward oracle stores it.
    rng = np.random.default_rng(4)
    E, d, H = 3, 16, 8
    off = np.array([0, 4, 4, 9], np.int32)
    R = 9
    X, dY = (O.to_bf16(grid_values(rng, (R, d)).astype(np.float64)) for _ in range(2))
    W_gu = O.to_bf16(grid_values(rng, (E, 2 * H, d), 0.3).astype(np.float64))
    W_d = O.to_bf16(grid_values(rng, (E, d, H), 0.3).astype(np.float64))
    _, _, dWd = O.expert_rows_bwd(X, dY, off, W_gu, W_d)
    ex = np.repeat(np.arange(E, dtype=np.int32), np.diff(off))
    _, h = O.expert_rows(X, ex, list(W_gu), list(W_d), H, want_h=True)
    dWd_ref = O.ragged_drhs(O.to_bf16(h), dY, off)     # h is already bf16-exact
    np.testing.assert_allclose(dWd, dWd_ref, rtol=1e-13, atol=1e-13)
    assert np.all(dWd[1] == 0.0)


def test_zero_output_gradient_gives_zero_gradients():
    rng = np.random.default_rng(5)
    E, d, H = 2, 8, 4
    off = np.array([0, 2, 5], np.int32)
    X = grid_values(rng, (5, d))
    W_gu, W_d = grid_values(rng, (E, 2 * H, d)), grid_values(rng, (E, d, H))
    dX, dWgu, dWd = O.expert_rows_bwd(X, np.zeros((5, d), np.float32), off, W_gu, W_d)
    assert not np.any(dX) and not np.any(dWgu) and not np.any(dWd)

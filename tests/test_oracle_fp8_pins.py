"""Pins for the oracle's OCP E4M3 codec, its per-tensor quantisation and the
grouped matmul on E4M3 operands, each against something other than the oracle:
torch's float8_e4m3fn type, exhaustive checks over all 256 codes, and numpy
block matmuls on the decoded values."""
import numpy as np
import pytest
import torch

from oracle import oracle as O


def torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = np.array([O.e4m3_value(c) for c in codes])
    ref = torch_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert nan.sum() == 2                              # S.1111.111 only


def test_encode_is_the_inverse_on_every_finite_code():
    for c in range(256):
        v = O.e4m3_value(c)
        if np.isnan(v):
            continue
        assert O.to_e4m3(v) == c, c


def test_midpoints_round_to_the_even_code():
    # between two neighbouring positive codes the midpoint goes to the even one
    for c in range(0, 0x7E):
        lo, hi = O.e4m3_value(c), O.e4m3_value(c + 1)
        mid = (lo + hi) / 2
        assert O.to_e4m3(mid) == (c if c % 2 == 0 else c + 1), c
        assert O.to_e4m3(np.nextafter(mid, 0)) == c
        assert O.to_e4m3(np.nextafter(mid, np.inf)) == c + 1


def test_rounding_matches_torch_below_the_saturation_point():
    g = torch.Generator().manual_seed(3)
    x = torch.randn(20000, generator=g) * torch.exp(3 * torch.randn(20000, generator=g))
    x = x[x.abs() < 460]                               # torch turns >= 464 into NaN
    ref = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([O.to_e4m3(float(v)) for v in x.double()], np.uint8)
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("x,code", [(464.0, 0x7E), (480.0, 0x7E), (1e30, 0x7E), (float("inf"), 0x7E),
                                    (-1e30, 0xFE), (float("nan"), 0x7F), (-0.0, 0x80),
                                    (2.0 ** -10, 0x00), (3 * 2.0 ** -11, 0x01)])
def test_saturation_nan_and_tiny_values(x, code):
    # magnitudes past 448 saturate (the reading taken for training tensors)
    assert O.to_e4m3(x) == code


def test_quantize_decides_in_float32():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(5000) * 3).astype(np.float32)
    inv = np.float32(37.3)
    q, amax = O.quantize_e4m3(x, float(inv))
    prod = (x * inv).astype(np.float32)                  # one float32 rounding
    ok = np.abs(prod) < 460
    ref = torch.from_numpy(prod[ok]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q[ok], ref)
    assert np.all(q[~ok] & 0x7F == 0x7E)                 # saturated
    assert amax == float(np.abs(x).max())
    qb, _ = O.quantize_e4m3(O.to_bf16(x.astype(np.float64)), float(inv))
    xb = O.bf16_to_f64(O.to_bf16(x.astype(np.float64))).astype(np.float32)
    okb = np.abs(xb * inv) < 460
    refb = torch.from_numpy((xb * inv).astype(np.float32)[okb]).to(torch.float8_e4m3fn)
    assert np.array_equal(qb[okb], refb.view(torch.uint8).numpy())


def test_e4m3_ragged_dot_is_a_block_matmul_of_decoded_values():
    rng = np.random.default_rng(5)
    sizes = [5, 0, 9, 3]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    R, N, K, E = 20, 6, 16, 4
    X = rng.integers(0, 0x7E, (R, K)).astype(np.uint8) | (rng.integers(0, 2, (R, K)) << 7).astype(np.uint8)
    W = rng.integers(0, 0x60, (E, N, K)).astype(np.uint8)
    Z = O.ragged_dot_e4m3(X, W, off, 0.125)
    Xd, Wd = torch_decode(X), torch_decode(W)
    for e in range(E):
        rows = slice(off[e], off[e + 1])
        np.testing.assert_allclose(Z[rows], 0.125 * Xd[rows] @ Wd[e].T, rtol=1e-13, atol=1e-300)
    assert np.all(np.isnan(Z[off[-1]:]))


def test_ragged_dot_is_a_block_matmul():
    rng = np.random.default_rng(6)
    off = np.array([0, 4, 4, 11], np.int32)
    X = rng.standard_normal((13, 8)).astype(np.float32)
    W = rng.standard_normal((3, 5, 8)).astype(np.float32)
    Z = O.ragged_dot(X, W, off)
    for e in range(3):
        rows = slice(off[e], off[e + 1])
        np.testing.assert_allclose(Z[rows], X[rows].astype(np.float64) @ W[e].T.astype(np.float64),
                                   rtol=1e-13, atol=1e-13)
    assert np.all(np.isnan(Z[11:]))

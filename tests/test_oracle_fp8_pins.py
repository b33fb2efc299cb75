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


def _torch_h_codes(gu_bf16_bits, inv):
    """Codes of float32(silu(g) u) * inv by torch's silu and float8_e4m3fn cast, with
    the saturation the oracle reads (torch gives NaN past 464)."""
    t = torch.from_numpy(gu_bf16_bits.view(np.int16)).view(torch.bfloat16).double()
    H = t.shape[1] // 2
    h32 = (torch.nn.functional.silu(t[:, :H]) * t[:, H:]).float()
    p = h32 * torch.tensor(inv, dtype=torch.float32)
    codes = p.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    big = p.abs().numpy() >= 464
    codes[big] = np.where(p.numpy()[big] < 0, 0xFE, 0x7E)
    return codes, float(h32.abs().max()) if h32.numel() else 0.0, h32.numpy()


@pytest.mark.parametrize("inv", [1.0, 23.5, 0.01])
def test_swiglu_quantize_matches_torch_silu_and_cast(inv):
    g = torch.Generator().manual_seed(7)
    gu = (torch.randn(37, 2 * 48, generator=g) * 3).to(torch.bfloat16)
    bits = gu.view(torch.int16).numpy().view(np.uint16)
    q, amax, h = O.swiglu_quantize_e4m3(bits, inv, want_h=True)
    ref, ref_amax, h32 = _torch_h_codes(bits, inv)
    # torch's and the oracle's float32(h) are both the double rounded once, except where
    # the two silu evaluations differ in the last double bits across a float32 midpoint
    same = h.astype(np.float32) == h32
    assert same.mean() > 0.999
    assert np.array_equal(q[same], ref[same])
    assert amax == pytest.approx(ref_amax, rel=2 ** -23)


def test_swiglu_quantize_gate_first_and_special_values():
    H = 4
    g = np.array([[0.0, 10.0, -40.0, 2.0]])
    u = np.array([[3.0, 1.0, 5.0, 0.0]])
    bits = O.to_bf16(np.concatenate([g, u], axis=1))
    q, amax = O.swiglu_quantize_e4m3(bits, 1.0)
    vals = np.array([O.e4m3_value(c) for c in q.ravel()])
    # silu(0) = 0; silu(10) u = 10/(1+e^-10) -> 10 in E4M3; silu(-40) ~ -1.7e-16 -> -0;
    # u = 0 -> 0.  Swapping the halves would give silu(3)*0, silu(1)*10, ... instead.
    assert vals.tolist() == [0.0, 10.0, 0.0, 0.0]
    assert q[0, 2] == 0x80
    assert amax == np.float32(10 / (1 + np.exp(-10.0)))


def test_expert_mlp_e4m3_stages_are_block_matmuls():
    rng = np.random.default_rng(8)
    sizes = [3, 0, 5]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    E, d, H = 3, 16, 8
    R = int(off[-1])

    def codes(shape):
        c = rng.integers(0x20, 0x48, shape).astype(np.uint8)
        return c | (rng.integers(0, 2, shape) << 7).astype(np.uint8)

    Xq, Wgu, Wd = codes((R, d)), codes((E, 2 * H, d)), codes((E, d, H))
    sgu, inv_h, sd = 0.03125, 4.0, 0.5
    out = O.expert_mlp_e4m3(Xq, Wgu, Wd, off, sgu, inv_h, sd)
    Xd, Wgud, Wdd = torch_decode(Xq), torch_decode(Wgu), torch_decode(Wd)
    for e in range(E):
        rows = slice(off[e], off[e + 1])
        gu = sgu * Xd[rows] @ Wgud[e].T
        gu_bits = torch.from_numpy(gu).float().to(torch.bfloat16).view(torch.int16).numpy()
        # float32 then bfloat16 rounds twice; the values here are exact in float32
        assert np.array_equal(gu.astype(np.float32).astype(np.float64), gu)
        assert np.array_equal(out["gu"][rows].view(np.int16), gu_bits)
        ref, _, _ = _torch_h_codes(gu_bits.view(np.uint16), inv_h)
        assert np.array_equal(out["hq"][rows], ref)
        np.testing.assert_allclose(out["Y"][rows], sd * torch_decode(ref) @ Wdd[e].T, rtol=1e-13,
                                   atol=1e-300)
    assert np.all(np.isnan(out["Y"][R:]))


def test_delayed_scale_update_by_hand():
    h, s, inv = O.fp8_scale_update([3.0, 7.0, 1.0, 0.0], 2.0)
    assert h.tolist() == [2.0, 3.0, 7.0, 1.0]                 # newest first, oldest dropped
    assert s == np.float32(7.0) / np.float32(448.0) and inv == np.float32(1.0) / np.float32(s)
    h, s, _ = O.fp8_scale_update([0.0, 0.0], 0.0)
    assert s == 1.0                                           # nothing seen yet
    h, s, _ = O.fp8_scale_update([5.0, float("inf")], float("nan"))
    assert s == np.float32(5.0) / np.float32(448.0)           # non-finite entries ignored
    h, s, _ = O.fp8_scale_update([448.0 * 3], 896.0)
    assert h.tolist() == [896.0] and s == 2.0                 # history of one: this amax alone

"""Parity of the fp8 path (per-tensor E4M3 quantisation and the grouped matmul on
E4M3 operands) and of the plain grouped matmul against the CPU oracle, through the
C ABI.  Quantised codes are integers decided in float32 on both sides, so they
must match bit for bit.  The plain grouped matmul meets the usual bound for its
storage type (bf16 2e-2 x RMS, fp32 1e-5 x RMS); the E4M3 one the bound the fp8
MFMA's accumulation allows (see assert_fp8_close).  Output rows past the groups
hold a sentinel that must survive."""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as O
from oracle import torch_bridge as TB

from gpu_util import assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.fixture(scope="module")
def M():
    import mixture_experts_transformer_amd as m
    return m


def _special_values():
    """Exact midpoints between neighbouring codes (ties), their neighbours, the
    saturation edge, subnormals, signed zeros, NaN and infinities."""
    vals = []
    for c in range(0, 0x7E):
        lo, hi = O.e4m3_value(c), O.e4m3_value(c + 1)
        mid = np.float32((lo + hi) / 2)
        vals += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9)), lo]
    vals += [448, 463.99, 464, 480, 1e30, np.inf, -np.inf, np.nan, 0.0, -0.0, 2 ** -10, 2 ** -12]
    v = np.array(vals, np.float32)
    return np.concatenate([v, -v])


@pytest.mark.parametrize("dt,n,inv", [("f32", 0, 1.0), ("f32", 1, 1.0), ("f32", 1237, 1.0),
                                      ("bf16", 4099, 1.0), ("f32", 65536 + 5, 37.25),
                                      ("bf16", 300001, 0.0625)])
def test_quantize_e4m3_bit_exact(M, dt, n, inv):
    rng = np.random.default_rng(n)
    x = (rng.standard_normal(n) * np.exp(3 * rng.standard_normal(n))).astype(np.float32)
    sp = _special_values()
    k = min(n, sp.size)
    x[:k] = sp[:k]
    xt = torch.from_numpy(x).to(TDT[dt])
    host = TB.host(xt)
    q_ref, amax_ref = O.quantize_e4m3(host, inv)
    amax = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    q = M.moe_quantize_e4m3(xt.to(DEV), inv, amax=amax)
    torch.cuda.synchronize()
    got = q.cpu().numpy()
    assert np.array_equal(got, q_ref), f"{int((got != q_ref).sum())} codes differ"
    assert float(amax.item()) == (amax_ref if n > 0 else 0.0)


# The E4M3 MFMA (v_mfma_f32_32x32x64_f8f6f4) does not sum its 64 products in full
# float32: measured on MI355X, its error stays within 2^-14.3 of sum_k |a_k b_k|.
# The bound below allows 2^-12 of that sum plus one storage rounding of the output,
# against the oracle's exact product of the same codes (a wrong row, column or
# code gives errors of order one); E4M3's own quantisation step is 2^-4.
STORE_REL = {"bf16": 2.0 ** -8, "f32": 2.0 ** -23}


def assert_fp8_close(got, Xq, Wq, off, scale, out, what):
    R = int(off[-1])
    ref = O.ragged_dot_e4m3(Xq[:R], Wq, off, scale)[:R]
    absum = O.ragged_dot_e4m3(Xq[:R] & 0x7F, Wq & 0x7F, off, abs(scale))[:R]
    err = np.abs(got[:R] - ref)
    allow = 2.0 ** -12 * absum + STORE_REL[out] * np.abs(ref)
    worst = int(np.argmax(err - allow)) if err.size else 0
    assert np.all(err <= allow), (f"{what}: |err| {err.flat[worst]:.3e} over the bound "
                                  f"{allow.flat[worst]:.3e} (sum|ab| {absum.flat[worst]:.3e})")
    return ref


def _offsets(rng, E, kind, scale):
    c = rng.poisson(scale, E)
    if kind == "skewed":
        c[rng.choice(E, max(1, E // 4), replace=False)] *= 5
    if kind == "sparse":
        c[:] = 0
        c[rng.choice(E, 2, replace=False)] = rng.integers(1, 400, 2)
    return np.concatenate([[0], np.cumsum(c)]).astype(np.int32)


FP8_CASES = [  # out, E, N, K, kind, scale
    ("bf16", 4, 128, 256, "uniform", 150),      # two K steps
    ("f32", 3, 192, 384, "skewed", 200),        # three K steps, float32 output
    ("bf16", 6, 64, 128, "sparse", 0),          # one K step, empty groups
    ("f32", 2, 256, 512, "uniform", 700),       # A's steps ahead (>= 2 row tiles per group)
    ("bf16", 2, 128, 128, "uniform", 4200),     # 8-row-tile swizzle (>= 16 row tiles per group)
]


@pytest.mark.parametrize("out,E,N,K,kind,scale", FP8_CASES)
def test_ragged_dot_e4m3_parity(M, out, E, N, K, kind, scale):
    rng = np.random.default_rng(E * N + K)
    off = _offsets(rng, E, kind, scale)
    R = int(off[-1])
    R_phys = R + 31
    Xq = rng.integers(0, 0xFF, (R_phys, K)).astype(np.uint8)
    Xq[(Xq & 0x7F) == 0x7F] = 0x38                       # no NaN codes in the operands
    Wq = rng.integers(0, 0xFF, (E, N, K)).astype(np.uint8)
    Wq[(Wq & 0x7F) == 0x7F] = 0x30
    Wq[(Wq & 0x78) > 0x50] &= 0xC7                        # keep products moderate
    Xq[:, :][(Xq & 0x78) > 0x50] &= 0xC7
    scale = 2.0 ** -6
    Z = torch.full((R_phys, N), 9.0, dtype=TDT[out], device=DEV)
    M.moe_ragged_dot_e4m3(torch.from_numpy(Xq).to(DEV), torch.from_numpy(off).to(DEV),
                          torch.from_numpy(Wq).to(DEV), scale, Z=Z)
    torch.cuda.synchronize()
    got = Z.float().cpu().numpy()
    assert_fp8_close(got, Xq, Wq, off, scale, out, "Z")
    assert np.all(got[R:] == 9.0), "rows past offsets[E] were written"


@pytest.mark.parametrize("dt,out,E,N,K,kind,scale", [
    ("bf16", "bf16", 4, 128, 192, "uniform", 150), ("f32", "f32", 3, 64, 96, "skewed", 120),
    ("bf16", "f32", 2, 256, 256, "uniform", 700)])
def test_ragged_dot_parity(M, dt, out, E, N, K, kind, scale):
    rng = np.random.default_rng(E * N + K + 7)
    off = _offsets(rng, E, kind, scale)
    R = int(off[-1])
    g = torch.Generator().manual_seed(21)
    X = torch.randn((R + 17, K), generator=g).to(TDT[dt])
    W = (torch.randn((E, N, K), generator=g) / math.sqrt(K)).to(TDT[dt])
    Z = torch.full((R + 17, N), 9.0, dtype=TDT[out], device=DEV)
    M.moe_ragged_dot(X.to(DEV), torch.from_numpy(off).to(DEV), W.to(DEV), Z=Z)
    torch.cuda.synchronize()
    ref = O.ragged_dot(TB.host(X)[:R], TB.host(W), off)
    got = Z.float().cpu().numpy()
    assert_close(got[:R], ref[:R], out, "Z")
    assert np.all(got[R:] == 9.0)


def test_fp8_expert_gemm_from_quantised_bf16(M):
    """The delayed-scaling flow at a 535B-like width: bf16 rows and weights are
    quantised with scales from their amax, multiplied in E4M3, and the result is
    checked against the oracle's product of the same codes."""
    rng = np.random.default_rng(11)
    E, N, K = 4, 256, 1024
    off = _offsets(rng, E, "uniform", 300)
    R = int(off[-1])
    g = torch.Generator().manual_seed(5)
    X = torch.randn((R, K), generator=g).to(torch.bfloat16).to(DEV)
    W = (torch.randn((E, N, K), generator=g) / math.sqrt(K)).to(torch.bfloat16).to(DEV)
    ax = torch.zeros(1, device=DEV)
    aw = torch.zeros(1, device=DEV)
    M.moe_quantize_e4m3(X, 1.0, amax=ax)          # this step's amax: the next step's scale
    M.moe_quantize_e4m3(W, 1.0, amax=aw)
    torch.cuda.synchronize()
    sx, sw = float(ax.item()) / 448.0, float(aw.item()) / 448.0
    Xq = M.moe_quantize_e4m3(X, 1.0 / sx)
    Wq = M.moe_quantize_e4m3(W, 1.0 / sw)
    Z = M.moe_ragged_dot_e4m3(Xq, torch.from_numpy(off).to(DEV), Wq, sx * sw,
                              z_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_fp8_close(Z.cpu().numpy(), Xq.cpu().numpy(), Wq.cpu().numpy(), off, sx * sw, "f32",
                     "Z")
    # and the quantisation error against the bf16 product stays at E4M3's level
    exact = O.ragged_dot(TB.host(X.cpu()), TB.host(W.cpu()), off)
    rel = float(np.sqrt(np.mean((Z.cpu().numpy() - exact) ** 2)) / np.sqrt(np.mean(exact ** 2)))
    assert rel < 0.08, rel

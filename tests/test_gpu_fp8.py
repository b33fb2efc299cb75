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


def dev_scale(v):
    """A per-tensor scale in device memory (None stays None: scale 1)."""
    return None if v is None else torch.tensor([v], dtype=torch.float32, device=DEV)


def inv_f32(s):
    """1 / s rounded to float32, as the kernels form it from a device scale."""
    return 1.0 if s is None else float(np.float32(1.0) / np.float32(s))


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


@pytest.mark.parametrize("dt,n,scale", [("f32", 0, None), ("f32", 1, 1.0), ("f32", 1237, None),
                                        ("bf16", 4099, 1.0), ("f32", 65536 + 5, 1 / 37.25),
                                        ("bf16", 300001, 16.0)])
def test_quantize_e4m3_bit_exact(M, dt, n, scale):
    inv = inv_f32(scale)
    rng = np.random.default_rng(n)
    x = (rng.standard_normal(n) * np.exp(3 * rng.standard_normal(n))).astype(np.float32)
    sp = _special_values()
    k = min(n, sp.size)
    x[:k] = sp[:k]
    xt = torch.from_numpy(x).to(TDT[dt])
    host = TB.host(xt)
    q_ref, amax_ref = O.quantize_e4m3(host, inv)
    amax = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    q = M.moe_quantize_e4m3(xt.to(DEV), dev_scale(scale), amax=amax)
    torch.cuda.synchronize()
    got = q.cpu().numpy()
    bad = np.flatnonzero(got != q_ref)
    assert bad.size == 0, (f"{bad.size} codes differ: " + ", ".join(
        f"x={x[i]!r} (x*inv={np.float32(x[i]) * np.float32(inv)!r}) got {got[i]:#04x} "
        f"want {q_ref[i]:#04x}" for i in bad[:6]))
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
    return ref, absum


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
    ("bf16", 1024, 64, 128, "sparse", 0),       # the most groups, two of them non-empty
    ("f32", 2, 64, 4096, "uniform", 100),       # a long reduction (32 K steps)
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
                          torch.from_numpy(Wq).to(DEV), dev_scale(2.0 ** -3), dev_scale(2.0 ** -3),
                          Z=Z)
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
    M.moe_quantize_e4m3(X, amax=ax)               # this step's amax: the next step's scale
    M.moe_quantize_e4m3(W, amax=aw)
    sx_t, sw_t = ax / 448.0, aw / 448.0           # scales stay on the device
    Xq = M.moe_quantize_e4m3(X, sx_t)
    Wq = M.moe_quantize_e4m3(W, sw_t)
    Z = M.moe_ragged_dot_e4m3(Xq, torch.from_numpy(off).to(DEV), Wq, sx_t, sw_t,
                              z_dtype=torch.float32)
    torch.cuda.synchronize()
    sx, sw = np.float32(sx_t.item()), np.float32(sw_t.item())
    assert sx == np.float32(ax.item()) / np.float32(448.0)
    xq_o, _ = O.quantize_e4m3(TB.host(X.cpu()), inv_f32(sx))
    wq_o, _ = O.quantize_e4m3(TB.host(W.cpu()), inv_f32(sw))
    assert np.array_equal(Xq.cpu().numpy(), xq_o) and np.array_equal(Wq.cpu().numpy(), wq_o)
    assert_fp8_close(Z.cpu().numpy(), xq_o, wq_o, off, float(sx * sw), "f32", "Z")
    # and the quantisation error against the bf16 product stays at E4M3's level
    exact = O.ragged_dot(TB.host(X.cpu()), TB.host(W.cpu()), off)
    rel = float(np.sqrt(np.mean((Z.cpu().numpy() - exact) ** 2)) / np.sqrt(np.mean(exact ** 2)))
    assert rel < 0.08, rel


_LUT = None


def e4m3_values(codes):
    global _LUT
    if _LUT is None:
        _LUT = np.array([O.e4m3_value(c) for c in range(256)])
    return _LUT[codes]


def h_code_window(h, dh, inv):
    """Decoded values of the E4M3 codes at the two ends of [h - dh, h + dh] * inv (in
    float32, as the kernels decide them): every h in the window gets a code between."""
    lo, _ = O.quantize_e4m3(((h - dh) * inv).astype(np.float32), 1.0)
    hi, _ = O.quantize_e4m3(((h + dh) * inv).astype(np.float32), 1.0)
    return e4m3_values(lo), e4m3_values(hi)


@pytest.mark.parametrize("dt,E,H,kind,scale,s_h", [
    ("bf16", 4, 256, "uniform", 150, 1 / 37.0), ("f32", 3, 64, "skewed", 120, None),
    ("bf16", 6, 48, "sparse", 0, 8.0)])
def test_swiglu_quantize_e4m3_parity(M, dt, E, H, kind, scale, s_h):
    inv = inv_f32(s_h)
    rng = np.random.default_rng(E * H)
    off = _offsets(rng, E, kind, scale)
    R = int(off[-1])
    R_phys = R + 13
    g = torch.Generator().manual_seed(E + H)
    gu = (torch.randn((R_phys, 2 * H), generator=g) * 3).to(TDT[dt])
    hq = torch.full((R_phys, H), 0x55, dtype=torch.uint8, device=DEV)
    amax = torch.full((1,), -1.0, device=DEV)
    M.moe_swiglu_quantize_e4m3(gu.to(DEV), torch.from_numpy(off).to(DEV), dev_scale(s_h), hq=hq,
                               amax=amax)
    torch.cuda.synchronize()
    q_ref, amax_ref, h = O.swiglu_quantize_e4m3(TB.host(gu)[:R], inv, want_h=True)
    got = hq.cpu().numpy()
    # the kernel's float32 silu(g) u is within a few units of the last place of h
    lo, hi = h_code_window(h, 2.0 ** -20 * np.abs(h), inv)
    sure = lo == hi
    assert np.array_equal(got[:R][sure], q_ref[sure]), "codes differ away from a midpoint"
    v = e4m3_values(got[:R])
    assert np.all((v >= np.minimum(lo, hi)) & (v <= np.maximum(lo, hi)))
    assert np.all(got[R:] == 0x55), "rows past offsets[E] were written"
    assert abs(float(amax.item()) - amax_ref) <= 2.0 ** -20 * amax_ref


def _codes(rng, shape, top=0x50):
    c = rng.integers(0, top, shape).astype(np.uint8)
    return c | (rng.integers(0, 2, shape) << 7).astype(np.uint8)


# E4M3 codes of 0, 1/2, 1, 2, 3, 4: products of two are multiples of 1/4 up to 16, so
# every partial sum of a gate/up reduction (d <= 4096) is exact in any accumulator the
# fp8 instruction could use, and [g | u] is exact up to its bf16 storage.
SMALL_INT_CODES = np.array([0x00, 0x30, 0x38, 0x40, 0x44, 0x48], np.uint8)


def _small_int_codes(rng, shape):
    c = SMALL_INT_CODES[rng.integers(0, len(SMALL_INT_CODES), shape)]
    return c | (rng.integers(0, 2, shape) << 7).astype(np.uint8)


def ws_views(ws, E, R_phys, H):
    """[g | u] (bf16 bits, int16) and h's codes as moe_grouped_ffn_e4m3 lays them out in
    its workspace: after the row-tile prefix, each region 256-byte aligned."""
    base = ((E + 1) * 4 + 255) // 256 * 256
    gu_bytes = R_phys * 2 * H * 2
    hq_at = base + (gu_bytes + 255) // 256 * 256
    return (ws[base:base + gu_bytes].view(torch.int16).view(R_phys, 2 * H),
            ws[hq_at:hq_at + R_phys * H].view(R_phys, H))


def check_ffn_e4m3(Xq, Wgu, Wd, off, sgu, inv_h, sd, Y, ws, amax_h, out, R_phys, ref=None):
    """The fp8 expert MLP against the oracle, stage by stage, for X and W_gu of small
    integer values (exact gate/up sums) and a power-of-two scale_gu:
      [g | u] (read from the workspace) bit for bit;
      h's codes equal the oracle's except where the kernel's float32 silu(g) u (within
      2^-20 of h) can cross a rounding midpoint, and there lie between the two codes;
      amax_h within 2^-20;
      Y within the E4M3 matmul bound plus, for each such h, |W_d| times the width."""
    E, twoH, d = Wgu.shape
    H = twoH // 2
    R = int(off[-1])
    if ref is None:
        ref = O.expert_mlp_e4m3(Xq, Wgu, Wd, off, sgu, inv_h, sd)
    if isinstance(ws, tuple):                 # rows already taken out
        gu_gpu, hq_gpu = ws
    else:
        gv, hv_ = ws_views(ws, E, R_phys, H)
        gu_gpu, hq_gpu = gv[:R].cpu().numpy(), hv_[:R].cpu().numpy()
    bad = gu_gpu.view(np.uint16) != ref["gu"]
    assert not bad.any(), f"[g | u] differs in {int(bad.sum())} places"
    lo, hi = h_code_window(ref["h"], 2.0 ** -20 * np.abs(ref["h"]), inv_h)
    sure = lo == hi
    assert np.array_equal(hq_gpu[sure], ref["hq"][sure]), "h codes differ away from a midpoint"
    v = e4m3_values(hq_gpu)
    assert np.all((v >= np.minimum(lo, hi)) & (v <= np.maximum(lo, hi))), "h code out of window"
    if amax_h is not None:
        assert abs(float(amax_h.item()) - ref["amax_h"]) <= 2.0 ** -20 * ref["amax_h"]
    width = np.abs(hi - lo)
    Wdd = e4m3_values(Wd)
    hv = e4m3_values(ref["hq"])
    slack = np.zeros((R, d))
    absY = np.zeros((R, d))
    for e in range(E):
        rows = slice(off[e], off[e + 1])
        slack[rows] = abs(sd) * width[rows] @ np.abs(Wdd[e]).T
        absY[rows] = abs(sd) * (np.abs(hv[rows]) + width[rows]) @ np.abs(Wdd[e]).T
    got = Y[:R].float().cpu().numpy() if isinstance(Y, torch.Tensor) else Y[:R]
    err = np.abs(got - ref["Y"][:R])
    allow = 2.0 ** -12 * absY + slack + STORE_REL[out] * np.abs(ref["Y"][:R])
    worst = int(np.argmax(err - allow)) if err.size else 0
    assert np.all(err <= allow), f"Y: |err| {err.flat[worst]:.3e} over {allow.flat[worst]:.3e}"
    return float(sure.mean()) if sure.size else 1.0


@pytest.mark.parametrize("out,E,d,H,kind,scale", [
    ("bf16", 4, 256, 128, "uniform", 150), ("f32", 3, 128, 384, "skewed", 100),
    ("bf16", 6, 128, 128, "sparse", 0), ("bf16", 2, 128, 256, "uniform", 700)])
def test_grouped_ffn_e4m3_parity(M, out, E, d, H, kind, scale):
    rng = np.random.default_rng(E * d + H)
    off = _offsets(rng, E, kind, scale)
    R = int(off[-1])
    R_phys = R + 19
    Xq, Wgu = _small_int_codes(rng, (R_phys, d)), _small_int_codes(rng, (E, 2 * H, d))
    Wd = _codes(rng, (E, d, H))
    sgu = 2.0 ** -round(math.log2(math.sqrt(d) * 2.6))   # [g | u] ~ 1..2 in RMS
    inv_h = 16.0                                          # h * inv_h up to a few hundred
    sd = 2.0 ** -9
    Y = torch.full((R_phys, d), 9.0, dtype=TDT[out], device=DEV)
    ws = torch.zeros(M.moe_grouped_ffn_e4m3_workspace_size(E, R_phys, H), dtype=torch.uint8,
                     device=DEV)
    amax_h = torch.full((1,), -1.0, device=DEV)
    # scales as a training step holds them: s_x s_gu = sgu, 1 / s_h = inv_h, s_h s_d = sd
    M.moe_grouped_ffn_e4m3(torch.from_numpy(Xq).to(DEV), torch.from_numpy(off).to(DEV),
                           torch.from_numpy(Wgu).to(DEV), torch.from_numpy(Wd).to(DEV),
                           dev_scale(2.0), dev_scale(sgu / 2.0), dev_scale(1.0 / inv_h),
                           dev_scale(sd * inv_h), Y=Y, amax_h=amax_h, ws=ws)
    torch.cuda.synchronize()
    sure = check_ffn_e4m3(Xq, Wgu, Wd, off, sgu, inv_h, sd, Y, ws, amax_h, out, R_phys)
    assert sure > 0.999
    assert np.all(Y[R:].float().cpu().numpy() == 9.0), "rows past offsets[E] were written"


def test_grouped_ffn_e4m3_full_size_sampled(M):
    """The 535B expert shape in the benchmark's launch configuration (65,536 rows, 384
    experts, d = H = 3,072), with X and W_gu of small integer values quantised by the
    library (scale 1) and W_d ~ N(0, 1/H) quantised with its amax: the quantised codes,
    [g | u], h's codes and Y of every row of one expert and two rows of five others
    against the oracle, which quantises those rows and experts itself."""
    from moe_synth import by_name, expert_mlp_routing, small_int_tensor

    cfg = by_name("marin535b_experts_bf16_T8192_L3072_H3072_E384_k8")
    R, d, H, E = cfg.R, cfg.d, cfg.H, cfg.E
    counts, off = expert_mlp_routing(cfg)
    X = small_int_tensor((R, d), 71, DEV)
    W_gu = small_int_tensor((E, 2 * H, d), 72, DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(73)
    W_d = (torch.randn((E, d, H), generator=g, device=DEV) * H ** -0.5).to(torch.bfloat16)
    aw = torch.zeros(1, device=DEV)
    Xq = M.moe_quantize_e4m3(X)
    Wguq = M.moe_quantize_e4m3(W_gu)
    M.moe_quantize_e4m3(W_d, q=torch.empty(W_d.shape, dtype=torch.uint8, device=DEV), amax=aw)
    sw_t = aw / 448.0
    Wdq = M.moe_quantize_e4m3(W_d, sw_t)
    sgu, inv_h = 2.0 ** -8, 16.0
    ws = torch.empty(M.moe_grouped_ffn_e4m3_workspace_size(E, R, H), dtype=torch.uint8,
                     device=DEV)
    off_d = torch.from_numpy(off).to(DEV)
    Y = M.moe_grouped_ffn_e4m3(Xq, off_d, Wguq, Wdq, None, dev_scale(sgu), dev_scale(1 / inv_h),
                               sw_t, ws=ws)
    torch.cuda.synchronize()
    sw = float(np.float32(sw_t.item()))
    sd = sw / inv_h                               # exact: a power of two times sw

    rng = np.random.default_rng(9)
    e_full = 201
    others = rng.choice([e for e in range(E) if e != e_full and counts[e] >= 2], 5, replace=False)
    experts = np.sort(np.concatenate([[e_full], others]))
    take = [np.arange(off[e], off[e + 1]) if e == e_full
            else np.sort(rng.choice(np.arange(off[e], off[e + 1]), 2, replace=False))
            for e in experts]
    rows = np.concatenate(take)
    sub_off = np.concatenate([[0], np.cumsum([len(t) for t in take])]).astype(np.int32)
    idx = torch.from_numpy(rows).to(DEV)
    sel = torch.from_numpy(experts).to(DEV)
    # the oracle's own codes from the generator's values
    xq_o, _ = O.quantize_e4m3(TB.host(X[idx]), 1.0)
    wgu_o, _ = O.quantize_e4m3(TB.host(W_gu[sel]), 1.0)
    wd_o, amax_sel = O.quantize_e4m3(TB.host(W_d[sel]), inv_f32(sw))
    assert amax_sel <= float(aw.item())
    assert np.array_equal(Xq[idx].cpu().numpy(), xq_o), "X codes"
    assert np.array_equal(Wguq[sel].cpu().numpy(), wgu_o), "W_gu codes"
    assert np.array_equal(Wdq[sel].cpu().numpy(), wd_o), "W_d codes"
    gv, hv = ws_views(ws, E, R, H)
    ref = O.expert_mlp_e4m3(xq_o, wgu_o, wd_o, sub_off, sgu, inv_h, sd)
    sure = check_ffn_e4m3(xq_o, wgu_o, wd_o, sub_off, sgu, inv_h, sd,
                          Y[idx].float().cpu().numpy(),
                          (gv[idx].cpu().numpy(), hv[idx].cpu().numpy()), None, "bf16",
                          len(rows), ref)
    assert sure > 0.999


@pytest.mark.parametrize("R_phys", [0, 37])
def test_fp8_entry_points_with_no_routed_rows(M, R_phys):
    """No rows at all, and rows whose groups are all empty: nothing is written past
    offsets[E] (here 0) and the amax outputs are cleared to zero."""
    E, d, H = 5, 128, 128
    off = torch.zeros(E + 1, dtype=torch.int32, device=DEV)
    Xq = torch.full((R_phys, d), 0x38, dtype=torch.uint8, device=DEV)
    Wgu = torch.full((E, 2 * H, d), 0x38, dtype=torch.uint8, device=DEV)
    Wd = torch.full((E, d, H), 0x38, dtype=torch.uint8, device=DEV)
    Y = torch.full((R_phys, d), 9.0, dtype=torch.bfloat16, device=DEV)
    Z = torch.full((R_phys, 2 * H), 9.0, dtype=torch.float32, device=DEV)
    gu = torch.ones((R_phys, 2 * H), dtype=torch.bfloat16, device=DEV)
    hq = torch.full((R_phys, H), 0x55, dtype=torch.uint8, device=DEV)
    a1 = torch.full((1,), -1.0, device=DEV)
    a2 = torch.full((1,), -1.0, device=DEV)
    M.moe_grouped_ffn_e4m3(Xq, off, Wgu, Wd, Y=Y, amax_h=a1)
    M.moe_ragged_dot_e4m3(Xq, off, Wgu, Z=Z)
    M.moe_swiglu_quantize_e4m3(gu, off, hq=hq, amax=a2)
    torch.cuda.synchronize()
    assert bool((Y == 9.0).all()) and bool((Z == 9.0).all()) and bool((hq == 0x55).all())
    assert float(a1.item()) == 0.0 and float(a2.item()) == 0.0


@pytest.mark.parametrize("length", [1, 16, 1000, 1024])
def test_fp8_scale_update_parity(M, length):
    """Delayed scaling's update on the device, three steps in a row, against the oracle:
    the history bit for bit (with infinities and NaN among the entries) and the scale."""
    rng = np.random.default_rng(length)
    hist = (np.abs(rng.standard_normal(length)) * 10).astype(np.float32)
    if length > 3:
        hist[1], hist[2] = np.inf, np.nan
    h_dev = torch.from_numpy(hist.copy()).to(DEV)
    sc = torch.full((1,), -1.0, device=DEV)
    for amax in (np.float32(3.5), np.float32(0.0), np.float32(1e4)):
        M.moe_fp8_scale_update(h_dev, torch.tensor([amax], device=DEV), sc)
        hist, s_ref, _ = O.fp8_scale_update(hist, float(amax))
        torch.cuda.synchronize()
        got = h_dev.cpu().numpy()
        assert np.array_equal(got, hist, equal_nan=True)
        assert float(sc.item()) == s_ref


def test_fp8_step_with_device_delayed_scaling_in_a_graph(M):
    """One fp8 expert-MLP step whose scales never leave the device: the rows quantised
    with the scale the history gives, the E4M3 MLP, then both histories updated.  The
    step is captured in a HIP graph and replayed; each replay must equal the same step
    run eagerly from the same state, with eager work and synchronisation in between."""
    rng = np.random.default_rng(31)
    E, d, H = 4, 128, 128
    off = torch.from_numpy(_offsets(rng, E, "uniform", 120)).to(DEV)
    R = 600
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    X = torch.randn((R, d), generator=g, device=DEV).to(torch.bfloat16)
    W_gu = (torch.randn((E, 2 * H, d), generator=g, device=DEV) / d ** 0.5).to(torch.bfloat16)
    W_d = (torch.randn((E, d, H), generator=g, device=DEV) / H ** 0.5).to(torch.bfloat16)
    aw = torch.zeros(2, device=DEV)
    M.moe_quantize_e4m3(W_gu, amax=aw[0:1])
    M.moe_quantize_e4m3(W_d, amax=aw[1:2])
    s_w = aw / 448.0
    Wguq, Wdq = M.moe_quantize_e4m3(W_gu, s_w[0:1]), M.moe_quantize_e4m3(W_d, s_w[1:2])
    L = 16
    hist_x, hist_h = torch.zeros(L, device=DEV), torch.zeros(L, device=DEV)
    s_x, s_h = torch.ones(1, device=DEV), torch.ones(1, device=DEV)
    a_x, a_h = torch.zeros(1, device=DEV), torch.zeros(1, device=DEV)
    Xq = torch.empty((R, d), dtype=torch.uint8, device=DEV)
    Y = torch.zeros((R, d), dtype=torch.bfloat16, device=DEV)   # rows past the groups stay 0
    ws = torch.empty(M.moe_grouped_ffn_e4m3_workspace_size(E, R, H), dtype=torch.uint8,
                     device=DEV)

    def bits(t):
        return t.view(torch.int16) if t.dtype == torch.bfloat16 else t

    def step():
        M.moe_quantize_e4m3(X, s_x, q=Xq, amax=a_x)
        M.moe_grouped_ffn_e4m3(Xq, off, Wguq, Wdq, s_x, s_w[0:1], s_h, s_w[1:2], Y=Y,
                               amax_h=a_h, ws=ws)
        M.moe_fp8_scale_update(hist_x, a_x, s_x)
        M.moe_fp8_scale_update(hist_h, a_h, s_h)

    state = [hist_x, hist_h, s_x, s_h]
    for _ in range(2):                            # warm the histories eagerly
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    saved = [t.clone() for t in state]
    with torch.cuda.graph(graph):
        step()
    for t, v in zip(state, saved):                # capture must not have run the step
        t.copy_(v)
    torch.cuda.synchronize()
    for rep in range(3):
        before = [t.clone() for t in state]
        graph.replay()
        torch.cuda.synchronize()
        got = [Y.clone(), Xq.clone()] + [t.clone() for t in state]
        for t, v in zip(state, before):           # the same step, eagerly, from the same state
            t.copy_(v)
        step()
        torch.cuda.synchronize()
        want = [Y, Xq] + state
        for a, b in zip(got, want):
            assert torch.equal(bits(a), bits(b)), f"replay {rep} differs from the eager step"
        assert float(s_x.item()) > 0 and float(s_h.item()) > 0


@pytest.mark.parametrize("dt,width,div,n,E,cap,pad,s", [
    ("bf16", 3072, 8, 4000, 24, -1, 0.0, 1 / 64),   # one source row per token, k = 8
    ("f32", 128, 2, 4000, 24, -1, 0.0, None),
    ("bf16", 64, 1, 4000, 24, -1, 0.0, 0.25),       # one source row per assignment
    ("bf16", 3072, 8, 4003, 24, -1, 0.0, 1 / 64),   # last source row has 3 assignments
    ("bf16", 256, 3, 6000, 16, 200, 0.1, 2.0),      # capacity drops and padding ids
    ("f32", 64, 70, 7000, 5, -1, 0.3, 1 / 8),       # more than 64 assignments per source row
    ("bf16", 128, 4, 4096, 8, 0, 0.0, None),        # capacity 0: nothing kept, nothing copied
    ("f32", 1040, 1, 3000, 12, 300, 0.2, 1 / 3),    # pool rows with padding, a ragged pass
])
def test_permute_e4m3_bit_exact(M, dt, width, div, n, E, cap, pad, s):
    """The grouping as moe_permute's, and every kept row as the oracle's E4M3 codes of
    its source row; amax over the source rows with a kept assignment."""
    rng = np.random.default_rng(width + n + 1)
    ids = rng.integers(0, E, n).astype(np.int32)
    ids[rng.random(n) < pad] = -1
    n_src = -(-n // div)
    src = (torch.randn((n_src, width), generator=torch.Generator().manual_seed(2)) * 20).to(TDT[dt])
    dst = torch.full((n, width), 0x55, dtype=torch.uint8, device=DEV)
    amax = torch.full((1,), -1.0, device=DEV)
    out = M.moe_permute_e4m3(torch.from_numpy(ids).to(DEV), E, src.to(DEV), dst, capacity=cap,
                             src_div=div, scale=dev_scale(s), amax=amax)
    torch.cuda.synchronize()
    ref = O.permute(ids, E, capacity=cap, R_phys=n)
    kept = int(ref["offsets"][-1])
    for key in ("counts", "offsets", "slot_row"):
        assert np.array_equal(out[key].cpu().numpy(), ref[key]), key
    assert np.array_equal(out["row_src"].cpu().numpy()[:kept], ref["row_src"][:kept])
    rows = ref["row_src"][:kept] // div
    host = TB.host(src)
    q_ref, _ = O.quantize_e4m3(host[rows], inv_f32(s))
    got = dst.cpu().numpy()
    assert np.array_equal(got[:kept], q_ref), f"{int((got[:kept] != q_ref).sum())} codes differ"
    assert np.all(got[kept:] == 0x55), "rows past the kept total were written"
    read = np.unique(rows)
    _, amax_ref = O.quantize_e4m3(host[read], 1.0) if read.size else (None, 0.0)
    assert float(amax.item()) == amax_ref


def test_dispatch_pack_e4m3_bit_exact(M):
    """The fp8 wire format of the dispatch: the grouping by peer as moe_dispatch_pack's,
    each sent row the oracle's E4M3 codes of its token row, amax over the rows sent."""
    rng = np.random.default_rng(77)
    T, k, E, P, width = 2048, 8, 384, 64, 512
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    cap = int(np.ceil(0.9 * T * k / P))                  # some sender drops
    x = (torch.randn((T, width), generator=torch.Generator().manual_seed(4)) * 5).to(torch.bfloat16)
    amax = torch.full((1,), -1.0, device=DEV)
    s = 1 / 32
    out = M.moe_dispatch_pack_e4m3(torch.from_numpy(ids).to(DEV), E, P, x.to(DEV), capacity=cap,
                                   scale=dev_scale(s), amax=amax)
    torch.cuda.synchronize()
    ref = O.permute(ids // (E // P), P, capacity=cap, R_phys=T * k)
    kept = int(ref["offsets"][-1])
    assert ref["n_dropped"] > 0 and int(out["n_dropped"].item()) == ref["n_dropped"]
    assert np.array_equal(out["offsets"].cpu().numpy(), ref["offsets"])
    rs = ref["row_src"][:kept]
    host = TB.host(x)
    q_ref, _ = O.quantize_e4m3(host[rs // k], inv_f32(s))
    assert np.array_equal(out["send_rows"][:kept].cpu().numpy(), q_ref)
    assert np.array_equal(out["send_expert"].cpu().numpy()[:kept], ids.ravel()[rs] % (E // P))
    _, amax_ref = O.quantize_e4m3(host[np.unique(rs // k)], 1.0)
    assert float(amax.item()) == amax_ref


def test_fp8_pool_step_full_size_sampled(M):
    """The receiver pool's fp8 step in the benchmark's launch configuration (65,536-row
    pool with padding, 6 local experts, latent and hidden 3,072): the E4M3 permute and
    the E4M3 expert MLP, with pool rows and W_gu of small integer values (exact gate/up
    sums) and W_d ~ N(0, 1/H) at its amax scale.  Checked on two rows of every expert:
    their codes bit for bit, and [g | u], h's codes and Y as in check_ffn_e4m3, against
    the oracle, which quantises those rows and all six experts itself."""
    from moe_synth import by_name, gen_pool, small_int_tensor

    cfg = by_name("marin535b_ep_share_bf16_P65536_E6")
    P, L, H, E = cfg.P, cfg.L, cfg.H, cfg.E
    pool = gen_pool(cfg, DEV)
    ids = pool["ids"]
    X = small_int_tensor((P, L), 81, DEV)
    W_gu = small_int_tensor((E, 2 * H, L), 82, DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(83)
    W_d = (torch.randn((E, L, H), generator=g, device=DEV) * H ** -0.5).to(torch.bfloat16)
    aw = torch.zeros(1, device=DEV)
    M.moe_quantize_e4m3(W_d, amax=aw)
    sw_t = aw / 448.0
    Wguq, Wdq = M.moe_quantize_e4m3(W_gu), M.moe_quantize_e4m3(W_d, sw_t)
    Xq = torch.empty((P, L), dtype=torch.uint8, device=DEV)
    a_x = torch.zeros(1, device=DEV)
    grp = M.moe_permute_e4m3(ids, E, X, Xq, src_div=1, R_phys=P, amax=a_x)
    sgu, inv_h = 2.0 ** -8, 16.0
    ws = torch.empty(M.moe_grouped_ffn_e4m3_workspace_size(E, P, H), dtype=torch.uint8,
                     device=DEV)
    Y = M.moe_grouped_ffn_e4m3(Xq, grp["offsets"], Wguq, Wdq, None, dev_scale(sgu),
                               dev_scale(1 / inv_h), sw_t, ws=ws)
    torch.cuda.synchronize()
    sw = float(np.float32(sw_t.item()))
    ids_h = ids.cpu().numpy()
    ref = O.permute(ids_h, E, R_phys=P)
    off = ref["offsets"]
    assert np.array_equal(grp["offsets"].cpu().numpy(), off)
    rng = np.random.default_rng(21)
    take = np.concatenate([np.sort(rng.choice(np.arange(off[e], off[e + 1]), 2, replace=False))
                           for e in range(E)])
    sub_off = np.arange(0, 2 * E + 1, 2, dtype=np.int32)
    src_rows = ref["row_src"][take]
    xq_o, _ = O.quantize_e4m3(TB.host(X[torch.from_numpy(src_rows.astype(np.int64)).to(DEV)]), 1.0)
    idx = torch.from_numpy(take.astype(np.int64)).to(DEV)
    assert np.array_equal(Xq[idx].cpu().numpy(), xq_o), "permuted E4M3 rows"
    wgu_o, _ = O.quantize_e4m3(TB.host(W_gu), 1.0)
    wd_o, _ = O.quantize_e4m3(TB.host(W_d), inv_f32(sw))
    assert np.array_equal(Wguq.cpu().numpy(), wgu_o) and np.array_equal(Wdq.cpu().numpy(), wd_o)
    gv, hv = ws_views(ws, E, P, H)
    ref_mlp = O.expert_mlp_e4m3(xq_o, wgu_o, wd_o, sub_off, sgu, inv_h, sw / inv_h)
    sure = check_ffn_e4m3(xq_o, wgu_o, wd_o, sub_off, sgu, inv_h, sw / inv_h,
                          Y[idx].float().cpu().numpy(),
                          (gv[idx].cpu().numpy(), hv[idx].cpu().numpy()), None, "bf16",
                          len(take), ref_mlp)
    assert sure > 0.99

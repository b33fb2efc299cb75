"""Parity of the backward entry points (the grouped matmul's VJP and the gated
expert MLP's backward) against the CPU oracle, through the C ABI.

Tolerance as for the forward: max |err| <= 2e-2 x RMS(ref) for bfloat16
outputs, 1e-5 x RMS(ref) for float32.  Rows past the groups hold NaN in every
input, so a read past a group's end shows up as NaN in the results, and output
rows past the groups hold a sentinel that must survive."""
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


def _offsets(rng, E, kind, scale):
    if kind == "uniform":
        c = rng.poisson(scale, E)
    elif kind == "skewed":
        c = rng.poisson(scale, E)
        c[rng.choice(E, max(1, E // 4), replace=False)] *= 5
    elif kind == "tails":            # reductions of 0, 1, 63, 64, 65, ... rows
        c = np.array([0, 1, 63, 64, 65, 127, 129, 300][:E])
    elif kind == "sparse":
        c = np.zeros(E, np.int64)
        c[rng.choice(E, 2, replace=False)] = rng.integers(1, 400, 2)
    else:
        raise ValueError(kind)
    return np.concatenate([[0], np.cumsum(c)]).astype(np.int32)


def _with_nan_tail(t, R):
    t = t.clone()
    t[R:] = float("nan")
    return t


DLHS_CASES = [  # dt, E, N, K, kind, scale
    ("bf16", 4, 128, 192, "uniform", 150),       # two and three reduction steps
    ("bf16", 3, 320, 64, "skewed", 200),         # several row tiles in one group
    ("bf16", 8, 64, 320, "tails", 0),            # partial column tile, empty group
    ("f32", 3, 96, 64, "uniform", 120),
    ("f32", 5, 32, 160, "sparse", 0),
    ("bf16", 2, 256, 256, "uniform", 700),       # A's steps ahead (>= 2 row tiles per group)
]


@pytest.mark.parametrize("dt,E,N,K,kind,scale", DLHS_CASES)
def test_ragged_dot_dlhs_parity(M, dt, E, N, K, kind, scale):
    rng = np.random.default_rng(E * N + K)
    off = _offsets(rng, E, kind, scale)
    R = int(off[-1])
    R_phys = R + 29
    g = torch.Generator().manual_seed(11)
    dZ = _with_nan_tail(torch.randn((R_phys, N), generator=g), R).to(TDT[dt])
    W = (torch.randn((E, N, K), generator=g) / math.sqrt(N)).to(TDT[dt])
    dX = torch.full((R_phys, K), 5.0, dtype=TDT[dt], device=DEV)
    M.moe_ragged_dot_dlhs(dZ.to(DEV), torch.from_numpy(off).to(DEV), W.to(DEV), dX=dX)
    torch.cuda.synchronize()
    ref = O.ragged_dlhs(TB.host(dZ)[:R], TB.host(W), off)
    got = dX.float().cpu().numpy()
    assert_close(got[:R], ref[:R], dt, "dX")
    assert np.all(got[R:] == 5.0), "rows past offsets[E] were written"


DRHS_CASES = [  # dt, out, E, N, K, kind, scale
    ("bf16", "f32", 8, 128, 192, "tails", 0),     # ragged reductions incl. 0 and 1 rows
    ("bf16", "bf16", 4, 320, 64, "uniform", 200),  # partial row tile of dW
    ("bf16", "f32", 3, 64, 320, "skewed", 150),    # partial column tile of dW
    ("f32", "f32", 8, 96, 64, "tails", 0),
    ("f32", "f32", 3, 32, 160, "uniform", 90),
    ("bf16", "f32", 2, 256, 256, "uniform", 1500),  # long reductions (about 24 steps)
    # groups of 8 to 15 tiles (the XCD ranges split groups between XCDs)
    ("bf16", "f32", 5, 640, 1088, "tails", 0),     # 15 tiles a group, partial row and column
    ("bf16", "bf16", 3, 512, 1024, "skewed", 150),  # 8 tiles a group
    ("f32", "f32", 4, 768, 768, "uniform", 100),   # 9 tiles a group
]


@pytest.mark.parametrize("dt,out,E,N,K,kind,scale", DRHS_CASES)
def test_ragged_dot_drhs_parity(M, dt, out, E, N, K, kind, scale):
    rng = np.random.default_rng(E * N + K + 1)
    off = _offsets(rng, E, kind, scale)
    R = int(off[-1])
    R_phys = R + 29
    g = torch.Generator().manual_seed(12)
    X = _with_nan_tail(torch.randn((R_phys, K), generator=g), R).to(TDT[dt])
    dZ = _with_nan_tail(torch.randn((R_phys, N), generator=g), R).to(TDT[dt])
    dW = torch.full((E, N, K), 7.0, dtype=TDT[out], device=DEV)
    M.moe_ragged_dot_drhs(X.to(DEV), dZ.to(DEV), torch.from_numpy(off).to(DEV), dW=dW)
    torch.cuda.synchronize()
    ref = O.ragged_drhs(TB.host(X)[:R], TB.host(dZ)[:R], off)
    got = dW.float().cpu().numpy()
    for e in range(E):
        if off[e + 1] == off[e]:
            assert np.all(got[e] == 0.0), f"empty group {e} not zeroed"
        else:
            assert_close(got[e], ref[e], out, f"dW[{e}]")


FFN_BWD_CASES = [  # dt, dw, E, d, H, kind, scale
    ("bf16", "f32", 4, 128, 64, "uniform", 150),
    ("bf16", "bf16", 3, 64, 128, "skewed", 120),
    ("bf16", "f32", 8, 64, 64, "tails", 0),
    ("f32", "f32", 3, 64, 96, "uniform", 100),
    ("f32", "f32", 5, 32, 64, "sparse", 0),
    ("bf16", "f32", 2, 128, 128, "uniform", 700),
    ("bf16", "f32", 3, 512, 512, "uniform", 300),  # dW_gu of 8 tiles a group
]


@pytest.mark.parametrize("dt,dw,E,d,H,kind,scale", FFN_BWD_CASES)
def test_grouped_ffn_bwd_parity(M, dt, dw, E, d, H, kind, scale):
    rng = np.random.default_rng(E * d + H + 2)
    off = _offsets(rng, E, kind, scale)
    R = int(off[-1])
    R_phys = R + 29
    g = torch.Generator().manual_seed(13)
    X = _with_nan_tail(torch.randn((R_phys, d), generator=g), R).to(TDT[dt])
    dY = _with_nan_tail(torch.randn((R_phys, d), generator=g), R).to(TDT[dt])
    W_gu = (torch.randn((E, 2 * H, d), generator=g) / math.sqrt(d)).to(TDT[dt])
    W_d = (torch.randn((E, d, H), generator=g) / math.sqrt(H)).to(TDT[dt])
    dX = torch.full((R_phys, d), 5.0, dtype=TDT[dt], device=DEV)
    dX, dWgu, dWd = M.moe_grouped_ffn_bwd(X.to(DEV), dY.to(DEV), torch.from_numpy(off).to(DEV),
                                          W_gu.to(DEV), W_d.to(DEV), dX=dX, dw_dtype=TDT[dw])
    torch.cuda.synchronize()
    rX, rWgu, rWd = O.expert_rows_bwd(TB.host(X)[:R], TB.host(dY)[:R], off, TB.host(W_gu),
                                      TB.host(W_d))
    gX = dX.float().cpu().numpy()
    assert_close(gX[:R], rX[:R], dt, "dX")
    assert np.all(gX[R:] == 5.0), "rows past offsets[E] were written"
    gWgu, gWd = dWgu.float().cpu().numpy(), dWd.float().cpu().numpy()
    for e in range(E):
        if off[e + 1] == off[e]:
            assert np.all(gWgu[e] == 0.0) and np.all(gWd[e] == 0.0), f"empty group {e}"
            continue
        # a bf16 path stores [g | u], [dg | du] and h in bf16 before the weight
        # gradients reduce them, so those meet the bf16 bound whatever dW's type
        assert_close(gWgu[e], rWgu[e], dt, f"dW_gu[{e}]")
        assert_close(gWd[e], rWd[e], dt, f"dW_d[{e}]")


def test_grouped_ffn_bwd_full_size_sampled(M):
    """The 535B expert shape in the benchmark's launch configuration (65,536 rows, 384
    experts, d = H = 3,072, bf16, fp32 weight gradients): dX on sampled rows of every part
    of the row range, and the whole dW_gu and dW_d of one expert, against the oracle."""
    from moe_synth import by_name, gen_expert_mlp

    cfg = by_name("marin535b_experts_bf16_T8192_L3072_H3072_E384_k8")
    data = gen_expert_mlp(cfg, DEV)
    off_d = data["offsets"]
    dX, dWgu, dWd = M.moe_grouped_ffn_bwd(data["X"], data["dY"], off_d, data["W_gu"],
                                          data["W_d"], dw_dtype=torch.float32)
    torch.cuda.synchronize()
    off = off_d.cpu().numpy()
    rng = np.random.default_rng(9)
    e_full = 201                                    # every row of this expert
    others = rng.choice([e for e in range(cfg.E) if e != e_full], 12, replace=False)
    experts = np.sort(np.concatenate([[e_full], others]))
    take = [np.arange(off[e], off[e + 1]) if e == e_full
            else np.sort(rng.choice(np.arange(off[e], off[e + 1]), 2, replace=False))
            for e in experts]
    rows = np.concatenate(take)
    sub_off = np.concatenate([[0], np.cumsum([len(t) for t in take])]).astype(np.int32)
    idx = torch.from_numpy(rows).to(DEV)
    sel = torch.from_numpy(experts).to(DEV)
    rX, rWgu, rWd = O.expert_rows_bwd(TB.host(data["X"][idx]), TB.host(data["dY"][idx]), sub_off,
                                      TB.host(data["W_gu"][sel]), TB.host(data["W_d"][sel]))
    assert_close(dX[idx].float().cpu().numpy(), rX, "bf16", "dX (sampled rows)")
    j = int(np.flatnonzero(experts == e_full)[0])
    assert_close(dWgu[e_full].cpu().numpy(), rWgu[j], "bf16", "dW_gu (one whole expert)")
    assert_close(dWd[e_full].cpu().numpy(), rWd[j], "bf16", "dW_d (one whole expert)")

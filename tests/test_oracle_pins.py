"""Pins for the CPU oracle: each test checks it against something other than
itself -- closed forms, a hand-derived example, brute force, library routines
and invariants -- chosen so that a dropped term, a wrong sign or index, or a
transposed operand fails at least one of them."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------ bf16 storage --

def test_bf16_rounding_matches_torch_on_float_values():
    # On values that are exact float32s there is a single rounding, and torch's
    # float32 -> bfloat16 conversion is round-to-nearest-even.
    g = torch.Generator().manual_seed(11)
    v = torch.randn(20000, generator=g) * torch.exp(4 * torch.randn(20000, generator=g))
    ref = bf16_bits(v.to(torch.bfloat16))
    got = O.to_bf16(v.double().numpy())
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3F80),
    (1.0 + 2 ** -8, 0x3F80),              # halfway, ties to even (down)
    (1.0 + 3 * 2 ** -8, 0x3F82),          # halfway, ties to even (up)
    (1.0 + 2 ** -8 + 2 ** -40, 0x3F81),   # just above halfway; a float detour would tie down
    (-(1.0 + 2 ** -8 + 2 ** -40), 0xBF81),
    (2.0 ** -130, 0x0008),                # subnormal
    (3.0e38, 0x7F62),
    (3.4e38, 0x7F80),                     # above the largest bfloat16 + half ulp: infinity
    (-0.0, 0x8000),
])
def test_bf16_rounding_hand_cases(x, bits):
    assert int(O.to_bf16(np.array([x]))[0]) == bits


# ----------------------------------------------------------------- RMSNorm --

def test_rmsnorm_matches_torch():
    g = torch.Generator().manual_seed(1)
    v = torch.randn(3072, generator=g, dtype=torch.float64) * 3
    gain = (1 + 0.1 * torch.randn(3072, generator=g)).float()
    ref = torch.nn.functional.rms_norm(v, (3072,), gain.double(), eps=1e-5)
    got = O.rmsnorm_row(v.numpy(), gain.numpy(), 1e-5)
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-14, atol=0)


# ------------------------------------------------------------------- top-k --

def _topk_brute(lg: np.ndarray, k: int):
    T, E = lg.shape
    ids = np.empty((T, k), np.int64)
    for t in range(T):
        # NaN ranks last; larger first; equal values by lower id.  lexsort keys
        # go from least to most significant.
        v = lg[t].astype(np.float64)
        nan = np.isnan(v)
        key = np.where(nan, 0.0, -v)
        order = np.lexsort((np.arange(E), key, nan))
        ids[t] = order[:k]
    return ids


def test_topk_matches_stable_sort_with_many_ties():
    rng = np.random.default_rng(3)
    lg = rng.integers(-3, 4, size=(500, 24)).astype(np.float32)  # heavy ties
    ids, w = O.topk(lg, 5)
    assert np.array_equal(ids, _topk_brute(lg, 5))


def test_topk_signed_zero_and_nan():
    lg = np.array([[-0.0, 0.0, -1.0, np.nan, 0.0],
                   [np.nan, np.nan, -np.inf, -np.inf, 5.0]], np.float32)
    ids, _ = O.topk(lg, 4)
    assert ids[0].tolist() == [0, 1, 4, 2]      # +0 == -0: lower id first; NaN last
    assert ids[1].tolist() == [4, 2, 3, 0]      # -inf above NaN


def test_topk_weights_softmax_then_renormalise():
    rng = np.random.default_rng(4)
    lg = (rng.standard_normal((300, 64)) * 2).astype(np.float32)
    k = 6
    ids, w = O.topk(lg, k)
    p = torch.softmax(torch.from_numpy(lg).double(), dim=1).numpy()
    sel = np.take_along_axis(p, ids, axis=1)
    ref = sel / sel.sum(1, keepdims=True)
    np.testing.assert_allclose(w, ref, rtol=1e-6, atol=0)
    np.testing.assert_allclose(w.astype(np.float64).sum(1), 1.0, atol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)      # best expert first


def test_topk_k_equals_E_is_softmax():
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((50, 16)).astype(np.float32)
    ids, w = O.topk(lg, 16)
    p = torch.softmax(torch.from_numpy(lg).double(), dim=1).numpy()
    full = np.zeros_like(p)
    np.put_along_axis(full, ids, w.astype(np.float64), axis=1)
    np.testing.assert_allclose(full, p, rtol=1e-6, atol=1e-7)


# ----------------------------------------------------------------- permute --

@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (37, 3, 7), (512, 4, 16), (300, 8, 384)])
def test_permute_dropless_matches_stable_argsort(T, k, E):
    rng = np.random.default_rng(T + E)
    ids = rng.integers(0, E, size=T * k).astype(np.int32)
    r = O.permute(ids, E)
    order = np.argsort(ids, kind="stable")          # rows in expert order, arrival within
    counts = np.bincount(ids, minlength=E)
    assert np.array_equal(r["counts"], counts)
    assert np.array_equal(r["offsets"], np.concatenate([[0], np.cumsum(counts)]))
    assert np.array_equal(r["row_src"], order)
    assert np.array_equal(r["slot_row"][order], np.arange(T * k))
    assert r["n_dropped"] == 0
    # every token appears exactly k times; the map is a bijection
    assert np.array_equal(np.bincount(r["row_src"] // k, minlength=T), np.full(T, k))
    assert np.array_equal(np.sort(r["slot_row"]), np.arange(T * k))


@pytest.mark.parametrize("cf", [(110, 100), (115, 100), (1, 2)])
def test_permute_capacity_drop_rule(cf):
    rng = np.random.default_rng(9)
    E, n = 12, 2000
    p = 1 / np.arange(1, E + 1)
    ids = rng.choice(E, size=n, p=p / p.sum()).astype(np.int32)
    C = O.capacity(cf[0], cf[1], n, E)
    assert C == math.ceil(Fraction(cf[0], cf[1]) * n / E)
    r = O.permute(ids, E, capacity=C)
    counts = np.bincount(ids, minlength=E)
    kept = np.minimum(counts, C)
    assert r["n_dropped"] == int(np.sum(np.maximum(0, counts - C)))
    assert np.array_equal(r["offsets"], np.concatenate([[0], np.cumsum(kept)]))
    for e in range(E):
        arrivals = np.flatnonzero(ids == e)
        keep, drop = arrivals[:C], arrivals[C:]
        assert np.array_equal(r["slot_row"][keep], r["offsets"][e] + np.arange(keep.size))
        assert np.all(r["slot_row"][drop] == -1)
    assert np.all(r["row_src"][r["offsets"][E]:] == -1)


def test_capacity_formula_against_exact_fractions():
    for n in [1, 7, 65536, 524288, 57673]:
        for E in [1, 6, 64, 384]:
            for num, den in [(110, 100), (115, 100), (100, 100), (3, 2)]:
                assert O.capacity(num, den, n, E) == math.ceil(Fraction(num, den) * n / E)


def test_permute_padding_rows_take_no_part():
    ids = np.array([2, -1, 0, 2, -1, 1, 0], np.int32)
    r = O.permute(ids, 3, R_phys=7)
    assert r["counts"].tolist() == [2, 1, 2]
    assert r["offsets"].tolist() == [0, 2, 3, 5]
    assert r["slot_row"].tolist() == [3, -1, 0, 4, -1, 2, 1]
    assert r["row_src"].tolist() == [2, 6, 5, 0, 3, -1, -1]


# ------------------------------------------------------------- expert FFN --

def _swiglu_torch(x, Wgu, Wd, H, store):
    u = x @ Wgu.T
    h = store(torch.nn.functional.silu(u[:, :H]) * u[:, H:])
    return h @ Wd.T, h


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_single_expert_is_dense_swiglu(dt):
    # E = 1, k = 1, no latent: the routed path is a dense SwiGLU MLP.
    g = torch.Generator().manual_seed(2)
    n, d, H = 40, 96, 64
    x = torch.randn(n, d, generator=g)
    Wgu = torch.randn(2 * H, d, generator=g) / math.sqrt(d)
    Wd = torch.randn(d, H, generator=g) / math.sqrt(H)
    if dt == "f32":
        X, A, B = x.numpy(), Wgu.numpy(), Wd.numpy()
        xd, Ad, Bd = x.double(), Wgu.double(), Wd.double()
        store = lambda v: v.float().double()
    else:
        xb, Ab, Bb = x.bfloat16(), Wgu.bfloat16(), Wd.bfloat16()
        X, A, B = bf16_bits(xb), bf16_bits(Ab), bf16_bits(Bb)
        xd, Ad, Bd = xb.double(), Ab.double(), Bb.double()
        store = lambda v: torch.from_numpy(O.bf16_to_f64(O.to_bf16(v.numpy())))
    Y, h = O.expert_rows(X, np.zeros(n, np.int32), [A], [B], H, want_h=True)
    Yr, hr = _swiglu_torch(xd, Ad, Bd, H, store)
    # h is stored: allow a one-unit storage flip from a different summation order
    ulp = 2.0 ** -23 if dt == "f32" else 2.0 ** -7
    assert np.mean(np.abs(h - hr.numpy()) > 0) < 1e-3
    np.testing.assert_allclose(h, hr.numpy(), rtol=ulp, atol=1e-30)
    np.testing.assert_allclose(Y, Yr.numpy(), rtol=0, atol=4 * ulp * float(Yr.abs().max()))


def test_expert_rows_pick_their_own_expert():
    rng = np.random.default_rng(6)
    d, H, E = 16, 8, 4
    Wgu = [rng.standard_normal((2 * H, d)).astype(np.float32) for _ in range(E)]
    Wd = [rng.standard_normal((d, H)).astype(np.float32) for _ in range(E)]
    X = rng.standard_normal((10, d)).astype(np.float32)
    ex = rng.integers(-1, E, size=10).astype(np.int32)
    Y = O.expert_rows(X, ex, Wgu, Wd, H)
    for r in range(10):
        if ex[r] < 0:
            assert np.all(Y[r] == 0)
            continue
        Yr = O.expert_rows(X[r:r + 1], np.zeros(1, np.int32), [Wgu[ex[r]]], [Wd[ex[r]]], H)
        assert np.array_equal(Y[r], Yr[0])


def test_combine_ordered_weighted_gather():
    rng = np.random.default_rng(8)
    T, k, d = 9, 3, 5
    Y = rng.standard_normal((T * k, d)).astype(np.float32)
    slot = rng.permutation(T * k).astype(np.int32)
    slot[[1, 5, 6]] = -1
    w = rng.random((T, k)).astype(np.float32)
    c = O.combine(Y, slot, w, T, k)
    ref = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            if slot[t * k + j] >= 0:
                ref[t] += float(w[t, j]) * Y[slot[t * k + j]].astype(np.float64)
    assert np.array_equal(c, ref)


# ------------------------------------------------------------- full layer --

def _hand_layer():
    with open(os.path.join(GOLDEN, "hand_three_experts.json")) as f:
        return json.load(f)


def test_hand_worked_three_expert_example():
    """Three experts on 8-wide rows with diagonal weights: the output has a
    closed form (derivation in the fixture)."""
    G = _hand_layer()
    D, E, k, H = G["D"], G["E"], G["k"], G["H"]
    I = np.eye(D, dtype=np.float32)
    a, b, c = G["gate_scale"], G["up_scale"], G["down_scale"]
    W_gu = [np.concatenate([a[e] * I, b[e] * I]).astype(np.float32) for e in range(E)]
    W_d = [(c[e] * I).astype(np.float32) for e in range(E)]
    W_r = np.array(G["W_r"], np.float32)
    x = np.array(G["x"], np.float32)
    W = O.LayerWeights(None, None, W_r, None, W_gu, W_d, None,
                       np.concatenate([I, I])[None].copy(), I[None].copy())
    dm = O.dims(T=x.shape[0], D=D, L=0, E=E, k=k, H=H, n_shared=1, Hs=D, dtype=O.DT_F32)
    r = O.route_tokens(dm, W, x, np.arange(x.shape[0]))
    assert r["ids"].tolist() == G["expected_ids"]
    np.testing.assert_allclose(r["w"], np.array(G["expected_w"]), rtol=1e-7)
    y = O.output_tokens(dm, W, x, np.arange(x.shape[0]), r["ids"], r["w"])
    np.testing.assert_allclose(y, np.array(G["expected_y"]), rtol=1e-6, atol=1e-7)


def _dense_masked_layer(cfg, inp, ids_override=None, parts=False):
    """Brute force in numpy: evaluate EVERY expert on EVERY token and combine
    with a mask of routing weights -- no permutation, no gather.  parts=True also
    returns the weights and every expert's stored output on every token."""
    f32 = cfg["dtype"] == "f32"

    def val(t):
        return t.double().numpy()

    def store(v):
        if f32:
            return v.astype(np.float32).astype(np.float64)
        return O.bf16_to_f64(O.to_bf16(v))

    x = val(inp["x"])
    if cfg["L"] > 0:
        zp = x @ val(inp["W_dn"]).T
        z = zp / np.sqrt((zp ** 2).mean(1, keepdims=True) + 1e-5) * inp["norm_g"].double().numpy()
    else:
        z = x
    lg = (z.astype(np.float32).astype(np.float64) @ inp["W_r"].double().numpy().T
          + inp["b_r"].double().numpy()).astype(np.float32)
    ids = _topk_brute(lg, cfg["k"]) if ids_override is None else ids_override
    p = torch.softmax(torch.from_numpy(lg).double(), 1).numpy()
    sel = np.take_along_axis(p, ids, 1)
    w = (sel / sel.sum(1, keepdims=True)).astype(np.float32).astype(np.float64)
    ze = store(z) if cfg["L"] > 0 else z
    T, E, H = x.shape[0], cfg["E"], cfg["H"]
    M = np.zeros((T, E))
    np.put_along_axis(M, ids, w, 1)
    c = np.zeros((T, ze.shape[1]))
    Y_all = []
    for e in range(E):
        u = ze @ val(inp["W_gu"][e]).T
        h = store(u[:, :H] / (1 + np.exp(-u[:, :H])) * u[:, H:])
        Ye = store(h @ val(inp["W_d"][e]).T)
        Y_all.append(Ye)
        c += M[:, e:e + 1] * Ye
    c = store(c)
    y = c @ val(inp["W_up"]).T if cfg["L"] > 0 else c.copy()
    Hs = cfg["Hs"]
    for s in range(cfg["n_shared"]):
        u = x @ val(inp["W_gu_s"][s]).T
        h = store(u[:, :Hs] / (1 + np.exp(-u[:, :Hs])) * u[:, Hs:])
        y += h @ val(inp["W_d_s"][s]).T
    if parts:
        return dict(y=y, ids=ids, lg=lg, w=w, Y_all=Y_all)
    return y, ids, lg


def _oracle_layer(cfg, inp, tok=None):
    dt = O.DT_F32 if cfg["dtype"] == "f32" else O.DT_BF16

    def host(t):
        if t is None:
            return None
        return t.numpy() if t.dtype != torch.bfloat16 else bf16_bits(t)

    E = cfg["E"]
    W = O.LayerWeights(host(inp.get("W_dn")), host(inp.get("norm_g")), host(inp["W_r"]),
                       host(inp["b_r"]), [host(inp["W_gu"][e]) for e in range(E)],
                       [host(inp["W_d"][e]) for e in range(E)], host(inp.get("W_up")),
                       host(inp["W_gu_s"]), host(inp["W_d_s"]))
    T = inp["x"].shape[0]
    dm = O.dims(T=T, D=cfg["D"], L=cfg["L"], E=E, k=cfg["k"], H=cfg["H"],
                n_shared=cfg["n_shared"], Hs=cfg["Hs"], dtype=dt)
    tok = np.arange(T) if tok is None else tok
    x = host(inp["x"])
    r = O.route_tokens(dm, W, x, tok)
    y = O.output_tokens(dm, W, x, tok, r["ids"], r["w"])
    return y, r


def _small(dtype, L, gain_noise=True, seed=0, bias=0.0):
    from moe_synth import LayerConfig, gen_layer
    cfg = LayerConfig("pin", T=48, D=64, L=L, E=6, k=2, H=32, n_shared=2, Hs=16, dtype=dtype,
                      seed=seed)
    inp = gen_layer(cfg, "cpu", gain_noise=gain_noise, bias_std=bias)
    return dict(dtype=dtype, L=L, E=6, k=2, H=32, n_shared=2, Hs=16, D=64), inp


@pytest.mark.parametrize("dtype,L", [("f32", 32), ("bf16", 32), ("bf16", 0), ("f32", 0)])
def test_sparse_oracle_equals_dense_every_expert_masked(dtype, L):
    cfg, inp = _small(dtype, L, bias=0.3)
    y_dense, ids_dense, lg_dense = _dense_masked_layer(cfg, inp)
    y, r = _oracle_layer(cfg, inp)
    assert np.array_equal(r["ids"], ids_dense)
    np.testing.assert_array_equal(r["logits32"], lg_dense)
    scale = np.sqrt(np.mean(y_dense ** 2))
    np.testing.assert_allclose(y, y_dense, rtol=0, atol=1e-12 * scale)


def test_zero_input_gives_zero_output():
    cfg, inp = _small("bf16", 32)
    inp["x"].zero_()
    y, _ = _oracle_layer(cfg, inp)
    assert np.all(y == 0)


def test_down_weights_scale_the_routed_part_exactly():
    cfg, inp = _small("bf16", 32)
    inp["W_d_s"].zero_()                     # routed part only
    y1, _ = _oracle_layer(cfg, inp)
    inp["W_d"].mul_(2)                       # exact in bfloat16
    y2, _ = _oracle_layer(cfg, inp)
    assert np.array_equal(y2, 2 * y1)


def test_relabelling_experts_leaves_output_unchanged():
    cfg, inp = _small("f32", 32)
    y1, r1 = _oracle_layer(cfg, inp)
    perm = torch.tensor([3, 0, 5, 1, 4, 2])
    inp2 = dict(inp)
    for name in ["W_r", "b_r", "W_gu", "W_d"]:
        inp2[name] = inp[name][perm].contiguous()
    y2, r2 = _oracle_layer(cfg, inp2)
    assert np.array_equal(perm.numpy()[r2["ids"]], r1["ids"])
    assert np.array_equal(y1, y2)


def test_permuting_tokens_permutes_output():
    cfg, inp = _small("bf16", 32)
    y1, _ = _oracle_layer(cfg, inp)
    perm = torch.randperm(inp["x"].shape[0], generator=torch.Generator().manual_seed(1))
    inp["x"] = inp["x"][perm].contiguous()
    y2, _ = _oracle_layer(cfg, inp)
    assert np.array_equal(y2, y1[perm.numpy()])


def test_dropped_assignment_skips_only_that_expert():
    cfg, inp = _small("f32", 32)
    y_full, r = _oracle_layer(cfg, inp)
    dt = O.DT_F32
    E = cfg["E"]
    W = O.LayerWeights(inp["W_dn"].numpy(), inp["norm_g"].numpy(), inp["W_r"].numpy(),
                       inp["b_r"].numpy(), [inp["W_gu"][e].numpy() for e in range(E)],
                       [inp["W_d"][e].numpy() for e in range(E)], inp["W_up"].numpy(),
                       inp["W_gu_s"].numpy(), inp["W_d_s"].numpy())
    T = inp["x"].shape[0]
    dm = O.dims(T=T, D=64, L=32, E=E, k=2, H=32, n_shared=2, Hs=16, dtype=dt)
    keep = np.ones((T, 2), np.int32)
    keep[:, 1] = 0                              # drop every second choice
    y_drop = O.output_tokens(dm, W, inp["x"].numpy(), np.arange(T), r["ids"], r["w"], keep)
    # with only the first choice kept and no renormalisation, the routed part is
    # w_0 * FFN_0; shared experts unchanged
    keep0 = np.zeros((T, 2), np.int32)
    y_none = O.output_tokens(dm, W, inp["x"].numpy(), np.arange(T), r["ids"], r["w"], keep0)
    r1 = r["ids"][:, :1].copy()
    w1 = r["w"][:, :1].copy()
    dm1 = O.dims(T=T, D=64, L=32, E=E, k=1, H=32, n_shared=0, Hs=16, dtype=dt)
    y_first = O.output_tokens(dm1, W, inp["x"].numpy(), np.arange(T), r1, w1)
    np.testing.assert_allclose(y_drop - y_none, y_first, rtol=0, atol=1e-12)
    assert not np.allclose(y_drop, y_full)


@pytest.mark.parametrize("dtype,L,cf", [("bf16", 32, None), ("f32", 0, None), ("bf16", 32, 110),
                                        ("f32", 32, 100)])
def test_combine_equals_dense_masked_sum(dtype, L, cf):
    """The oracle's ordered gather over the grouped rows (moe_ref_combine through
    the oracle's own permutation, optionally with a capacity cut) equals the
    brute-force sum over EVERY expert of mask x that expert's output, where the
    mask holds the routing weight of each kept (token, expert) pair and zero
    elsewhere (dropped pairs contribute nothing and nothing is renormalised)."""
    cfg, inp = _small(dtype, L, bias=0.3)
    dn = _dense_masked_layer(cfg, inp, parts=True)
    ids, w, Y_all = dn["ids"], dn["w"], dn["Y_all"]
    T, k, E = ids.shape[0], cfg["k"], cfg["E"]
    cap = O.capacity(cf, 100, T * k, E) if cf else -1
    g = O.permute(ids.ravel(), E, capacity=cap)
    if cf:
        assert g["n_dropped"] > 0
    R = int(g["offsets"][E])
    rows = np.zeros((T * k, Y_all[0].shape[1]))
    for r in range(R):
        t, j = divmod(int(g["row_src"][r]), k)
        rows[r] = Y_all[ids[t, j]][t]
    stored = rows.astype(np.float32) if dtype == "f32" else O.to_bf16(rows)
    c = O.combine(stored, g["slot_row"], w.astype(np.float32).ravel(), T, k)
    mask = np.zeros((T, E))
    kept = g["slot_row"].reshape(T, k) >= 0
    for t in range(T):
        for j in range(k):
            if kept[t, j]:
                mask[t, ids[t, j]] = w[t, j]
    dense = sum(mask[:, e:e + 1] * Y_all[e] for e in range(E))
    scale = np.sqrt(np.mean(dense ** 2))
    np.testing.assert_allclose(c, dense, rtol=0, atol=1e-12 * scale)


def test_combine_with_one_unit_weight_is_the_inverse_permutation():
    """k = 1 and no weights: the combine scatters each grouped row back to the
    pool row it came from (row_src is the permutation's inverse); padding rows,
    which have no grouped row, come out zero."""
    rng = np.random.default_rng(12)
    P, E, d = 200, 5, 7
    ids = rng.integers(0, E, size=P).astype(np.int32)
    ids[rng.choice(P, 40, replace=False)] = -1
    g = O.permute(ids, E, R_phys=P)
    Y = rng.standard_normal((P, d)).astype(np.float32)
    c = O.combine(Y, g["slot_row"], None, P, 1)
    R = int(g["offsets"][E])
    assert R == int((ids >= 0).sum())
    assert np.array_equal(c[g["row_src"][:R]], Y[:R].astype(np.float64))
    assert np.all(c[ids < 0] == 0)

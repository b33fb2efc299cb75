"""Per-entry-point parity of the HIP path against the CPU oracle, through the C ABI.

Integer work (top-k ids given identical float32 logits, permutation, offsets,
drops) must match bit for bit; float outputs within the spec's tolerance:
max |err| <= 2e-2 x RMS(ref) for bfloat16 storage, <= 1e-5 x RMS(ref) for float32.
Inputs are seeded synthetic data from moe_synth or built here from closed forms.
"""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as O
from oracle import torch_bridge as TB

from gpu_util import assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"bf16": 2e-2, "f32": 1e-5}
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.fixture(scope="module")
def M():
    import mixture_experts_transformer_amd as m
    return m


def _rms(a):
    return float(np.sqrt(np.mean(np.square(a, dtype=np.float64))))


# ---------------------------------------------------------------- route ----

ROUTE_SHAPES = [  # T, d_r, E, k
    (1, 32, 1, 1),          # narrowest router width
    (33, 64, 16, 2),        # ragged token tile
    (65, 48, 130, 3),       # K = 1.5 stages (a 16-value tail), E just over a 128 multiple
    (40, 80, 256, 5),       # K = 2.5 stages
    (1000, 128, 64, 4),
    (8192, 64, 384, 8),     # 535B router width and expert count, full token count
    (300, 32, 512, 16),     # largest E and k
    # expert-split form (E > 256 with a logits output): halves of ceil(E/2) experts,
    # 64-token workgroups
    (129, 48, 257, 3),      # odd E (halves of 129 and 128), a 16-value K tail, ragged tokens
    (70, 1040, 300, 6),     # K = 32.5 stages, halves of 150
    (200, 96, 449, 9),      # the four-column-block form (halves of 225)
]


@pytest.mark.parametrize("T,d,E,k", ROUTE_SHAPES)
@pytest.mark.parametrize("hdt", ["f32", "bf16"])
def test_route_topk_bit_exact_on_exact_logits(M, T, d, E, k, hdt):
    """Integer-valued router inputs make every float32 logit exact whatever the
    summation order, so GPU and oracle select from identical logits: ids must be
    identical (heavy ties exercise the lower-id rule) and weights within 1e-6."""
    g = torch.Generator().manual_seed(T * 7 + E)
    h = torch.randint(-2, 3, (T, d), generator=g).to(TDT[hdt])
    W = torch.randint(-3, 4, (E, d), generator=g).float()
    b = torch.randint(-2, 3, (E,), generator=g).float() * 0.5
    exact = (h.double() @ W.double().T + b.double()).float().numpy()
    logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
    ids, w = M.moe_route(h.to(DEV), W.to(DEV), k, b_r=b.to(DEV), logits_out=logits)
    torch.cuda.synchronize()
    assert np.array_equal(logits.cpu().numpy(), exact)
    ref_ids, ref_w = O.topk(exact, k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=0, atol=1e-6)


def test_route_signed_zero_and_ties(M):
    h = torch.ones((1, 32), dtype=torch.float32)
    W = torch.zeros((8, 32))
    W[3, 0] = -0.0
    W[5, 0] = 1.0
    W[6, 0] = 1.0
    b = torch.tensor([0.0, -0.0, -1.0, 0.0, 0.0, 0.0, 0.0, -2.0])
    ids, w = M.moe_route(h.to(DEV), W.to(DEV), 5, b_r=b.to(DEV))
    torch.cuda.synchronize()
    exact = (h.double() @ W.double().T + b.double()).float().numpy()
    ref_ids, _ = O.topk(exact, 5)
    assert ids.cpu().numpy().tolist() == ref_ids.tolist() == [[5, 6, 0, 1, 3]]


@pytest.mark.parametrize("T,d,E,k,hdt,rdt", [(777, 3072, 384, 8, "f32", "bf16"),
                                              (301, 1040, 384, 8, "bf16", "f32"),
                                              (97, 2064, 512, 16, "f32", "f32"),
                                              (256, 128, 16, 2, "f32", "f32"),
                                              (500, 2048, 64, 4, "bf16", "f32"),
                                              (129, 1040, 96, 6, "bf16", "bf16")])
def test_route_rmsnorm_router_on_real_distribution(M, T, d, E, k, hdt, rdt):
    """RMSNorm + router on Gaussian inputs: normalised rows within one storage
    rounding, logits within float32 accumulation error, ids equal wherever the
    oracle's k-th/(k+1)-th logit gap exceeds twice that error."""
    g = torch.Generator().manual_seed(d + T)
    h = (torch.randn((T, d), generator=g) * 3).to(TDT[hdt])
    gain = (1 + 0.1 * torch.randn(d, generator=g)).float()
    W = (torch.randn((E, d), generator=g) / math.sqrt(d)).float()
    b = 0.1 * torch.randn(E, generator=g)
    r_out = torch.empty((T, d), dtype=TDT[rdt], device=DEV)
    logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
    ids, w = M.moe_route(h.to(DEV), W.to(DEV), k, b_r=b.to(DEV), norm_g=gain.to(DEV), eps=1e-5,
                         apply_norm=True, r_out=r_out, logits_out=logits)
    torch.cuda.synchronize()
    # oracle: z = RMSNorm(h) * g in double, logits from float32(z)
    hd = TB.host(h)
    hv = O.bf16_to_f64(hd) if hdt == "bf16" else hd.astype(np.float64)
    z = np.stack([O.rmsnorm_row(hv[t], gain.numpy(), 1e-5) for t in range(T)])
    lg64 = z.astype(np.float32).astype(np.float64) @ W.double().numpy().T + b.double().numpy()
    lg32 = lg64.astype(np.float32)
    zg = r_out.float().cpu().numpy()
    ulp = 2.0 ** -7 if rdt == "bf16" else 1e-5
    assert np.all(np.abs(zg - z) <= ulp * np.abs(z) + 1e-30)
    tol_l = 2e-5 * max(1.0, _rms(lg64))
    lgg = logits.cpu().numpy()
    assert np.max(np.abs(lgg - lg64)) <= tol_l
    ref_ids, ref_w = O.topk(lg32, k)
    srt = -np.sort(-lg64, axis=1)
    clear = (srt[:, k - 1] - srt[:, k]) > 2 * tol_l if k < E else np.ones(T, bool)
    gi = ids.cpu().numpy()
    assert clear.mean() > 0.9
    assert np.array_equal(gi[clear], ref_ids[clear])
    np.testing.assert_allclose(w.cpu().numpy()[clear], ref_w[clear], rtol=0, atol=4 * tol_l)
    # the rest is valid: every chosen expert is within the tolerance of the k-th logit
    for t in np.flatnonzero(~clear):
        assert np.all(lg64[t, gi[t]] >= srt[t, k - 1] - 2 * tol_l)


@pytest.mark.parametrize("hdt", ["f32", "bf16"])
@pytest.mark.parametrize("E", [384, 512])
def test_route_forms_agree(M, E, hdt):
    """A wide router runs in its expert-split form (two kernels) when it has a logits
    output and in the one-kernel form without: on exactly representable logits both
    must give the same ids and bit-identical weights, and the same router input r."""
    g = torch.Generator().manual_seed(E)
    T, d, k = 333, 80, 8
    h = torch.randint(-2, 3, (T, d), generator=g).to(TDT[hdt])
    W = torch.randint(-3, 4, (E, d), generator=g).float()
    b = torch.randint(-2, 3, (E,), generator=g).float() * 0.5
    r1 = torch.empty((T, d), dtype=torch.float32, device=DEV)
    r2 = torch.empty((T, d), dtype=torch.float32, device=DEV)
    logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
    ids1, w1 = M.moe_route(h.to(DEV), W.to(DEV), k, b_r=b.to(DEV), r_out=r1, logits_out=logits)
    ids2, w2 = M.moe_route(h.to(DEV), W.to(DEV), k, b_r=b.to(DEV), r_out=r2)
    torch.cuda.synchronize()
    assert torch.equal(ids1.cpu(), ids2.cpu())
    assert torch.equal(w1.cpu(), w2.cpu())
    assert torch.equal(r1.cpu(), r2.cpu()) and torch.equal(r1.cpu(), h.float())


def test_route_split_form_logits_do_not_depend_on_the_router_input_output(M):
    """In the expert-split form the inverse RMS scales the logits in the first
    kernel whether or not the router input r is asked for (only then is it handed to
    the second kernel): logits, ids and weights are bit-identical either way."""
    g = torch.Generator().manual_seed(5)
    T, d, E, k = 515, 3072, 384, 8
    h = (torch.randn((T, d), generator=g) * 3).to(DEV)
    W = (torch.randn((E, d), generator=g) / math.sqrt(d)).to(DEV)
    b = (0.1 * torch.randn(E, generator=g)).to(DEV)
    gain = (1 + 0.1 * torch.randn(d, generator=g)).to(DEV)
    out = []
    for with_r in (True, False):
        r_out = torch.empty((T, d), dtype=torch.bfloat16, device=DEV) if with_r else None
        logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
        ids, w = M.moe_route(h, W, k, b_r=b, norm_g=gain, eps=1e-5, apply_norm=True,
                             r_out=r_out, logits_out=logits)
        out.append((logits, ids, w))
    torch.cuda.synchronize()
    for a, c in zip(out[0], out[1]):
        assert torch.equal(a.cpu(), c.cpu())


@pytest.mark.parametrize("hdt,rdt", [("f32", "f32"), ("f32", "bf16"), ("bf16", "bf16")])
def test_route_writes_router_input_without_norm(M, hdt, rdt):
    """Without the norm the router input r is h itself, stored in r's dtype."""
    g = torch.Generator().manual_seed(11)
    T, d, E, k = 70, 112, 24, 3
    h = torch.randn((T, d), generator=g).to(TDT[hdt])
    W = torch.randn((E, d), generator=g).float()
    r_out = torch.full((T, d), 7.0, dtype=TDT[rdt], device=DEV)
    M.moe_route(h.to(DEV), W.to(DEV), k, r_out=r_out)
    torch.cuda.synchronize()
    assert torch.equal(r_out.cpu(), h.float().to(TDT[rdt]))


# -------------------------------------------------------------- permute ----

def _ids_cases():
    rng = np.random.default_rng(0)
    yield "uniform", rng.integers(0, 384, 65536).astype(np.int32), 384, -1
    p = 1 / np.arange(1, 7)
    yield "zipf6", rng.choice(6, 57713, p=p / p.sum()).astype(np.int32), 6, -1
    yield "one_expert", np.full(10000, 3, np.int32), 16, -1
    yield "empty_experts", rng.choice([0, 5, 63], 4097).astype(np.int32), 64, -1
    z = rng.choice(6, 65536, p=p / p.sum()).astype(np.int32)
    z[rng.random(65536) < 0.12] = -1
    yield "padding", z, 6, -1
    u = rng.integers(0, 64, 32768).astype(np.int32)
    yield "cap110", u, 64, O.capacity(110, 100, u.size, 64)
    yield "cap_tight", rng.choice(16, 5000, p=np.r_[0.5, np.full(15, 0.5 / 15)]).astype(np.int32), 16, 200
    yield "single", np.array([0], np.int32), 1, -1
    yield "E1024", rng.integers(0, 1024, 100000).astype(np.int32), 1024, -1
    yield "empty", np.zeros(0, np.int32), 8, -1


@pytest.mark.parametrize("case", list(_ids_cases()), ids=lambda c: c[0])
def test_permute_bit_exact(M, case):
    name, ids, E, cap = case
    n = ids.size
    ref = O.permute(ids, E, capacity=cap, R_phys=n)
    gi = torch.from_numpy(ids).to(DEV)
    out = M.moe_permute(gi, E, capacity=cap, R_phys=n)
    out2 = M.moe_permute(gi, E, capacity=cap, R_phys=n)
    torch.cuda.synchronize()
    for key in ["counts", "offsets", "slot_row", "row_src"]:
        got = out[key].cpu().numpy()[: ref[key].size]
        assert np.array_equal(got, ref[key]), key
        assert torch.equal(out[key], out2[key]), f"{key} not deterministic"
    assert int(out["n_dropped"].item()) == ref["n_dropped"]


@pytest.mark.parametrize("dt,width,div,n,E,cap,pad", [
    ("bf16", 3072, 8, 4000, 24, -1, 0.0),      # one source row per token, k = 8
    ("f32", 128, 2, 4000, 24, -1, 0.0),
    ("bf16", 64, 1, 4000, 24, -1, 0.0),        # one source row per assignment
    ("bf16", 3072, 8, 4003, 24, -1, 0.0),      # last source row has 3 assignments
    ("bf16", 256, 3, 6000, 16, 200, 0.1),      # capacity drops and padding ids
    ("f32", 64, 70, 7000, 5, -1, 0.3),         # more than 64 assignments per source row
    ("bf16", 128, 4, 4096, 8, 0, 0.0),         # capacity 0: nothing kept, nothing copied
    ("bf16", 4096, 8, 2000, 24, -1, 0.0),      # 8 KB rows: 8 chunks per lane, shared rows
    ("bf16", 4096, 1, 3000, 24, 100, 0.1),     # 8 KB rows, one source row per assignment
])
def test_permute_row_copy(M, dt, width, div, n, E, cap, pad):
    rng = np.random.default_rng(width + n)
    ids = rng.integers(0, E, n).astype(np.int32)
    ids[rng.random(n) < pad] = -1
    n_src = -(-n // div)
    src = torch.randn((n_src, width), generator=torch.Generator().manual_seed(1)).to(TDT[dt])
    dst = torch.full((n, width), -7.0, dtype=TDT[dt], device=DEV)
    M.moe_permute(torch.from_numpy(ids).to(DEV), E, capacity=cap, src=src.to(DEV), src_div=div,
                  dst=dst)
    torch.cuda.synchronize()
    ref = O.permute(ids, E, capacity=cap, R_phys=n)
    kept = int(ref["offsets"][-1])
    got = dst.cpu()
    assert torch.equal(got[:kept], src[torch.from_numpy(ref["row_src"][:kept] // div).long()])
    assert bool((got[kept:] == -7.0).all()), "rows past the kept total were written"


# ----------------------------------------------------------- grouped FFN ----

def _group_counts(rng, E, kind, scale):
    if kind == "uniform":
        return rng.poisson(scale, E)
    if kind == "skewed":
        c = rng.poisson(scale, E)
        c[rng.choice(E, max(1, E // 10), replace=False)] *= 5
        return c
    if kind == "sparse":
        c = np.zeros(E, np.int64)
        c[rng.choice(E, 3, replace=False)] = rng.integers(1, 600, 3)
        return c
    raise ValueError(kind)


@pytest.mark.parametrize("dt,E,d,H,kind,scale", [
    ("bf16", 8, 128, 64, "uniform", 40),
    ("bf16", 16, 256, 256, "skewed", 150),     # several 256-row tiles, ragged tails
    ("bf16", 6, 3072, 3072, "sparse", 0),      # 535B expert shape, empty groups
    ("f32", 8, 128, 96, "uniform", 70),
    ("f32", 5, 64, 32, "sparse", 0),
    ("bf16", 3, 64, 64, "uniform", 300),       # one K step in both GEMMs
    ("bf16", 4, 128, 192, "skewed", 200),      # two and three K steps
    ("f32", 3, 32, 64, "uniform", 90),         # one and two K steps in float32
    # two or more row tiles per expert on average: the GEMMs run A's K steps ahead
    ("bf16", 2, 128, 128, "uniform", 700),     # 2.7 tiles per expert, ragged
    ("bf16", 4, 256, 256, "uniform", 600),     # four K steps
    ("f32", 3, 64, 96, "skewed", 300),         # one expert five times the others
    # 16 or more row tiles per expert: tiles swizzled in groups of 8 row tiles
    ("bf16", 2, 64, 64, "uniform", 4200),
])
def test_grouped_ffn_parity(M, dt, E, d, H, kind, scale):
    rng = np.random.default_rng(E * d + H)
    counts = _group_counts(rng, E, kind, scale)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    R_phys = R + 37                              # spare rows must stay untouched
    g = torch.Generator().manual_seed(5)
    X = torch.randn((R_phys, d), generator=g).to(TDT[dt])
    W_gu = (torch.randn((E, 2 * H, d), generator=g) / math.sqrt(d)).to(TDT[dt])
    W_d = (torch.randn((E, d, H), generator=g) / math.sqrt(H)).to(TDT[dt])
    Y = torch.full((R_phys, d), 3.0, dtype=TDT[dt], device=DEV)
    M.moe_grouped_ffn(X.to(DEV), torch.from_numpy(offsets).to(DEV), W_gu.to(DEV), W_d.to(DEV), Y=Y)
    torch.cuda.synchronize()
    expert = np.full(R_phys, -1, np.int32)
    for e in range(E):
        expert[offsets[e]:offsets[e + 1]] = e
    Xh = TB.host(X)
    sample = np.arange(R) if R <= 3000 else np.sort(rng.choice(R, 3000, replace=False))
    Yref = O.expert_rows(Xh[sample], expert[sample], [TB.host(W_gu[e]) for e in range(E)],
                         [TB.host(W_d[e]) for e in range(E)], H)
    Yg = Y.float().cpu().numpy()
    assert_close(Yg[sample], Yref, dt, "Y")
    assert np.all(Yg[R:] == 3.0), "rows past offsets[E] were written"


# --------------------------------------------------------------- combine ----

@pytest.mark.parametrize("dt,T,k,width", [
    ("bf16", 8192, 8, 3072),     # two row segments of 3 chunks per lane
    ("f32", 256, 2, 128),        # one segment of 2 chunks, most lanes idle
    ("bf16", 1000, 4, 2048),     # two segments of 2 chunks
    ("bf16", 700, 3, 1536),      # one segment of 3 chunks
    ("bf16", 3000, 1, 4096),     # k = 1: one segment of 8 chunks
    ("bf16", 2000, 1, 3072),     # k = 1: one segment of 6 chunks
    ("f32", 500, 1, 96),         # k = 1: 4 chunks, most lanes idle
])
def test_combine_parity(M, dt, T, k, width):
    rng = np.random.default_rng(T + k)
    slot = rng.permutation(T * k).astype(np.int32)
    slot[rng.random(T * k) < 0.05] = -1
    slot[:k] = -1                                     # a token with every slot dropped
    w = rng.random((T, k)).astype(np.float32)
    Y = torch.randn((T * k, width), generator=torch.Generator().manual_seed(3)).to(TDT[dt])
    out = M.moe_combine(Y.to(DEV), torch.from_numpy(slot).to(DEV), torch.from_numpy(w).to(DEV),
                        T, k)
    out2 = M.moe_combine(Y.to(DEV), torch.from_numpy(slot).to(DEV), torch.from_numpy(w).to(DEV),
                         T, k)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "combine not bitwise repeatable"
    ref = O.combine(TB.host(Y), slot, w, T, k)
    got = out.float().cpu().numpy()
    assert_close(got, ref, dt, "c")
    assert np.all(got[0] == 0)


def test_combine_unpermute_keeps_unrouted_rows(M):
    rng = np.random.default_rng(2)
    P, width = 5000, 256
    slot = rng.permutation(P).astype(np.int32)
    slot[rng.random(P) < 0.2] = -1
    Y = torch.randn((P, width), generator=torch.Generator().manual_seed(4)).bfloat16()
    out = torch.full((P, width), 11.0, dtype=torch.bfloat16, device=DEV)
    M.moe_combine(Y.to(DEV), torch.from_numpy(slot).to(DEV), None, P, 1, out=out,
                  flags=M.MOE_COMBINE_KEEP_UNROUTED)
    torch.cuda.synchronize()
    got = out.cpu()
    valid = slot >= 0
    assert torch.equal(got[torch.from_numpy(valid)], Y[torch.from_numpy(slot[valid]).long()])
    assert torch.all(got[torch.from_numpy(~valid)] == 11.0)


# ------------------------------------------------------------- argument checks ----

def test_errors_are_reported_not_launched(M):
    h = torch.zeros((4, 16), device=DEV)
    W = torch.zeros((4, 16), device=DEV)
    with pytest.raises(M.MoeError) as e:
        M.moe_route(h, W, 5)                       # k > E
    assert "shape" in str(e.value)
    with pytest.raises(M.MoeError):
        M.moe_route(torch.zeros((4, 24), device=DEV), torch.zeros((4, 24), device=DEV), 2)


@pytest.mark.parametrize("T,k,E,P,cap_f,pad,width", [
    (2048, 8, 384, 64, 1.10, 0.0, 256),     # the 535B layer's 64-way split, sender cap 1.10
    (1000, 4, 16, 4, None, 0.05, 128),      # no cap, some assignments absent
    (3000, 2, 24, 8, 0.5, 0.0, 64),         # heavy sender drops
])
def test_dispatch_pack_bit_exact(M, T, k, E, P, cap_f, pad, width):
    """The sender's half of the expert-parallel dispatch: the grouping by peer as the
    oracle's permutation of ids // (E / P) with the sender capacity, every kept row the
    token's row, and the payload each row's local expert id."""
    rng = np.random.default_rng(T + E)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    ids[rng.random((T, k)) < pad] = -1
    epp = E // P
    cap = -1 if cap_f is None else int(np.ceil(cap_f * T * k / P))
    x = torch.randn((T, width), generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    out = M.moe_dispatch_pack(torch.from_numpy(ids).to(DEV), E, P, x.to(DEV), capacity=cap)
    torch.cuda.synchronize()
    peer = np.where(ids < 0, -1, ids // epp)
    ref = O.permute(peer, P, capacity=cap, R_phys=T * k)
    for key in ("counts", "offsets", "slot_row"):
        assert np.array_equal(out[key].cpu().numpy(), ref[key]), key
    assert int(out["n_dropped"].item()) == ref["n_dropped"]
    kept = int(ref["offsets"][-1])
    rs = ref["row_src"][:kept]
    assert np.array_equal(out["row_src"].cpu().numpy()[:kept], rs)
    assert torch.equal(out["send_rows"][:kept].cpu(), x[torch.from_numpy(rs // k).long()])
    se = out["send_expert"].cpu().numpy()
    assert np.array_equal(se[:kept], ids.ravel()[rs] % epp)
    assert np.all(se[kept:] == -1)


def test_expert_parallel_legs_reproduce_the_local_routed_output(M):
    """The expert-parallel path on one GPU with the exchange as the identity: the sender's
    dispatch pack, each peer's receiver grouping by local expert, its grouped FFN and
    unpermute, the rows returned to their slots, and the sender's ordered combine give
    the same routed output, bit for bit, as the single-GPU permute, grouped FFN and
    combine (each output row depends only on its own row and expert, with a fixed
    reduction order)."""
    rng = np.random.default_rng(12)
    T, k, E, P, L, H = 768, 8, 64, 8, 256, 128
    epp = E // P
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    g = torch.Generator().manual_seed(8)
    X = torch.randn((T, L), generator=g).to(torch.bfloat16).to(DEV)
    W_gu = (torch.randn((E, 2 * H, L), generator=g) / L ** 0.5).to(torch.bfloat16).to(DEV)
    W_d = (torch.randn((E, L, H), generator=g) / H ** 0.5).to(torch.bfloat16).to(DEV)
    ids_d, w_d = torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
    # single GPU
    rows = torch.empty((T * k, L), dtype=torch.bfloat16, device=DEV)
    loc = M.moe_permute(ids_d, E, src=X, src_div=k, dst=rows)
    Y = M.moe_grouped_ffn(rows, loc["offsets"], W_gu, W_d)
    c_local = M.moe_combine(Y, loc["slot_row"], w_d, T, k)
    # expert parallel, exchange = identity
    d = M.moe_dispatch_pack(ids_d, E, P, X)
    off = d["offsets"].cpu().numpy()
    ret = torch.zeros((T * k, L), dtype=torch.bfloat16, device=DEV)
    for p in range(P):
        n_p = int(off[p + 1] - off[p])
        if n_p == 0:
            continue
        recv = d["send_rows"][off[p]:off[p + 1]].clone()        # what peer p receives
        recv_ids = d["send_expert"][off[p]:off[p + 1]].clone()
        pool_rows = torch.empty_like(recv)
        grp = M.moe_permute(recv_ids, epp, src=recv, src_div=1, dst=pool_rows)
        Y_p = M.moe_grouped_ffn(pool_rows, grp["offsets"], W_gu[p * epp:(p + 1) * epp].contiguous(),
                                W_d[p * epp:(p + 1) * epp].contiguous())
        M.moe_combine(Y_p, grp["slot_row"], None, n_p, 1, out=ret[off[p]:off[p + 1]],
                      flags=M.MOE_COMBINE_KEEP_UNROUTED)
    c_ep = M.moe_combine(ret, d["slot_row"], w_d, T, k)
    torch.cuda.synchronize()
    assert torch.equal(c_ep.view(torch.int16), c_local.view(torch.int16))


def test_swiglu_activation_accuracy(M):
    """The expert MLP's activation on its own, through moe_grouped_ffn in float32
    with identity-structured weights: the gate row i picks x_i, the up row i picks
    a column of ones and the down projection picks h_i, so every product and sum
    is exact and Y = silu(x) as the GEMM epilogue computes it.  Against silu in
    double precision over 2^20 values from -80 to 80 (dense near 0): within 4
    units in the last place of float32 (an exact exp and an exact division; the
    pages report that an approximate fused activation broke parity).  Below -80
    the result is below 1e-30 in magnitude, as is the exact value."""
    H, R = 128, 8192
    d = 2 * H
    n = R * H
    g = np.random.default_rng(5)
    x = np.concatenate([np.linspace(-80.0, 80.0, n // 2),
                        g.standard_normal(n // 2 - 1024) * 4.0,
                        -80.0 - np.arange(1024) * 0.05]).astype(np.float32)
    X = np.zeros((R, d), np.float32)
    X[:, :H] = x.reshape(R, H)
    X[:, H:] = 1.0
    W_gu = np.zeros((1, 2 * H, d), np.float32)
    W_gu[0, np.arange(H), np.arange(H)] = 1.0            # gate row i: x_i
    W_gu[0, H + np.arange(H), H + np.arange(H)] = 1.0    # up row i: 1
    W_d = np.zeros((1, d, H), np.float32)
    W_d[0, np.arange(H), np.arange(H)] = 1.0             # Y[:, i] = h_i
    off = torch.tensor([0, R], dtype=torch.int32, device=DEV)
    Y = M.moe_grouped_ffn(torch.from_numpy(X).to(DEV), off, torch.from_numpy(W_gu).to(DEV),
                          torch.from_numpy(W_d).to(DEV))
    torch.cuda.synchronize()
    got = Y.cpu().numpy()[:, :H].ravel().astype(np.float64)
    assert np.all(Y.cpu().numpy()[:, H:] == 0)
    xd = x.astype(np.float64)
    ref = xd / (1.0 + np.exp(-xd))
    main = xd >= -80.0
    ulp = np.spacing(np.abs(ref[main]).astype(np.float32)).astype(np.float64)
    err_ulp = np.abs(got[main] - ref[main]) / ulp
    print(f"silu: max error {err_ulp.max():.2f} ulp, mean {err_ulp.mean():.3f} ulp over "
          f"{main.sum()} values")
    assert err_ulp.max() <= 4.0
    assert np.all(np.abs(got[~main]) < 1e-30) and np.all(np.abs(ref[~main]) < 1e-30)


@pytest.mark.parametrize("tiles,pieces", [(320, 4), (384, 2), (8 * 36 + 8 * 9, 2)])
def test_partial_last_round_split_by_rows(M, tiles, pieces):
    """A GEMM whose last round of tiles is at most half full splits those tiles
    by rows (into `pieces` parts per XCD's range): one 256-row x 256-column tile
    per 256 rows of a single group, on the full 256-CU grid.  Against the oracle's
    grouped matmul; the rows are computed the same way as in an unsplit tile."""
    K, N = 128, 256
    R = tiles * 256 - 100                      # a ragged last tile
    g = torch.Generator().manual_seed(tiles)
    X = torch.randn((R, K), generator=g).to(torch.bfloat16)
    W = (torch.randn((1, N, K), generator=g) / K ** 0.5).to(torch.bfloat16)
    off = torch.tensor([0, R], dtype=torch.int32)
    Z = M.moe_ragged_dot(X.to(DEV), off.to(DEV), W.to(DEV), z_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = O.ragged_dot(TB.host(X), TB.host(W), off.numpy())
    # bf16 products summed in float32 and stored in float32: the float32 bound
    assert_close(Z.cpu().numpy(), ref, "f32", f"split last round ({tiles} tiles)")

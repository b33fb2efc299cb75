"""Seeded generators for the layer's inputs (random numbers and layout only).

Recipe (one torch generator per tensor, sub-seed = seed*1000 + tensor index, in
the fixed order x, W_dn, norm_g, W_r, b_r, W_gu, W_d, W_up, W_gu_s, W_d_s):
  x ~ N(0, 1); every weight ~ N(0, 1/fan_in); norm gain g = 1 (or 1 + 0.1 N(0,1)
  when asked); router bias 0, except that a `hot_frac` share of the experts -- the
  first ones of a seed-5 permutation -- get +HOT_BIAS so that each receives about
  `hot_load` times the mean load.  Values are drawn in float32 and stored in the
  workload's dtype (bfloat16 by round-to-nearest-even).  The router weight and
  bias stay float32.

The same seed gives the same bytes on a given device; CPU and GPU generators
differ, so a test draws once and hands the identical bytes to both sides.

Layout (row-major, [out, in] for every projection, so both operands of every
matmul are contiguous along the reduction):
  x [T, D]; W_dn [L, D]; norm_g [L]; W_r [E, d_r]; b_r [E];
  W_gu [E, 2H, d_e]  (rows [0, H) gate, [H, 2H) up);  W_d [E, d_e, H];
  W_up [D, L]; W_gu_s [n_shared, 2Hs, D]; W_d_s [n_shared, D, Hs]
with d_r = d_e = L (latent) or D (no latent).
"""
from __future__ import annotations

import math

import numpy as np
import torch

from .configs import ExpertMlpConfig, LayerConfig, PoolConfig

# Router bias for the hot experts of the long-context workload.  With the
# latent RMS-normalised and W_r ~ N(0, 1/L), a token's logits are iid N(0, 1)
# across experts; a Monte-Carlo bisection over 40,000 such draws (384 experts,
# 38 hot, top-8) puts the hot experts' mean load at 5.00x the mean for this
# offset.  The tests measure the load the kernels actually see.
HOT_BIAS = 1.0147

_ORDER = ["x", "W_dn", "norm_g", "W_r", "b_r", "W_gu", "W_d", "W_up", "W_gu_s", "W_d_s"]
_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + _ORDER.index(name))
    return g


def _normal(shape, std, g, device, dtype, chunk_rows=None):
    """N(0, std^2) drawn in float32, stored in dtype; drawn in slices along dim 0
    to bound the float32 temporary for very large banks."""
    out = torch.empty(shape, dtype=dtype, device=device)
    n0 = shape[0]
    step = n0 if chunk_rows is None else max(1, chunk_rows)
    for s in range(0, n0, step):
        e = min(n0, s + step)
        tmp = torch.randn((e - s,) + tuple(shape[1:]), generator=g, device=device,
                          dtype=torch.float32)
        tmp.mul_(std)
        out[s:e].copy_(tmp)
        del tmp
    return out


def layer_shapes(cfg: LayerConfig) -> dict:
    de = cfg.d_e
    s = dict(x=(cfg.T, cfg.D), W_r=(cfg.E, de), b_r=(cfg.E,), W_gu=(cfg.E, 2 * cfg.H, de),
             W_d=(cfg.E, de, cfg.H), W_gu_s=(cfg.n_shared, 2 * cfg.Hs, cfg.D),
             W_d_s=(cfg.n_shared, cfg.D, cfg.Hs))
    if cfg.L > 0:
        s.update(W_dn=(cfg.L, cfg.D), norm_g=(cfg.L,), W_up=(cfg.D, cfg.L))
    return s


def hot_experts(cfg: LayerConfig) -> np.ndarray:
    n_hot = int(round(cfg.hot_frac * cfg.E))
    return np.sort(np.random.default_rng(5).permutation(cfg.E)[:n_hot]).astype(np.int64)


def gen_tokens(cfg: LayerConfig, device="cpu", seed: int | None = None) -> torch.Tensor:
    """The layer's input x alone (the same bytes gen_layer draws for it)."""
    seed = cfg.seed if seed is None else seed
    return _normal((cfg.T, cfg.D), 1.0, _gen(seed, "x", device), device, _TORCH_DT[cfg.dtype],
                   chunk_rows=4096)


def router_bias(cfg: LayerConfig, device="cpu", seed: int | None = None,
                bias_std: float = 0.0) -> torch.Tensor:
    """The router bias alone (the same values gen_layer draws for it)."""
    seed = cfg.seed if seed is None else seed
    b = torch.zeros((cfg.E,), dtype=torch.float32, device=device)
    if bias_std > 0:
        b += bias_std * torch.randn((cfg.E,), generator=_gen(seed, "b_r", device), device=device)
    if cfg.hot_frac > 0:
        b[torch.as_tensor(hot_experts(cfg), device=device)] += HOT_BIAS
    return b


def gen_layer(cfg: LayerConfig, device="cpu", seed: int | None = None, gain_noise: bool = False,
              bias_std: float = 0.0) -> dict:
    """All inputs of one layer forward, on `device`."""
    seed = cfg.seed if seed is None else seed
    dt = _TORCH_DT[cfg.dtype]
    sh = layer_shapes(cfg)
    de = cfg.d_e
    out = {}
    out["x"] = gen_tokens(cfg, device, seed)
    if cfg.L > 0:
        out["W_dn"] = _normal(sh["W_dn"], 1 / math.sqrt(cfg.D), _gen(seed, "W_dn", device),
                              device, dt, chunk_rows=1024)
        g = torch.ones(sh["norm_g"], dtype=torch.float32, device=device)
        if gain_noise:
            g += 0.1 * torch.randn(sh["norm_g"], generator=_gen(seed, "norm_g", device),
                                   device=device)
        out["norm_g"] = g
    out["W_r"] = _normal(sh["W_r"], 1 / math.sqrt(de), _gen(seed, "W_r", device), device,
                         torch.float32)
    out["b_r"] = router_bias(cfg, device, seed, bias_std)
    rows_per_chunk = max(1, (1 << 27) // max(1, 2 * cfg.H * de))
    out["W_gu"] = _normal(sh["W_gu"], 1 / math.sqrt(de), _gen(seed, "W_gu", device), device, dt,
                          chunk_rows=rows_per_chunk)
    out["W_d"] = _normal(sh["W_d"], 1 / math.sqrt(cfg.H), _gen(seed, "W_d", device), device, dt,
                         chunk_rows=rows_per_chunk)
    if cfg.L > 0:
        out["W_up"] = _normal(sh["W_up"], 1 / math.sqrt(cfg.L), _gen(seed, "W_up", device),
                              device, dt, chunk_rows=2048)
    out["W_gu_s"] = _normal(sh["W_gu_s"], 1 / math.sqrt(cfg.D), _gen(seed, "W_gu_s", device),
                            device, dt, chunk_rows=1)
    out["W_d_s"] = _normal(sh["W_d_s"], 1 / math.sqrt(cfg.Hs), _gen(seed, "W_d_s", device),
                           device, dt, chunk_rows=1)
    return out


def gen_pool(cfg: PoolConfig, device="cpu", seed: int | None = None) -> dict:
    """A receiver pool: P = n_senders * slot_rows rows of width L.

    Sender s filled the first n_s rows of its slot, n_s = round(mu * exp(sigma*N(0,1)
    - sigma^2/2)) clipped to the slot (the excess was dropped at the sender and is
    counted in `sender_dropped`).  Valid rows: N(0,1) scaled to unit RMS, stored as
    bfloat16, with a local expert id drawn iid from Zipf(s) over the E experts,
    P(e) proportional to 1/(e+1)^s.  Padding rows: id -1 and NaN activations (a
    poison that must never reach a valid output)."""
    seed = cfg.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    n_raw = np.rint(cfg.mu * np.exp(cfg.sigma * rng.standard_normal(cfg.n_senders)
                                    - cfg.sigma ** 2 / 2)).astype(np.int64)
    n_s = np.minimum(n_raw, cfg.slot_rows)
    P = cfg.P
    ids = np.full(P, -1, np.int32)
    p = 1.0 / np.arange(1, cfg.E + 1, dtype=np.float64) ** cfg.zipf_s
    p /= p.sum()
    for s in range(cfg.n_senders):
        base = s * cfg.slot_rows
        ids[base:base + n_s[s]] = rng.choice(cfg.E, size=int(n_s[s]), p=p).astype(np.int32)
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000)
    dt = _TORCH_DT[cfg.dtype]
    X = torch.empty((P, cfg.L), dtype=dt, device=device)
    valid = torch.as_tensor(ids >= 0, device=device)
    step = 8192
    for s0 in range(0, P, step):
        tmp = torch.randn((min(step, P - s0), cfg.L), generator=g, device=device)
        tmp = tmp / tmp.pow(2).mean(dim=1, keepdim=True).sqrt()
        X[s0:s0 + tmp.shape[0]].copy_(tmp)
    X[~valid] = float("nan")
    ge = _gen(seed, "W_gu", device)
    W_gu = _normal((cfg.E, 2 * cfg.H, cfg.L), 1 / math.sqrt(cfg.L), ge, device, dt, chunk_rows=1)
    W_d = _normal((cfg.E, cfg.L, cfg.H), 1 / math.sqrt(cfg.H), _gen(seed, "W_d", device), device,
                  dt, chunk_rows=1)
    return dict(X=X, ids=torch.as_tensor(ids, device=device), W_gu=W_gu, W_d=W_d,
                sender_rows=n_s, sender_dropped=int((n_raw - n_s).sum()))


def expert_mlp_routing(cfg: ExpertMlpConfig):
    """Per-expert row counts and offsets [E+1] (int32) of an expert-MLP workload:
    each token draws k distinct experts uniformly at random (k > 1), or one expert
    with P(e) proportional to 1 / (e + 1)^zipf_s (k = 1).  Seed cfg.seed * 1000."""
    rng = np.random.default_rng(cfg.seed * 1000)
    if cfg.k == 1 and cfg.zipf_s > 0:
        p = 1.0 / np.arange(1, cfg.E + 1) ** cfg.zipf_s
        ids = rng.choice(cfg.E, size=cfg.T, p=p / p.sum())
    else:
        ids = np.argsort(rng.random((cfg.T, cfg.E)), axis=1)[:, :cfg.k].ravel()
    counts = np.bincount(ids, minlength=cfg.E)
    return counts, np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


SMALL_INT_VALUES = (0.0, 0.5, 1.0, 2.0, 3.0, 4.0)


def small_int_tensor(shape, seed: int, device="cpu", dtype=torch.bfloat16):
    """Values drawn uniformly from +-{0, 1/2, 1, 2, 3, 4} (each exact in bf16 and in
    E4M3), for matmuls whose partial sums must be exact.  Drawn in 64 MB slices."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    vals = torch.tensor(SMALL_INT_VALUES, dtype=torch.float32, device=device)
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    step = 16 << 20
    for i in range(0, flat.numel(), step):
        n = min(step, flat.numel() - i)
        idx = torch.randint(0, len(SMALL_INT_VALUES), (n,), generator=g, device=device)
        sign = torch.randint(0, 2, (n,), generator=g, device=device).float() * 2 - 1
        flat[i:i + n] = (vals[idx] * sign).to(dtype)
    return out


def gen_expert_mlp(cfg: ExpertMlpConfig, device="cpu") -> dict:
    """Rows grouped by expert for the expert MLP forward and backward.

    Routing: each token draws k distinct experts uniformly at random (k > 1), or
    one expert with P(e) proportional to 1 / (e + 1)^zipf_s (k = 1); the rows are
    laid out grouped by expert, so `offsets` [E+1] is the exclusive prefix of the
    per-expert counts.  X, dY ~ N(0, 1) [R, d]; W_gu ~ N(0, 1/d) [E, 2H, d];
    W_d ~ N(0, 1/H) [E, d, H]; all stored in cfg.dtype.  Sub-seeds seed*1000 + 0..4
    in the order routing, X, dY, W_gu, W_d."""
    dt = _TORCH_DT[cfg.dtype]
    counts, offsets = expert_mlp_routing(cfg)
    out = {"counts": counts, "offsets": torch.from_numpy(offsets).to(device)}
    for i, (name, shape, std) in enumerate([("X", (cfg.R, cfg.d), 1.0),
                                            ("dY", (cfg.R, cfg.d), 1.0),
                                            ("W_gu", (cfg.E, 2 * cfg.H, cfg.d), cfg.d ** -0.5),
                                            ("W_d", (cfg.E, cfg.d, cfg.H), cfg.H ** -0.5)]):
        g = torch.Generator(device=device)
        g.manual_seed(cfg.seed * 1000 + 1 + i)
        row_elems = int(np.prod(shape[1:]))
        out[name] = _normal(shape, std, g, device, dt,
                            chunk_rows=max(1, (64 << 20) // (4 * row_elems)))
    return out

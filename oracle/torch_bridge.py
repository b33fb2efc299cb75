"""Hands torch tensors (on any device) to the CPU oracle.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).  It
copies inputs to the host and calls oracle.py; it imports nothing from the GPU
library and computes nothing itself.
"""
from __future__ import annotations

import numpy as np
import torch

from . import oracle as O


def host(t: torch.Tensor | None) -> np.ndarray | None:
    """Host numpy copy: float32 stays float32, bfloat16 becomes its uint16 bits."""
    if t is None:
        return None
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def oracle_dtype(t: torch.Tensor) -> int:
    return O.DT_BF16 if t.dtype == torch.bfloat16 else O.DT_F32


def layer_weights(inp: dict, experts=None) -> O.LayerWeights:
    """Oracle weights from the generator's tensors; only `experts` (iterable of
    ids, default all) of the routed banks are copied to the host."""
    E = inp["W_gu"].shape[0]
    sel = set(range(E)) if experts is None else set(int(e) for e in experts)
    gu = [host(inp["W_gu"][e]) if e in sel else None for e in range(E)]
    dn = [host(inp["W_d"][e]) if e in sel else None for e in range(E)]
    return O.LayerWeights(host(inp.get("W_dn")), host(inp.get("norm_g")), host(inp["W_r"]),
                          host(inp.get("b_r")), gu, dn, host(inp.get("W_up")),
                          host(inp["W_gu_s"]), host(inp["W_d_s"]))


def dims(cfg, T=None) -> O.Dims:
    dt = O.DT_BF16 if cfg.dtype == "bf16" else O.DT_F32
    return O.dims(T=cfg.T if T is None else T, D=cfg.D, L=cfg.L, E=cfg.E, k=cfg.k, H=cfg.H,
                  n_shared=cfg.n_shared, Hs=cfg.Hs, dtype=dt, eps=cfg.eps)


def route_tokens(cfg, inp: dict, tok, x_host=None) -> dict:
    """Oracle router for tokens `tok` (the weights it needs are small)."""
    W = layer_weights(inp, experts=[])
    x = host(inp["x"]) if x_host is None else x_host
    return O.route_tokens(dims(cfg), W, x, np.asarray(tok, np.int32))


def layer_tokens(cfg, inp: dict, tok, keep=None, x_host=None) -> dict:
    """Oracle layer output for tokens `tok`, with the oracle's own routing;
    keep [n, k] optionally marks capacity drops.  Copies to the host only the
    expert banks those tokens use."""
    x = host(inp["x"]) if x_host is None else x_host
    tok = np.asarray(tok, np.int32)
    r = O.route_tokens(dims(cfg), layer_weights(inp, experts=[]), x, tok)
    W = layer_weights(inp, experts=np.unique(r["ids"]))
    y, c = O.output_tokens(dims(cfg), W, x, tok, r["ids"], r["w"], keep=keep, want_c=True)
    r.update(y=y, c=c)
    return r

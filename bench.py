"""Benchmark of the routed MoE layer forward on one MI355X.

One step = one moe_layer_fwd over a batch of seeded synthetic inputs already in
HBM: down-projection, RMSNorm + router + top-k, grouping, gate/up + SwiGLU and
down grouped GEMMs, ordered combine, shared experts and the output projection.
Prints one JSON line.  Default workload: the 535B-A23B-shaped layer (8,192
tokens, width 6,144, latent 3,072, 384 experts top-8, two shared experts).
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

DEFAULT_WORKLOAD = "marin535b_bf16_T8192_D6144_L3072_E384_k8"
PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run one 1 GiB device copy (a kernel of known "
                         "traffic, to scale the FETCH_SIZE / WRITE_SIZE counters) and report "
                         "its bandwidth")
    return ap.parse_args()


class HipEvents:
    """hipEvent_t handles for the library's per-stage timing hook."""

    def __init__(self):
        self.hip = C.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            h = C.c_void_p()
            assert self.hip.hipEventCreate(C.byref(h)) == 0
            evs.append(h.value)
        return evs

    def elapsed_ms(self, a, b) -> float:
        ms = C.c_float()
        assert self.hip.hipEventElapsedTime(C.byref(ms), C.c_void_p(a), C.c_void_p(b)) == 0
        return ms.value


def grouped_gemm1_bytes(cfg, counts) -> int:
    """Algorithmic HBM bytes of the gate/up + SwiGLU grouped GEMM: the weights of
    every expert that received a row, each routed row of the expert input once,
    each hidden row written once."""
    es = 2 if cfg.dtype == "bf16" else 4
    active = int((counts > 0).sum())
    rows = int(counts.sum())
    return active * 2 * cfg.H * cfg.d_e * es + rows * cfg.d_e * es + rows * cfg.H * es


def cpu_baseline(cfg, inp, target_s: float) -> dict:
    """The oracle as it stands, on a bounded sample of the same workload's tokens."""
    import numpy as np

    from oracle import oracle as O
    from oracle import torch_bridge as TB

    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    x_host = TB.host(inp["x"])
    base = TB.layer_weights(inp, experts=[])        # dense weights, copied once
    gu = [None] * cfg.E
    dn = [None] * cfg.E

    def weights(experts):
        for e in experts:
            if gu[e] is None:
                gu[e] = TB.host(inp["W_gu"][e])
                dn[e] = TB.host(inp["W_d"][e])
        return O.LayerWeights(base.W_dn, base.norm_g, base.W_r, base.b_r, gu, dn, base.W_up,
                              base.W_gu_s, base.W_d_s)

    rng = np.random.default_rng(0)
    n = 8
    spent = 0.0
    done = 0
    while spent < target_s and done < cfg.T:
        tok = np.sort(rng.choice(cfg.T, size=n, replace=False)).astype(np.int32)
        r = O.route_tokens(TB.dims(cfg), base, x_host, tok)
        W = weights(np.unique(r["ids"]))
        t0 = time.perf_counter()
        r = O.route_tokens(TB.dims(cfg), W, x_host, tok)
        O.output_tokens(TB.dims(cfg), W, x_host, tok, r["ids"], r["w"])
        dt = time.perf_counter() - t0
        spent += dt
        done += n
        n = max(8, int(n * min(4.0, max(1.0, (target_s - spent) / max(dt, 1e-3)))))
        n = min(n, 256)
    return {"value": done / spent, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} random tokens of the same workload (seed 0), full layer per token "
                      f"(routing, experts, combine, up-projection, shared experts) in double "
                      f"precision; host copies of weights not timed"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for "
              f"--gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import mixture_experts_transformer_amd as M
    from moe_synth import by_name, gen_layer

    cfg = by_name(args.workload)
    dev = torch.device("cuda:0")
    inp = gen_layer(cfg, dev)
    desc = M.layer_desc(cfg.T, cfg.D, cfg.L, cfg.E, cfg.k, cfg.H, cfg.n_shared, cfg.Hs,
                        cfg.dtype, cfg.eps)
    ws = torch.empty(M.moe_layer_workspace_size(desc), dtype=torch.uint8, device=dev)
    y = torch.empty_like(inp["x"])
    counts = torch.empty(cfg.E, dtype=torch.int32, device=dev)
    n_dropped = torch.empty(1, dtype=torch.int64, device=dev)
    aux = dict(counts=counts, n_dropped=n_dropped)

    for _ in range(args.warmup):
        M.moe_layer_fwd(desc, inp, inp["x"], y=y, aux=aux, ws=ws)
    torch.cuda.synchronize()

    hip = HipEvents()
    evs = [hip.create(M.MOE_EV_COUNT) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        M.moe_layer_fwd(desc, inp, inp["x"], y=y, aux=aux, ws=ws, events=evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    stage_ms = {n: 0.0 for n in M.EV_NAMES[1:]}
    for s in range(args.steps):
        for i in range(1, M.MOE_EV_COUNT):
            stage_ms[M.EV_NAMES[i]] += hip.elapsed_ms(evs[s][i - 1], evs[s][i]) / args.steps
    gpu_ms = sum(hip.elapsed_ms(evs[s][0], evs[s][-1]) for s in range(args.steps)) / args.steps

    cnt = counts.cpu().numpy().astype(np.int64)
    kept = int(cnt.sum()) - int(n_dropped.item())
    ms = wall * 1e3 / args.steps
    flops = cfg.flops(kept)
    tflops = flops / (ms * 1e-3) / 1e12
    g1_bytes = grouped_gemm1_bytes(cfg, cnt)
    g1_ms = stage_ms["gemm1"]
    g1_flops = 2 * kept * cfg.d_e * 2 * cfg.H
    achieved = g1_bytes / (g1_ms * 1e-3) / 1e9
    line = {
        "metric": "MoE layer fwd TFLOP/s + tokens/s, % of bf16 MFMA peak (1 MI355X)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s (model FLOPs)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded; x ~ N(0,1), weights ~ N(0,1/fan_in))",
        "config": {"workload": cfg.name, "tokens": cfg.T, "d_model": cfg.D, "latent": cfg.L,
                   "experts": cfg.E, "top_k": cfg.k, "expert_hidden": cfg.H,
                   "shared_experts": cfg.n_shared, "shared_hidden": cfg.Hs, "router": "f32",
                   "parallelism": "none (1 GPU)"},
        "tokens_per_s": round(cfg.T / (ms * 1e-3), 1),
        "pct_bf16_mfma_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "gpu_ms_per_step_events": round(gpu_ms, 4),
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "roofline": {"kernel": "grouped gate/up + SwiGLU GEMM", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "bytes_per_launch": g1_bytes, "avg_launch_ms": round(g1_ms, 4),
                     "mfma_frac": round(g1_flops / (g1_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
    }
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)                           # warm-up copy
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        line["copy_1GiB"] = {"ms": round(e0.elapsed_time(e1), 4),
                             "GB_per_s": round(2 * (1 << 30) / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the routed MoE layer forward on one MI355X.

One step = one pass of the whole path over a batch of seeded synthetic inputs
already resident in HBM.  For a layer workload that is one moe_layer_fwd:
down-projection, RMSNorm + router + top-k, grouping, gate/up + SwiGLU and down
grouped GEMMs, ordered combine, shared experts and the output projection.  For
the expert-parallel share (a receiver pool of rows with packed local expert
ids) it is moe_permute (with the row copy), moe_grouped_ffn and the unpermute
(moe_combine, k = 1).  Prints one JSON line.

Default workload: the 535B-A23B-shaped layer (8,192 tokens, width 6,144,
latent 3,072, 384 experts top-8, two shared experts).

Other modes, each printing its own JSON line:
  --backward  the expert MLP forward + backward (moe_grouped_ffn, moe_grouped_ffn_bwd)
              on an expert-MLP workload;
  --fp8       the expert MLP with E4M3 ragged dots and delayed scaling kept on the
              device (moe_quantize_e4m3, moe_grouped_ffn_e4m3, moe_fp8_scale_update), or,
              on a pool workload, the pool step with the E4M3 permute; each beside its
              bf16 counterpart.
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import os
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

DEFAULT_WORKLOAD = "marin535b_bf16_T8192_D6144_L3072_E384_k8"
EP_SHARE_WORKLOAD = "marin535b_ep_share_bf16_P65536_E6"
LONGCTX_WORKLOAD = "marin535b_longctx_bf16_T65536_D6144_L3072_E384_k8"
METRIC = "MoE layer fwd TFLOP/s + tokens/s, % of bf16 MFMA peak (1 MI355X)"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3, "fp8": 5000.0}   # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0                          # MI355X HBM3E
GEMM_TILE_M = 256                              # rows per grouped-GEMM tile
GEMM_SOURCES = ["gemm.hip", "common.h", "kernels.h"]
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles",
                               "grouped_gate_up_gemm_marin535b_T8192_hbm_traffic.txt")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-kernel-extras", action="store_true",
                    help="skip the stand-alone permute-with-copy measurement after the timed steps")
    ap.add_argument("--backward", action="store_true",
                    help="time the expert MLP forward + backward (moe_grouped_ffn, "
                         "moe_grouped_ffn_bwd) on an expert-MLP workload instead of the layer "
                         "forward; default workload: the pages' custom-VJP microbench shape")
    ap.add_argument("--fp8", action="store_true",
                    help="time the expert MLP forward with E4M3 ragged dots (moe_quantize_e4m3 "
                         "of the rows, moe_grouped_ffn_e4m3) beside the bf16 one on an expert-MLP "
                         "workload; default workload: the 535B expert shape")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run one 1 GiB device copy (a kernel of known "
                         "traffic, to scale the FETCH_SIZE / WRITE_SIZE counters) and a 1 GiB "
                         "fill, and report their bandwidths")
    return ap.parse_args()


class HipEvents:
    """hipEvent_t handles for the library's per-stage timing hook."""

    def __init__(self):
        self.hip = C.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]

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

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(C.c_void_p(e))


def gemm_source_hash() -> str:
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "mixture_experts_transformer_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch of the gate/up grouped GEMM from the committed counter
    summary, if it was taken on this workload with the current GEMM source."""
    try:
        with open(TRAFFIC_PROFILE) as f:
            text = f.read()
    except OSError:
        return None
    fields = dict(re.findall(r"^([a-z_0-9]+):\s*(\S+)\s*$", text, flags=re.M))
    if fields.get("workload") != workload or fields.get("gemm_source_sha256") != gemm_source_hash():
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def gemm_roofline(name, flops, nbytes, ms, dtype, traffic=None) -> dict:
    """Roofline entry for one kernel: bound by HBM or by the MFMA rate, whichever
    its arithmetic intensity puts it under."""
    peak_f = PEAK_TFLOPS[dtype]
    ridge = peak_f * 1e12 / (PEAK_HBM_GBS * 1e9)
    tflops = flops / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    if flops / nbytes < ridge:
        r = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(gbs / PEAK_HBM_GBS, 4)}
    else:
        r = {"bound": "mfma", "achieved": round(tflops, 1), "peak": peak_f, "unit": "TFLOP/s",
             "frac": round(tflops / peak_f, 4)}
    r.update({"traffic": traffic, "kernel": name, "algorithmic_bytes_per_launch": int(nbytes),
              "flops_per_launch": int(flops), "avg_launch_ms": round(ms, 4),
              "mfma_frac": round(tflops / peak_f, 4), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)})
    return r


def hbm_entry(nbytes, ms) -> dict:
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "bytes": int(nbytes), "GB_per_s": round(gbs, 1),
            "frac": round(gbs / PEAK_HBM_GBS, 4)}


def padded_rows(counts) -> int:
    return int(sum(-(-int(c) // GEMM_TILE_M) * GEMM_TILE_M for c in counts))


def time_ms(fn, reps=20) -> float:
    """Mean device time of fn() over reps back-to-back calls, torch events on the
    current stream.  One untimed call is queued before the first event so the
    GPU is busy while the host queues the timed calls: the figure is the
    kernels' time, not the binding's argument checks."""
    import torch
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


# ---------------------------------------------------------------- CPU oracle --
def cpu_model() -> str:
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_both(fn, target_s: float) -> dict:
    """The oracle timed with all its threads and with one; fn(target_s) runs one
    bounded sample and returns its figures."""
    from oracle import oracle as O

    full = fn(target_s)
    prev = O.set_threads(1)
    try:
        one = fn(target_s / 2)
    finally:
        O.set_threads(prev)
    full["single_thread"] = {"value": one["value"], "unit": one["unit"], "cores": 1,
                             "sample": one["sample"]}
    full["cpu_model"] = cpu_model()
    full["host_cpus"] = os.cpu_count()
    return full


def cpu_baseline_layer(cfg, inp, target_s: float) -> dict:
    """The oracle as it stands, on a bounded sample of the same workload's tokens."""
    import numpy as np

    from oracle import oracle as O
    from oracle import torch_bridge as TB

    threads = int(O.lib().moe_ref_max_threads())
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
        tok = np.sort(rng.choice(cfg.T, size=min(n, cfg.T), replace=False)).astype(np.int32)
        r = O.route_tokens(TB.dims(cfg), base, x_host, tok)
        W = weights(np.unique(r["ids"]))
        t0 = time.perf_counter()
        r = O.route_tokens(TB.dims(cfg), W, x_host, tok)
        O.output_tokens(TB.dims(cfg), W, x_host, tok, r["ids"], r["w"])
        dt = time.perf_counter() - t0
        spent += dt
        done += len(tok)
        n = max(8, int(n * min(4.0, max(1.0, (target_s - spent) / max(dt, 1e-3)))))
        n = min(n, 256)
    return {"value": round(done / spent, 2), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} random tokens of the same workload (seed 0), full layer per token "
                      f"(routing, experts, combine, up-projection, shared experts) in double "
                      f"precision; host copies of weights not timed"}


def cpu_baseline_pool(cfg, pool, target_s: float) -> dict:
    import numpy as np

    from oracle import oracle as O
    from oracle import torch_bridge as TB

    threads = int(O.lib().moe_ref_max_threads())
    ids = pool["ids"].cpu().numpy()
    valid = np.flatnonzero(ids >= 0)
    W_gu = [TB.host(pool["W_gu"][e]) for e in range(cfg.E)]
    W_d = [TB.host(pool["W_d"][e]) for e in range(cfg.E)]
    rng = np.random.default_rng(0)
    n, spent, done = 16, 0.0, 0
    while spent < target_s and done < len(valid):
        rows = np.sort(rng.choice(valid, size=min(n, len(valid)), replace=False))
        Xh = TB.host(pool["X"][rows])
        t0 = time.perf_counter()
        O.expert_rows(Xh, ids[rows], W_gu, W_d, cfg.H)
        dt = time.perf_counter() - t0
        spent += dt
        done += len(rows)
        n = min(1024, max(16, int(n * min(4.0, max(1.0, (target_s - spent) / max(dt, 1e-3))))))
    return {"value": round(done / spent, 2), "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} random valid pool rows (seed 0) through their local expert's "
                      f"SwiGLU FFN in double precision; host copies not timed"}


# ------------------------------------------------------------------ workloads --
def stats_ms(vals) -> dict:
    import numpy as np
    a = np.asarray(vals, np.float64)
    return {"mean": round(float(a.mean()), 4), "median": round(float(np.median(a)), 4),
            "min": round(float(a.min()), 4), "max": round(float(a.max()), 4)}


def layer_rooflines(cfg, kept, cnt, stage_ms, dtype):
    """Rooflines of the two grouped GEMMs of a layer step from their mean stage times."""
    es = 2 if dtype == "bf16" else 4
    de, H = cfg.d_e, cfg.H
    active = int((cnt > 0).sum())
    # gate/up + SwiGLU: every active expert's [2H, de] weights, each routed row of
    # the expert input read once, each hidden row written once.
    g1_bytes = active * 2 * H * de * es + kept * de * es + kept * H * es
    g1_flops = 2 * kept * de * 2 * H
    g2_bytes = active * de * H * es + kept * H * es + kept * de * es
    g2_flops = 2 * kept * H * de
    return (gemm_roofline("grouped gate/up + SwiGLU GEMM", g1_flops, g1_bytes, stage_ms["gemm1"],
                          dtype),
            gemm_roofline("grouped down GEMM", g2_flops, g2_bytes, stage_ms["gemm2"], dtype))


N_ROTATE = 3     # input/output copies used in turn (each x is 100 MB at the 535B layer)


def time_layer(M, desc, W, xs, ys, aux, ws, warmup, steps):
    """warmup + steps layer calls, the inputs and outputs taken in turn from xs/ys so
    that no step finds the previous one's x or y in the 256 MB last-level cache.
    Returns the wall time of the timed steps and each step's per-stage event times."""
    import torch

    def run(s, ev=None):
        M.moe_layer_fwd(desc, W, xs[s % len(xs)], y=ys[s % len(ys)], aux=aux, ws=ws, events=ev)

    for s in range(warmup):
        run(s)
    torch.cuda.synchronize()
    hip = HipEvents()
    evs = [hip.create(M.MOE_EV_COUNT) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        run(warmup + s, evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_stage = {n: [hip.elapsed_ms(evs[s][i - 1], evs[s][i]) for s in range(steps)]
                 for i, n in enumerate(M.EV_NAMES) if i > 0}
    per_step = [hip.elapsed_ms(evs[s][0], evs[s][-1]) for s in range(steps)]
    hip.destroy([e for ev in evs for e in ev])
    return wall, per_stage, per_step


def bench_layer(args, cfg, M, dev):
    import numpy as np
    import torch

    from moe_synth import gen_layer

    inp = gen_layer(cfg, dev)
    desc = M.layer_desc(cfg.T, cfg.D, cfg.L, cfg.E, cfg.k, cfg.H, cfg.n_shared, cfg.Hs,
                        cfg.dtype, cfg.eps)
    ws = torch.empty(M.moe_layer_workspace_size(desc), dtype=torch.uint8, device=dev)
    xs = [inp["x"]] + [inp["x"].clone() for _ in range(N_ROTATE - 1)]
    ys = [torch.empty_like(inp["x"]) for _ in range(N_ROTATE)]
    i32 = dict(dtype=torch.int32, device=dev)
    aux = dict(ids=torch.empty((cfg.T, cfg.k), **i32),
               w=torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev),
               counts=torch.empty(cfg.E, **i32),
               n_dropped=torch.empty(1, dtype=torch.int64, device=dev),
               slot_row=torch.empty(cfg.T * cfg.k, **i32))
    wall, per_stage, per_step = time_layer(M, desc, inp, xs, ys, aux, ws, args.warmup,
                                           args.steps)
    stage_ms = {n: float(np.mean(v)) for n, v in per_stage.items()}

    cnt = aux["counts"].cpu().numpy().astype(np.int64)
    kept = int(cnt.sum()) - int(aux["n_dropped"].item())
    ms = wall * 1e3 / args.steps
    flops = cfg.flops(kept)
    tflops = flops / (ms * 1e-3) / 1e12
    pad = padded_rows(cnt)
    hw_flops = cfg.flops(kept) + 2 * (pad - kept) * cfg.d_e * cfg.H * 3
    es = 2 if cfg.dtype == "bf16" else 4
    de, H, T, k = cfg.d_e, cfg.H, cfg.T, cfg.k
    active = int((cnt > 0).sum())
    g1, g2 = layer_rooflines(cfg, kept, cnt, stage_ms, cfg.dtype)
    g1["traffic"] = measured_traffic(cfg.name)
    # the dense GEMMs: down-projection (x W_dn^T), the shared experts' gate/up +
    # SwiGLU, and the K-concatenated output GEMM [c | h_s] [W_up | W2_s]^T
    dense = {}
    if cfg.L > 0:
        dense["down_projection"] = gemm_roofline(
            "down-projection GEMM", 2 * T * cfg.D * cfg.L,
            (T * cfg.D + cfg.L * cfg.D) * es + T * cfg.L * 4, stage_ms["downproj"], cfg.dtype)
    if cfg.n_shared > 0:
        sh = cfg.n_shared * cfg.Hs
        dense["shared_gate_up"] = gemm_roofline(
            "shared experts' gate/up + SwiGLU GEMM", 2 * T * cfg.D * 2 * sh,
            (T * cfg.D + 2 * sh * cfg.D + T * sh) * es, stage_ms["shared"], cfg.dtype)
        kk = (cfg.L if cfg.L > 0 else 0) + sh
        dense["output"] = gemm_roofline(
            "output GEMM [c | h_s] [W_up | W2_s]^T", 2 * T * kk * cfg.D,
            (T * kk + cfg.D * kk + T * cfg.D) * es, stage_ms["output"], cfg.dtype)
    line = {
        "metric": METRIC,
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
        "config": {"workload": cfg.name, "tokens": T, "d_model": cfg.D, "latent": cfg.L,
                   "experts": cfg.E, "top_k": k, "expert_hidden": H,
                   "shared_experts": cfg.n_shared, "shared_hidden": cfg.Hs, "router": "f32",
                   "parallelism": "none (1 GPU)"},
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "pct_peak_mfma": round(100 * tflops / PEAK_TFLOPS[cfg.dtype], 2),
        "hw_tflops": round(hw_flops / (ms * 1e-3) / 1e12, 2),
        "timing": {"inputs_rotated": N_ROTATE, "step_ms_events": stats_ms(per_step)},
        "gpu_ms_per_step_events": round(float(np.mean(per_step)), 4),
        "stage_ms": {n: round(v, 4) for n, v in stage_ms.items()},
        "stage_ms_median": {n: round(float(np.median(v)), 4) for n, v in per_stage.items()},
        "roofline": g1,
        "grouped_down_gemm": g2,
        "dense_gemms": dense,
        "routed_rows": {"kept": kept, "padded_to_tiles": pad, "active_experts": active,
                        "max_per_expert": int(cnt.max()), "min_per_expert": int(cnt.min())},
    }
    # ordered combine: every kept Y row read once, slot_row and weights, c written once
    comb_bytes = kept * de * es + T * k * 8 + T * de * es
    # The combine timed alone, back to back on the layer's own expert rows (Y, read
    # from the workspace) and routing: its kernel time.  The in-layer figure also
    # holds the gap between the stage events and the kernel.
    lay = M.moe_layer_workspace_layout(desc)
    y_rows = ws[lay["Y"]:lay["Y"] + T * k * de * es].view(inp["x"].dtype).view(T * k, de)
    c_out = torch.empty((T, de), dtype=inp["x"].dtype, device=dev)
    cms = time_ms(lambda: M.moe_combine(y_rows, aux["slot_row"], aux["w"], T, k, out=c_out))
    hbm = {"combine": hbm_entry(comb_bytes, cms),
           "combine_in_layer": hbm_entry(comb_bytes, stage_ms["combine"])}
    if not args.no_kernel_extras:
        # The layer's grouping copies no rows (the expert GEMM gathers them); the
        # stand-alone moe_permute with the row copy is timed here at the same shape.
        src = torch.randn((T, de), device=dev).to(inp["x"].dtype)
        dst = torch.empty((T * k, de), dtype=src.dtype, device=dev)
        pws = torch.empty(M.moe_permute_workspace_size(T * k, cfg.E), dtype=torch.uint8,
                          device=dev)
        pout = dict(slot_row=torch.empty(T * k, **i32), row_src=torch.empty(T * k, **i32),
                    counts=torch.empty(cfg.E, **i32), offsets=torch.empty(cfg.E + 1, **i32),
                    n_dropped=torch.empty(1, dtype=torch.int64, device=dev))
        pms = time_ms(lambda: M.moe_permute(aux["ids"], cfg.E, src=src, src_div=k, dst=dst,
                                            ws=pws, out=pout))
        perm_bytes = T * de * es + T * k * de * es + T * k * 4 * 4
        hbm["permute_with_row_copy"] = hbm_entry(perm_bytes, pms)
        hbm["permute_grouping_only"] = {"ms": round(stage_ms["permute"], 4),
                                        "bytes": T * k * 4 * 4}
        # the sender's half of an expert-parallel dispatch to 64 peers (6 experts each)
        # with the pages' 1.10 sender capacity, on the same rows
        if cfg.E % 64 == 0:
            cap = -(-11 * T * k // (10 * 64))
            sent = torch.empty((T * k, de), dtype=src.dtype, device=dev)
            sexp = torch.empty(T * k, **i32)
            dws = torch.empty(M.moe_dispatch_pack_workspace_size(T * k, 64), dtype=torch.uint8,
                              device=dev)
            dout = dict(slot_row=torch.empty(T * k, **i32), row_src=torch.empty(T * k, **i32),
                        counts=torch.empty(64, **i32), offsets=torch.empty(65, **i32),
                        n_dropped=torch.empty(1, dtype=torch.int64, device=dev))
            dms = time_ms(lambda: M.moe_dispatch_pack(aux["ids"], cfg.E, 64, src, capacity=cap,
                                                      send_rows=sent, send_expert=sexp, ws=dws,
                                                      out=dout))
            kept = int(dout["offsets"][64].item())
            hbm["dispatch_pack_64_peers"] = hbm_entry(T * de * es + kept * (de * es + 4)
                                                      + T * k * 4 * 5, dms)
            hbm["dispatch_pack_64_peers"]["sender_drops"] = int(dout["n_dropped"].item())
            # the same with the rows sent as E4M3 codes (the fp8 wire format)
            sent8 = torch.empty((T * k, de), dtype=torch.uint8, device=dev)
            s8 = torch.ones(1, dtype=torch.float32, device=dev)
            a8 = torch.zeros(1, dtype=torch.float32, device=dev)
            d8ms = time_ms(lambda: M.moe_dispatch_pack_e4m3(aux["ids"], cfg.E, 64, src,
                                                            capacity=cap, scale=s8, amax=a8,
                                                            send_rows=sent8, send_expert=sexp,
                                                            ws=dws))
            hbm["dispatch_pack_e4m3_64_peers"] = hbm_entry(T * de * es + kept * (de + 4)
                                                           + T * k * 4 * 5, d8ms)
            del sent, sent8, sexp, dws
        del src, dst
    line["hbm_kernels"] = hbm
    return line, inp


def bench_longctx_leg(args, M, dev, inp3):
    """The long-context batch's layer (65,536 tokens, 10% of the experts biased to
    about 5x the mean load) on the 535B layer's weights, so that no second 22 GB
    bank is drawn: the same shapes and distributions as that workload, with its own
    tokens and router bias.  Times the layer and reports its grouped GEMMs against
    the MFMA peak (at 524,288 routed rows they are MFMA-bound)."""
    import numpy as np
    import torch

    from moe_synth import by_name
    from moe_synth.gen import gen_tokens, hot_experts, router_bias

    cfg = by_name(LONGCTX_WORKLOAD)
    x = gen_tokens(cfg, dev)
    W = dict(inp3)
    W["b_r"] = router_bias(cfg, dev)
    desc = M.layer_desc(cfg.T, cfg.D, cfg.L, cfg.E, cfg.k, cfg.H, cfg.n_shared, cfg.Hs,
                        cfg.dtype, cfg.eps)
    ws = torch.empty(M.moe_layer_workspace_size(desc), dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    i32 = dict(dtype=torch.int32, device=dev)
    aux = dict(counts=torch.empty(cfg.E, **i32),
               n_dropped=torch.empty(1, dtype=torch.int64, device=dev))
    steps = max(5, args.steps // 5)
    wall, per_stage, per_step = time_layer(M, desc, W, [x], [y], aux, ws, 2, steps)
    stage_ms = {n: float(np.mean(v)) for n, v in per_stage.items()}
    cnt = aux["counts"].cpu().numpy().astype(np.int64)
    kept = int(cnt.sum()) - int(aux["n_dropped"].item())
    ms = wall * 1e3 / steps
    g1, g2 = layer_rooflines(cfg, kept, cnt, stage_ms, cfg.dtype)
    hot = hot_experts(cfg)
    out = {"workload": cfg.name, "weights": "the 535B layer's banks (same shapes and "
                                            "distributions), this workload's tokens and bias",
           "steps": steps, "ms_per_step": round(ms, 3),
           "tflops": round(cfg.flops(kept) / (ms * 1e-3) / 1e12, 1),
           "tokens_per_s": round(cfg.T / (ms * 1e-3), 1),
           "step_ms_events": stats_ms(per_step),
           "stage_ms": {n: round(v, 4) for n, v in stage_ms.items()},
           "hot_expert_load": round(float(cnt[hot].mean() / cnt.mean()), 2),
           "rows_per_expert": {"max": int(cnt.max()), "min": int(cnt.min())},
           "gate_up_gemm": g1, "down_gemm": g2}
    del ws, x, y
    torch.cuda.empty_cache()
    return out


def bench_pool_leg(args, M, dev):
    """The expert-parallel share's step (the receiver pool), timed after the headline."""
    from moe_synth import by_name

    cfg = by_name(EP_SHARE_WORKLOAD)
    a = argparse.Namespace(**vars(args))
    line, pool = bench_pool(a, cfg, M, dev)
    out = {k: line[k] for k in ["ms_per_step", "value", "rows_per_s", "stage_ms",
                                "stage_ms_median", "step_ms_events"] if k in line}
    out["tflops"] = out.pop("value")
    out.update(workload=cfg.name, steps=a.steps, grouped_ffn=line["roofline"],
               hbm_kernels=line["hbm_kernels"])
    del pool
    return out


def bench_pool(args, cfg, M, dev):
    import numpy as np
    import torch

    from moe_synth import gen_pool

    pool = gen_pool(cfg, dev)
    P, L, H, E = cfg.P, cfg.L, cfg.H, cfg.E
    ids = pool["ids"]
    i32 = dict(dtype=torch.int32, device=dev)
    X_perm = torch.empty((P, L), dtype=torch.bfloat16, device=dev)
    Y_perm = torch.empty_like(X_perm)
    out = torch.full((P, L), 0.0, dtype=torch.bfloat16, device=dev)
    pws = torch.empty(M.moe_permute_workspace_size(P, E), dtype=torch.uint8, device=dev)
    fws = torch.empty(M.moe_grouped_ffn_workspace_size(E, P, H, torch.bfloat16),
                      dtype=torch.uint8, device=dev)
    g = dict(slot_row=torch.empty(P, **i32), row_src=torch.empty(P, **i32),
             counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
             n_dropped=torch.empty(1, dtype=torch.int64, device=dev))

    def step(ev=None):
        if ev:
            ev[0].record()
        M.moe_permute(ids, E, src=pool["X"], src_div=1, dst=X_perm, R_phys=P, ws=pws, out=g)
        if ev:
            ev[1].record()
        M.moe_grouped_ffn(X_perm, g["offsets"], pool["W_gu"], pool["W_d"], Y=Y_perm, ws=fws)
        if ev:
            ev[2].record()
        M.moe_combine(Y_perm, g["slot_row"], None, P, 1, out=out,
                      flags=M.MOE_COMBINE_KEEP_UNROUTED)
        if ev:
            ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    names = ["permute", "grouped_ffn", "unpermute"]
    per_stage = {n: [e[i].elapsed_time(e[i + 1]) for e in evs] for i, n in enumerate(names)}
    stage_ms = {n: float(np.mean(v)) for n, v in per_stage.items()}
    per_step = [e[0].elapsed_time(e[3]) for e in evs]
    cnt = g["counts"].cpu().numpy().astype(np.int64)
    valid = int(cnt.sum())
    ms = wall * 1e3 / args.steps
    flops = cfg.flops(valid)
    tflops = flops / (ms * 1e-3) / 1e12
    es = 2
    ffn_bytes = E * 3 * H * L * es + valid * (L + H + H + L) * es
    perm_bytes = P * 4 + valid * L * es * 2 + valid * 4 * 2 + P * 4
    unperm_bytes = valid * L * es * 2 + P * 4
    line = {
        "metric": METRIC,
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
        "data": "synthetic (seeded receiver pool; rows ~ N(0,1) at unit RMS, Zipf(1) local "
                "expert ids, weights ~ N(0,1/fan_in))",
        "config": {"workload": cfg.name, "pool_rows": P, "valid_rows": valid, "latent": L,
                   "local_experts": E, "expert_hidden": H, "parallelism": "none (1 GPU)"},
        "rows_per_s": round(valid / (ms * 1e-3), 1),
        "pct_peak_mfma": round(100 * tflops / PEAK_TFLOPS[cfg.dtype], 2),
        "step_ms_events": stats_ms(per_step),
        "stage_ms": {n: round(v, 4) for n, v in stage_ms.items()},
        "stage_ms_median": {n: round(float(np.median(v)), 4) for n, v in per_stage.items()},
        "roofline": gemm_roofline("grouped FFN (gate/up + SwiGLU and down GEMMs)", flops,
                                  ffn_bytes, stage_ms["grouped_ffn"], cfg.dtype),
        "hbm_kernels": {"permute_with_row_copy": hbm_entry(perm_bytes, stage_ms["permute"]),
                        "unpermute": hbm_entry(unperm_bytes, stage_ms["unpermute"])},
        "routed_rows": {"valid": valid, "padded_to_tiles": padded_rows(cnt),
                        "per_expert": cnt.tolist()},
    }
    return line, pool


BWD_METRIC = "expert MLP fwd+bwd TFLOP/s (model FLOPs), % of bf16 MFMA peak (1 MI355X)"
BWD_DEFAULT = "grug_vjp_bf16_T4096_D1024_H2048_E64_k4"


def bench_backward(args, cfg, M, dev):
    """Forward (moe_grouped_ffn) then backward (moe_grouped_ffn_bwd) of the gated
    expert MLP over rows grouped by expert; weight gradients in float32."""
    import numpy as np
    import torch

    from moe_synth import gen_expert_mlp

    data = gen_expert_mlp(cfg, dev)
    X, dY, W_gu, W_d, off = data["X"], data["dY"], data["W_gu"], data["W_d"], data["offsets"]
    R, d, H, E = cfg.R, cfg.d, cfg.H, cfg.E
    Y = torch.empty_like(X)
    dX = torch.empty_like(X)
    dWgu = torch.empty(W_gu.shape, dtype=torch.float32, device=dev)
    dWd = torch.empty(W_d.shape, dtype=torch.float32, device=dev)
    fws = torch.empty(M.moe_grouped_ffn_workspace_size(E, R, H, X.dtype), dtype=torch.uint8,
                      device=dev)
    bws = torch.empty(M.moe_grouped_ffn_bwd_workspace_size(E, R, H, X.dtype), dtype=torch.uint8,
                      device=dev)

    def step(ev=None):
        if ev:
            ev[0].record()
        M.moe_grouped_ffn(X, off, W_gu, W_d, Y=Y, ws=fws)
        if ev:
            ev[1].record()
        M.moe_grouped_ffn_bwd(X, dY, off, W_gu, W_d, dX=dX, dW_gu=dWgu, dW_d=dWd, ws=bws)
        if ev:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / args.steps
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    ff, fb = cfg.flops_fwd(), cfg.flops_bwd()
    tflops = (ff + fb) / (ms * 1e-3) / 1e12
    es = 2 if cfg.dtype == "bf16" else 4
    # The two VJP GEMMs of the largest reduction, each timed alone: the input
    # gradient dX = [dg | du] W_gu[e] and the weight gradient dW_gu[e] = [dg | du]^T X
    dgu = torch.randn((R, 2 * H), device=dev).to(X.dtype)
    dlhs_ms = time_ms(lambda: M.moe_ragged_dot_dlhs(dgu, off, W_gu, dX=dX))
    drhs_ms = time_ms(lambda: M.moe_ragged_dot_drhs(X, dgu, off, dW=dWgu))
    mm = 2 * R * 2 * H * d
    dlhs_bytes = E * 2 * H * d * es + R * (2 * H + d) * es
    drhs_bytes = R * (2 * H + d) * es + E * 2 * H * d * 4
    del dgu
    line = {
        "metric": BWD_METRIC,
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
        "data": "synthetic (seeded; rows and output gradients ~ N(0,1), weights ~ "
                "N(0,1/fan_in), uniform top-k routing or Zipf(1) for a pool)",
        "config": {"workload": cfg.name, "tokens": cfg.T, "top_k": cfg.k, "rows": R, "width": d,
                   "expert_hidden": H, "experts": E, "weight_grad_dtype": "f32",
                   "parallelism": "none (1 GPU)"},
        "pct_peak_mfma": round(100 * tflops / PEAK_TFLOPS[cfg.dtype], 2),
        "stage_ms": {"forward": round(fwd_ms, 4), "backward": round(bwd_ms, 4)},
        "fwd_tflops": round(ff / (fwd_ms * 1e-3) / 1e12, 2),
        "bwd_tflops": round(fb / (bwd_ms * 1e-3) / 1e12, 2),
        "roofline": gemm_roofline("ragged-dot weight gradient dW_gu (moe_ragged_dot_drhs)", mm,
                                  drhs_bytes, drhs_ms, cfg.dtype),
        "vjp_kernels": {
            "dlhs_dX": gemm_roofline("ragged-dot input gradient dX (moe_ragged_dot_dlhs)", mm,
                                     dlhs_bytes, dlhs_ms, cfg.dtype),
            "drhs_dW_gu": gemm_roofline("ragged-dot weight gradient dW_gu", mm, drhs_bytes,
                                        drhs_ms, cfg.dtype),
        },
        "routed_rows": {"per_expert_min": int(data["counts"].min()),
                        "per_expert_max": int(data["counts"].max())},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_backward(cfg, data, args.cpu_seconds)
    return line


def cpu_baseline_backward(cfg, data, target_s: float) -> dict:
    """The oracle's forward and backward of the expert MLP on a bounded random sample:
    rows of four experts (the weight gradients of those experts over the sampled
    rows)."""
    import numpy as np

    from oracle import oracle as O
    from oracle import torch_bridge as TB

    counts = data["counts"]
    off = np.concatenate([[0], np.cumsum(counts)])
    rng = np.random.default_rng(0)
    experts = np.sort(rng.choice(np.flatnonzero(counts), min(4, int(np.count_nonzero(counts))),
                                 replace=False))
    W_gu = TB.host(data["W_gu"][experts.tolist()])
    W_d = TB.host(data["W_d"][experts.tolist()])

    def run(per_expert):
        take = [np.sort(rng.choice(counts[e], min(per_expert, counts[e]), replace=False))
                + off[e] for e in experts]
        rows = np.concatenate(take).astype(np.int64)
        sub_counts = np.array([len(t) for t in take])
        sub_off = np.concatenate([[0], np.cumsum(sub_counts)]).astype(np.int32)
        X = TB.host(data["X"][rows])
        dY = TB.host(data["dY"][rows])
        ex = np.repeat(np.arange(len(experts), dtype=np.int32), sub_counts)
        t0 = time.perf_counter()
        O.expert_rows(X, ex, list(W_gu), list(W_d), cfg.H)
        O.expert_rows_bwd(X, dY, sub_off, W_gu, W_d)
        return time.perf_counter() - t0, int(len(rows))

    t, n = run(2)
    per = max(2, int(2 * target_s / max(t, 1e-3)))
    t, n = run(per)
    return {"value": round(n / t, 2), "unit": "rows/s (forward + backward)",
            "cores": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)),
            "kind": "oracle",
            "sample": f"{n} rows of experts {experts.tolist()} (up to {per} random rows each, "
                      f"seed 0) of the same workload through the oracle's expert forward and "
                      f"backward in double precision"}


FP8_METRIC = ("expert MLP fwd TFLOP/s with E4M3 ragged dots (model FLOPs), % of fp8 MFMA peak "
              "(1 MI355X)")
FP8_DEFAULT = "marin535b_experts_bf16_T8192_L3072_H3072_E384_k8"


def bench_fp8(args, cfg, M, dev):
    """The expert MLP forward on E4M3 operands with delayed scaling kept on the device:
    per step, the rows are quantised with the scale their amax history gives
    (moe_quantize_e4m3, recording this step's amax), moe_grouped_ffn_e4m3 runs the
    gate/up ragged dot, the activation quantised to E4M3 with h's history scale and the
    down ragged dot, and moe_fp8_scale_update rolls both histories (16 steps) into the
    next step's scales.  No host round trip.  The weights are quantised once per
    optimizer step (timed separately, not part of the step).  The bf16 expert MLP
    (moe_grouped_ffn) is timed on the same data."""
    import numpy as np
    import torch

    from moe_synth import gen_expert_mlp

    data = gen_expert_mlp(cfg, dev)
    del data["dY"]
    X, W_gu, W_d, off = data["X"], data["W_gu"], data["W_d"], data["offsets"]
    R, d, H, E = cfg.R, cfg.d, cfg.H, cfg.E
    u8 = dict(dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    Xq, Wguq, Wdq = torch.empty(X.shape, **u8), torch.empty(W_gu.shape, **u8), \
        torch.empty(W_d.shape, **u8)
    a_x, a_h, a_gu, a_d = (torch.zeros(1, **f32) for _ in range(4))
    HIST = 16
    hist_x, hist_h = torch.zeros(HIST, **f32), torch.zeros(HIST, **f32)
    hist_gu, hist_d = torch.zeros(1, **f32), torch.zeros(1, **f32)
    s_x, s_h, s_gu, s_d = (torch.ones(1, **f32) for _ in range(4))

    def quantize_weights():
        # once per optimizer step, delayed as well: quantised with the scale the last
        # step's amax gave (a history of one), recording this step's amax
        M.moe_quantize_e4m3(W_gu, s_gu, q=Wguq, amax=a_gu)
        M.moe_quantize_e4m3(W_d, s_d, q=Wdq, amax=a_d)
        M.moe_fp8_scale_update(hist_gu, a_gu, s_gu)
        M.moe_fp8_scale_update(hist_d, a_d, s_d)

    quantize_weights()                            # the first pass only records the amax
    wq_ms = time_ms(quantize_weights, reps=2)     # the weights stay as they are, so the
    quantize_weights()                            # codes match the scales in s_gu, s_d
    Y = torch.empty_like(X)
    ws = torch.empty(M.moe_grouped_ffn_e4m3_workspace_size(E, R, H), **u8)

    def step(ev=None):
        if ev:
            ev[0].record()
        M.moe_quantize_e4m3(X, s_x, q=Xq, amax=a_x)
        if ev:
            ev[1].record()
        M.moe_grouped_ffn_e4m3(Xq, off, Wguq, Wdq, s_x, s_gu, s_h, s_d, Y=Y, amax_h=a_h, ws=ws)
        if ev:
            ev[2].record()
        M.moe_fp8_scale_update(hist_x, a_x, s_x)
        M.moe_fp8_scale_update(hist_h, a_h, s_h)
        if ev:
            ev[3].record()

    # warm-up: the first step runs with unit scales and fills the histories
    for _ in range(max(2, args.warmup)):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / args.steps
    q_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    mlp_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    su_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps
    ff = cfg.flops_fwd()
    tflops = ff / (ms * 1e-3) / 1e12
    scale = {"x": float(s_x.item()), "h": float(s_h.item())}
    s_gu_v, s_d_v = float(s_gu.item()), float(s_d.item())
    # h's last amax against the largest its history held before it (1 = no saturation)
    hh = hist_h.cpu().numpy()
    h_over = float(hh[0] / max(hh[1:].max(), 1e-30))
    # the gate/up ragged dot alone in E4M3 and in bf16, and the bf16 expert MLP
    gu8 = torch.empty((R, 2 * H), dtype=torch.bfloat16, device=dev)
    g8_ms = time_ms(lambda: M.moe_ragged_dot_e4m3(Xq, off, Wguq, s_x, s_gu, Z=gu8))
    g16_ms = time_ms(lambda: M.moe_ragged_dot(X, off, W_gu, Z=gu8))
    del gu8
    fws = torch.empty(M.moe_grouped_ffn_workspace_size(E, R, H, X.dtype), **u8)
    Y16 = torch.empty_like(X)
    bf16_ms = time_ms(lambda: M.moe_grouped_ffn(X, off, W_gu, W_d, Y=Y16, ws=fws))
    rel = float((Y.float() - Y16.float()).pow(2).mean().sqrt() / Y16.float().pow(2).mean().sqrt())
    del fws, Y16
    mm = 2 * R * 2 * H * d
    g8_bytes = E * 2 * H * d + R * d + R * 2 * H * 2
    g16_bytes = E * 2 * H * d * 2 + R * d * 2 + R * 2 * H * 2
    line = {
        "metric": FP8_METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s (model FLOPs)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic (seeded; rows ~ N(0,1), weights ~ N(0,1/fan_in) in bf16, uniform "
                "top-k routing), quantised to E4M3 with per-tensor scales",
        "config": {"workload": cfg.name, "tokens": cfg.T, "top_k": cfg.k, "rows": R, "width": d,
                   "expert_hidden": H, "experts": E, "operands": "E4M3",
                   "intermediate": "[g | u] bf16", "output": "bf16",
                   "scaling": f"per tensor, delayed: amax history of {HIST} steps on the device",
                   "parallelism": "none (1 GPU)"},
        "pct_peak_mfma": round(100 * tflops / PEAK_TFLOPS["fp8"], 2),
        "stage_ms": {"quantize_rows": round(q_ms, 4), "expert_mlp_e4m3": round(mlp_ms, 4),
                     "scale_updates": round(su_ms, 4)},
        "weight_quantization_ms": round(wq_ms, 4),
        "bf16_expert_mlp_ms": round(bf16_ms, 4),
        "speedup_vs_bf16": round(bf16_ms / ms, 3),
        "rel_rms_diff_vs_bf16": round(rel, 5),
        "h_amax_vs_history": round(h_over, 4),
        "roofline": gemm_roofline("E4M3 gate/up ragged dot (moe_ragged_dot_e4m3)", mm, g8_bytes,
                                  g8_ms, "fp8"),
        "gate_up_ragged_dot": {
            "e4m3": gemm_roofline("E4M3 gate/up ragged dot", mm, g8_bytes, g8_ms, "fp8"),
            "bf16": gemm_roofline("bf16 gate/up ragged dot (moe_ragged_dot)", mm, g16_bytes,
                                  g16_ms, "bf16"),
            "speedup": round(g16_ms / g8_ms, 3),
        },
        "routed_rows": {"per_expert_min": int(data["counts"].min()),
                        "per_expert_max": int(data["counts"].max())},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_fp8(cfg, data, scale, s_gu_v, s_d_v, args.cpu_seconds)
    return line


def cpu_baseline_fp8(cfg, data, scale, s_gu, s_d, target_s: float) -> dict:
    """The oracle's quantisation of sampled rows and its E4M3 expert MLP over them, for
    the rows of two experts (whose weights the oracle quantises first, untimed, as the
    GPU path quantises weights once per optimizer step)."""
    import numpy as np

    from oracle import oracle as O
    from oracle import torch_bridge as TB

    counts = data["counts"]
    off = np.concatenate([[0], np.cumsum(counts)])
    rng = np.random.default_rng(0)
    experts = np.sort(rng.choice(np.flatnonzero(counts), min(2, int(np.count_nonzero(counts))),
                                 replace=False))
    inv = lambda v: float(np.float32(1.0) / np.float32(v))
    wgu, _ = O.quantize_e4m3(TB.host(data["W_gu"][experts.tolist()]), inv(s_gu))
    wd, _ = O.quantize_e4m3(TB.host(data["W_d"][experts.tolist()]), inv(s_d))

    def run(per_expert):
        take = [np.sort(rng.choice(counts[e], min(per_expert, counts[e]), replace=False))
                + off[e] for e in experts]
        rows = np.concatenate(take).astype(np.int64)
        sub_off = np.concatenate([[0], np.cumsum([len(t) for t in take])]).astype(np.int32)
        X = TB.host(data["X"][rows])
        t0 = time.perf_counter()
        xq, _ = O.quantize_e4m3(X, inv(scale["x"]))
        O.expert_mlp_e4m3(xq, wgu, wd, sub_off, float(np.float32(scale["x"]) * np.float32(s_gu)),
                          inv(scale["h"]), float(np.float32(scale["h"]) * np.float32(s_d)))
        return time.perf_counter() - t0, int(len(rows))

    t, n = run(2)
    per = max(2, int(2 * target_s / max(t, 1e-3)))
    t, n = run(per)
    return {"value": round(n / t, 2), "unit": "rows/s (E4M3 expert MLP forward)",
            "cores": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)),
            "kind": "oracle",
            "sample": f"{n} rows of experts {experts.tolist()} (up to {per} random rows each, "
                      f"seed 0) of the same workload: the oracle's E4M3 quantisation of the rows "
                      f"and its E4M3 expert MLP (products of decoded codes summed in double); "
                      f"the two experts' weights quantised beforehand, untimed"}


POOL_FP8_METRIC = ("EP-share pool step (permute, expert MLP, unpermute) TFLOP/s with E4M3 "
                   "ragged dots (model FLOPs), % of fp8 MFMA peak (1 MI355X)")


def bench_pool_fp8(args, cfg, M, dev):
    """The receiver pool's step with the fp8 permutation leg and E4M3 expert MLP: the
    pool rows are grouped and quantised in one pass (moe_permute_e4m3, with the rows'
    delayed scale), the expert MLP runs on E4M3 operands (moe_grouped_ffn_e4m3), the
    output rows go back to pool order (moe_combine, k = 1), and both amax histories
    roll into the next step's scales on the device.  The bf16 step (moe_permute with
    the row copy, moe_grouped_ffn, moe_combine) is timed on the same pool."""
    import numpy as np
    import torch

    from moe_synth import gen_pool
    from oracle import oracle as O

    pool = gen_pool(cfg, dev)
    P, L, H, E = cfg.P, cfg.L, cfg.H, cfg.E
    ids = pool["ids"]
    i32 = dict(dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    u8 = dict(dtype=torch.uint8, device=dev)
    W_gu, W_d = pool["W_gu"], pool["W_d"]
    Wguq, Wdq = torch.empty(W_gu.shape, **u8), torch.empty(W_d.shape, **u8)
    HIST = 16
    hist_x, hist_h = torch.zeros(HIST, **f32), torch.zeros(HIST, **f32)
    hist_gu, hist_d = torch.zeros(1, **f32), torch.zeros(1, **f32)
    s_x, s_h, s_gu, s_d = (torch.ones(1, **f32) for _ in range(4))
    a_x, a_h, a_gu, a_d = (torch.zeros(1, **f32) for _ in range(4))

    def quantize_weights():
        M.moe_quantize_e4m3(W_gu, s_gu, q=Wguq, amax=a_gu)
        M.moe_quantize_e4m3(W_d, s_d, q=Wdq, amax=a_d)
        M.moe_fp8_scale_update(hist_gu, a_gu, s_gu)
        M.moe_fp8_scale_update(hist_d, a_d, s_d)

    quantize_weights()
    quantize_weights()
    Xq_perm = torch.empty((P, L), **u8)
    Y_perm = torch.empty((P, L), dtype=torch.bfloat16, device=dev)
    out = torch.full((P, L), 0.0, dtype=torch.bfloat16, device=dev)
    pws = torch.empty(M.moe_permute_workspace_size(P, E), **u8)
    fws = torch.empty(M.moe_grouped_ffn_e4m3_workspace_size(E, P, H), **u8)
    g = dict(slot_row=torch.empty(P, **i32), row_src=torch.empty(P, **i32),
             counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
             n_dropped=torch.empty(1, dtype=torch.int64, device=dev))

    def step(ev=None):
        if ev:
            ev[0].record()
        M.moe_permute_e4m3(ids, E, pool["X"], Xq_perm, src_div=1, R_phys=P, scale=s_x,
                           amax=a_x, ws=pws, out=g)
        if ev:
            ev[1].record()
        M.moe_grouped_ffn_e4m3(Xq_perm, g["offsets"], Wguq, Wdq, s_x, s_gu, s_h, s_d, Y=Y_perm,
                               amax_h=a_h, ws=fws)
        if ev:
            ev[2].record()
        M.moe_combine(Y_perm, g["slot_row"], None, P, 1, out=out,
                      flags=M.MOE_COMBINE_KEEP_UNROUTED)
        M.moe_fp8_scale_update(hist_x, a_x, s_x)
        M.moe_fp8_scale_update(hist_h, a_h, s_h)
        if ev:
            ev[3].record()

    for _ in range(max(2, args.warmup)):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for st in range(args.steps):
        step(evs[st])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    names = ["permute_e4m3", "expert_mlp_e4m3", "unpermute_and_scale_updates"]
    stage_ms = {n: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / args.steps
                for i, n in enumerate(names)}
    cnt = g["counts"].cpu().numpy().astype(np.int64)
    valid = int(cnt.sum())
    ms = wall * 1e3 / args.steps
    flops = cfg.flops(valid)
    tflops = flops / (ms * 1e-3) / 1e12
    # the bf16 step on the same pool
    X_perm = torch.empty((P, L), dtype=torch.bfloat16, device=dev)
    bws = torch.empty(M.moe_grouped_ffn_workspace_size(E, P, H, torch.bfloat16), **u8)
    g2 = {k: torch.empty_like(v) for k, v in g.items()}

    def step16():
        M.moe_permute(ids, E, src=pool["X"], src_div=1, dst=X_perm, R_phys=P, ws=pws, out=g2)
        M.moe_grouped_ffn(X_perm, g2["offsets"], W_gu, W_d, Y=Y_perm, ws=bws)
        M.moe_combine(Y_perm, g2["slot_row"], None, P, 1, out=out,
                      flags=M.MOE_COMBINE_KEEP_UNROUTED)

    bf16_ms = time_ms(step16, reps=10)
    ffn_bytes = E * 3 * H * L + valid * (L + H) + valid * (2 * H * 2 * 2 + L * 2)
    line = {
        "metric": POOL_FP8_METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s (model FLOPs)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic (seeded receiver pool; rows ~ N(0,1) at unit RMS, Zipf(1) local "
                "expert ids, weights ~ N(0,1/fan_in)), quantised to E4M3 with per-tensor scales",
        "config": {"workload": cfg.name, "pool_rows": P, "valid_rows": valid, "latent": L,
                   "local_experts": E, "expert_hidden": H, "operands": "E4M3",
                   "scaling": f"per tensor, delayed: amax history of {HIST} steps on the device",
                   "parallelism": "none (1 GPU)"},
        "rows_per_s": round(valid / (ms * 1e-3), 1),
        "pct_peak_mfma": round(100 * tflops / PEAK_TFLOPS["fp8"], 2),
        "stage_ms": {n: round(v, 4) for n, v in stage_ms.items()},
        "bf16_step_ms": round(bf16_ms, 4),
        "speedup_vs_bf16": round(bf16_ms / ms, 3),
        "roofline": gemm_roofline("E4M3 expert MLP (gate/up and down ragged dots, activation "
                                  "quantisation)", flops, ffn_bytes,
                                  stage_ms["expert_mlp_e4m3"], "fp8"),
    }
    if not args.no_cpu_baseline:
        # the oracle's own grouping of the pool picks the rows it samples
        ref = O.permute(ids.cpu().numpy(), E, R_phys=P)
        kept = int(ref["offsets"][-1])
        rows = torch.from_numpy(ref["row_src"][:kept].astype(np.int64)).to(dev)
        data = {"counts": np.diff(ref["offsets"]).astype(np.int64), "X": pool["X"][rows],
                "W_gu": W_gu, "W_d": W_d}
        sc = {"x": float(s_x.item()), "h": float(s_h.item())}
        line["cpu_baseline"] = cpu_baseline_fp8(cfg, data, sc, float(s_gu.item()),
                                                float(s_d.item()), args.cpu_seconds)
    return line


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this library has no multi-GPU path (asked for "
              f"--gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import mixture_experts_transformer_amd as M
    from moe_synth import PoolConfig, by_name

    dev = torch.device("cuda:0")
    cfg = data = None
    if args.backward:
        name = args.workload if args.workload != DEFAULT_WORKLOAD else BWD_DEFAULT
        line = bench_backward(args, by_name(name), M, dev)
    elif args.fp8:
        name = args.workload if args.workload != DEFAULT_WORKLOAD else FP8_DEFAULT
        cfg8 = by_name(name)
        if isinstance(cfg8, PoolConfig):
            line = bench_pool_fp8(args, cfg8, M, dev)
        else:
            line = bench_fp8(args, cfg8, M, dev)
    else:
        cfg = by_name(args.workload)
        if isinstance(cfg, PoolConfig):
            line, data = bench_pool(args, cfg, M, dev)
        else:
            line, data = bench_layer(args, cfg, M, dev)
            if cfg.name == DEFAULT_WORKLOAD and not args.no_kernel_extras:
                # the workloads where the grouped GEMMs are MFMA-bound, timed after
                # the headline: the expert-parallel share's pool and the
                # long-context batch
                line["ep_share_pool"] = bench_pool_leg(args, M, dev)
                line["long_context"] = bench_longctx_leg(args, M, dev, data)
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        cms = time_ms(lambda: dst.copy_(src), reps=1)
        line["copy_1GiB"] = {"ms": round(cms, 4),
                             "GB_per_s": round(2 * (1 << 30) / (cms * 1e-3) / 1e9, 1)}
        # the write ceiling that a write-dominated kernel (a row copy fanning each
        # source row out to k destinations) is held to
        fms = time_ms(lambda: dst.fill_(1), reps=3)
        line["fill_1GiB"] = {"ms": round(fms, 4),
                             "GB_per_s": round((1 << 30) / (fms * 1e-3) / 1e9, 1)}
        del src, dst
    if not args.no_cpu_baseline and cfg is not None:
        if isinstance(cfg, PoolConfig):
            line["cpu_baseline"] = cpu_baseline_both(
                lambda t: cpu_baseline_pool(cfg, data, t), args.cpu_seconds)
        else:
            line["cpu_baseline"] = cpu_baseline_both(
                lambda t: cpu_baseline_layer(cfg, data, t), args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Throughput of the fused MoE expert layer on one MI355X.

Workload: the Mixtral-8x7B-shaped MoE layer (H=4096, F=14336, E=8 experts,
top-2, SwiGLU experts, bf16) at a batch of T=32 tokens, router logits
~ N(0,1), inputs already resident in HBM. A step is one moe_forward_packed
call (route -> permute -> gate/up+SwiGLU -> down -> combine, 5 launches) on
weights packed once beforehand (moe_pack_weights, as at model load; its time
is reported as `pack_ms`, outside the steps); `rowmajor_ms_per_step` is the
same step on the row-major weights (moe_forward), for comparison.

Metric: MoE-layer HBM GB/s (algorithmic bytes / time), with TFLOP/s and the
roofline fractions beside it. `roofline` describes the dominant kernel (the
gate/up+SwiGLU grouped GEMM), timed with HIP events on its launch stream.
`cpu_baseline` is the CPU oracle timed on a bounded sample of the same
workload. `--sweep 1,128,512` repeats the measurement at other batch sizes of
the same layer shape (listed under `sweep`).

`--weights mxfp4` likewise on MXFP4 weights (E2M1 codes, one E8M0 scale per
32 K-values of a column; moe_forward_mxfp4), 4.25 bits per weight.
`--weights fp8` times the layer on FP8 (E4M3) weights with per-column
scales (moe_forward_fp8; bf16 activations and MFMA), which computes exactly
the bf16 layer on the dequantized weights at half the weight bytes.
`--router` instead times the router projection fused with routing
(moe_router_route) at every layer shape, against the unfused sequence.
`--backward` times the training backward (moe_backward) of --config at --T.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer TFLOP/s and HBM GB/s (roofline %) vs tokens T, 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="mixtral")
    ap.add_argument("--T", type=int, default=32)
    ap.add_argument("--sweep", default="",
                    help="other batch sizes of the same layer to measure, e.g. '1,128,512' "
                         "(off by default, so that a kernel-trace of the default run "
                         "averages the headline kernels only)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=32,
                    help="tokens in the oracle's timed sample")
    ap.add_argument("--weights", choices=("packed", "rowmajor", "fp8", "mxfp4"),
                    default="packed",
                    help="weight layout of the timed steps (fp8: E4M3 codes with per-column "
                         "scales, moe_forward_fp8; mxfp4: E2M1 codes with a scale byte per "
                         "32 K-values, moe_forward_mxfp4; bf16 arithmetic in every case)")
    ap.add_argument("--router", action="store_true",
                    help="only time the router row: moe_router_route (router GEMM + "
                         "top-k routing) against torch's matmul + fp32 cast + moe_route, "
                         "for every layer shape, one JSON line each, and exit")
    ap.add_argument("--backward", action="store_true",
                    help="only time the training backward (moe_backward: forward "
                         "recompute, dx and the weight gradients) at --config/--T against "
                         "the forward on the same row-major weights, one JSON line, and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy three times (the "
                         "known-size reference for HBM byte counters) and exit")
    return ap.parse_args()


def work_model(cfg, T, counts, wb=2):
    """Algorithmic FLOPs and HBM bytes of one forward, per kernel.
    counts: rows per routed expert (E_touched = experts with rows); wb: bytes
    per weight (2 bf16, 1 fp8, 0.5 + 1/32 mxfp4: a 4-bit code and a scale
    byte per 32 K-values; fp8 adds a 4-byte scale per output column)."""
    H, F, E, k, Fs = cfg.H, cfg.F, cfg.E, cfg.k, cfg.Fs
    A = T * k
    Et = int((counts > 0).sum())
    m = {}
    m["route"] = dict(bytes=4 * T * E + 8 * A, flops=0)
    m["permute"] = dict(bytes=4 * A + 2 * T * H + 2 * A * H + 8 * A, flops=0)
    sc = 4 if wb == 1 else 0                # fp8 column scales
    # (mxfp4's scale bytes are inside wb; byte counts are rounded to integers)
    g1 = 2 * wb * H * F * Et + 2 * sc * F * Et + 2 * A * H + 2 * A * F
    g1f = 4 * A * H * F
    # routed part of the gate/up GEMM alone (what moe_gateup_swiglu runs)
    m["gateup_swiglu_routed"] = dict(bytes=int(g1), flops=g1f)
    g2 = wb * F * H * Et + sc * H * Et + 2 * A * F + 2 * A * H
    g2f = 2 * A * F * H
    cb = 2 * A * H + 8 * A + 2 * T * H
    if Fs:
        g1 += 2 * wb * H * Fs + 2 * sc * Fs + 2 * T * H + 2 * T * Fs
        g1f += 4 * T * H * Fs
        g2 += wb * Fs * H + sc * H + 2 * T * Fs + 2 * T * H
        g2f += 2 * T * Fs * H
        cb += 2 * T * H + (4 * T if cfg.shared_gated else 0)
    m["gateup_swiglu"] = dict(bytes=int(g1), flops=g1f)
    m["down"] = dict(bytes=int(g2), flops=g2f)
    m["combine"] = dict(bytes=cb, flops=0)
    total_b = sum(v["bytes"] for n, v in m.items() if n != "gateup_swiglu_routed")
    total_f = sum(v["flops"] for n, v in m.items() if n != "gateup_swiglu_routed")
    return total_b, total_f, m, Et


def measured_traffic(workload_is_default: bool, weights: str):
    """HBM bytes per launch of the gate/up kernel from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE counters (copy-calibrated), or None when they were
    taken on other kernel sources or another workload."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gateup_swiglu_mixtral_t32_traffic.json")
    if not workload_is_default or not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("weights", "rowmajor") != weights:
        return None
    h = hashlib.sha256()
    for src in d["kernel_sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return d["traffic_bytes_per_launch"] if h.hexdigest() == d["kernel_sources_sha256"] else None


def roof(bytes_, flops, ms):
    s = ms * 1e-3
    gbs = bytes_ / s / 1e9
    tfl = flops / s / 1e12
    t_hbm = bytes_ / (PEAK_HBM_GBS * 1e9)
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    return dict(gbs=gbs, tflops=tfl, hbm_frac=gbs / PEAK_HBM_GBS,
                mfma_frac=tfl / PEAK_BF16_TFLOPS, bound=bound,
                roofline_frac=max(t_hbm, t_mfma) / s)


ROUTER_SHAPES = [("mixtral", 1), ("mixtral", 32), ("mixtral", 512), ("mixtral_large", 8192),
                 ("qwen2", 16), ("qwen2", 1024), ("qwen2", 16384), ("dsv3", 128),
                 ("dsv3", 4096)]


def router_table(args, torch, B, synth):
    """Router projection + routing of each layer shape: the fused library call
    and the unfused sequence (bf16 matmul, cast to fp32, moe_route), each timed
    over a burst of calls with HIP events on the launch stream. At small T the
    host's call rate can bound both; the kernel trace of this command gives
    the device times."""
    stream = torch.cuda.current_stream()

    def timed(fn, n):
        for _ in range(5):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    for name, T in ROUTER_SHAPES:
        cfg = synth.CONFIGS[name]
        x = synth.router_input(cfg, T, args.seed, "cuda")
        w = synth.router_weight(cfg, args.seed, "cuda")
        wt = w.t().contiguous()
        ids = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
        tw = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(B.moe_router_workspace_bytes(T, cfg.H, cfg.E, cfg.k), 16),
                         dtype=torch.uint8, device="cuda")

        def fused():
            B.moe_router_route(x, w, cfg.k, ws=ws, out=(ids, tw, None))

        def unfused():
            B.moe_route(torch.matmul(x, wt).float(), cfg.k, ids, tw)

        n = max(20, args.steps)
        us_f, us_u = timed(fused, n), timed(unfused, n)
        nbytes = 2 * (T + cfg.E) * cfg.H + 8 * T * cfg.k
        print(json.dumps({"router": cfg.name, "T": T, "H": cfg.H, "E": cfg.E, "k": cfg.k,
                          "fused_us": round(us_f, 2), "matmul_cast_route_us": round(us_u, 2),
                          "alg_bytes": nbytes, "fused_GBs": round(nbytes / us_f / 1e3, 1),
                          "workspace_bytes": ws.numel() if ws.numel() > 16 else 0}),
              flush=True)


def backward_line(args, torch, B, synth):
    """moe_backward of the routed layer at one batch size: HIP events around
    `steps` calls on the launch stream. Its work is eight A*H*F products
    (2*A*H*F FLOPs each, A = T*k): the recomputed gate and up products, dh
    (on the unweighted dout), the two dx products and the three weight
    gradients."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.CONFIGS[args.config]
    T, H, F, E, k = args.T, cfg.H, cfg.F, cfg.E, cfg.k
    stream = torch.cuda.current_stream()
    layer = synth.make_layer(cfg.name, T, seed=args.seed, device=dev, with_shared=False)
    ids, w = B.moe_route(layer.logits, k, stream=stream)
    g = torch.Generator(device=dev).manual_seed(args.seed + 1)
    dout = torch.randn((T, H), generator=g, device=dev).to(torch.bfloat16)
    ws = torch.empty(B.moe_backward_workspace_bytes(T, H, F, E, k), dtype=torch.uint8,
                     device=dev)
    fws = torch.empty(B.moe_forward_workspace_bytes(T, H, F, E, k, 0), dtype=torch.uint8,
                      device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    def bwd():
        B.moe_backward(layer.x, ids, w, layer.w_gate, layer.w_up, layer.w_down, dout, ws=ws,
                       stream=stream)

    def fwd():
        B.moe_forward_routed(layer.x, ids, w, layer.w_gate, layer.w_up, layer.w_down,
                             out=out, ws=fws, stream=stream)

    def timed(fn, n, warm):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b) / n

    ms_b = timed(bwd, args.steps, args.warmup)
    ms_f = timed(fwd, args.steps, args.warmup)
    A = T * k
    flops = 8 * 2 * A * H * F
    print(json.dumps({"backward": cfg.name, "T": T, "H": H, "F": F, "E": E, "k": k,
                      "ms": round(ms_b, 4), "TFLOPs": round(flops / ms_b / 1e9, 1),
                      "mfma_frac": round(flops / ms_b / 1e9 / PEAK_BF16_TFLOPS, 4),
                      "forward_rowmajor_ms": round(ms_f, 4), "alg_flops": flops,
                      "workspace_bytes": ws.numel(), "dtype": "bf16 (fp32 weight gradients)",
                      "data": "synthetic"}), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        n = 1 << 29                                  # 2^29 bf16 = 1 GiB
        src = torch.ones(n, dtype=torch.bfloat16, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 2 * n, "launches": 3}))
        return

    from grouped_gemm_softmax_amd import binding as B
    from grouped_gemm_softmax_amd import synth

    if args.router:
        torch.cuda.set_device(0)
        router_table(args, torch, B, synth)
        return
    if args.backward:
        backward_line(args, torch, B, synth)
        return

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.CONFIGS[args.config]
    stream = torch.cuda.current_stream()

    def layer_for(T, weights_from=None):
        if weights_from is None:
            return synth.make_layer(cfg.name, T, seed=args.seed, device=dev)
        lay = synth.make_layer(cfg.name, T, seed=args.seed, device=dev, with_weights=False)
        lay.w_gate, lay.w_up, lay.w_down = (weights_from.w_gate, weights_from.w_up,
                                            weights_from.w_down)
        if lay.shared is not None:
            lay.shared = dict(weights_from.shared, gate_logits=lay.shared["gate_logits"])
        return lay

    def weights_of(layer, mode):
        """(w_gate, w_up, w_down, shared) of a layer in the timed layout."""
        if mode == "rowmajor":
            return layer.w_gate, layer.w_up, layer.w_down, layer.shared
        src = pk8 if mode in ("fp8", "mxfp4") else pk
        return (src["wg"], src["wu"], src["wd"],
                None if layer.shared is None else dict(src["shared"],
                                                       gate_logits=layer.shared["gate_logits"]))

    def measure(layer, steps, warmup, mode):
        T, H, F, E, k = layer.T, cfg.H, cfg.F, cfg.E, cfg.k
        wg, wu, wd, sh = weights_of(layer, mode)
        Fs = cfg.Fs
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        ws = torch.empty(B.moe_forward_workspace_bytes(T, H, F, E, k, Fs),
                         dtype=torch.uint8, device=dev)

        def step():
            B.moe_forward(layer.x, layer.logits, k, wg, wu, wd, shared=sh, out=out,
                          topk_ids=ids, topk_w=w, ws=ws, stream=stream)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        counts = torch.bincount(ids.flatten().long(), minlength=E).cpu().numpy()
        return ms, counts

    def time_gateup(layer, steps, mode):
        """Average duration of the gate/up+SwiGLU grouped GEMM alone, with the
        same inputs, weights and launch configuration as inside the step."""
        k = cfg.k
        wg, wu, _, _ = weights_of(layer, mode)
        ids, w = B.moe_route(layer.logits, k, stream=stream)
        off, rt, rd, xp = B.moe_permute(layer.x, ids, cfg.E, stream=stream)
        h = torch.empty((xp.shape[0], cfg.F), dtype=torch.bfloat16, device=dev)
        for _ in range(3):
            B.moe_gateup_swiglu(xp, off, wg, wu, h=h, stream=stream)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            B.moe_gateup_swiglu(xp, off, wg, wu, h=h, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    # ---- headline workload ----
    layer = layer_for(args.T)
    mode = args.weights
    torch.cuda.synchronize()
    # one-off weight packing (model-load time), timed on its own
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    pk = dict(wg=B.moe_pack_weights(layer.w_gate, stream=stream),
              wu=B.moe_pack_weights(layer.w_up, stream=stream),
              wd=B.moe_pack_weights(layer.w_down, stream=stream))
    if layer.shared is not None:
        pk["shared"] = {n: B.moe_pack_weights(layer.shared[n], stream=stream)
                        for n in ("w_gate", "w_up", "w_down")}
    e1.record(stream)
    torch.cuda.synchronize()
    pack_ms = e0.elapsed_time(e1)
    pk8, quant_ms = None, None
    if mode in ("fp8", "mxfp4"):
        quant = B.moe_quantize_fp8 if mode == "fp8" else B.moe_quantize_mxfp4
        e0.record(stream)
        pk8 = dict(wg=quant(layer.w_gate, stream=stream),
                   wu=quant(layer.w_up, stream=stream),
                   wd=quant(layer.w_down, stream=stream))
        if layer.shared is not None:
            pk8["shared"] = {n: quant(layer.shared[n], stream=stream)
                             for n in ("w_gate", "w_up", "w_down")}
        e1.record(stream)
        torch.cuda.synchronize()
        quant_ms = e0.elapsed_time(e1)
    other = {"packed": "rowmajor", "rowmajor": "packed", "fp8": "packed", "mxfp4": "packed"}[mode]
    WBYTES = {"fp8": 1, "mxfp4": 0.5 + 1 / 32}.get(mode, 2)
    ms, counts = measure(layer, args.steps, args.warmup, mode)
    ms_other, _ = measure(layer, max(10, args.steps // 2), 5, other)
    total_b, total_f, per_kernel, Et = work_model(cfg, args.T, counts, WBYTES)
    r = roof(total_b, total_f, ms)

    g1_ms = time_gateup(layer, max(args.steps, 20), mode)
    g1 = per_kernel["gateup_swiglu_routed"]
    g1r = roof(g1["bytes"], g1["flops"], g1_ms)
    if g1r["bound"] == "hbm":
        roofline = dict(bound="hbm", achieved=round(g1r["gbs"], 1), peak=PEAK_HBM_GBS,
                        unit="GB/s", frac=round(g1r["gbs"] / PEAK_HBM_GBS, 4), traffic=None)
    else:
        roofline = dict(bound="mfma", achieved=round(g1r["tflops"], 1), peak=PEAK_BF16_TFLOPS,
                        unit="TFLOP/s", frac=round(g1r["tflops"] / PEAK_BF16_TFLOPS, 4),
                        traffic=None)
    roofline["traffic"] = measured_traffic(args.config == "mixtral" and args.T == 32 and
                                           args.seed == 0, args.weights)
    # the gate/up launch of the step: rs_gateup_kernel (register-streaming)
    # for packed bf16 weights at decode sizes, grouped_gemm_kernel otherwise
    roofline.update(kernel="gate/up + SwiGLU grouped GEMM over the routed experts "
                           "(moe_gateup_swiglu" + ("" if mode == "rowmajor" else "_" + mode) +
                           "; rs_gateup_kernel for packed bf16 weights at up to 16 items "
                           "per CU, grouped_gemm_kernel otherwise)",
                    kernel_ms=round(g1_ms, 5),
                    alg_bytes=g1["bytes"], alg_flops=g1["flops"])

    # ---- the other batch sizes of the same layer shape ----
    sweep = []
    for tok in [int(s) for s in args.sweep.split(",") if s.strip()]:
        if tok == args.T:
            continue
        lay = layer_for(tok, weights_from=layer)
        ms_t, counts_t = measure(lay, max(10, args.steps // 2), 5, mode)
        b_t, f_t, _, et_t = work_model(cfg, tok, counts_t, WBYTES)
        rr = roof(b_t, f_t, ms_t)
        sweep.append(dict(T=tok, ms_per_step=round(ms_t, 5), GBs=round(rr["gbs"], 1),
                          TFLOPs=round(rr["tflops"], 2), hbm_frac=round(rr["hbm_frac"], 4),
                          mfma_frac=round(rr["mfma_frac"], 4), bound=rr["bound"],
                          roofline_frac=round(rr["roofline_frac"], 4),
                          experts_touched=et_t))
        del lay

    # ---- CPU oracle on a bounded sample of the headline workload ----
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import oracle
        n = min(args.cpu_tokens, args.T)
        x = synth.u16(layer.x[:n])
        lg = synth.f32(layer.logits[:n])
        wg, wu, wd = synth.u16(layer.w_gate), synth.u16(layer.w_up), synth.u16(layer.w_down)
        # repeated until about 10 s of CPU work have been timed (a short
        # sample is run several times and averaged)
        runs, t0 = 0, time.perf_counter()
        while True:
            oracle.forward(x, lg, cfg.k, wg, wu, wd, keep_intermediates=False)
            runs += 1
            t_all = time.perf_counter() - t0
            if t_all >= 10.0 or runs >= 500:
                break
        t_cpu = t_all / runs
        t_full = t_cpu * args.T / n        # the oracle's cost is linear in tokens
        cpu = dict(value=round(total_b / t_full / 1e9, 3), unit="GB/s",
                   cores=oracle.num_threads(), kind="oracle",
                   sample=f"first {n} of {args.T} tokens, whole layer (oracle.forward, fp64), "
                          f"{runs} runs in {t_all:.1f} s ({t_cpu:.3f} s each); scaled "
                          f"linearly to the {args.T}-token step",
                   seconds_sample=round(t_cpu, 3))

    line = {
        "metric": METRIC,
        "value": round(r["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "weight_dtype": {"fp8": "fp8_e4m3", "mxfp4": "mxfp4_e2m1"}.get(mode, "bf16"),
        "data": "synthetic (seeded; x~N(0,1), weights~N(0,0.02), logits~N(0,1))",
        "config": {"workload": f"{cfg.desc}: T={args.T}, H={cfg.H}, F={cfg.F}, E={cfg.E}, "
                               f"top-{cfg.k}, bf16, "
                               + ({"fp8": "fp8 E4M3 weights with per-column scales",
                                   "mxfp4": "MXFP4 weights (E2M1, E8M0 scale per 32)"}
                                  .get(mode, f"{args.weights} weights")),
                   "weights": args.weights,
                   "T": args.T, "H": cfg.H, "F": cfg.F, "E": cfg.E, "k": cfg.k,
                   "Fs": cfg.Fs, "experts_touched": Et, "parallelism": "none (1 GPU)"},
        "TFLOPs": round(r["tflops"], 3),
        "hbm_frac": round(r["hbm_frac"], 4),
        "mfma_frac": round(r["mfma_frac"], 4),
        "layer_bound": r["bound"],
        "layer_roofline_frac": round(r["roofline_frac"], 4),
        "alg_bytes": total_b,
        "alg_flops": total_f,
        other + "_ms_per_step": round(ms_other, 5),
        "pack_ms": round(pack_ms, 3),
        "quantize_ms": None if quant_ms is None else round(quant_ms, 3),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "sweep": sweep,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

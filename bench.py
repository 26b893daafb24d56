#!/usr/bin/env python3
"""Throughput of the fused MoE expert layer on one MI355X, against T.

Headline workload: the Mixtral-8x7B-shaped MoE layer at large batch (H=4096,
F=14336, E=8 experts, top-2, SwiGLU experts, bf16) at T=8192 tokens, router
logits ~ N(0,1) plus a per-expert bias ~ N(0,0.5), inputs already resident in
HBM: the largest-FLOP configuration, bound by the matrix cores. A step is one
moe_forward_packed call (route -> permute -> gate/up+SwiGLU -> down ->
combine, 5 launches) on weights packed once beforehand (moe_pack_weights, as
at model load; `pack_ms`, outside the steps); `rowmajor_ms_per_step` is the
same step on the row-major weights (moe_forward).

Timing: before every timed step a 512 MiB buffer is read (outside the timed
interval), so that neither the 4 MB L2s nor the 256 MB Infinity Cache hold
the previous step's weights; each step is timed alone with HIP events on
its stream. `ms_per_step` is the median, with p10/p90 and the mean beside it.
`value` is the layer's algorithmic TFLOP/s at the median. `roofline`
describes the dominant kernel (the gate/up+SwiGLU grouped GEMM, 2/3 of the
FLOPs and of the weight bytes), its launches timed the same way.

`sweep` (default: every configured layer and batch size, `--sweep none` to
skip) repeats the measurement for the tiny, Mixtral-, DeepSeek-V3- and
Qwen2-MoE-shaped layers at each of their batch sizes: ms, TFLOP/s, GB/s,
binding roof, roofline fraction, gate/up kernel time, and the row-major
step. `cpu_baseline` is the CPU oracle timed on a bounded sample of the
headline workload.

`--weights fp8` / `--weights mxfp4` time the layer on FP8 (E4M3, per-column
scales; moe_forward_fp8) or MXFP4 (E2M1 with an E8M0 scale per 32 K-values
of a column; moe_forward_mxfp4) weights instead, which compute exactly the
bf16 layer on the dequantized weights. `--router` instead times the router
projection fused with routing (moe_router_route) at every layer shape,
against the unfused sequence. `--backward` times the training backward
(moe_backward) of --config at --T.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C --T t]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer TFLOP/s and HBM GB/s (roofline %) vs tokens T, 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
FLUSH_BYTES = 512 << 20     # read before every timed step (L2 + MALL flush)
SWEEP_ALL = [("tiny", 64), ("mixtral", 1), ("mixtral", 32), ("mixtral", 128), ("mixtral", 512),
             ("mixtral_large", 2048), ("mixtral_large", 8192), ("dsv3", 128), ("dsv3", 4096),
             ("qwen2", 16), ("qwen2", 1024), ("qwen2", 16384)]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mixtral_large")
    ap.add_argument("--T", type=int, default=8192)
    ap.add_argument("--sweep", default="all",
                    help="'all' (every configured layer and batch size), 'none', or a list "
                         "like 'mixtral:1,qwen2:16'")
    ap.add_argument("--sweep-steps", type=int, default=10)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=64,
                    help="tokens in the oracle's timed sample")
    ap.add_argument("--weights", choices=("packed", "rowmajor", "fp8", "mxfp4", "mxfp8"),
                    default="packed",
                    help="weight layout of the timed steps (fp8: E4M3 codes with per-column "
                         "scales, moe_forward_fp8; mxfp4 / mxfp8: E2M1 / E4M3 codes with a "
                         "scale byte per 32 K-values, moe_forward_mxfp4 / _mxfp8; bf16 "
                         "arithmetic in every case)")
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


def measured_traffic(config: str, T: int, weights: str):
    """HBM bytes per launch of the gate/up kernel of this workload from the
    committed rocprofv3 FETCH_SIZE/WRITE_SIZE counters (copy-calibrated,
    profiles/gateup_swiglu_<config>_t<T>_traffic.json), or None when there
    are none or they were taken on other kernel sources or weights."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"gateup_swiglu_{config}_t{T}_traffic.json")
    if not os.path.exists(path):
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


def activation_bytes(cfg, T):
    """Activation bytes moved between the layer's steps (weights excluded):
    the fused path as built against an unfused one. Fused, large batch: the
    gate/up tiles read x through the row map (no x_perm copy), h is written
    and read once in bf16, the down projection's fp32 output is written and
    read once by the combine, out written once. Unfused (each step its own
    kernel over HBM): x_perm written, read by the gate and by the up GEMM, G
    and U written and read by a SwiGLU kernel that writes h, h read by the
    down GEMM, y written and read by the combine (all bf16), out written.
    Shared expert and routing excluded (the same in both)."""
    A, H, F = T * cfg.k, cfg.H, cfg.F
    unfused = 2 * A * (5 * H + 6 * F) + 2 * T * H
    fused = 2 * A * H + 4 * A * F + 8 * A * H + 2 * T * H
    return fused, unfused


def pct(xs, q):
    import numpy as np
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


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
    """moe_backward of the layer at one batch size (with its shared expert,
    through moe_backward_shared, where the config has one): HIP events
    around `steps` calls on the launch stream. Its work is eight A*H*F
    products (2*A*H*F FLOPs each, A = T*k): the recomputed gate and up
    products, dh (on the unweighted dout), the two dx products and the three
    weight gradients; the shared expert adds eight T*H*Fs products."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.CONFIGS[args.config]
    T, H, F, E, k = args.T, cfg.H, cfg.F, cfg.E, cfg.k
    stream = torch.cuda.current_stream()
    Fs = cfg.Fs or 0
    layer = synth.make_layer(cfg.name, T, seed=args.seed, device=dev, with_shared=Fs > 0)
    shared = layer.shared if Fs > 0 else None
    ids, w = B.moe_route(layer.logits, k, stream=stream)
    g = torch.Generator(device=dev).manual_seed(args.seed + 1)
    dout = torch.randn((T, H), generator=g, device=dev).to(torch.bfloat16)
    ws = torch.empty(B.moe_backward_shared_workspace_bytes(T, H, F, E, k, Fs), dtype=torch.uint8,
                     device=dev)
    fws = torch.empty(B.moe_forward_workspace_bytes(T, H, F, E, k, Fs), dtype=torch.uint8,
                      device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    def bwd():
        B.moe_backward(layer.x, ids, w, layer.w_gate, layer.w_up, layer.w_down, dout,
                       shared=shared, ws=ws, stream=stream)

    def fwd():
        B.moe_forward_routed(layer.x, ids, w, layer.w_gate, layer.w_up, layer.w_down,
                             shared=shared, out=out, ws=fws, stream=stream)

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
    flops = 8 * 2 * A * H * F + 8 * 2 * T * H * Fs
    print(json.dumps({"backward": cfg.name, "T": T, "H": H, "F": F, "E": E, "k": k, "Fs": Fs,
                      "ms": round(ms_b, 4), "TFLOPs": round(flops / ms_b / 1e9, 1),
                      "mfma_frac": round(flops / ms_b / 1e9 / PEAK_BF16_TFLOPS, 4),
                      "forward_rowmajor_ms": round(ms_f, 4), "alg_flops": flops,
                      "workspace_bytes": ws.numel(), "dtype": "bf16 (fp32 weight gradients)",
                      "data": "synthetic"}), flush=True)


def host_cpu():
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return model, usable


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
    stream = torch.cuda.current_stream()
    flush_buf = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    mode = args.weights
    WBYTES = {"fp8": 1, "mxfp4": 0.5 + 1 / 32, "mxfp8": 1 + 1 / 32}.get(mode, 2)

    def flush():
        # read (not write) the buffer: the caches then hold other, clean lines,
        # and no write-back of dirty flush data competes with the timed step
        torch.sum(flush_buf)

    def timed_steps(fn, steps, warmup):
        """Per-step milliseconds (HIP events on the launch stream around each
        step alone, the cache flush before it outside the events), and the
        wall time of the whole timed region (flushes included)."""
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        t0 = time.perf_counter()
        for a, b in ev:
            flush()
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return [a.elapsed_time(b) for a, b in ev], wall

    def stats(ms):
        return dict(ms_median=round(pct(ms, 50), 5), ms_p10=round(pct(ms, 10), 5),
                    ms_p90=round(pct(ms, 90), 5), ms_mean=round(float(np.mean(ms)), 5))

    class Workload:
        """One layer's weights (row-major and in the timed layout)."""

        def __init__(self, cfg_name):
            self.cfg = synth.CONFIGS[cfg_name]
            self.layer = synth.make_layer(cfg_name, 1, seed=args.seed, device=dev)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pack = B.moe_pack_weights
            L = self.layer
            self.pk = dict(wg=pack(L.w_gate), wu=pack(L.w_up), wd=pack(L.w_down))
            if L.shared is not None:
                self.pk["shared"] = {n: pack(L.shared[n]) for n in ("w_gate", "w_up", "w_down")}
            e1.record(stream)
            torch.cuda.synchronize()
            self.pack_ms = e0.elapsed_time(e1)
            self.q, self.quant_ms = None, None
            if mode in ("fp8", "mxfp4", "mxfp8"):
                quant = {"fp8": B.moe_quantize_fp8, "mxfp4": B.moe_quantize_mxfp4,
                         "mxfp8": B.moe_quantize_mxfp8}[mode]
                e0.record(stream)
                self.q = dict(wg=quant(L.w_gate), wu=quant(L.w_up), wd=quant(L.w_down))
                if L.shared is not None:
                    self.q["shared"] = {n: quant(L.shared[n]) for n in ("w_gate", "w_up", "w_down")}
                e1.record(stream)
                torch.cuda.synchronize()
                self.quant_ms = e0.elapsed_time(e1)

        def weights(self, m, batch):
            L = self.layer
            if m == "rowmajor":
                src = dict(wg=L.w_gate, wu=L.w_up, wd=L.w_down,
                           shared=None if L.shared is None else
                           {n: L.shared[n] for n in ("w_gate", "w_up", "w_down")})
            else:
                src = self.q if m in ("fp8", "mxfp4", "mxfp8") else self.pk
            sh = None
            if self.cfg.Fs:
                sh = dict(src["shared"], gate_logits=batch.shared["gate_logits"])
            return src["wg"], src["wu"], src["wd"], sh

        def batch(self, T):
            return synth.make_layer(self.cfg.name, T, seed=args.seed, device=dev,
                                    with_weights=False)

    def measure(wl, batch, m, steps, warmup):
        cfg, T = wl.cfg, batch.T
        wg, wu, wd, sh = wl.weights(m, batch)
        out = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=dev)
        ids = torch.empty((T, cfg.k), dtype=torch.int32, device=dev)
        w = torch.empty((T, cfg.k), dtype=torch.float32, device=dev)
        ws = torch.empty(max(B.moe_forward_workspace_bytes(T, cfg.H, cfg.F, cfg.E, cfg.k, cfg.Fs),
                             16), dtype=torch.uint8, device=dev)

        def step():
            B.moe_forward(batch.x, batch.logits, cfg.k, wg, wu, wd, shared=sh, out=out,
                          topk_ids=ids, topk_w=w, ws=ws, stream=stream)

        ms, wall = timed_steps(step, steps, warmup)
        counts = torch.bincount(ids.flatten().long(), minlength=cfg.E).cpu().numpy()
        return ms, wall, counts

    def gateup_ms(wl, batch, m, steps):
        """Launches of the gate/up+SwiGLU grouped GEMM over the routed experts
        alone (moe_gateup_swiglu with the layer's weights and routing), each
        timed like a step."""
        cfg = wl.cfg
        wg, wu, _, _ = wl.weights(m, batch)
        ids, _ = B.moe_route(batch.logits, cfg.k, stream=stream)
        off, _, _, xp = B.moe_permute(batch.x, ids, cfg.E, stream=stream)
        h = torch.empty((xp.shape[0], cfg.F), dtype=torch.bfloat16, device=dev)
        ms, _ = timed_steps(lambda: B.moe_gateup_swiglu(xp, off, wg, wu, h=h, stream=stream),
                            steps, 2)
        return ms

    def row(wl, T, steps, warmup, with_rowmajor=True):
        batch = wl.batch(T)
        ms, wall, counts = measure(wl, batch, mode, steps, warmup)
        st = stats(ms)
        tb, tf, per, et = work_model(wl.cfg, T, counts, WBYTES)
        r = roof(tb, tf, st["ms_median"])
        g_ms = gateup_ms(wl, batch, mode, steps)
        g = per["gateup_swiglu_routed"]
        gr = roof(g["bytes"], g["flops"], float(np.mean(g_ms)))
        d = dict(config=wl.cfg.name, T=T, **st, TFLOPs=round(r["tflops"], 2),
                 GBs=round(r["gbs"], 1), bound=r["bound"], hbm_frac=round(r["hbm_frac"], 4),
                 mfma_frac=round(r["mfma_frac"], 4), roofline_frac=round(r["roofline_frac"], 4),
                 gateup_ms=round(float(np.mean(g_ms)), 5), gateup_bound=gr["bound"],
                 gateup_frac=round(gr["hbm_frac"] if gr["bound"] == "hbm" else gr["mfma_frac"], 4),
                 experts_touched=et)
        if with_rowmajor and mode == "packed":
            ms_rm, _, _ = measure(wl, batch, "rowmajor", max(3, steps // 2), 2)
            d["rowmajor_ms_median"] = round(pct(ms_rm, 50), 5)
        return d, dict(ms=ms, wall=wall, counts=counts, work=(tb, tf, per, et), r=r,
                       g_ms=g_ms, g=g, gr=gr)

    # ---- headline workload ----
    wl = Workload(args.config)
    cfg, T = wl.cfg, args.T
    head, raw = row(wl, T, args.steps, args.warmup)
    tb, tf, per, Et = raw["work"]
    r, gr, g = raw["r"], raw["gr"], raw["g"]
    g_mean = float(np.mean(raw["g_ms"]))
    if gr["bound"] == "hbm":
        roofline = dict(bound="hbm", achieved=round(gr["gbs"], 1), peak=PEAK_HBM_GBS,
                        unit="GB/s", frac=round(gr["gbs"] / PEAK_HBM_GBS, 4))
    else:
        roofline = dict(bound="mfma", achieved=round(gr["tflops"], 1), peak=PEAK_BF16_TFLOPS,
                        unit="TFLOP/s", frac=round(gr["tflops"] / PEAK_BF16_TFLOPS, 4))
    roofline["traffic"] = measured_traffic(args.config, T, mode)
    roofline.update(kernel="gate/up + SwiGLU grouped GEMM over the routed experts "
                           "(moe_gateup_swiglu" + ("" if mode == "rowmajor" else "_" + mode) +
                           "; grouped_gemm_kernel, or rs_gateup_kernel for packed bf16/fp8 "
                           "weights at decode sizes)",
                    kernel_ms=round(g_mean, 5), kernel_ms_p10=round(pct(raw["g_ms"], 10), 5),
                    kernel_ms_p90=round(pct(raw["g_ms"], 90), 5),
                    alg_bytes=g["bytes"], alg_flops=g["flops"])
    act_f, act_u = activation_bytes(cfg, T)
    pack_ms, quant_ms = wl.pack_ms, wl.quant_ms
    host_layer = wl.layer if not args.no_cpu_baseline else None
    head_batch = wl.batch(min(T, args.cpu_tokens)) if host_layer is not None else None
    del wl
    torch.cuda.empty_cache()

    # ---- every configured layer and batch size ----
    sweep = []
    if args.sweep != "none":
        if args.sweep == "all":
            todo = SWEEP_ALL
        else:
            todo = [(a.split(":")[0], int(a.split(":")[1])) for a in args.sweep.split(",") if a]
        cur = None
        for name, t in todo:
            if cur is None or cur.cfg.name != name:
                cur = None
                torch.cuda.empty_cache()
                cur = Workload(name)
            d, _ = row(cur, t, args.sweep_steps, 3)
            sweep.append(d)
            print(json.dumps({"sweep_row": d}), file=sys.stderr, flush=True)
        cur = None
        torch.cuda.empty_cache()

    # ---- CPU oracle on a bounded sample of the headline workload ----
    cpu = None
    if host_layer is not None:
        from oracle import oracle
        n = head_batch.T
        x = synth.u16(head_batch.x)
        lg = synth.f32(head_batch.logits)
        wg, wu, wd = (synth.u16(host_layer.w_gate), synth.u16(host_layer.w_up),
                      synth.u16(host_layer.w_down))
        sh = None
        if cfg.Fs:
            gl = head_batch.shared["gate_logits"]
            sh = dict(w_gate=synth.u16(host_layer.shared["w_gate"]),
                      w_up=synth.u16(host_layer.shared["w_up"]),
                      w_down=synth.u16(host_layer.shared["w_down"]),
                      gate_logits=None if gl is None else synth.f32(gl))
        # the sample's FLOPs: the same per-token work as the layer
        f_tok = tf / T

        def run_for(seconds, ntok):
            shn = None if sh is None else dict(
                sh, gate_logits=None if sh["gate_logits"] is None else sh["gate_logits"][:ntok])
            runs, t0 = 0, time.perf_counter()
            while True:
                oracle.forward(x[:ntok], lg[:ntok], cfg.k, wg, wu, wd, shared=shn,
                               keep_intermediates=False)
                runs += 1
                t_all = time.perf_counter() - t0
                if t_all >= seconds or runs >= 500:
                    return runs, t_all

        runs, t_all = run_for(10.0, n)
        t_cpu = t_all / runs
        threads = oracle.num_threads()
        oracle.set_num_threads(1)
        n1 = min(n, 4)                      # single thread: a 4-token sample
        runs1, t_all1 = run_for(2.0, n1)
        oracle.set_num_threads(threads)
        model, usable = host_cpu()
        cpu = dict(value=round(f_tok * n / t_cpu / 1e12, 5), unit="TFLOP/s", cores=threads,
                   kind="oracle",
                   sample=f"first {n} of {T} tokens of the headline layer, whole layer "
                          f"(oracle.forward, fp64, OpenMP over rows), {runs} runs in "
                          f"{t_all:.1f} s ({t_cpu:.3f} s each); the layer's FLOPs per token "
                          f"times {n} tokens per run",
                   seconds_sample=round(t_cpu, 4),
                   single_thread_value=round(f_tok * n1 / (t_all1 / runs1) / 1e12, 5),
                   single_thread_sample=f"first {n1} tokens, {runs1} runs in {t_all1:.1f} s",
                   host_cpu=model, host_cpus_usable=usable)

    line = {
        "metric": METRIC,
        "value": head["TFLOPs"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_median"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "weight_dtype": {"fp8": "fp8_e4m3", "mxfp4": "mxfp4_e2m1",
                         "mxfp8": "mxfp8_e4m3"}.get(mode, "bf16"),
        "data": "synthetic (seeded; x~N(0,1), weights~N(0,0.02), logits~N(0,1) "
                "(+ per-expert bias N(0,0.5) at large batch, Zipf(1.2)+Gumbel for the "
                "DeepSeek-V3 shape))",
        "config": {"workload": f"{cfg.desc}: T={T}, H={cfg.H}, F={cfg.F}, E={cfg.E}, "
                               f"top-{cfg.k}, bf16, " +
                               ({"fp8": "fp8 E4M3 weights with per-column scales",
                                 "mxfp4": "MXFP4 weights (E2M1, E8M0 scale per 32)",
                                 "mxfp8": "MXFP8 weights (E4M3, E8M0 scale per 32)"}
                                .get(mode, f"{mode} weights")),
                   "weights": mode, "T": T, "H": cfg.H, "F": cfg.F, "E": cfg.E, "k": cfg.k,
                   "Fs": cfg.Fs, "experts_touched": Et, "parallelism": "none (1 GPU)"},
        "timing": "median of per-step HIP-event times, a 512 MiB read before each step to "
                  "flush L2 and the Infinity Cache (outside the events)",
        "ms_p10": head["ms_p10"], "ms_p90": head["ms_p90"], "ms_mean": head["ms_mean"],
        "timed_region_s": round(raw["wall"], 4),
        "GBs": head["GBs"],
        "hbm_frac": head["hbm_frac"],
        "mfma_frac": head["mfma_frac"],
        "layer_bound": head["bound"],
        "layer_roofline_frac": head["roofline_frac"],
        "alg_bytes": tb,
        "alg_flops": tf,
        "rowmajor_ms_per_step": head.get("rowmajor_ms_median"),
        "pack_ms": round(pack_ms, 3),
        "quantize_ms": None if quant_ms is None else round(quant_ms, 3),
        "activation_bytes_fused": act_f,
        "activation_bytes_unfused": act_u,
        "activation_bytes_ratio": round(act_f / act_u, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "sweep": sweep,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

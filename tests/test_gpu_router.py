"""GPU parity of the router projection fused with routing (moe_router_route)
against the CPU oracle.

The logits are an fp32 sum whose order the kernel chooses, so they are checked
against the oracle's fp64 logits within the worst-case bound of any fp32
summation order. The routing decision is an integer result taken on those fp32
logits: the ids and weights must equal what the oracle's routing returns on
the kernel's own fp32 logits (same precision on both sides), and the chosen
experts must also be a valid top-k of the fp64 logits up to that bound. With
integer-valued inputs every logit is exact, so there the ids must equal the
oracle's on its own logits.

The layer entry that takes a routing (moe_forward_routed) must equal
moe_forward bit for bit given the same ids and weights, and the chain router
-> routed layer is checked against the oracle's layer on the router's logits.
"""
import numpy as np
import pytest
import torch

from grouped_gemm_softmax_amd import binding as B
from grouped_gemm_softmax_amd import synth
from helpers import (U, assert_close, bf16_to_f64, gpu_bf16_f64, host_layer, route_weight_bound,
                     say)

pytestmark = pytest.mark.gpu

# name -> (H, E, k, T, kind). A block holds 16..64 tokens x 16..64 experts;
# H is cut into K-slices while the blocks cannot fill the chip. One slice
# with all experts in the block ranks inside the GEMM kernel ("fused");
# otherwise the slices go through the workspace to the finalize launch.
CASES = {
    "mixtral_t1": (4096, 8, 2, 1, "normal"),            # 16 slices, one token
    "mixtral_t32": (4096, 8, 2, 32, "normal"),
    "mixtral_t200": (4096, 8, 2, 200, "normal"),        # ragged token blocks
    "qwen2_t16": (2048, 60, 4, 16, "normal"),           # E ragged in the block
    "qwen2_t300": (2048, 60, 4, 300, "normal"),
    "dsv3_t40": (7168, 256, 8, 40, "normal"),           # 4 expert blocks
    "dsv3_t128": (7168, 256, 8, 128, "normal"),
    "ragged_h": (200, 33, 3, 70, "normal"),             # fused, K tail inside a chunk
    "ragged_h_slices": (1000, 33, 3, 9, "normal"),      # K tail in the last slice
    "max_e_k": (256, 1024, 16, 20, "normal"),           # one slice, 64 expert blocks
    "e1024_t130": (128, 1024, 16, 130, "normal"),       # K shorter than one wave step
    "k_equals_e": (64, 5, 5, 50, "normal"),             # fused
    "one_expert": (64, 1, 1, 5, "normal"),              # fused
    "ties_fused": (256, 16, 4, 64, "ties_int"),         # exact integer logits, fused
    "ties_slices": (264, 60, 4, 33, "ties_int"),
    "ties_expert_blocks": (128, 200, 8, 150, "ties_int"),
}


def inputs(name):
    H, E, k, T, kind = CASES[name]
    cfg = synth.small_config("rt_" + name, H=H, E=E, k=k)
    return cfg, T, kind


def logit_bound(x, w):
    """Worst case of an fp32 sum of the H exact products in any order (with
    rounding that need not be to nearest): 2 H u sum_h |x w|."""
    H = x.shape[1]
    return 2.0 * H * U * (np.abs(bf16_to_f64(x)) @ np.abs(bf16_to_f64(w)).T) + 1e-30


def check_valid_topk(ref64, ids, bound):
    """Every chosen expert's fp64 logit is at least every unchosen one's, up
    to the two logits' bounds."""
    T, E = ref64.shape
    for t in range(T):
        chosen = np.zeros(E, bool)
        chosen[ids[t]] = True
        assert len(set(ids[t].tolist())) == ids.shape[1]
        if chosen.all():
            continue
        lo = (ref64[t, chosen] + bound[t, chosen]).min()
        hi = (ref64[t, ~chosen] - bound[t, ~chosen]).max()
        assert lo >= hi, (t, lo, hi)


@pytest.mark.parametrize("name", list(CASES))
def test_router_route(name, orc):
    cfg, T, kind = inputs(name)
    x = synth.router_input(cfg, T, 0, "cuda", kind)
    w = synth.router_weight(cfg, 0, "cuda", kind)
    xh, wh = synth.u16(x), synth.u16(w)
    say("moe_router_route", name, (T, cfg.H, cfg.E, cfg.k),
        "ws", B.moe_router_workspace_bytes(T, cfg.H, cfg.E, cfg.k))
    ids, tw, lg = B.moe_router_route(x, w, cfg.k, logits=True)
    ids2, tw2 = B.moe_router_route(x, w, cfg.k)
    torch.cuda.synchronize()
    ids, tw, lg = ids.cpu().numpy(), tw.cpu().numpy(), lg.cpu().numpy()

    ref64 = orc.router_logits(xh, wh)
    bound = logit_bound(xh, wh)
    err = np.abs(lg.astype(np.float64) - ref64)
    assert (err <= bound).all(), (err.max(), bound[err > bound][:4])
    if kind == "ties_int":
        assert (lg.astype(np.float64) == ref64).all()      # integer sums are exact

    # the routing decision, taken on the kernel's fp32 logits
    rids, rw = orc.route(lg, cfg.k)
    assert (ids == rids).all()
    wb = route_weight_bound(lg, rids, rw)
    assert (np.abs(tw.astype(np.float64) - rw) <= wb).all()
    check_valid_topk(ref64, ids, bound)
    if kind == "ties_int":
        oids, _ = orc.route(ref64.astype(np.float32), cfg.k)
        assert (ids == oids).all()

    # without the logits output the routing result is the same, bit for bit
    assert (ids2.cpu().numpy() == ids).all()
    assert (tw2.cpu().numpy().view(np.uint32) == tw.view(np.uint32)).all()


def test_router_route_matches_moe_route_on_its_logits():
    """Routing inside the router kernel equals moe_route's kernel on the same
    fp32 logits, bit for bit (ids and weights)."""
    for name in ("qwen2_t16", "dsv3_t128", "mixtral_t200", "ragged_h", "ties_slices"):
        cfg, T, kind = inputs(name)
        x = synth.router_input(cfg, T, 1, "cuda", kind)
        w = synth.router_weight(cfg, 1, "cuda", kind)
        say("moe_router_route vs moe_route", name)
        ids, tw, lg = B.moe_router_route(x, w, cfg.k, logits=True)
        ids_r, tw_r = B.moe_route(lg, cfg.k)
        torch.cuda.synchronize()
        assert torch.equal(ids, ids_r)
        assert torch.equal(tw.view(torch.int32), tw_r.view(torch.int32))


def test_router_route_empty_batch():
    cfg, _, _ = inputs("qwen2_t16")
    x = torch.empty((0, cfg.H), dtype=torch.bfloat16, device="cuda")
    w = synth.router_weight(cfg, 0, "cuda")
    ids, tw = B.moe_router_route(x, w, cfg.k)
    torch.cuda.synchronize()
    assert ids.shape == (0, cfg.k) and tw.shape == (0, cfg.k)


@pytest.mark.parametrize("cfg_name,T", [("dsv3", 4096), ("qwen2", 16384), ("qwen2", 32768),
                                        ("mixtral", 32), ("mixtral", 8192)])
def test_router_route_full_size_sampled(cfg_name, T, orc):
    """Full-size batches; the oracle's logits are computed for a sample of
    tokens (every 61st plus the last) and checked as above."""
    base = synth.CONFIGS[cfg_name]
    cfg = synth.small_config(cfg_name, H=base.H, E=base.E, k=base.k)
    x = synth.router_input(cfg, T, 0, "cuda")
    w = synth.router_weight(cfg, 0, "cuda")
    say("moe_router_route full size", cfg_name, T)
    ids, tw, lg = B.moe_router_route(x, w, cfg.k, logits=True)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[np.arange(0, T, 61), T - 1])
    xh = synth.u16(x)[rows]
    wh = synth.u16(w)
    ids, tw, lg = ids.cpu().numpy()[rows], tw.cpu().numpy()[rows], lg.cpu().numpy()[rows]
    ref64 = orc.router_logits(xh, wh)
    bound = logit_bound(xh, wh)
    assert (np.abs(lg.astype(np.float64) - ref64) <= bound).all()
    rids, rw = orc.route(lg, cfg.k)
    assert (ids == rids).all()
    assert (np.abs(tw.astype(np.float64) - rw) <= route_weight_bound(lg, rids, rw)).all()
    check_valid_topk(ref64, ids, bound)


# The layer from the router's routing (moe_forward_routed): name -> (config, T)
ROUTED_CASES = {
    # T*k <= 128: moe_forward routes and permutes in one launch; the routed
    # layer takes the histogram + permute launches instead
    "small_batch_shared": (synth.small_config("fr_s", H=136, F=120, E=7, k=3, Fs=64,
                                              shared_gated=True), 20),
    "many_experts": (synth.small_config("fr_m", H=192, F=96, E=32, k=8, Fs=160), 70),
    # ~170 rows per expert: large-batch tiles gather x rows through the map
    "large_batch_gather": (synth.small_config("fr_l", H=200, F=328, E=6, k=2), 500),
}


def _routed_layer(name):
    cfg, T = ROUTED_CASES[name]
    layer = synth.make_layer(cfg.name, T, seed=4, device="cuda", cfg=cfg)
    return cfg, T, layer


@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
@pytest.mark.parametrize("name", list(ROUTED_CASES))
def test_forward_routed_equals_forward(name, packed):
    """Given moe_route's ids and weights, the routed layer's output equals
    moe_forward's on the same logits bit for bit."""
    cfg, T, layer = _routed_layer(name)
    wg, wu, wd, sh = layer.w_gate, layer.w_up, layer.w_down, layer.shared
    if packed:
        wg, wu, wd = (B.moe_pack_weights(t) for t in (wg, wu, wd))
        if sh is not None:
            sh = dict(w_gate=B.moe_pack_weights(sh["w_gate"]), w_up=B.moe_pack_weights(sh["w_up"]),
                      w_down=B.moe_pack_weights(sh["w_down"]), gate_logits=sh["gate_logits"])
    say("moe_forward_routed vs moe_forward", name, T, "packed" if packed else "rowmajor")
    ids, tw = B.moe_route(layer.logits, cfg.k)
    out_ref = B.moe_forward(layer.x, layer.logits, cfg.k, wg, wu, wd, shared=sh)
    out = B.moe_forward_routed(layer.x, ids, tw, wg, wu, wd, shared=sh)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16))


@pytest.mark.parametrize("name", list(ROUTED_CASES))
def test_router_then_routed_layer_vs_oracle(name, orc):
    """x and the router weights through moe_router_route and
    moe_forward_routed, against the oracle's layer on the router's fp32
    logits (whose routing the router kernel reproduces exactly)."""
    cfg, T, layer = _routed_layer(name)
    wr = synth.router_weight(cfg, 4, "cuda")
    say("moe_router_route -> moe_forward_routed", name, T)
    ids, tw, lg = B.moe_router_route(layer.x, wr, cfg.k, logits=True)
    out = B.moe_forward_routed(layer.x, ids, tw, layer.w_gate, layer.w_up, layer.w_down,
                               shared=layer.shared)
    torch.cuda.synchronize()
    d, sh = host_layer(layer)
    lg_h = lg.cpu().numpy()
    ref = orc.forward(d["x"], lg_h, cfg.k, d["wg"], d["wu"], d["wd"], shared=sh,
                      keep_intermediates=False)
    rids, _ = orc.route(lg_h, cfg.k)
    assert (ids.cpu().numpy() == rids).all()
    assert_close(gpu_bf16_f64(out), ref["out"], f"out[{name}]")

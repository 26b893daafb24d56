"""GPU parity of each step of the layer through the C ABI, against the CPU
oracle, at sizes the oracle finishes in seconds. Shapes are chosen so that the
grouped GEMMs see several tiles per expert, ragged M, N and K tails, empty
experts, and every tile class (small, mid, large128 and large)."""
import numpy as np
import pytest
import torch

from grouped_gemm_softmax_amd import binding as B
from grouped_gemm_softmax_amd import synth
from helpers import (assert_close, bf16_to_f64, gpu_bf16_f64, host_layer, route_weight_bound,
                     say, to_dev)

pytestmark = pytest.mark.gpu

# name -> (config, T, logits kind); H/F values make K and N tails for BK=64/128/256
CASES = {
    "tiny": (synth.CONFIGS["tiny"], 64, None),
    "ragged_small_batch": (synth.small_config("rs", H=200, F=328, E=6, k=2), 90, None),
    "ragged_large_batch": (synth.small_config("rl", H=200, F=328, E=6, k=2), 500, None),
    "zipf_many_experts": (synth.small_config("zm", H=256, F=128, E=64, k=8, logits="zipf"), 60, None),
    "qwen_like": (synth.small_config("ql", H=128, F=88, E=60, k=4), 33, None),
    "single_token": (synth.small_config("st", H=136, F=72, E=8, k=2), 1, None),
    "one_expert": (synth.small_config("oe", H=64, F=64, E=1, k=1), 40, None),
    "k_equals_E": (synth.small_config("ke", H=64, F=48, E=5, k=5), 23, None),
    "k16": (synth.small_config("k16", H=64, F=40, E=32, k=16), 17, None),
    # 120 assignments over 200 experts with Zipf-skewed logits: the forward
    # routes and permutes them in one launch (two waves of assignments, hot
    # experts in both)
    "small_batch_many_experts": (synth.small_config("sbm", H=64, F=64, E=200, k=4,
                                                    logits="zipf"), 30, None),
    "all_equal_logits": (synth.small_config("eq", H=72, F=56, E=12, k=3), 45, "equal"),
    "ties_int": (synth.small_config("ti", H=64, F=64, E=16, k=4), 80, "ties_int"),
    "signed_zero": (synth.small_config("sz", H=64, F=64, E=10, k=3), 50, "signed_zero"),
    # ~100 rows per expert and enough column tiles: both GEMMs take the
    # 128-row large tiles; F = 64 is narrower than one 128-column tile
    "large128_tiles": (synth.small_config("l128", H=2048, F=64, E=64, k=4), 1600, None),
    # >= 192 rows per expert: the 256-row large tiles, with ragged K and N
    "ragged_large256": (synth.small_config("rl256", H=200, F=328, E=4, k=2), 500, None),
    # ... and with K a whole number of steps (the ping-pong tiles' main path,
    # fp8's widening one included)
    "large256_whole_k": (synth.small_config("l256", H=256, F=384, E=4, k=2), 500, None),
    # 96..191 rows per expert on average, Zipf-skewed (128-row tiles): hot
    # experts with several row tiles beside cold ones far below one
    "skewed_mid_zipf": (synth.small_config("srz", H=256, F=384, E=16, k=2, logits="zipf"), 1000,
                        None),
    # ... with K and N not whole tiles (the K-tail kernels)
    "skewed_mid_ragged": (synth.small_config("srr", H=200, F=328, E=12, k=2, logits="zipf"),
                          700, None),
    # decode-size groups on row-major weights with enough expected items for
    # the 256-column gate/up tile and the 128-column down tile (64 touched
    # experts), K and N not whole tiles
    "rowmajor_wide256": (synth.small_config("rw256", H=200, F=1480, E=64, k=2), 200, None),
    # ... few tokens: the 128-column gate/up tile (about 7 touched experts)
    "rowmajor_wide128": (synth.small_config("rw128", H=328, F=2344, E=8, k=2), 8, None),
    # the ABI's limits: 1024 experts (16 logits per lane of the routing
    # kernel, the permutation's and the GEMMs' group tables at full size) and
    # k = 16
    "max_experts_k16": (synth.small_config("mek", H=64, F=64, E=1024, k=16, logits="zipf"),
                        100, None),
}


@pytest.fixture(scope="module", params=sorted(CASES))
def case(request, orc):
    cfg, T, kind = CASES[request.param]
    layer = synth.make_layer(cfg.name, T, seed=1, device="cuda", cfg=cfg, logits_kind=kind)
    d, _ = host_layer(layer)
    ref = orc.forward(d["x"], d["logits"], cfg.k, d["wg"], d["wu"], d["wd"])
    return request.param, layer, d, ref


def test_route(case):
    name, layer, d, ref = case
    say("moe_route", name, tuple(layer.logits.shape))
    ids, w = B.moe_route(layer.logits, layer.cfg.k)
    torch.cuda.synchronize()
    ids, w = ids.cpu().numpy(), w.cpu().numpy().astype(np.float64)
    assert (ids == ref["ids"]).all()
    bound = route_weight_bound(d["logits"], ref["ids"], ref["w"])
    assert (np.abs(w - ref["w"]) <= bound).all(), np.abs(w - ref["w"]).max()


def test_permute(case, orc):
    name, layer, d, ref = case
    say("moe_permute", name, tuple(layer.x.shape))
    ids = to_dev(ref["ids"])
    off, rt, rd, xp = B.moe_permute(layer.x, ids, layer.cfg.E)
    torch.cuda.synchronize()
    assert (off.cpu().numpy() == ref["offsets"]).all()
    assert (rt.cpu().numpy() == ref["row_token"]).all()
    assert (rd.cpu().numpy() == ref["row_dest"]).all()
    assert (synth.u16(xp) == orc.gather(d["x"], ref["row_token"])).all()


def test_gateup_swiglu(case, orc):
    name, layer, d, ref = case
    x_perm = orc.gather(d["x"], ref["row_token"])
    say("moe_gateup_swiglu", name, x_perm.shape, layer.w_gate.shape)
    h = B.moe_gateup_swiglu(to_dev(x_perm), to_dev(ref["offsets"]), layer.w_gate, layer.w_up)
    torch.cuda.synchronize()
    assert_close(gpu_bf16_f64(h), ref["h"], f"h[{name}]")


def test_down(case, orc):
    name, layer, d, ref = case
    A, F = ref["h"].shape
    h_in = synth.u16(synth.randn_bf16((A, F), 1.0, "cpu", name, "h_in"))
    y_ref = orc.grouped_down(bf16_to_f64(h_in), ref["offsets"], d["wd"])
    say("moe_down", name, (A, F), layer.w_down.shape)
    y = B.moe_down(to_dev(h_in), to_dev(ref["offsets"]), layer.w_down)
    torch.cuda.synchronize()
    assert_close(gpu_bf16_f64(y), y_ref, f"y_perm[{name}]")


def test_grouped_ffn(case, orc):
    name, layer, d, ref = case
    x_perm = orc.gather(d["x"], ref["row_token"])
    say("moe_grouped_ffn", name, x_perm.shape)
    h, y = B.moe_grouped_ffn(to_dev(x_perm), to_dev(ref["offsets"]), layer.w_gate, layer.w_up,
                             layer.w_down)
    torch.cuda.synchronize()
    assert_close(gpu_bf16_f64(h), ref["h"], f"h[{name}]")
    assert_close(gpu_bf16_f64(y), ref["y"], f"y_perm[{name}]")


def test_combine(case, orc):
    name, layer, d, ref = case
    T, k = ref["ids"].shape
    H = layer.cfg.H
    y_in = synth.u16(synth.randn_bf16((T * k, H), 1.0, "cpu", name, "y_in"))
    w32 = ref["w"].astype(np.float32)
    out_ref = orc.combine(bf16_to_f64(y_in), ref["row_dest"], w32.astype(np.float64))
    say("moe_combine", name, (T, H, k))
    out = B.moe_combine(to_dev(y_in), to_dev(ref["row_dest"]), to_dev(w32))
    torch.cuda.synchronize()
    assert_close(gpu_bf16_f64(out), out_ref, f"out[{name}]")


def test_forward(case):
    """The fused layer; small batches (T*k <= 128, E <= 256) route and
    permute in one launch, larger ones in two, large-batch tiles gather rows
    of x."""
    name, layer, d, ref = case
    T, k = ref["ids"].shape
    say("moe_forward", name, (T, layer.cfg.H, layer.cfg.F, layer.cfg.E, k))
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    out = B.moe_forward(layer.x, layer.logits, k, layer.w_gate, layer.w_up, layer.w_down,
                        topk_ids=ids, topk_w=w)
    torch.cuda.synchronize()
    assert (ids.cpu().numpy() == ref["ids"]).all()
    bound = route_weight_bound(d["logits"], ref["ids"], ref["w"])
    assert (np.abs(w.cpu().numpy().astype(np.float64) - ref["w"]) <= bound).all()
    assert_close(gpu_bf16_f64(out), ref["out"], f"out[{name}]")

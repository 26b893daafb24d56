"""GPU parity of the whole layer (moe_forward) with shared experts, its exact
invariants (determinism, power-of-two scaling, zero input, T = 0) and the
empty/degenerate cases."""
import numpy as np
import pytest
import torch

from grouped_gemm_softmax_amd import binding as B
from grouped_gemm_softmax_amd import synth
from helpers import assert_close, gpu_bf16_f64, host_layer, say

pytestmark = pytest.mark.gpu

SHARED_CASES = {
    "dsv3_like": (synth.small_config("d3", H=192, F=96, E=32, k=8, Fs=160, logits="zipf"), 70),
    "qwen2_like_gated": (synth.small_config("q2", H=128, F=88, E=60, k=4, Fs=352,
                                            shared_gated=True), 37),
    "qwen2_like_large_batch": (synth.small_config("q2l", H=128, F=88, E=12, k=4, Fs=176,
                                                  shared_gated=True), 400),
    # shared K three times the routed K: the shared expert's down projection
    # is split into 3 K-slices (small tile) ...
    "shared_long_k": (synth.small_config("slk", H=128, F=256, E=16, k=2, Fs=768,
                                         shared_gated=True), 40),
    # ... and into 4 with the large tile
    "shared_long_k_large_batch": (synth.small_config("slkl", H=128, F=256, E=4, k=2, Fs=1024,
                                                     shared_gated=True), 200),
    # 1024 routed experts and the shared one: every group table at its limit
    "max_groups_shared": (synth.small_config("mgs", H=64, F=64, E=1024, k=8, Fs=128,
                                             shared_gated=True), 50),
}


def _fwd(layer):
    return B.moe_forward(layer.x, layer.logits, layer.cfg.k, layer.w_gate, layer.w_up,
                         layer.w_down, shared=layer.shared)


@pytest.mark.parametrize("name", sorted(SHARED_CASES))
def test_forward_shared_expert(name, orc):
    cfg, T = SHARED_CASES[name]
    layer = synth.make_layer(cfg.name, T, seed=2, device="cuda", cfg=cfg)
    d, sh = host_layer(layer)
    ref = orc.forward(d["x"], d["logits"], cfg.k, d["wg"], d["wu"], d["wd"], shared=sh,
                      keep_intermediates=False)
    say("moe_forward+shared", name, T)
    out = _fwd(layer)
    torch.cuda.synchronize()
    assert_close(gpu_bf16_f64(out), ref["out"], f"out[{name}]")


def _layer(T=96, shared=True):
    cfg = synth.small_config("inv", H=136, F=120, E=7, k=3, Fs=64 if shared else 0,
                             shared_gated=shared)
    return synth.make_layer("inv", T, seed=3, device="cuda", cfg=cfg)


def _double(t):
    return (t.float() * 2).to(torch.bfloat16)     # exact for normal bf16 values


def test_deterministic_bitwise():
    layer = _layer()
    say("determinism")
    a = _fwd(layer).clone()
    b = _fwd(layer)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_power_of_two_scaling_is_exact():
    """out(2 W_down) = 2 out and out(2 W_up) = 2 out bit for bit: scaling by
    two is exact at every fp32 and bf16 rounding of the path."""
    layer = _layer(shared=False)
    say("scaling")
    base = _fwd(layer).float()
    layer.w_down = _double(layer.w_down)
    out_d = _fwd(layer).float()
    layer.w_down = (layer.w_down.float() / 2).to(torch.bfloat16)
    layer.w_up = _double(layer.w_up)
    out_u = _fwd(layer).float()
    torch.cuda.synchronize()
    assert torch.equal(out_d, 2 * base)
    assert torch.equal(out_u, 2 * base)


def test_zero_input_gives_zero():
    layer = _layer()
    layer.x.zero_()
    say("zero input")
    out = _fwd(layer)
    torch.cuda.synchronize()
    assert (out.float() == 0).all()


def test_empty_batch_is_noop():
    cfg = synth.small_config("e0", H=64, F=64, E=4, k=2)
    layer = synth.make_layer("e0", 0, seed=0, device="cuda", cfg=cfg)
    say("T=0")
    out = _fwd(layer)
    torch.cuda.synchronize()
    assert out.shape == (0, 64)


def test_shared_gate_zero_logit_is_half(orc):
    """g_t = 0 gives s_t = 1/2 exactly; with routed W_down zeroed the output is
    half the shared expert's FFN."""
    layer = _layer(T=40)
    layer.shared["gate_logits"].zero_()
    layer.w_down.zero_()
    d, sh = host_layer(layer)
    ref = orc.forward(d["x"], d["logits"], layer.cfg.k, d["wg"], d["wu"], d["wd"], shared=sh,
                      keep_intermediates=False)
    sh_one = dict(sh, gate_logits=None)
    ref_one = orc.forward(d["x"], d["logits"], layer.cfg.k, d["wg"], d["wu"], d["wd"],
                          shared=sh_one, keep_intermediates=False)
    assert np.array_equal(ref["out"], 0.5 * ref_one["out"])
    say("shared gate 0")
    out = _fwd(layer)
    torch.cuda.synchronize()
    assert_close(gpu_bf16_f64(out), ref["out"], "out[gate=0]")


def test_down_projection_k_slices_all_nonempty(orc):
    """A down projection whose K = F = 2056 is 33 steps of 64 for the small
    tile, split 8 ways (a handful of output tiles): each slice covers
    floor((s+1) 33 / 8) - floor(s 33 / 8) >= 4 steps (an equal ceil-sized
    split would leave the last slice at -2 steps). The layer still matches
    the oracle."""
    nk, ks = 33, 8
    sizes = [(s + 1) * nk // ks - s * nk // ks for s in range(ks)]
    assert min(sizes) >= 4 and sum(sizes) == nk
    cfg = synth.small_config("kss", H=128, F=2056, E=4, k=1)
    T = 2
    layer = synth.make_layer("kss", T, seed=4, device="cuda", cfg=cfg)
    # the workspace holds 8 fp32 K-slices of y [T*k, H] (beside the rest)
    assert B.moe_forward_workspace_bytes(T, cfg.H, cfg.F, cfg.E, cfg.k, 0) >= 8 * T * cfg.H * 4
    d, _ = host_layer(layer)
    ref = orc.forward(d["x"], d["logits"], cfg.k, d["wg"], d["wu"], d["wd"],
                      keep_intermediates=False)
    say("moe_forward uneven K-slices", cfg.F)
    out = _fwd(layer)
    torch.cuda.synchronize()
    assert_close(gpu_bf16_f64(out), ref["out"], "out[K-split 8 of 33 steps]")


def test_side_stream_call_keeps_its_workspace():
    """A call on a stream other than torch's current one allocates its
    workspace on that stream: current-stream allocations made right after the
    call (while its kernels may still run) cannot take that memory, and the
    result equals the same call on the current stream."""
    layer = _layer(T=300)
    say("side stream")
    ref = _fwd(layer).clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    out = B.moe_forward(layer.x, layer.logits, layer.cfg.k, layer.w_gate, layer.w_up,
                        layer.w_down, shared=layer.shared, stream=side)
    junk = [torch.full((1 << 20,), 3.0, device="cuda") for _ in range(8)]   # current stream
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))

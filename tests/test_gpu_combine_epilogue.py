"""GPU: with the testing hook moe_set_combine_override(1) the fused layer
combines at decode sizes in the down projection's epilogue (each workgroup
counts its rows into per-(token, column tile) arrival counters, and the one
that completes a tile adds the token's rows in the combine's order). Its
output must equal, bit for bit, the default separate combine launch, for
every weight layout, with and without a (gated) shared expert, with K-sliced
down projections, output widths that are not whole column tiles, k from 1
to 8 and T = 1; and the launch trace must show that no combine kernel ran.
Its results are also checked against the oracle."""
import pytest
import torch

from grouped_gemm_softmax_amd import binding as B
from grouped_gemm_softmax_amd import synth
from helpers import assert_close, gpu_bf16_f64, host_layer, say

pytestmark = pytest.mark.gpu

# every case has fewer than 16 rows per expert (the decode-size tiles)
CASES = {
    "single_token": (synth.small_config("ce1", H=136, F=200, E=8, k=2), 1),
    "k1": (synth.small_config("cek1", H=200, F=96, E=16, k=1), 20),
    "k8_many_experts": (synth.small_config("cek8", H=192, F=96, E=64, k=8, logits="zipf"), 12),
    # routed down projection in 4 K-slices, the shared expert's in 8
    "shared_gated_k_slices": (synth.small_config("cesh", H=200, F=1024, E=8, k=2, Fs=2048,
                                                 shared_gated=True), 6),
    "shared_ungated": (synth.small_config("ceshu", H=128, F=512, E=12, k=4, Fs=256), 9),
    # about 60 touched experts: the 128-column row-major down tile
    "wide_rowmajor_down": (synth.small_config("cewr", H=520, F=256, E=64, k=2), 100),
}
LAYOUTS = ("rowmajor", "packed", "fp8", "mxfp8", "mxfp4")


@pytest.fixture(autouse=True)
def _restore_hooks():
    yield
    B.moe_set_combine_override(-1)
    B.moe_set_diagnostics(0, -1)


def _weights(layer, layout):
    sh = layer.shared
    if layout == "rowmajor":
        return (layer.w_gate, layer.w_up, layer.w_down), sh
    conv = {"packed": B.moe_pack_weights, "fp8": B.moe_quantize_fp8,
            "mxfp8": B.moe_quantize_mxfp8, "mxfp4": B.moe_quantize_mxfp4}[layout]
    w = tuple(conv(t) for t in (layer.w_gate, layer.w_up, layer.w_down))
    if sh is not None:
        sh = dict(w_gate=conv(sh["w_gate"]), w_up=conv(sh["w_up"]), w_down=conv(sh["w_down"]),
                  gate_logits=sh["gate_logits"])
    return w, sh


def _fwd(layer, w, sh):
    return B.moe_forward(layer.x, layer.logits, layer.cfg.k, *w, shared=sh)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("name", sorted(CASES))
def test_epilogue_combine_equals_separate_combine(name, layout, capfd):
    cfg, T = CASES[name]
    assert T * cfg.k < 16 * cfg.E
    layer = synth.make_layer(cfg.name, T, seed=4, device="cuda", cfg=cfg)
    w, sh = _weights(layer, layout)
    say("combine placement", name, layout, T)
    sep = _fwd(layer, w, sh).clone()
    torch.cuda.synchronize()
    B.moe_set_combine_override(1)
    capfd.readouterr()
    B.moe_set_diagnostics(1, -1)
    epi = _fwd(layer, w, sh).clone()
    again = _fwd(layer, w, sh)
    torch.cuda.synchronize()
    B.moe_set_diagnostics(0, -1)
    log = capfd.readouterr().err
    assert "launch grouped_gemm_kernel" in log and "combine_kernel" not in log, log[-2000:]
    assert torch.equal(epi.view(torch.int16), sep.view(torch.int16)), \
        (epi.float() - sep.float()).abs().max().item()
    assert torch.equal(again.view(torch.int16), epi.view(torch.int16))


@pytest.mark.parametrize("name", sorted(CASES))
def test_epilogue_combine_matches_oracle(name, orc):
    cfg, T = CASES[name]
    layer = synth.make_layer(cfg.name, T, seed=5, device="cuda", cfg=cfg)
    d, shh = host_layer(layer)
    ref = orc.forward(d["x"], d["logits"], cfg.k, d["wg"], d["wu"], d["wd"], shared=shh,
                      keep_intermediates=False)
    say("epilogue combine vs oracle", name, T)
    B.moe_set_combine_override(1)
    out = _fwd(layer, (layer.w_gate, layer.w_up, layer.w_down), layer.shared)
    torch.cuda.synchronize()
    assert_close(gpu_bf16_f64(out), ref["out"], f"out[{name}]")


def test_epilogue_combine_from_given_routing():
    """moe_forward_routed (the caller's ids and weights; the permutation
    launch without routing clears the counters) against the default."""
    cfg, T = CASES["shared_gated_k_slices"]
    layer = synth.make_layer(cfg.name, T, seed=6, device="cuda", cfg=cfg)
    ids, w = B.moe_route(layer.logits, cfg.k)
    say("epilogue combine, given routing", T)
    sep = B.moe_forward_routed(layer.x, ids, w, layer.w_gate, layer.w_up, layer.w_down,
                               shared=layer.shared).clone()
    torch.cuda.synchronize()
    B.moe_set_combine_override(1)
    epi = B.moe_forward_routed(layer.x, ids, w, layer.w_gate, layer.w_up, layer.w_down,
                               shared=layer.shared)
    torch.cuda.synchronize()
    assert torch.equal(epi.view(torch.int16), sep.view(torch.int16))

"""The two decode-size gate/up paths give the same bits: the
register-streaming kernel (weights streamed straight into registers) and
the LDS-ring small tile compute the same products in the same order. Both
are selected per launch through the library's testing hook
moe_set_dispatch_override (1: the register-streaming kernel, 0: the ring
tile), on packed bf16 and FP8
weights, with ragged K and N, several row tiles per group and empty
groups. The values themselves are checked against the oracle by the other
GPU tests (which run whichever path the launch rules pick)."""
import pytest
import torch

from grouped_gemm_softmax_amd import binding as B
from grouped_gemm_softmax_amd import synth
from helpers import say, to_dev

pytestmark = pytest.mark.gpu

CASES = {
    # name: (config, T)
    "tiny": (synth.CONFIGS["tiny"], 40),
    "ragged_k_n": (synth.small_config("rk", H=200, F=328, E=6, k=2), 30),
    "many_groups": (synth.small_config("mg", H=256, F=192, E=64, k=8, logits="zipf"), 20),
    "hot_group": (synth.small_config("hg", H=128, F=96, E=4, k=1, logits="zipf"), 60),
}


def gateup(x_perm, off, wg, wu, rs):
    B.moe_set_dispatch_override(rs, -1)
    try:
        h = B.moe_gateup_swiglu(x_perm, off, wg, wu)
        torch.cuda.synchronize()
    finally:
        B.moe_set_dispatch_override(-1, -1)
    return h


@pytest.mark.parametrize("fmt", ["packed", "fp8"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_decode_paths_bit_identical(name, fmt, orc):
    cfg, T = CASES[name]
    layer = synth.make_layer(cfg.name, T, seed=3, device="cuda", cfg=cfg, with_shared=False)
    ids, _ = orc.route(synth.f32(layer.logits), cfg.k)
    off, rt, rd, xp = B.moe_permute(layer.x, to_dev(ids), cfg.E)
    if fmt == "fp8":
        wg, wu = B.moe_quantize_fp8(layer.w_gate), B.moe_quantize_fp8(layer.w_up)
    else:
        wg, wu = B.moe_pack_weights(layer.w_gate), B.moe_pack_weights(layer.w_up)
    say("gate/up decode paths", name, fmt, tuple(xp.shape))
    h_rs = gateup(xp, off, wg, wu, 1)
    h_ring = gateup(xp, off, wg, wu, 0)
    assert torch.equal(h_rs.view(torch.int16), h_ring.view(torch.int16)), (name, fmt)

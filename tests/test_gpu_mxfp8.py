"""GPU tests of the MXFP8 weights (E4M3 codes, one E8M0 scale per 32
K-values of a column): moe_quantize_mxfp8 against the oracle's quantizer
(codes and scale bytes bit for bit, through the documented layouts), and
every mxfp8 call against the bf16 packed call on the dequantized weights
(exact bf16 values, so the same products are summed in the same order: bit
for bit) and against the oracle's layer on the dequantized weights."""
import numpy as np
import pytest
import torch

from grouped_gemm_softmax_amd import binding as B
from grouped_gemm_softmax_amd import synth
from helpers import assert_close, gpu_bf16_f64, say
from test_gpu_forward import SHARED_CASES
from test_gpu_fp8 import _same_bits, bf16_of, to_dev_bf16, unpack_codes
from test_gpu_steps import CASES

pytestmark = pytest.mark.gpu


def unpack_scales(sb: np.ndarray, G: int, K: int, N: int) -> np.ndarray:
    """[G][NB][SKB][64] -> scale bytes [G, ceil(K/32), N] (127 in the padding)."""
    NB, SKB, KB32 = -(-N // 64), 4 * -(-K // 128), -(-K // 32)
    full = sb[:G * NB * SKB * 64].reshape(G, NB, SKB, 64).transpose(0, 2, 1, 3).reshape(
        G, SKB, NB * 64)
    assert (full[:, KB32:, :] == 127).all() and (full[:, :, N:] == 127).all()
    return full[:, :KB32, :N]


@pytest.mark.parametrize("G,K,N", [(3, 200, 328), (2, 64, 128), (1, 136, 72), (2, 8, 16)])
def test_quantize_matches_oracle(G, K, N, orc):
    w = synth.randn_bf16((G, K, N), 0.02, "cuda", "mxq", G, K, N)
    w[:, :32, 1] = 0                                     # an all-zero block
    w[0, :, 2] *= 3000                                   # a wide column
    w[-1, :, 3] *= 1e-30                                 # a tiny column (X raised)
    w[0, :32, 4] = -0.0                                  # a negative-zero block
    w[1 % G, 0, 5] = 30.0                                # a block with saturated codes
    w[1 % G, 1, 5] = 29.0
    say("moe_quantize_mxfp8", (G, K, N))
    q = B.moe_quantize_mxfp8(w)
    torch.cuda.synchronize()
    assert q.codes.numel() == G * -(-N // 64) * -(-K // 64) * 4096
    codes_ref, sb_ref = orc.quantize_mxfp8(synth.u16(w))
    assert (unpack_scales(q.scales.cpu().numpy(), G, K, N) == sb_ref).all()
    assert (unpack_codes(q.codes.cpu().numpy(), G, K, N) == codes_ref).all()


def _dequant_bf16(orc, q: B.Mxfp8Weight, G, K, N) -> torch.Tensor:
    codes = unpack_codes(q.codes.cpu().numpy(), G, K, N)
    d = orc.dequant_mxfp8(codes, unpack_scales(q.scales.cpu().numpy(), G, K, N))
    return to_dev_bf16(bf16_of(d))


@pytest.fixture(scope="module", params=sorted(CASES))
def mx_case(request, orc):
    cfg, T, kind = CASES[request.param]
    layer = synth.make_layer(cfg.name, T, seed=1, device="cuda", cfg=cfg, logits_kind=kind)
    E, H, F = cfg.E, cfg.H, cfg.F
    q = dict(wg=B.moe_quantize_mxfp8(layer.w_gate), wu=B.moe_quantize_mxfp8(layer.w_up),
             wd=B.moe_quantize_mxfp8(layer.w_down))
    torch.cuda.synchronize()
    dq = dict(wg=_dequant_bf16(orc, q["wg"], E, H, F), wu=_dequant_bf16(orc, q["wu"], E, H, F),
              wd=_dequant_bf16(orc, q["wd"], E, F, H))
    return request.param, layer, q, dq


def test_mxfp8_steps_match_bf16_on_dequantized(mx_case, orc):
    name, layer, q, dq = mx_case
    k, E = layer.cfg.k, layer.cfg.E
    say("mxfp8 steps", name)
    ids, _ = B.moe_route(layer.logits, k)
    off, _, _, xp = B.moe_permute(layer.x, ids, E)
    pk = dict(wg=B.moe_pack_weights(dq["wg"]), wu=B.moe_pack_weights(dq["wu"]),
              wd=B.moe_pack_weights(dq["wd"]))
    h8 = B.moe_gateup_swiglu(xp, off, q["wg"], q["wu"])
    h = B.moe_gateup_swiglu(xp, off, pk["wg"], pk["wu"])
    y8 = B.moe_down(h, off, q["wd"])
    y = B.moe_down(h, off, pk["wd"])
    torch.cuda.synchronize()
    _same_bits(h8, h, f"h[{name}]")
    _same_bits(y8, y, f"y_perm[{name}]")


def test_mxfp8_forward(mx_case, orc):
    name, layer, q, dq = mx_case
    k = layer.cfg.k
    say("moe_forward_mxfp8", name, layer.x.shape[0])
    out8 = B.moe_forward(layer.x, layer.logits, k, q["wg"], q["wu"], q["wd"])
    out = B.moe_forward(layer.x, layer.logits, k, B.moe_pack_weights(dq["wg"]),
                        B.moe_pack_weights(dq["wu"]), B.moe_pack_weights(dq["wd"]))
    torch.cuda.synchronize()
    _same_bits(out8, out, f"out[{name}]")
    ref = orc.forward(synth.u16(layer.x), synth.f32(layer.logits), k, synth.u16(dq["wg"]),
                      synth.u16(dq["wu"]), synth.u16(dq["wd"]), keep_intermediates=False)
    assert_close(gpu_bf16_f64(out8), ref["out"], f"out[{name}]")


@pytest.mark.parametrize("name", sorted(SHARED_CASES))
def test_mxfp8_forward_shared_expert(name, orc):
    cfg, T = SHARED_CASES[name]
    layer = synth.make_layer(cfg.name, T, seed=2, device="cuda", cfg=cfg)
    E, H, F, Fs = cfg.E, cfg.H, cfg.F, cfg.Fs
    sh = layer.shared
    qw = [B.moe_quantize_mxfp8(t) for t in (layer.w_gate, layer.w_up, layer.w_down)]
    qs = [B.moe_quantize_mxfp8(sh[n]) for n in ("w_gate", "w_up", "w_down")]
    torch.cuda.synchronize()
    dw = [_dequant_bf16(orc, qw[0], E, H, F), _dequant_bf16(orc, qw[1], E, H, F),
          _dequant_bf16(orc, qw[2], E, F, H)]
    ds = [_dequant_bf16(orc, qs[0], 1, H, Fs)[0], _dequant_bf16(orc, qs[1], 1, H, Fs)[0],
          _dequant_bf16(orc, qs[2], 1, Fs, H)[0]]
    say("moe_forward_mxfp8 + shared", name, T)
    g = sh["gate_logits"]
    out8 = B.moe_forward(layer.x, layer.logits, cfg.k, *qw,
                         shared=dict(w_gate=qs[0], w_up=qs[1], w_down=qs[2], gate_logits=g))
    pk = [B.moe_pack_weights(t) for t in dw]
    pks = [B.moe_pack_weights(t) for t in ds]
    out = B.moe_forward(layer.x, layer.logits, cfg.k, *pk,
                        shared=dict(w_gate=pks[0], w_up=pks[1], w_down=pks[2], gate_logits=g))
    torch.cuda.synchronize()
    _same_bits(out8, out, f"out[{name}]")
    shh = dict(w_gate=synth.u16(ds[0]), w_up=synth.u16(ds[1]), w_down=synth.u16(ds[2]),
               gate_logits=None if g is None else synth.f32(g))
    ref = orc.forward(synth.u16(layer.x), synth.f32(layer.logits), cfg.k, synth.u16(dw[0]),
                      synth.u16(dw[1]), synth.u16(dw[2]), shared=shh, keep_intermediates=False)
    assert_close(gpu_bf16_f64(out8), ref["out"], f"out[{name}]")

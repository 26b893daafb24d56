"""GPU tests of the FP8 (OCP E4M3) weights: moe_quantize_fp8 against the
oracle's quantizer (codes bit for bit, through the documented block layout,
and the per-column scales), and every fp8 call against the bf16 packed call
on the dequantized weights (which are exact bf16 values, so the kernels sum
the same products in the same order: bit for bit) and against the oracle's
layer on the dequantized weights."""
import numpy as np
import pytest
import torch

from grouped_gemm_softmax_amd import binding as B
from grouped_gemm_softmax_amd import synth
from helpers import assert_close, gpu_bf16_f64, say
from test_gpu_forward import SHARED_CASES
from test_gpu_steps import CASES

pytestmark = pytest.mark.gpu


def unpack_codes(codes: np.ndarray, G: int, K: int, N: int) -> np.ndarray:
    """Block layout -> codes [G,K,N]: byte h*2048 + c*32 + p*8 + j of block
    (g, nb, kb) holds row kb*64 + h*32 + 8*(p ^ ((c >> 2) & 3)) + j of
    column nb*64 + c."""
    NB, KB = -(-N // 64), -(-K // 64)
    b = codes[:G * NB * KB * 4096].reshape(G, NB, KB, 2, 64, 4, 8)
    c = np.arange(64)[:, None]
    q = np.arange(4)[None, :] ^ ((c >> 2) & 3)            # [64, 4] logical chunk
    out = np.empty((G, NB, KB, 2, 64, 4, 8), np.uint8)
    out[:, :, :, :, c, q, :] = b                           # physical p -> logical q
    # [G, NB, KB, h, c, q, j] -> [G, KB, h, q, j, NB, c] = [G, K', N']
    full = out.transpose(0, 2, 3, 5, 6, 1, 4).reshape(G, KB * 64, NB * 64)
    assert (full[:, K:, :] == 0).all() and (full[:, :, N:] == 0).all()
    return full[:, :K, :N]


def to_dev_bf16(u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_of(d: np.ndarray) -> np.ndarray:
    """float64 values that are bf16 values -> their bit patterns (checked)."""
    f = d.astype(np.float32)
    u = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert ((u.astype(np.uint32) << 16).view(np.float32) == f).all()
    return u


def _same_bits(a: torch.Tensor, b: torch.Tensor, what: str):
    assert a.shape == b.shape, what
    assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b), what


@pytest.mark.parametrize("G,K,N", [(3, 200, 328), (2, 64, 128), (1, 136, 72), (2, 8, 16)])
def test_quantize_matches_oracle(G, K, N, orc):
    w = synth.randn_bf16((G, K, N), 0.02, "cuda", "fp8q", G, K, N)
    w[:, :, 1] = 0                                      # an all-zero column
    w[0, :, 2] *= 3000                                  # a wide column
    say("moe_quantize_fp8", (G, K, N))
    q = B.moe_quantize_fp8(w)
    torch.cuda.synchronize()
    assert q.codes.numel() == G * -(-N // 64) * -(-K // 64) * 4096
    codes_ref, scales_ref = orc.quantize_e4m3(synth.u16(w))
    assert (q.scales.cpu().numpy().astype(np.float64) == scales_ref).all()
    assert (unpack_codes(q.codes.cpu().numpy(), G, K, N) == codes_ref).all()


def _dequant_bf16(orc, q: B.Fp8Weight, G, K, N) -> torch.Tensor:
    codes = unpack_codes(q.codes.cpu().numpy(), G, K, N)
    d = orc.dequant_e4m3(codes, q.scales.cpu().numpy().astype(np.float64))
    return to_dev_bf16(bf16_of(d))


@pytest.fixture(scope="module", params=sorted(CASES))
def fp8_case(request, orc):
    cfg, T, kind = CASES[request.param]
    layer = synth.make_layer(cfg.name, T, seed=1, device="cuda", cfg=cfg, logits_kind=kind)
    E, H, F = cfg.E, cfg.H, cfg.F
    q = dict(wg=B.moe_quantize_fp8(layer.w_gate), wu=B.moe_quantize_fp8(layer.w_up),
             wd=B.moe_quantize_fp8(layer.w_down))
    torch.cuda.synchronize()
    dq = dict(wg=_dequant_bf16(orc, q["wg"], E, H, F), wu=_dequant_bf16(orc, q["wu"], E, H, F),
              wd=_dequant_bf16(orc, q["wd"], E, F, H))
    return request.param, layer, q, dq


def test_fp8_steps_match_bf16_on_dequantized(fp8_case, orc):
    name, layer, q, dq = fp8_case
    k, E = layer.cfg.k, layer.cfg.E
    say("fp8 steps", name)
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


def test_fp8_forward(fp8_case, orc):
    name, layer, q, dq = fp8_case
    k = layer.cfg.k
    say("moe_forward_fp8", name, layer.x.shape[0])
    out8 = B.moe_forward(layer.x, layer.logits, k, q["wg"], q["wu"], q["wd"])
    out = B.moe_forward(layer.x, layer.logits, k, B.moe_pack_weights(dq["wg"]),
                        B.moe_pack_weights(dq["wu"]), B.moe_pack_weights(dq["wd"]))
    torch.cuda.synchronize()
    _same_bits(out8, out, f"out[{name}]")
    ref = orc.forward(synth.u16(layer.x), synth.f32(layer.logits), k, synth.u16(dq["wg"]),
                      synth.u16(dq["wu"]), synth.u16(dq["wd"]), keep_intermediates=False)
    assert_close(gpu_bf16_f64(out8), ref["out"], f"out[{name}]")


@pytest.mark.parametrize("name", sorted(SHARED_CASES))
def test_fp8_forward_shared_expert(name, orc):
    cfg, T = SHARED_CASES[name]
    layer = synth.make_layer(cfg.name, T, seed=2, device="cuda", cfg=cfg)
    E, H, F, Fs = cfg.E, cfg.H, cfg.F, cfg.Fs
    sh = layer.shared
    qw = [B.moe_quantize_fp8(t) for t in (layer.w_gate, layer.w_up, layer.w_down)]
    qs = [B.moe_quantize_fp8(sh[n]) for n in ("w_gate", "w_up", "w_down")]
    torch.cuda.synchronize()
    dw = [_dequant_bf16(orc, qw[0], E, H, F), _dequant_bf16(orc, qw[1], E, H, F),
          _dequant_bf16(orc, qw[2], E, F, H)]
    ds = [_dequant_bf16(orc, qs[0], 1, H, Fs)[0], _dequant_bf16(orc, qs[1], 1, H, Fs)[0],
          _dequant_bf16(orc, qs[2], 1, Fs, H)[0]]
    say("moe_forward_fp8 + shared", name, T)
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


def test_fp8_rejects_mixed_or_missing_scales():
    cfg = synth.small_config("fx", H=64, F=64, E=2, k=1)
    layer = synth.make_layer(cfg.name, 8, seed=0, device="cuda", cfg=cfg)
    q = B.moe_quantize_fp8(layer.w_gate)
    ids, _ = B.moe_route(layer.logits, 1)
    off, _, _, xp = B.moe_permute(layer.x, ids, 2)
    h = torch.empty((8, 64), dtype=torch.bfloat16, device="cuda")
    rc = B.lib().moe_gateup_swiglu_fp8(B._ptr(xp), B._ptr(off), 8, 64, 64, 2, B._ptr(q.codes),
                                       None, B._ptr(q.codes), B._ptr(q.scales), B._ptr(h), None)
    assert rc == -1                                      # null scales
    torch.cuda.synchronize()

"""GPU parity of the quantized weights (FP8 with per-column scales, MXFP8,
MXFP4) at the full sizes of every configured layer (Mixtral-8x7B-,
DeepSeek-V3- and Qwen2-MoE-shaped, every batch size, the shared expert
included), in the launch configuration bench.py times.

The quantized layer is compared bit for bit with the bf16 packed layer on the
dequantized weights: those are exact bf16 values (a code times a power of
two), so both sum the same products in the same order. The bf16 packed layer
is itself compared with the oracle at these sizes (test_gpu_configs), so this
carries that parity over to every quantized format at every size, including
the tile classes only the large shapes select.

Dequantizing full DeepSeek-V3 weights on the host would take minutes, so it
runs here as plain torch index and cast operations on the device, written
from the documented block layouts; test_device_dequant_matches_oracle checks
those against the oracle's own dequantization."""
import numpy as np
import pytest
import torch

from grouped_gemm_softmax_amd import binding as B
from grouped_gemm_softmax_amd import synth
from helpers import say
from test_gpu_fp8 import _dequant_bf16 as fp8_dequant_oracle
from test_gpu_fp8 import _same_bits
from test_gpu_mxfp4 import _dequant_bf16 as mxfp4_dequant_oracle
from test_gpu_mxfp8 import _dequant_bf16 as mxfp8_dequant_oracle

pytestmark = pytest.mark.gpu

FORMATS = ("fp8", "mxfp8", "mxfp4")
QUANTIZE = dict(fp8=B.moe_quantize_fp8, mxfp8=B.moe_quantize_mxfp8, mxfp4=B.moe_quantize_mxfp4)
CHUNK = 16                      # groups dequantized at a time (bounds the temporaries)

# OCP E2M1: bit 3 is the sign, bits 2..0 index these magnitudes
E2M1 = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _cdiv(a, b):
    return -(-a // b)


def _codes8_gkn(codes: torch.Tensor, G: int, K: int, N: int) -> torch.Tensor:
    """E4M3 block layout -> codes [G,K,N]: byte h*2048 + c*32 + p*8 + j of
    block (g, nb, kb) holds row kb*64 + h*32 + 8*(p ^ ((c >> 2) & 3)) + j of
    column nb*64 + c."""
    NB, KB = _cdiv(N, 64), _cdiv(K, 64)
    b = codes.view(G, NB, KB, 2, 64, 4, 8)
    c = torch.arange(64, device=codes.device)[:, None]
    p = torch.arange(4, device=codes.device)[None, :] ^ ((c >> 2) & 3)   # physical of logical
    logical = b[:, :, :, :, c, p, :]                                    # [G,NB,KB,h,c,q,j]
    full = logical.permute(0, 2, 3, 5, 6, 1, 4).reshape(G, KB * 64, NB * 64)
    return full[:, :K, :N]


def _codes4_gkn(codes: torch.Tensor, G: int, K: int, N: int) -> torch.Tensor:
    """E2M1 block layout -> codes [G,K,N] (0..15): byte h*1024 + c*16 + q*4 +
    i/2 of block (g, nb, kb) holds rows kb*64 + h*32 + 8q + i of column
    nb*64 + c, even i in the low nibble."""
    NB, KB = _cdiv(N, 64), _cdiv(K, 64)
    b = codes.view(G, NB, KB, 2, 64, 4, 4)
    nib = torch.stack([b & 15, b >> 4], dim=-1).reshape(G, NB, KB, 2, 64, 4, 8)
    full = nib.permute(0, 2, 3, 5, 6, 1, 4).reshape(G, KB * 64, NB * 64)
    return full[:, :K, :N]


def _e8m0_scale_gkn(sb: torch.Tensor, G: int, K: int, N: int) -> torch.Tensor:
    """[G][NB][SKB][64] scale bytes -> fp32 scales 2^(s - 127) broadcast to
    [G,K,N] (each byte covers 32 consecutive K-values of one column)."""
    NB, SKB = _cdiv(N, 64), 4 * _cdiv(K, 128)
    s = sb.view(G, NB, SKB, 64).permute(0, 2, 1, 3).reshape(G, SKB, NB * 64)
    s = s[:, :_cdiv(K, 32), :N]
    assert int(s.max()) < 255                                           # no NaN scale
    f = torch.exp2(s.to(torch.float32) - 127.0)
    return f.repeat_interleave(32, dim=1)[:, :K, :]


def _to_bf16_exact(v: torch.Tensor) -> torch.Tensor:
    b = v.to(torch.bfloat16)
    assert torch.equal(b.to(torch.float32), v), "dequantized value is not a bf16 value"
    return b


def dequant_device(fmt: str, q, G: int, K: int, N: int) -> torch.Tensor:
    """Quantized weight -> its exact bf16 values [G,K,N] on the device."""
    out = torch.empty((G, K, N), dtype=torch.bfloat16, device=q.codes.device)
    NB, KB = _cdiv(N, 64), _cdiv(K, 64)
    cblock = (2048 if fmt == "mxfp4" else 4096) * NB * KB
    sblock = NB * 4 * _cdiv(K, 128) * 64
    lut = torch.tensor(E2M1, dtype=torch.float32, device=q.codes.device)
    for g0 in range(0, G, CHUNK):
        g1 = min(G, g0 + CHUNK)
        n = g1 - g0
        cod = q.codes[g0 * cblock:g1 * cblock]
        if fmt == "mxfp4":
            c = _codes4_gkn(cod, n, K, N).to(torch.int64)
            v = lut[c & 7] * (1.0 - 2.0 * (c >> 3).to(torch.float32))
        else:
            v = _codes8_gkn(cod, n, K, N).contiguous().view(torch.float8_e4m3fn).to(
                torch.float32)
        if fmt == "fp8":
            v = v * q.scales[g0:g1, None, :]
        else:
            v = v * _e8m0_scale_gkn(q.scales[g0 * sblock:g1 * sblock], n, K, N)
        out[g0:g1] = _to_bf16_exact(v)
    return out


ORACLE_DEQUANT = dict(fp8=fp8_dequant_oracle, mxfp8=mxfp8_dequant_oracle,
                      mxfp4=mxfp4_dequant_oracle)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("G,K,N", [(3, 200, 328), (20, 72, 136)])
def test_device_dequant_matches_oracle(fmt, G, K, N, orc):
    """The device dequantization used below equals the oracle's (ragged K and
    N, and more groups than one chunk)."""
    w = synth.randn_bf16((G, K, N), 0.02, "cuda", "qfull", fmt, G, K, N)
    w[0, :, 2] *= 3000                                   # a wide column
    w[:, :32, 1] = 0                                     # an all-zero block
    q = QUANTIZE[fmt](w)
    torch.cuda.synchronize()
    got = dequant_device(fmt, q, G, K, N)
    ref = ORACLE_DEQUANT[fmt](orc, q, G, K, N)
    _same_bits(got, ref, f"dequant[{fmt}]")


CASES = [(name, fmt, T) for name in ("mixtral", "mixtral_large", "dsv3", "qwen2")
         for fmt in FORMATS for T in synth.CONFIGS[name].Ts]


@pytest.fixture(scope="module")
def quant_cache():
    cache = {}
    yield cache
    cache.clear()
    torch.cuda.empty_cache()


def _weights(cache, name, fmt):
    """Quantized weights of one config and the packed bf16 copies of their
    dequantized values (one (config, format) pair held at a time)."""
    key = (name, fmt)
    if key not in cache:
        cache.clear()
        torch.cuda.empty_cache()
        cfg = synth.CONFIGS[name]
        layer = synth.make_layer(name, 1, seed=0, device="cuda")
        src = dict(wg=(layer.w_gate, cfg.H, cfg.F), wu=(layer.w_up, cfg.H, cfg.F),
                   wd=(layer.w_down, cfg.F, cfg.H))
        if layer.shared is not None:
            src.update(sg=(layer.shared["w_gate"], cfg.H, cfg.Fs),
                       su=(layer.shared["w_up"], cfg.H, cfg.Fs),
                       sd=(layer.shared["w_down"], cfg.Fs, cfg.H))
        q, pk = {}, {}
        for n, (w, K, N) in src.items():
            G = w.shape[0] if w.dim() == 3 else 1
            say("quantize + device dequant", name, fmt, n, (G, K, N))
            q[n] = QUANTIZE[fmt](w)
            d = dequant_device(fmt, q[n], G, K, N)
            pk[n] = B.moe_pack_weights(d if w.dim() == 3 else d[0])
            del d
        del layer, src
        torch.cuda.synchronize()
        cache[key] = (q, pk)
    return cache[key]


def _shared(ws, g):
    if "sg" not in ws:
        return None
    return dict(w_gate=ws["sg"], w_up=ws["su"], w_down=ws["sd"], gate_logits=g)


@pytest.mark.parametrize("name,fmt,T", CASES, ids=[f"{n}-{f}-T{t}" for n, f, t in CASES])
def test_full_size_quantized_forward(name, fmt, T, quant_cache):
    cfg = synth.CONFIGS[name]
    q, pk = _weights(quant_cache, name, fmt)
    layer = synth.make_layer(name, T, seed=0, device="cuda", with_shared=False,
                             with_weights=False)
    g = synth.shared_gate_logits(cfg, T, 0, "cuda") if cfg.Fs else None
    say("moe_forward full size", name, fmt, T, (cfg.H, cfg.F, cfg.E, cfg.k, cfg.Fs))
    outq = B.moe_forward(layer.x, layer.logits, cfg.k, q["wg"], q["wu"], q["wd"],
                         shared=_shared(q, g))
    say("moe_forward_packed on the dequantized weights", name, fmt, T)
    outp = B.moe_forward(layer.x, layer.logits, cfg.k, pk["wg"], pk["wu"], pk["wd"],
                         shared=_shared(pk, g))
    torch.cuda.synchronize()
    assert torch.isfinite(outq.float()).all()
    _same_bits(outq, outp, f"out[{name}, {fmt}, T={T}]")

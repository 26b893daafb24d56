"""Seeded synthetic inputs for the fused MoE expert layer.

This module only draws random tensors of the layer shapes below. It holds no
step of the layer's arithmetic, and both the HIP path's tests and the CPU
oracle take their inputs from it.

Shapes follow the MoE layers the pages test on. The routed layers are
Mixtral-8x7B, DeepSeek-V3 and Qwen2-MoE, from the Triton MoE page (setupai.cc)
key points and the dispatch-kernel post (lumeric.app). The expert counts, top-k,
shared experts and value distributions are the workload definitions of this
project:

* x ~ N(0, 1), expert weights ~ N(0, 0.02) (the second parameter is the
  standard deviation), every value rounded to bf16 round-to-nearest-even;
* router logits ~ N(0, 1) in fp32, plus a per-expert bias ~ N(0, 0.5) for the
  large-batch Mixtral layer;
* DeepSeek-V3 logits with Zipf(s = 1.2) expert popularity: p_r ~ r^-1.2 over
  ranks r = 1..E, ranks assigned to experts by a seeded permutation, and
  logit[t, e] = ln p_rank(e) + Gumbel(0, 1) noise. Top-1 is then exactly
  Zipf-distributed, and top-k samples without replacement;
* the Qwen2 shared expert's gate logits ~ N(0, 1);
* router weights W_r [E, H] ~ N(0, 0.02) in bf16 (logit spread
  0.02 * sqrt(H): 0.9 at H = 2048, 1.3 at 4096, 1.7 at 7168), or, for the
  tie tests, small integers (exact logits with many ties).

Tensors are drawn with torch's seeded generator on the requested device.
The same (config, T, seed) on the same device always gives the same values.
Weights do not depend on T.
"""
from __future__ import annotations

import math
import zlib
from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

import torch


@dataclass(frozen=True)
class LayerConfig:
    name: str
    H: int
    F: int
    E: int
    k: int
    Ts: Tuple[int, ...]
    logits: str = "normal"          # normal | normal_bias | zipf
    Fs: int = 0                     # shared-expert intermediate size (0: none)
    shared_gated: bool = False      # sigmoid gate on the shared expert
    desc: str = ""


CONFIGS: Dict[str, LayerConfig] = {
    "tiny": LayerConfig("tiny", H=256, F=512, E=8, k=2, Ts=(64,),
                        desc="Tiny MoE layer, T=64, H=256, F=512, E=8, top-2"),
    "mixtral": LayerConfig("mixtral", H=4096, F=14336, E=8, k=2,
                           Ts=(1, 32, 128, 512),
                           desc="Mixtral-8x7B-shaped MoE layer, small batch"),
    "mixtral_large": LayerConfig("mixtral_large", H=4096, F=14336, E=8, k=2,
                                 Ts=(2048, 8192), logits="normal_bias",
                                 desc="Mixtral-8x7B-shaped MoE layer, large "
                                      "batch, per-expert logit bias"),
    "dsv3": LayerConfig("dsv3", H=7168, F=2048, E=256, k=8, Ts=(128, 4096),
                        logits="zipf", Fs=2048, shared_gated=False,
                        desc="DeepSeek-V3-shaped MoE layer, Zipf(1.2) routing "
                             "skew, one always-on shared expert"),
    "qwen2": LayerConfig("qwen2", H=2048, F=1408, E=60, k=4,
                         Ts=(16, 1024, 16384), Fs=5632, shared_gated=True,
                         desc="Qwen2-MoE-shaped layer with a sigmoid-gated "
                              "shared expert"),
}

WEIGHT_STD = 0.02
BIAS_STD = 0.5
ZIPF_S = 1.2


def _seed(*parts) -> int:
    """Stable 63-bit seed from the parts (crc32 of their text, twice)."""
    text = "/".join(str(p) for p in parts).encode()
    return (zlib.crc32(text) << 31) ^ zlib.crc32(text[::-1])


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def randn_bf16(shape, std: float, device, *seed_parts) -> torch.Tensor:
    """N(0, std) drawn in fp32, rounded to bf16 (round-to-nearest-even)."""
    g = _gen(device, *seed_parts)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch.bfloat16)


def expert_weights(shape_e, E: int, std: float, device, *seed_parts) -> torch.Tensor:
    """[E, *shape_e] bf16, drawn one expert at a time so that the fp32
    staging buffer stays one expert large."""
    out = torch.empty((E, *shape_e), dtype=torch.bfloat16, device=device)
    for e in range(E):
        out[e].copy_(randn_bf16(shape_e, std, device, *seed_parts, e))
    return out


def router_logits(cfg: LayerConfig, T: int, seed: int, device,
                  kind: Optional[str] = None) -> torch.Tensor:
    """fp32 [T, E] router logits for the config's distribution.

    kind overrides the config's: 'normal', 'normal_bias', 'zipf',
    'ties_int' (integers in -2..2: many exact ties), 'ties_bf16' (N(0,1)
    rounded to the bf16 grid: occasional ties), 'equal' (all zero),
    'signed_zero' (a mix of +0.0 and -0.0 with a few +-1)."""
    kind = kind or cfg.logits
    E = cfg.E
    g = _gen(device, cfg.name, T, seed, "logits", kind)
    if kind == "normal":
        return torch.randn((T, E), generator=g, device=device)
    if kind == "normal_bias":
        b = torch.randn((E,), generator=_gen(device, cfg.name, seed, "bias"),
                        device=device) * BIAS_STD
        return torch.randn((T, E), generator=g, device=device) + b
    if kind == "zipf":
        perm = torch.randperm(E, generator=_gen(device, cfg.name, seed, "ranks"),
                              device=device)
        ranks = (perm + 1).to(torch.float64)
        logp = -ZIPF_S * torch.log(ranks)
        logp = logp - torch.logsumexp(logp, 0)
        u = torch.rand((T, E), generator=g, device=device, dtype=torch.float64)
        u = u.clamp_(min=1e-300, max=1.0 - 1e-16)
        gumbel = -torch.log(-torch.log(u))
        return (logp[None, :] + gumbel).to(torch.float32)
    if kind == "ties_int":
        return torch.randint(-2, 3, (T, E), generator=g, device=device).float()
    if kind == "ties_bf16":
        return torch.randn((T, E), generator=g, device=device).to(
            torch.bfloat16).float()
    if kind == "equal":
        return torch.zeros((T, E), device=device)
    if kind == "signed_zero":
        r = torch.randint(0, 8, (T, E), generator=g, device=device)
        out = torch.zeros((T, E), device=device)
        out[r == 1] = -0.0
        out[r == 2] = 1.0
        out[r == 3] = -1.0
        out[(r >= 4)] = -0.0
        return out
    raise ValueError(f"unknown logits kind {kind!r}")


@dataclass
class Layer:
    cfg: LayerConfig
    T: int
    seed: int
    x: torch.Tensor                 # [T, H] bf16
    logits: torch.Tensor            # [T, E] fp32
    w_gate: torch.Tensor            # [E, H, F] bf16
    w_up: torch.Tensor              # [E, H, F] bf16
    w_down: torch.Tensor            # [E, F, H] bf16
    shared: Optional[dict] = field(default=None)  # w_gate/w_up [H,Fs], w_down [Fs,H], gate_logits [T]|None


def make_layer(name: str, T: int, seed: int = 0, device="cpu",
               logits_kind: Optional[str] = None, with_shared: bool = True,
               cfg: Optional[LayerConfig] = None, with_weights: bool = True) -> Layer:
    """Draw one layer's inputs. `cfg` overrides the named config's shapes.
    with_weights=False draws only the per-batch tensors (x, logits, gate
    logits) and leaves the weight fields None, for reuse of drawn weights
    (they do not depend on T)."""
    cfg = cfg or CONFIGS[name]
    H, F, E = cfg.H, cfg.F, cfg.E
    x = randn_bf16((T, H), 1.0, device, cfg.name, T, seed, "x")
    logits = router_logits(cfg, T, seed, device, logits_kind)
    if not with_weights:
        shared = None
        if with_shared and cfg.Fs > 0:
            shared = dict(w_gate=None, w_up=None, w_down=None,
                          gate_logits=shared_gate_logits(cfg, T, seed, device))
        return Layer(cfg, T, seed, x, logits, None, None, None, shared)
    wg = expert_weights((H, F), E, WEIGHT_STD, device, cfg.name, seed, "w_gate")
    wu = expert_weights((H, F), E, WEIGHT_STD, device, cfg.name, seed, "w_up")
    wd = expert_weights((F, H), E, WEIGHT_STD, device, cfg.name, seed, "w_down")
    shared = None
    if with_shared and cfg.Fs > 0:
        Fs = cfg.Fs
        shared = dict(
            w_gate=randn_bf16((H, Fs), WEIGHT_STD, device, cfg.name, seed, "ws_gate"),
            w_up=randn_bf16((H, Fs), WEIGHT_STD, device, cfg.name, seed, "ws_up"),
            w_down=randn_bf16((Fs, H), WEIGHT_STD, device, cfg.name, seed, "ws_down"),
            gate_logits=shared_gate_logits(cfg, T, seed, device),
        )
    return Layer(cfg, T, seed, x, logits, wg, wu, wd, shared)


def router_weight(cfg: LayerConfig, seed: int, device, kind: str = "normal") -> torch.Tensor:
    """bf16 [E, H] router weights (row e is expert e's router vector).
    kind 'normal': N(0, WEIGHT_STD); 'ties_int': integers in -2..2."""
    if kind == "normal":
        return randn_bf16((cfg.E, cfg.H), WEIGHT_STD, device, cfg.name, seed, "w_router")
    if kind == "ties_int":
        g = _gen(device, cfg.name, seed, "w_router", kind)
        return torch.randint(-2, 3, (cfg.E, cfg.H), generator=g, device=device).to(torch.bfloat16)
    raise ValueError(f"unknown router weight kind {kind!r}")


def router_input(cfg: LayerConfig, T: int, seed: int, device, kind: str = "normal") -> torch.Tensor:
    """bf16 [T, H] token rows for the router. 'normal' is the layer's x
    (make_layer draws the same values); 'ties_int': integers in -2..2."""
    if kind == "normal":
        return randn_bf16((T, cfg.H), 1.0, device, cfg.name, T, seed, "x")
    if kind == "ties_int":
        g = _gen(device, cfg.name, T, seed, "x", kind)
        return torch.randint(-2, 3, (T, cfg.H), generator=g, device=device).to(torch.bfloat16)
    raise ValueError(f"unknown router input kind {kind!r}")


def shared_gate_logits(cfg: LayerConfig, T: int, seed: int, device) -> Optional[torch.Tensor]:
    """fp32 [T] gate logits of a sigmoid-gated shared expert, else None."""
    if not (cfg.Fs > 0 and cfg.shared_gated):
        return None
    return torch.randn((T,), generator=_gen(device, cfg.name, T, seed, "gate"), device=device)


def small_config(name: str = "small", H=128, F=192, E=6, k=2, Fs=0,
                 shared_gated=False, logits="normal") -> LayerConfig:
    """An ad-hoc small config for tests (several tiles and ragged tails)."""
    return LayerConfig(name, H=H, F=F, E=E, k=k, Ts=(), logits=logits, Fs=Fs,
                       shared_gated=shared_gated)


def u16(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (on the host)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view("uint16")


def f32(t: torch.Tensor):
    return t.detach().contiguous().float().cpu().numpy()


def zipf_probs(E: int, s: float = ZIPF_S):
    """Normalised Zipf probabilities over ranks 1..E (for generator checks)."""
    w = [r ** -s for r in range(1, E + 1)]
    z = math.fsum(w)
    return [v / z for v in w]

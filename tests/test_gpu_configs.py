"""GPU parity at the full sizes of every configured layer (Mixtral-8x7B-,
DeepSeek-V3- and Qwen2-MoE-shaped, every batch size), in the launch
configuration bench.py times (moe_forward). Routing and the permutation are
compared with the oracle in full and bit for bit; layer outputs on a seeded
sample of tokens, which the oracle computes one token at a time (each
token's output depends on that token alone)."""
import numpy as np
import pytest
import torch

from grouped_gemm_softmax_amd import binding as B
from grouped_gemm_softmax_amd import synth
from helpers import assert_close, gpu_bf16_f64, rel_l2, route_weight_bound, say

pytestmark = pytest.mark.gpu

CASES = [(name, T) for name in ("mixtral", "mixtral_large", "dsv3", "qwen2")
         for T in synth.CONFIGS[name].Ts]
N_SAMPLE = 16


@pytest.fixture(scope="module")
def weights_cache():
    cache = {}
    yield cache
    cache.clear()


def _weights(cache, name):
    """Device weights and their host copies, drawn once per config."""
    if name not in cache:
        cache.clear()
        torch.cuda.empty_cache()
        layer = synth.make_layer(name, 1, seed=0, device="cuda")
        host = dict(wg=synth.u16(layer.w_gate), wu=synth.u16(layer.w_up),
                    wd=synth.u16(layer.w_down))
        if layer.shared is not None:
            host["shared"] = {k: synth.u16(v) for k, v in layer.shared.items()
                              if k != "gate_logits"}
        cache[name] = (layer, host)
    return cache[name]


def _packed(cache, name):
    """Packed copies of the cached device weights (made once per config)."""
    key = name + ":packed"
    if key not in cache:
        layer, _ = cache[name]
        pk = dict(wg=B.moe_pack_weights(layer.w_gate), wu=B.moe_pack_weights(layer.w_up),
                  wd=B.moe_pack_weights(layer.w_down))
        if layer.shared is not None:
            pk["shared"] = {n: B.moe_pack_weights(layer.shared[n])
                            for n in ("w_gate", "w_up", "w_down")}
        cache[key] = pk
    return cache[key]


@pytest.mark.parametrize("name,T", CASES, ids=[f"{n}-T{t}" for n, t in CASES])
def test_full_size_forward(name, T, weights_cache, orc):
    cfg = synth.CONFIGS[name]
    wl, host = _weights(weights_cache, name)
    layer = synth.make_layer(name, T, seed=0, device="cuda", with_shared=False, with_weights=False)
    layer.w_gate, layer.w_up, layer.w_down = wl.w_gate, wl.w_up, wl.w_down
    shared = None
    sh_host = None
    if cfg.Fs:
        g = synth.shared_gate_logits(cfg, T, 0, "cuda")
        shared = dict(wl.shared, gate_logits=g)
        sh_host = dict(host["shared"], gate_logits=None if g is None else synth.f32(g))
    k = cfg.k
    say("moe_forward full size", name, T, (cfg.H, cfg.F, cfg.E, k, cfg.Fs))
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    out = B.moe_forward(layer.x, layer.logits, k, layer.w_gate, layer.w_up, layer.w_down,
                        shared=shared, topk_ids=ids, topk_w=w)
    say("moe_permute full size", name, T)
    off, rt, rd, xp = B.moe_permute(layer.x, ids, cfg.E)
    torch.cuda.synchronize()

    x = synth.u16(layer.x)
    logits = synth.f32(layer.logits)
    ids_ref, w_ref = orc.route(logits, k)
    assert (ids.cpu().numpy() == ids_ref).all()
    bound = route_weight_bound(logits, ids_ref, w_ref)
    assert (np.abs(w.cpu().numpy().astype(np.float64) - w_ref) <= bound).all()
    off_ref, rt_ref, rd_ref = orc.permute(ids_ref, cfg.E)
    assert (off.cpu().numpy() == off_ref).all()
    assert (rt.cpu().numpy() == rt_ref).all()
    assert (rd.cpu().numpy() == rd_ref).all()
    assert (synth.u16(xp) == x[rt_ref]).all()

    rng = np.random.default_rng(T)
    toks = np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, N_SAMPLE)]))[:N_SAMPLE]
    ref, ids_s, _ = orc.forward_tokens(x, logits, k, host["wg"], host["wu"], host["wd"], toks,
                                       shared=sh_host)
    got = gpu_bf16_f64(out)[toks]
    assert_close(got, ref, f"out[{name}, T={T}]")
    assert rel_l2(got, ref) < 1e-2

    # the packed-weight layer (what bench.py times): bit-identical to the above
    pk = _packed(weights_cache, name)
    say("moe_forward_packed full size", name, T)
    outp = B.moe_forward(layer.x, layer.logits, k, pk["wg"], pk["wu"], pk["wd"],
                         shared=None if shared is None else dict(pk["shared"],
                                                                 gate_logits=shared["gate_logits"]))
    torch.cuda.synchronize()
    assert torch.equal(outp.view(torch.int16), out.view(torch.int16))
    assert_close(gpu_bf16_f64(outp)[toks], ref, f"packed out[{name}, T={T}]")

"""The forward without allocation (moe_forward_packed_noalloc, the library's
fixed device workspace) against moe_forward_packed (a caller-allocated
workspace), through the C ABI: two calls in a row on each layer shape, the
second with fewer tokens than the first, each bit-identical to the
workspace call on the same inputs (the same kernels and launch plan; the
leftovers of the first call in the fixed array must not reach the second).
A layer whose workspace exceeds the fixed array is rejected with
MOE_ERR_WORKSPACE_TOO_SMALL and its output is left untouched."""
import ctypes

import pytest
import torch

from grouped_gemm_softmax_amd import binding as B
from grouped_gemm_softmax_amd import synth
from helpers import say

pytestmark = pytest.mark.gpu

STATIC_BYTES = 128 << 20
WS_SMALL = -4


def _packed(layer):
    pk = dict(wg=B.moe_pack_weights(layer.w_gate), wu=B.moe_pack_weights(layer.w_up),
              wd=B.moe_pack_weights(layer.w_down))
    if layer.shared is not None:
        pk["shared"] = {n: B.moe_pack_weights(layer.shared[n])
                        for n in ("w_gate", "w_up", "w_down")}
    return pk


def _batch(wl, T, seed):
    """x, logits (and shared gate logits) of T tokens over the weights of wl."""
    cfg = wl.cfg
    lay = synth.make_layer(cfg.name, T, seed=seed, device="cuda", with_weights=False)
    return lay


@pytest.mark.parametrize("name,T1,T2", [("mixtral", 32, 1), ("qwen2", 64, 16)])
def test_noalloc_matches_workspace_call(name, T1, T2):
    cfg = synth.CONFIGS[name]
    wl = synth.make_layer(name, 1, seed=0, device="cuda")
    pk = _packed(wl)
    for T in (T1, T2):
        assert B.moe_forward_workspace_bytes(T, cfg.H, cfg.F, cfg.E, cfg.k, cfg.Fs) <= STATIC_BYTES
        lay = _batch(wl, T, seed=T)
        sh = None
        if cfg.Fs:
            sh = dict(pk["shared"], gate_logits=lay.shared["gate_logits"])
        k = cfg.k
        ids_a = torch.empty((T, k), dtype=torch.int32, device="cuda")
        w_a = torch.empty((T, k), dtype=torch.float32, device="cuda")
        ids_b, w_b = torch.empty_like(ids_a), torch.empty_like(w_a)
        say("moe_forward_packed_noalloc", name, T)
        out_b = B.moe_forward_packed_noalloc(lay.x, lay.logits, k, pk["wg"], pk["wu"], pk["wd"],
                                             shared=sh, topk_ids=ids_b, topk_w=w_b)
        torch.cuda.synchronize()
        say("moe_forward_packed", name, T)
        out_a = B.moe_forward(lay.x, lay.logits, k, pk["wg"], pk["wu"], pk["wd"], shared=sh,
                              topk_ids=ids_a, topk_w=w_a)
        torch.cuda.synchronize()
        assert torch.equal(ids_a, ids_b)
        assert torch.equal(w_a.view(torch.int32), w_b.view(torch.int32))
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), (name, T)


def test_noalloc_rejects_a_layer_beyond_the_fixed_workspace():
    cfg = synth.small_config("big", H=4096, F=14336, E=8, k=2)
    T = 2048
    assert B.moe_forward_workspace_bytes(T, cfg.H, cfg.F, cfg.E, cfg.k, 0) > STATIC_BYTES
    x = torch.zeros((T, cfg.H), dtype=torch.bfloat16, device="cuda")
    logits = torch.zeros((T, cfg.E), dtype=torch.float32, device="cuda")
    out = torch.full((T, cfg.H), 7.0, dtype=torch.bfloat16, device="cuda")
    fake = ctypes.c_void_p(x.data_ptr())          # never read: the call is rejected first
    say("moe_forward_packed_noalloc beyond the limit", T)
    rc = B.lib().moe_forward_packed_noalloc(ctypes.c_void_p(x.data_ptr()),
                                            ctypes.c_void_p(logits.data_ptr()), T, cfg.H, cfg.F,
                                            cfg.E, cfg.k, fake, fake, fake, None,
                                            ctypes.c_void_p(out.data_ptr()), None, None, None)
    torch.cuda.synchronize()
    assert rc == WS_SMALL
    assert (out.float() == 7.0).all()

"""GPU tests of the packed weight layout (moe_pack_weights and the *_packed
calls). The packed tensor must hold every weight exactly once, in its 64 x 64
block, each block as two 32-row halves of 64 column rows, each column row the
column's 32 K-values in whole chunks of 8 K-consecutive values, with zeros
past K and N; every
packed call must return bit for bit what the row-major call returns (the
kernels stage identical data in LDS and sum the same products in the same
order); and the packed layer must match the oracle like the row-major one."""
import numpy as np
import pytest
import torch

from grouped_gemm_softmax_amd import binding as B
from grouped_gemm_softmax_amd import synth
from helpers import assert_close, gpu_bf16_f64, host_layer, say
from test_gpu_forward import SHARED_CASES
from test_gpu_steps import CASES

pytestmark = pytest.mark.gpu


def _same_bits(a: torch.Tensor, b: torch.Tensor, what: str):
    assert a.shape == b.shape, what
    assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b), what


@pytest.mark.parametrize("G,K,N", [(3, 72, 136), (2, 64, 128), (1, 136, 72), (2, 8, 16)])
def test_pack_layout_block_rows(G, K, N):
    rng = np.random.default_rng(G * 1000 + K + N)
    # distinct non-zero bit patterns, so every value can be traced
    vals = rng.choice(np.arange(1, 65536, dtype=np.uint16), size=G * K * N, replace=False)
    w_host = vals.reshape(G, K, N)
    w = torch.from_numpy(w_host.view(np.int16).copy()).view(torch.bfloat16).cuda()
    say("moe_pack_weights", (G, K, N))
    p = B.moe_pack_weights(w)
    torch.cuda.synchronize()
    NB, KB = -(-N // 64), -(-K // 64)
    assert p.data.numel() == G * NB * KB * 8192
    got = p.data.cpu().numpy().view(np.uint16).reshape(G, NB, KB, 2, 64, 4, 8)
    # expected: per block, half h, column c, chunk q: W[kb*64 + 32h + 8q + e, nb*64 + c]
    exp = np.zeros((G, KB * 64, NB * 64), np.uint16)
    exp[:, :K, :N] = w_host
    exp = exp.reshape(G, KB, 2, 4, 8, NB, 64).transpose(0, 5, 1, 2, 6, 3, 4)  # [G,NB,KB,2,64,4,8]
    # each packed chunk is one whole chunk of its column row: order the
    # chunks of both by their first element (zero chunks are equal anyway)
    key_g = np.argsort(got[..., 0], axis=-1, kind="stable")
    key_e = np.argsort(exp[..., 0], axis=-1, kind="stable")
    got_s = np.take_along_axis(got, key_g[..., None], axis=-2)
    exp_s = np.take_along_axis(exp, key_e[..., None], axis=-2)
    assert (got_s == exp_s).all()


@pytest.fixture(scope="module", params=sorted(CASES))
def packed_case(request):
    cfg, T, kind = CASES[request.param]
    layer = synth.make_layer(cfg.name, T, seed=1, device="cuda", cfg=cfg, logits_kind=kind)
    pk = dict(wg=B.moe_pack_weights(layer.w_gate), wu=B.moe_pack_weights(layer.w_up),
              wd=B.moe_pack_weights(layer.w_down))
    return request.param, layer, pk


def test_packed_steps_match_rowmajor(packed_case):
    name, layer, pk = packed_case
    k, E = layer.cfg.k, layer.cfg.E
    say("packed steps", name)
    ids, _ = B.moe_route(layer.logits, k)
    off, _, _, xp = B.moe_permute(layer.x, ids, E)
    h = B.moe_gateup_swiglu(xp, off, layer.w_gate, layer.w_up)
    hp = B.moe_gateup_swiglu(xp, off, pk["wg"], pk["wu"])
    y = B.moe_down(h, off, layer.w_down)
    yp = B.moe_down(h, off, pk["wd"])
    torch.cuda.synchronize()
    _same_bits(hp, h, f"h[{name}]")
    _same_bits(yp, y, f"y_perm[{name}]")


def test_packed_forward(packed_case, orc):
    name, layer, pk = packed_case
    k = layer.cfg.k
    T = layer.x.shape[0]
    say("moe_forward_packed", name, T)
    out = B.moe_forward(layer.x, layer.logits, k, layer.w_gate, layer.w_up, layer.w_down)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    outp = B.moe_forward(layer.x, layer.logits, k, pk["wg"], pk["wu"], pk["wd"], topk_ids=ids)
    torch.cuda.synchronize()
    _same_bits(outp, out, f"out[{name}]")
    d, _ = host_layer(layer)
    ref = orc.forward(d["x"], d["logits"], k, d["wg"], d["wu"], d["wd"], keep_intermediates=False)
    assert (ids.cpu().numpy() == ref["ids"]).all()
    assert_close(gpu_bf16_f64(outp), ref["out"], f"out[{name}]")


@pytest.mark.parametrize("name", sorted(SHARED_CASES))
def test_packed_forward_shared_expert(name):
    cfg, T = SHARED_CASES[name]
    layer = synth.make_layer(cfg.name, T, seed=2, device="cuda", cfg=cfg)
    sh = layer.shared
    shp = dict(w_gate=B.moe_pack_weights(sh["w_gate"]), w_up=B.moe_pack_weights(sh["w_up"]),
               w_down=B.moe_pack_weights(sh["w_down"]), gate_logits=sh["gate_logits"])
    say("moe_forward_packed+shared", name, T)
    out = B.moe_forward(layer.x, layer.logits, cfg.k, layer.w_gate, layer.w_up, layer.w_down,
                        shared=sh)
    outp = B.moe_forward(layer.x, layer.logits, cfg.k, B.moe_pack_weights(layer.w_gate),
                         B.moe_pack_weights(layer.w_up), B.moe_pack_weights(layer.w_down),
                         shared=shp)
    torch.cuda.synchronize()
    _same_bits(outp, out, f"out[{name}]")


def test_mixed_layouts_rejected():
    layer = synth.make_layer("tiny", 8, seed=1, device="cuda", cfg=synth.CONFIGS["tiny"])
    with pytest.raises(TypeError):
        B.moe_forward(layer.x, layer.logits, layer.cfg.k, B.moe_pack_weights(layer.w_gate),
                      layer.w_up, layer.w_down)

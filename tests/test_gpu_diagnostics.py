"""GPU tests of the library's diagnostics: moe_check_topk_ids finds expert
ids outside [0, E); with the id check on (MOE_DEBUG, here through
moe_set_diagnostics) the calls that take caller ids return MOE_ERR_BAD_IDS
before launching anything that would use them, and give the same results as
with the check off on valid ids; the launch trace (MOE_TRACE) writes one line
per kernel launch naming the kernel and, for the grouped GEMMs, the tile.

Every call on invalid ids is made only after moe_check_topk_ids has been
shown to flag that very tensor, so no kernel ever reads an id outside
[0, E)."""
import pytest
import torch

from grouped_gemm_softmax_amd import binding as B
from grouped_gemm_softmax_amd import synth
from helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture
def diag():
    yield B
    B.moe_set_diagnostics(0, 0)
    B.moe_set_diagnostics(-1, -1)


def _layer():
    cfg = synth.small_config("dg", H=64, F=96, E=6, k=2)
    return cfg, synth.make_layer(cfg.name, 20, seed=4, device="cuda", cfg=cfg, with_shared=False)


def _bad(ids, where, value):
    b = ids.clone()
    b.view(-1)[where] = value
    return b


def test_check_topk_ids(diag):
    cfg, layer = _layer()
    ids, _ = B.moe_route(layer.logits, cfg.k)
    say("moe_check_topk_ids", tuple(ids.shape), cfg.E)
    assert B.moe_check_topk_ids(ids, cfg.E)
    n = ids.numel()
    for where, value in [(0, cfg.E), (n - 1, -1), (n // 2, 1 << 30), (3, -(1 << 31))]:
        assert not B.moe_check_topk_ids(_bad(ids, where, value), cfg.E), (where, value)
    # the count is cleared for every call
    assert B.moe_check_topk_ids(ids, cfg.E)
    assert B.moe_check_topk_ids(ids[:0], cfg.E)


def test_id_check_rejects_before_launching(diag):
    cfg, layer = _layer()
    E, k, T = cfg.E, cfg.k, layer.x.shape[0]
    ids, w = B.moe_route(layer.logits, k)
    bad = _bad(ids, 5, E)
    assert not B.moe_check_topk_ids(bad, E)        # the guard: the check flags this tensor
    off0, rt0, rd0, xp0 = B.moe_permute(layer.x, ids, E)
    out0 = B.moe_forward_routed(layer.x, ids, w, layer.w_gate, layer.w_up, layer.w_down)
    torch.cuda.synchronize()

    B.moe_set_diagnostics(-1, 1)
    say("id check on: valid ids")
    off, rt, rd, xp = B.moe_permute(layer.x, ids, E)
    out = B.moe_forward_routed(layer.x, ids, w, layer.w_gate, layer.w_up, layer.w_down)
    torch.cuda.synchronize()
    for a, b in [(off, off0), (rt, rt0), (rd, rd0), (xp.view(torch.int16), xp0.view(torch.int16)),
                 (out.view(torch.int16), out0.view(torch.int16))]:
        assert torch.equal(a, b)

    say("id check on: an id equal to E")
    sentinel = torch.full_like(off, -7)
    with pytest.raises(B.MoeError) as e:
        B.moe_permute(layer.x, bad, E, out=(sentinel, rt.clone(), rd.clone(), xp.clone()))
    assert e.value.status == B.MOE_ERR_BAD_IDS
    torch.cuda.synchronize()
    assert (sentinel == -7).all()                  # nothing was launched on the bad ids
    with pytest.raises(B.MoeError) as e:
        B.moe_forward_routed(layer.x, bad, w, layer.w_gate, layer.w_up, layer.w_down)
    assert e.value.status == B.MOE_ERR_BAD_IDS
    dout = torch.ones_like(layer.x)
    with pytest.raises(B.MoeError) as e:
        B.moe_backward(layer.x, bad, w, layer.w_gate, layer.w_up, layer.w_down, dout)
    assert e.value.status == B.MOE_ERR_BAD_IDS
    with pytest.raises(B.MoeError) as e:
        B.moe_route_backward(bad, w, torch.ones_like(w), E)
    assert e.value.status == B.MOE_ERR_BAD_IDS
    torch.cuda.synchronize()


def test_launch_trace(diag, capfd):
    cfg, layer = _layer()
    capfd.readouterr()
    B.moe_set_diagnostics(1, -1)
    out = B.moe_forward(layer.x, layer.logits, cfg.k, layer.w_gate, layer.w_up, layer.w_down)
    torch.cuda.synchronize()
    B.moe_set_diagnostics(0, -1)
    B.moe_forward(layer.x, layer.logits, cfg.k, layer.w_gate, layer.w_up, layer.w_down)
    torch.cuda.synchronize()
    err = capfd.readouterr().err
    lines = [l for l in err.splitlines() if l.startswith("moe: launch ")]
    say("trace lines", len(lines))
    names = [l.split()[2] for l in lines]
    # five launches: routing (+ permutation), gate/up, down, combine
    assert len(lines) in (4, 5), lines
    assert names[-1] == "combine_kernel" and " combine=0" in lines[-2], lines
    gemm = [l for l in lines if " grouped_gemm_kernel " in l or " rs_gateup_kernel " in l]
    assert len(gemm) == 2 and all(" tile=" in l and " grid=" in l for l in gemm), gemm
    assert out.shape == layer.x.shape
    # the combine in the down projection's epilogue (testing hook)
    B.moe_set_combine_override(1)
    try:
        B.moe_set_diagnostics(1, -1)
        B.moe_forward(layer.x, layer.logits, cfg.k, layer.w_gate, layer.w_up, layer.w_down)
        torch.cuda.synchronize()
    finally:
        B.moe_set_diagnostics(0, -1)
        B.moe_set_combine_override(-1)
    lines = [l for l in capfd.readouterr().err.splitlines() if l.startswith("moe: launch ")]
    assert len(lines) in (3, 4) and lines[-1].split()[2] == "grouped_gemm_kernel", lines
    assert " combine=1" in lines[-1], lines

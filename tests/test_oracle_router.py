"""Pins of the oracle's router projection logits[t,e] = sum_h x[t,h] W_r[e,h]
(fp64) against numpy's fp64 matrix product, exact integer arithmetic, exact
power-of-two scaling and the composition with the routing step. CPU only."""
import numpy as np
import pytest
import torch

from grouped_gemm_softmax_amd import synth


def f64(u):
    return (np.asarray(u, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_router_logits_hand_worked(orc):
    # x = [1, 2, -1, 0.5]; rows of W_r: [1,1,1,1], [3,-1,0,2], [0,0,0,0]
    # logits: 1+2-1+0.5 = 2.5; 3-2+0+1 = 2; 0 (bf16 bit patterns below)
    x = np.array([[0x3F80, 0x4000, 0xBF80, 0x3F00]], np.uint16)
    w = np.array([[0x3F80, 0x3F80, 0x3F80, 0x3F80],
                  [0x4040, 0xBF80, 0x0000, 0x4000],
                  [0x0000, 0x0000, 0x0000, 0x0000]], np.uint16)
    assert orc.router_logits(x, w).tolist() == [[2.5, 2.0, 0.0]]


@pytest.mark.parametrize("T,H,E", [(7, 96, 5), (33, 200, 60), (1, 4096, 8), (16, 8, 1)])
def test_router_logits_match_numpy_matmul(orc, T, H, E):
    cfg = synth.small_config(H=H, E=E)
    x = synth.u16(synth.router_input(cfg, T, 1, "cpu"))
    w = synth.u16(synth.router_weight(cfg, 1, "cpu"))
    got = orc.router_logits(x, w)
    ref = f64(x) @ f64(w).T          # [T,H] x [H,E]: a transposed W_r fails here
    # both sides are fp64 sums of the same exact products in different orders
    bound = 2 * H * 2.0 ** -53 * (np.abs(f64(x)) @ np.abs(f64(w)).T) + 1e-300
    assert got.shape == (T, E)
    assert (np.abs(got - ref) <= bound).all()


def test_router_logits_integer_inputs_exact(orc):
    cfg = synth.small_config(H=520, E=37)
    x = synth.router_input(cfg, 19, 2, "cpu", "ties_int")
    w = synth.router_weight(cfg, 2, "cpu", "ties_int")
    ref = x.to(torch.int64).numpy() @ w.to(torch.int64).numpy().T
    got = orc.router_logits(synth.u16(x), synth.u16(w))
    assert (got == ref.astype(np.float64)).all()


def test_router_logits_power_of_two_scaling_exact(orc):
    cfg = synth.small_config(H=136, E=12)
    x = synth.router_input(cfg, 9, 3, "cpu")
    w = synth.router_weight(cfg, 3, "cpu")
    base = orc.router_logits(synth.u16(x), synth.u16(w))
    # scaling one operand by 4 is exact in bf16 and in every fp64 partial sum
    assert (orc.router_logits(synth.u16(x * 4), synth.u16(w)) == 4 * base).all()
    assert (orc.router_logits(synth.u16(x), synth.u16(-w)) == -base).all()


def test_router_then_route_picks_largest_scores(orc):
    cfg = synth.small_config(H=256, E=60, k=4)
    x = synth.u16(synth.router_input(cfg, 40, 4, "cpu"))
    w = synth.u16(synth.router_weight(cfg, 4, "cpu"))
    lg = orc.router_logits(x, w)
    ids, _ = orc.route(lg.astype(np.float32), 4)
    # brute force: full sort of numpy's product, descending, stable
    ref = f64(x) @ f64(w).T
    brute = np.argsort(-ref.astype(np.float32).astype(np.float64), axis=1, kind="stable")[:, :4]
    assert (ids == brute).all()

"""GPU parity of the training backward at full layer sizes (Mixtral-8x7B-,
DeepSeek-V3- and Qwen2-MoE-shaped), in the configuration `bench.py
--backward` times: moe_backward on row-major weights for the routing of the
layer's own logits. The oracle computes sampled outputs one by one: dx and
the routing-weight gradient of sampled tokens (each depends on that token
alone: at least 1024 tokens, all of them when T <= 1024, with every 16-row
block of every expert's rows holding a sampled assignment) and 64 whole
columns of the three weight gradients (each a sum over one expert's rows:
the first, last, most and least loaded experts among them). The tolerance
is the one derived in test_gpu_backward.py (5 u times the root-sum-square of the GPU's bf16
rounding errors as they propagate, u = 2^-8), evaluated here for the
sampled elements only."""
import numpy as np
import pytest
import torch

from grouped_gemm_softmax_amd import binding as B
from grouped_gemm_softmax_amd import synth
from helpers import check_block_coverage, gpu_bf16_f64, rel_l2, say, stratified_tokens

pytestmark = pytest.mark.gpu

U_BF16 = 2.0 ** -8
LAMBDA = 5.0
CASES = [("mixtral", 512), ("mixtral_large", 2048), ("dsv3", 4096), ("qwen2", 1024)]
N_COL = 64


def f32w(u):
    return (np.asarray(u, np.uint16).astype(np.uint32) << 16).view(np.float32)


def silu_parts(G):
    sg = 1.0 / (1.0 + np.exp(-G))
    return G * sg, sg * (1.0 + G * (1.0 - sg))


def token_bounds(x, wg, wu, wd, ids, w, dout, toks, dx_ref):
    """Root-sum-square rounding scales (divided by u) of dx and d_topk_w for
    the sampled tokens, from each token's rows, taken expert by expert (a
    token picks an expert at most once; float32 is ample for a bound)."""
    H = x.shape[1]
    k = ids.shape[1]
    bdx2, bdw = np.zeros((len(toks), H)), np.zeros((len(toks), k))
    f32 = lambda v: v.astype(np.float32)
    sel = ids[toks]
    for e in np.unique(sel):
        si, sj = np.nonzero(sel == e)
        t = toks[si]
        X, DR = f32w(x[t]), f32w(dout[t])
        DY = w[t, sj][:, None].astype(np.float32) * DR
        Wg, Wu, Wd = f32w(wg[e]), f32w(wu[e]), f32w(wd[e])
        G, U = (X @ Wg).astype(np.float64), (X @ Wu).astype(np.float64)
        silu, dsilu = silu_parts(G)
        h = silu * U
        Wd2 = Wd * Wd
        dh = (DY @ Wd.T).astype(np.float64)
        dG, dU = dh * U * dsilu, dh * silu
        dGr2 = dG ** 2 + (dh * U * dsilu) ** 2 + (0.5 * dh * U * G) ** 2
        dUr2 = dU ** 2 + (1.1 * dh * G) ** 2
        bdx2[si] += f32(dGr2) @ (Wg * Wg).T + f32(dUr2) @ (Wu * Wu).T
        bdw[si, sj] = np.sqrt(np.sum((DR * DR) * (f32(h * h) @ Wd2), axis=1, dtype=np.float64))
    return np.sqrt(bdx2 + dx_ref ** 2), bdw


def column_bounds(x, wg, wu, wd, w, dout, ecol, fcol, offsets, row_token, row_dest):
    """Root-sum-square rounding scales (divided by u) of the sampled
    weight-gradient columns, from the expert's rows."""
    H = x.shape[1]
    wrow = np.empty(row_token.shape[0])
    wrow[row_dest.reshape(-1)] = w.reshape(-1)
    bg, bu, bd = (np.zeros((len(ecol), H)) for _ in range(3))
    for s, (e, f) in enumerate(zip(ecol, fcol)):
        r = slice(offsets[e], offsets[e + 1])
        xs = f32w(x[row_token[r]]).astype(np.float64)
        ds = f32w(dout[row_token[r]]).astype(np.float64) * wrow[r][:, None]   # dy rows
        wgc, wuc = f32w(wg[e][:, f]).astype(np.float64), f32w(wu[e][:, f]).astype(np.float64)
        wdr = f32w(wd[e][f]).astype(np.float64)
        G, U = xs @ wgc, xs @ wuc
        silu, dsilu = silu_parts(G)
        dh = ds @ wdr
        dG, dU = dh * U * dsilu, dh * silu
        dGr2 = dG ** 2 + (dh * U * dsilu) ** 2 + (0.5 * dh * U * G) ** 2
        dUr2 = dU ** 2 + (1.1 * dh * G) ** 2
        bg[s] = np.sqrt((xs * xs).T @ dGr2)
        bu[s] = np.sqrt((xs * xs).T @ dUr2)
        bd[s] = np.sqrt(2 * (ds * ds).T @ (silu * U) ** 2)
    return bg, bu, bd


def check(gpu, ref, bound, what):
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    allowed = LAMBDA * U_BF16 * bound + 1e-6 * rms + 1e-30
    err = np.abs(gpu - ref)
    assert np.isfinite(gpu).all(), what
    bad = err > allowed
    assert not bad.any(), (what, int(bad.sum()), float((err / allowed).max()))
    assert rel_l2(gpu, ref) <= 1e-2, (what, rel_l2(gpu, ref))


@pytest.mark.parametrize("name,T", CASES, ids=[f"{n}-T{t}" for n, t in CASES])
def test_full_size_backward(name, T, orc):
    cfg = synth.CONFIGS[name]
    E, k, H, F = cfg.E, cfg.k, cfg.H, cfg.F
    layer = synth.make_layer(name, T, seed=0, device="cuda", with_shared=False)
    # the routing of the layer's logits, from the oracle (an input of both sides)
    ids_h, w64 = orc.route(synth.f32(layer.logits), k)
    w_h = w64.astype(np.float32)
    ids, w = torch.from_numpy(ids_h).cuda(), torch.from_numpy(w_h).cuda()
    g = torch.Generator(device="cuda").manual_seed(1)
    dout = torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16)
    say("moe_backward full size", name, T, (H, F, E, k))
    grads = B.moe_backward(layer.x, ids, w, layer.w_gate, layer.w_up, layer.w_down, dout)
    torch.cuda.synchronize()

    host = dict(x=synth.u16(layer.x), wg=synth.u16(layer.w_gate), wu=synth.u16(layer.w_up),
                wd=synth.u16(layer.w_down), dout=synth.u16(dout))
    offsets, row_token, row_dest = orc.permute(ids_h, E)
    rng = np.random.default_rng(T + E)
    toks, _ = stratified_tokens(offsets, row_token, T, rng)
    check_block_coverage(toks, offsets, row_dest)
    used = np.flatnonzero(np.diff(offsets) > 0)
    # columns: the first and last used expert, the most and least loaded,
    # then random used experts; the first and last column among them
    cnt = np.diff(offsets)[used]
    ecol = np.concatenate([used[[0, -1, np.argmax(cnt), np.argmin(cnt)]],
                           rng.choice(used, N_COL - 4)])
    fcol = rng.integers(0, F, N_COL)
    fcol[0], fcol[1] = F - 1, 0
    say("oracle samples", name, T, len(toks), "tokens,", N_COL, "weight-gradient columns")
    dx_g = gpu_bf16_f64(grads["dx"])[toks]
    dw_g = grads["d_topk_w"].cpu().numpy().astype(np.float64)[toks]
    ei, fi = torch.from_numpy(ecol).long().cuda(), torch.from_numpy(fcol).long().cuda()
    cg_g = grads["dw_gate"][ei, :, fi].cpu().numpy().astype(np.float64)
    cu_g = grads["dw_up"][ei, :, fi].cpu().numpy().astype(np.float64)
    cd_g = grads["dw_down"][ei, fi, :].cpu().numpy().astype(np.float64)
    del grads, layer
    torch.cuda.empty_cache()

    dx, dw = orc.backward_tokens(host["x"], ids_h, w_h, host["wg"], host["wu"], host["wd"],
                                 host["dout"], toks)
    cg, cu, cd = orc.backward_wcols(host["x"], ids_h, w_h, host["wg"], host["wu"], host["wd"],
                                    host["dout"], ecol, fcol)
    bdx, bdw = token_bounds(host["x"], host["wg"], host["wu"], host["wd"], ids_h, w_h,
                            host["dout"], toks, dx)
    bg, bu, bd = column_bounds(host["x"], host["wg"], host["wu"], host["wd"], w_h, host["dout"],
                               ecol, fcol, offsets, row_token, row_dest)
    check(dx_g, dx, bdx, f"dx[{name}, T={T}]")
    check(dw_g, dw, bdw, f"d_topk_w[{name}, T={T}]")
    check(cg_g, cg, bg, f"dw_gate columns[{name}, T={T}]")
    check(cu_g, cu, bu, f"dw_up columns[{name}, T={T}]")
    check(cd_g, cd, bd, f"dw_down rows[{name}, T={T}]")

"""GPU parity of the training backward (moe_backward, moe_route_backward)
through the C ABI against the CPU oracle's fp64 chain rule, at sizes the
oracle finishes in seconds. The shapes make the backward's GEMMs (dh with the
SwiGLU backward, the two dx products, the three K-grouped weight gradients)
see every tile class, ragged M, N and K tails, empty experts, and a token
count of zero.

Tolerance, derived from the arithmetic: the GPU rounds G, U, h, dG, dU and
dx to bf16, and dy = w dout for the W_down gradient (relative error at most
u = 2^-8 each, spread evenly); dh = w (dout W_down^T) is formed in fp32 from
the unrounded dout, so no rounding of dy reaches dG, dU or dx. Every product
accumulates in fp32 (error ~K 2^-24, far below u); the oracle keeps fp64. Each rounding is an independent error of at most u times the
rounded value, so an element's error is a sum of such terms weighted by how
they propagate; its root-sum-square, u * rss (grad_bounds below: the
backward chain with every sum of products replaced by the root of the sum
of squares), sets the scale. The test allows 5 u * rss per element (the
uniform rounding model's standard deviation is u * rss / sqrt(3), so 5 u *
rss is 8.7 of them; measured maxima are 1.4 - 2.4 u * rss over millions of
elements), plus a relative L2 error under 1e-2 per gradient. A flat
per-element tolerance does not fit: gradients are not O(1), and with few
rows per expert one row's stacked roundings (U, G, dG; ~1 % of that
row's term) can set a weight-gradient element, while a worst-case
(absolute-value) bound is 3 - 60 times the values themselves because of
the cancellation in the long sums."""
import numpy as np
import pytest
import torch

from grouped_gemm_softmax_amd import binding as B
from grouped_gemm_softmax_amd import synth
from helpers import bf16_to_f64, gpu_bf16_f64, host_layer, rel_l2, say, to_dev
from test_gpu_fp8 import to_dev_bf16

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": (synth.CONFIGS["tiny"], 64),
    "ragged_small_batch": (synth.small_config("rs", H=200, F=328, E=6, k=2), 90),
    "ragged_large128": (synth.small_config("rl", H=200, F=328, E=6, k=2), 500),
    "ragged_large256": (synth.small_config("rl256", H=200, F=328, E=4, k=2), 500),
    "large256_whole_k": (synth.small_config("l256", H=256, F=384, E=4, k=2), 500),
    "zipf_empty_experts": (synth.small_config("zm", H=256, F=128, E=64, k=8, logits="zipf"), 60),
    "single_token": (synth.small_config("st", H=136, F=72, E=8, k=2), 1),
    "k_equals_E": (synth.small_config("ke", H=64, F=48, E=5, k=5), 23),
    # the ABI's limits: 1024 experts, k = 16 (the two dx products then take
    # one launch each: their 2048 groups exceed one launch's group table)
    "max_experts_k16": (synth.small_config("mek", H=64, F=64, E=1024, k=16, logits="zipf"), 100),
}


def dout_bf16(T, H, seed):
    g = torch.Generator().manual_seed(1000 + seed)
    return torch.randn((T, H), generator=g).to(torch.bfloat16)


U_BF16 = 2.0 ** -8   # bf16 unit roundoff (8-bit significand)
LAMBDA = 5.0


def grad_bounds(orc, x, ids, w, wg, wu, wd, dout):
    """Root-sum-square scale (divided by u) of the GPU's rounding error on
    each gradient: the backward chain in float64, dense per row, with each
    rounded quantity contributing its own magnitude and each sum of products
    the root of the sum of their squares (for the tolerance only, never as
    an expected value). |d silu'/dz| <= 1/2 and |d silu/dz| <= 1.1 carry the
    rounding of G."""
    f = lambda a: bf16_to_f64(a)
    x, wg, wu, wd, dout = f(x), f(wg), f(wu), f(wd), f(dout)
    w = np.asarray(w, np.float64)
    T, H = x.shape
    E, _, F = wg.shape
    k = ids.shape[1]
    offsets, row_token, row_dest = orc.permute(ids, E)
    A = T * k
    eid = np.repeat(np.arange(E), np.diff(offsets))
    wrow = np.empty(A)
    wrow[row_dest.reshape(-1)] = w.reshape(-1)
    xp = x[row_token]
    G = np.einsum("ph,phf->pf", xp, wg[eid])
    U = np.einsum("ph,phf->pf", xp, wu[eid])
    sg = 1.0 / (1.0 + np.exp(-G))
    silu, dsilu = G * sg, sg * (1.0 + G * (1.0 - sg))
    h = silu * U
    dy = wrow[:, None] * dout[row_token]
    dh = np.einsum("pc,pfc->pf", dy, wd[eid])
    dG, dU = dh * U * dsilu, dh * silu
    dGr2 = dG ** 2 + (dh * U * dsilu) ** 2 + (0.5 * dh * U * G) ** 2
    dUr2 = dU ** 2 + (1.1 * dh * G) ** 2
    b = dict(dwg=np.zeros((E, H, F)), dwu=np.zeros((E, H, F)), dwd=np.zeros((E, F, H)))
    for e in range(E):
        r = slice(offsets[e], offsets[e + 1])
        b["dwg"][e] = np.sqrt((xp[r] ** 2).T @ dGr2[r])
        b["dwu"][e] = np.sqrt((xp[r] ** 2).T @ dUr2[r])
        b["dwd"][e] = np.sqrt(2 * (h[r] ** 2).T @ dy[r] ** 2)       # h and dy rounded
    dxr2 = np.einsum("pf,phf->ph", dGr2, wg[eid] ** 2) + np.einsum("pf,phf->ph", dUr2,
                                                                   wu[eid] ** 2)
    dx2 = np.zeros((T, H))
    np.add.at(dx2, row_token, dxr2)
    dx = np.zeros((T, H))
    np.add.at(dx, row_token, np.einsum("pf,phf->ph", dG, wg[eid]) +
              np.einsum("pf,phf->ph", dU, wu[eid]))
    b["dx"] = np.sqrt(dx2 + dx ** 2)                                 # + dx's own rounding
    # <dout, y>, y from rounded h
    ya2 = np.einsum("pf,pfc->pc", h ** 2, wd[eid] ** 2)
    dwr = np.sqrt((dout[row_token] ** 2 * ya2).sum(axis=1))
    b["dw"] = np.empty((T, k))
    b["dw"].reshape(-1)[:] = dwr[row_dest.reshape(-1)]
    return b


def check_grad(gpu, ref, bound, what, l2=1e-2):
    gpu = np.asarray(gpu, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), what
    if ref.size == 0:
        return
    rms = float(np.sqrt(np.mean(ref * ref)))
    allowed = LAMBDA * U_BF16 * bound + 1e-6 * rms + 1e-30
    err = np.abs(gpu - ref)
    bad = err > allowed
    if bad.any():
        i = np.unravel_index(np.argmax(err / allowed), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {err.size} out of tolerance; worst at {i}: "
            f"gpu={gpu[i]!r} ref={ref[i]!r} allowed={allowed[i]:.3e} (rms {rms:.3e})")
    r = rel_l2(gpu, ref)
    assert r <= l2, f"{what}: relative L2 error {r:.3e} > {l2}"


@pytest.fixture(scope="module", params=sorted(CASES))
def case(request, orc):
    cfg, T = CASES[request.param]
    layer = synth.make_layer(cfg.name, T, seed=2, device="cuda", cfg=cfg,
                             with_shared=False)
    d, _ = host_layer(layer)
    ids, w = orc.route(d["logits"], cfg.k)
    w32 = w.astype(np.float32)
    dout = dout_bf16(T, cfg.H, 2)
    dout_u = synth.u16(dout)
    ref = orc.backward(d["x"], ids, w32, d["wg"], d["wu"], d["wd"], dout_u)
    ref["bound"] = grad_bounds(orc, d["x"], ids, w32, d["wg"], d["wu"], d["wd"], dout_u)
    return request.param, layer, ids, w32, dout.cuda(), ref


def test_backward(case):
    name, layer, ids, w32, dout, ref = case
    say("moe_backward", name, tuple(layer.x.shape), tuple(layer.w_gate.shape))
    g = B.moe_backward(layer.x, to_dev(ids), to_dev(w32), layer.w_gate, layer.w_up,
                       layer.w_down, dout)
    torch.cuda.synchronize()
    b = ref["bound"]
    check_grad(gpu_bf16_f64(g["dx"]), ref["dx"], b["dx"], f"dx[{name}]")
    check_grad(g["d_topk_w"].cpu().numpy(), ref["dw"], b["dw"], f"d_topk_w[{name}]")
    check_grad(g["dw_gate"].cpu().numpy(), ref["dwg"], b["dwg"], f"dw_gate[{name}]")
    check_grad(g["dw_up"].cpu().numpy(), ref["dwu"], b["dwu"], f"dw_up[{name}]")
    check_grad(g["dw_down"].cpu().numpy(), ref["dwd"], b["dwd"], f"dw_down[{name}]")
    # experts no token chose: exactly zero weight gradients
    used = np.zeros(layer.cfg.E, bool)
    used[np.unique(ids)] = True
    for n in ("dw_gate", "dw_up", "dw_down"):
        assert not g[n][torch.from_numpy(~used).cuda()].any(), n


def test_backward_deterministic(case):
    name, layer, ids, w32, dout, _ = case
    say("moe_backward twice", name)
    a = B.moe_backward(layer.x, to_dev(ids), to_dev(w32), layer.w_gate, layer.w_up,
                       layer.w_down, dout)
    b = B.moe_backward(layer.x, to_dev(ids), to_dev(w32), layer.w_gate, layer.w_up,
                       layer.w_down, dout)
    torch.cuda.synchronize()
    for n in a:
        assert torch.equal(a[n].view(torch.int16) if a[n].dtype == torch.bfloat16 else a[n],
                           b[n].view(torch.int16) if b[n].dtype == torch.bfloat16 else b[n]), n


def test_backward_no_tokens():
    cfg = synth.small_config("z0", H=64, F=48, E=3, k=2)
    layer = synth.make_layer(cfg.name, 0, seed=0, device="cuda", cfg=cfg, with_shared=False)
    say("moe_backward T=0")
    ids = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    w = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    dout = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    g = B.moe_backward(layer.x, ids, w, layer.w_gate, layer.w_up, layer.w_down, dout)
    torch.cuda.synchronize()
    for n in ("dw_gate", "dw_up", "dw_down"):
        assert g[n].numel() > 0 and not g[n].any(), n


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (300, 64, 8), (77, 5, 5), (50, 16, 1)])
def test_route_backward(orc, T, E, k):
    rng = np.random.default_rng(T + E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = orc.route(logits, k)
    w32 = w.astype(np.float32)
    dw = rng.standard_normal((T, k)).astype(np.float32)
    say("moe_route_backward", T, E, k)
    got = B.moe_route_backward(to_dev(ids), to_dev(w32), to_dev(dw), E)
    torch.cuda.synchronize()
    got = got.cpu().numpy().astype(np.float64)
    ref = orc.route_backward(ids, w32, dw.astype(np.float64), E)
    # fp32 arithmetic: k products and sums, one product and difference
    s = np.abs(w32.astype(np.float64) * dw).sum(axis=1, keepdims=True)
    bound = np.zeros_like(ref)
    wd = np.abs(w32.astype(np.float64)) * (np.abs(dw) + s) * (k + 4) * 2.0 ** -24
    np.put_along_axis(bound, ids.astype(np.int64), wd, 1)
    assert (np.abs(got - ref) <= bound + 1e-30).all(), np.abs(got - ref).max()
    mask = np.zeros((T, E), bool)
    np.put_along_axis(mask, ids.astype(np.int64), True, 1)
    assert not got[~mask].any()


# ---- with the shared expert (moe_backward_shared) ---------------------------

SHARED_CASES = {
    # Qwen2-MoE-like: a sigmoid gate on a shared expert 4x wider than F
    "gated_wide_shared": (synth.small_config("gw", H=128, F=96, E=8, k=2), 70, 384, True),
    # DeepSeek-V3-like: an always-on shared expert (s = 1), ragged sizes
    "ungated_ragged": (synth.small_config("ur", H=200, F=136, E=6, k=2), 90, 264, False),
    # many rows per expert: the 128- and 256-row tiles for both segments
    "gated_large_tiles": (synth.small_config("gl", H=256, F=128, E=4, k=2), 520, 256, True),
}


@pytest.mark.parametrize("name", sorted(SHARED_CASES))
def test_backward_shared(orc, name):
    """The shared expert's term is a one-expert layer over all tokens with
    routing weight s_t: its bounds are grad_bounds of that layer (s_t as the
    weight), and dx, the sum of the routed and the shared parts, is bounded
    by the root-sum-square of both."""
    cfg, T, Fs, gated = SHARED_CASES[name]
    layer = synth.make_layer(cfg.name, T, seed=4, device="cuda", cfg=cfg, with_shared=False)
    d, _ = host_layer(layer)
    rng = np.random.default_rng(T + Fs)
    mk = lambda *s: synth.u16(torch.from_numpy(rng.standard_normal(s) * 0.05).to(torch.bfloat16))
    wsg, wsu, wsd = mk(cfg.H, Fs), mk(cfg.H, Fs), mk(Fs, cfg.H)
    gl = rng.standard_normal(T).astype(np.float32) if gated else None
    ids, w = orc.route(d["logits"], cfg.k)
    w32 = w.astype(np.float32)
    dout = dout_bf16(T, cfg.H, 4)
    dout_u = synth.u16(dout)
    say("moe_backward_shared", name, T, Fs, gated)
    shared = dict(w_gate=to_dev_bf16(wsg), w_up=to_dev_bf16(wsu), w_down=to_dev_bf16(wsd),
                  gate_logits=None if gl is None else to_dev(gl))
    g = B.moe_backward(layer.x, to_dev(ids), to_dev(w32), layer.w_gate, layer.w_up,
                       layer.w_down, dout.cuda(), shared=shared)
    g0 = B.moe_backward(layer.x, to_dev(ids), to_dev(w32), layer.w_gate, layer.w_up,
                        layer.w_down, dout.cuda())
    torch.cuda.synchronize()
    ref = orc.backward(d["x"], ids, w32, d["wg"], d["wu"], d["wd"], dout_u)
    rs = orc.shared_backward(d["x"], wsg, wsu, wsd, gl, dout_u)
    b = grad_bounds(orc, d["x"], ids, w32, d["wg"], d["wu"], d["wd"], dout_u)
    s = np.ones(T) if gl is None else 1.0 / (1.0 + np.exp(-gl.astype(np.float64)))
    bs = grad_bounds(orc, d["x"], np.zeros((T, 1), np.int32), s.astype(np.float32)[:, None],
                     wsg[None], wsu[None], wsd[None], dout_u)
    check_grad(gpu_bf16_f64(g["dx"]), ref["dx"] + rs["dx"], np.sqrt(b["dx"] ** 2 + bs["dx"] ** 2),
               f"dx[{name}]")
    check_grad(g["dw_gate_sh"].cpu().numpy(), rs["dwsg"], bs["dwg"][0], f"dw_gate_sh[{name}]")
    check_grad(g["dw_up_sh"].cpu().numpy(), rs["dwsu"], bs["dwu"][0], f"dw_up_sh[{name}]")
    check_grad(g["dw_down_sh"].cpu().numpy(), rs["dwsd"], bs["dwd"][0], f"dw_down_sh[{name}]")
    if gated:
        check_grad(g["d_gate_logits"].cpu().numpy(), rs["dg"], bs["dw"][:, 0] * s * (1 - s),
                   f"d_gate_logits[{name}]")
    else:
        assert g["d_gate_logits"] is None
    # the routed gradients do not change with the shared expert beside them
    for n in ("d_topk_w", "dw_gate", "dw_up", "dw_down"):
        assert torch.equal(g[n], g0[n]), n


def test_backward_shared_no_tokens():
    cfg = synth.small_config("zs", H=64, F=48, E=3, k=2)
    layer = synth.make_layer(cfg.name, 0, seed=0, device="cuda", cfg=cfg, with_shared=False)
    say("moe_backward_shared T=0")
    ids = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    w = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    dout = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    sh = dict(w_gate=torch.ones((64, 32), dtype=torch.bfloat16, device="cuda"),
              w_up=torch.ones((64, 32), dtype=torch.bfloat16, device="cuda"),
              w_down=torch.ones((32, 64), dtype=torch.bfloat16, device="cuda"),
              gate_logits=torch.empty(0, dtype=torch.float32, device="cuda"))
    g = B.moe_backward(layer.x, ids, w, layer.w_gate, layer.w_up, layer.w_down, dout, shared=sh)
    torch.cuda.synchronize()
    for n in ("dw_gate", "dw_up", "dw_down", "dw_gate_sh", "dw_up_sh", "dw_down_sh"):
        assert g[n].numel() > 0 and not g[n].any(), n

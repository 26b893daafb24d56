"""Pins of the oracle's expert FFN, combine and whole forward against a numpy
fp64 dense brute force (every expert on every token, masked by the top-k set
and weighted), the E=1,k=1 textbook SwiGLU FFN, hand-worked fixtures and exact
invariants. CPU only."""
import json
import math
import os

import numpy as np
import pytest

from grouped_gemm_softmax_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f64(u16):
    return (np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_u16(vals):
    """Exact-in-bf16 float values -> uint16 bit patterns (asserts exactness)."""
    a = np.asarray(vals, np.float32)
    u = a.view(np.uint32)
    assert (u & 0xFFFF == 0).all(), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def dense_swiglu(x, wg, wu, wd):
    """Textbook SwiGLU FFN in numpy fp64 matmuls (a different evaluation order
    and code path from the oracle's loops)."""
    g = x @ wg
    u = x @ wu
    return (g / (1.0 + np.exp(-g)) * u) @ wd


def dense_moe(x, logits, k, wg, wu, wd, shared=None):
    """Brute force: run every expert on every token, keep the top-k experts
    (full stable sort), weight by the softmax over their logits, sum."""
    T = x.shape[0]
    E = wg.shape[0]
    xd = f64(x)
    l = logits.astype(np.float64)
    order = np.stack([np.argsort(-r, kind="stable") for r in l]) if T else np.zeros((0, E), int)
    mask = np.zeros((T, E))
    for t in range(T):
        top = order[t, :k]
        z = np.exp(l[t, top] - l[t, top].max())
        mask[t, top] = z / z.sum()
    out = np.zeros((T, wd.shape[2]))
    for e in range(E):
        ye = dense_swiglu(xd, f64(wg[e]), f64(wu[e]), f64(wd[e]))
        out += mask[:, e:e + 1] * ye
    if shared is not None:
        ysh = dense_swiglu(xd, f64(shared["w_gate"]), f64(shared["w_up"]), f64(shared["w_down"]))
        g = shared.get("gate_logits")
        s = np.ones(T) if g is None else 1.0 / (1.0 + np.exp(-g.astype(np.float64)))
        out += s[:, None] * ysh
    return out


def np_layer(layer):
    d = dict(x=synth.u16(layer.x), logits=synth.f32(layer.logits),
             wg=synth.u16(layer.w_gate), wu=synth.u16(layer.w_up), wd=synth.u16(layer.w_down))
    sh = None
    if layer.shared is not None:
        sh = dict(w_gate=synth.u16(layer.shared["w_gate"]), w_up=synth.u16(layer.shared["w_up"]),
                  w_down=synth.u16(layer.shared["w_down"]),
                  gate_logits=None if layer.shared["gate_logits"] is None else synth.f32(layer.shared["gate_logits"]))
    return d, sh


def test_golden_ffn_cases(orc):
    with open(os.path.join(GOLDEN, "ffn_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = to_u16(c["x"])
        wg, wu, wd = to_u16(c["w_gate"]), to_u16(c["w_up"]), to_u16(c["w_down"])
        r = orc.forward(x, np.array(c["logits"], np.float32), c["k"], wg, wu, wd)
        np.testing.assert_allclose(r["out"], c["out"], rtol=1e-14, atol=1e-15, err_msg=c["why"])
        if c["h"] is not None:
            np.testing.assert_allclose(r["h"], c["h"], rtol=1e-14, err_msg=c["why"])


@pytest.mark.parametrize("cfgname,T,shared", [("tiny", 64, False), ("small", 37, False),
                                              ("small_shared", 29, True), ("small_gated", 21, True)])
def test_oracle_matches_dense_brute_force(orc, cfgname, T, shared):
    cfgs = {"tiny": synth.CONFIGS["tiny"],
            "small": synth.small_config(H=96, F=80, E=7, k=3),
            "small_shared": synth.small_config("ss", H=64, F=48, E=9, k=4, Fs=112, logits="zipf"),
            "small_gated": synth.small_config("sg", H=80, F=32, E=5, k=2, Fs=64, shared_gated=True)}
    layer = synth.make_layer(cfgname, T, seed=4, cfg=cfgs[cfgname])
    d, sh = np_layer(layer)
    r = orc.forward(d["x"], d["logits"], layer.cfg.k, d["wg"], d["wu"], d["wd"], shared=sh)
    ref = dense_moe(d["x"], d["logits"], layer.cfg.k, d["wg"], d["wu"], d["wd"], shared=sh)
    scale = max(1.0, np.abs(ref).max())
    assert np.abs(r["out"] - ref).max() <= 1e-12 * scale


def test_e1_k1_is_textbook_swiglu_ffn(orc):
    cfg = synth.small_config("e1", H=72, F=40, E=1, k=1)
    layer = synth.make_layer("e1", 13, seed=7, cfg=cfg)
    d, _ = np_layer(layer)
    r = orc.forward(d["x"], d["logits"], 1, d["wg"], d["wu"], d["wd"])
    ref = dense_swiglu(f64(d["x"]), f64(d["wg"][0]), f64(d["wu"][0]), f64(d["wd"][0]))
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-14)
    assert (r["w"] == 1.0).all() and (r["row_dest"].ravel() == np.arange(13)).all()


def _small_layer(seed=11, shared=False):
    cfg = synth.small_config("inv", H=64, F=48, E=6, k=2, Fs=32 if shared else 0, shared_gated=shared)
    return np_layer(synth.make_layer("inv", 19, seed=seed, cfg=cfg)) + (cfg,)


def test_exact_scaling_invariants(orc):
    d, _, cfg = _small_layer()
    base = orc.forward(d["x"], d["logits"], cfg.k, d["wg"], d["wu"], d["wd"])["out"]
    two = lambda u: (u.astype(np.int32) + (1 << 7)).astype(np.uint16)  # exponent +1: exact *2 for normal bf16
    assert (f64(two(d["wd"]))[f64(d["wd"]) != 0] == 2 * f64(d["wd"])[f64(d["wd"]) != 0]).all()
    wd2 = np.where(f64(d["wd"]) == 0, d["wd"], two(d["wd"])).astype(np.uint16)
    wu2 = np.where(f64(d["wu"]) == 0, d["wu"], two(d["wu"])).astype(np.uint16)
    out_d = orc.forward(d["x"], d["logits"], cfg.k, d["wg"], d["wu"], wd2)["out"]
    out_u = orc.forward(d["x"], d["logits"], cfg.k, d["wg"], wu2, d["wd"])["out"]
    assert (out_d == 2 * base).all()
    assert (out_u == 2 * base).all()


def test_zero_input_gives_zero_output(orc):
    d, _, cfg = _small_layer()
    r = orc.forward(np.zeros_like(d["x"]), d["logits"], cfg.k, d["wg"], d["wu"], d["wd"])
    assert (r["out"] == 0).all()


def test_token_permutation_equivariance(orc):
    d, _, cfg = _small_layer(seed=3)
    T = d["x"].shape[0]
    perm = np.random.default_rng(0).permutation(T)
    a = orc.forward(d["x"], d["logits"], cfg.k, d["wg"], d["wu"], d["wd"])["out"]
    b = orc.forward(d["x"][perm], d["logits"][perm], cfg.k, d["wg"], d["wu"], d["wd"])["out"]
    assert (b == a[perm]).all()


def test_zeroed_expert_drops_its_term(orc):
    d, _, cfg = _small_layer(seed=5)
    r = orc.forward(d["x"], d["logits"], cfg.k, d["wg"], d["wu"], d["wd"])
    e0 = int(r["ids"][0, 0])
    wd0 = d["wd"].copy()
    wd0[e0] = 0
    r0 = orc.forward(d["x"], d["logits"], cfg.k, d["wg"], d["wu"], wd0)
    xd = f64(d["x"])
    ye = dense_swiglu(xd, f64(d["wg"][e0]), f64(d["wu"][e0]), f64(d["wd"][e0]))
    wt = np.where(r["ids"] == e0, r["w"], 0.0).sum(1)
    np.testing.assert_allclose(r0["out"], r["out"] - wt[:, None] * ye, rtol=1e-10, atol=1e-12)


def test_forward_tokens_equals_full_forward_rows(orc):
    for shared in (False, True):
        d, sh, cfg = _small_layer(seed=9, shared=shared)
        if shared:
            sh = dict(w_gate=synth.u16(synth.randn_bf16((64, 32), 0.02, "cpu", "s1")),
                      w_up=synth.u16(synth.randn_bf16((64, 32), 0.02, "cpu", "s2")),
                      w_down=synth.u16(synth.randn_bf16((32, 64), 0.02, "cpu", "s3")),
                      gate_logits=np.linspace(-2, 2, 19).astype(np.float32))
        full = orc.forward(d["x"], d["logits"], cfg.k, d["wg"], d["wu"], d["wd"], shared=sh)
        toks = [18, 0, 7, 7, 3]
        out, ids, w = orc.forward_tokens(d["x"], d["logits"], cfg.k, d["wg"], d["wu"], d["wd"], toks, shared=sh)
        assert (out == full["out"][toks]).all()
        assert (ids == full["ids"][toks]).all() and (w == full["w"][toks]).all()


def test_shared_gate_closed_forms(orc):
    s = orc.shared_gate(np.array([0.0, math.log(3.0)], np.float32), 2)
    assert s[0] == 0.5
    assert abs(s[1] - 0.75) < 1e-7
    assert (orc.shared_gate(None, 3) == 1.0).all()


def test_shared_only_equals_dense_shared_ffn(orc):
    """Routed down weights zeroed: the output is the shared expert's dense
    SwiGLU FFN (s = 1, the always-on form)."""
    cfg = synth.small_config("so", H=64, F=32, E=4, k=2, Fs=48)
    layer = synth.make_layer("so", 11, seed=2, cfg=cfg)
    d, sh = np_layer(layer)
    r = orc.forward(d["x"], d["logits"], 2, d["wg"], d["wu"], np.zeros_like(d["wd"]), shared=sh)
    ref = dense_swiglu(f64(d["x"]), f64(sh["w_gate"]), f64(sh["w_up"]), f64(sh["w_down"]))
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-14)


def test_grouped_steps_compose_to_forward(orc):
    d, _, cfg = _small_layer(seed=13)
    full = orc.forward(d["x"], d["logits"], cfg.k, d["wg"], d["wu"], d["wd"])
    ids, w = orc.route(d["logits"], cfg.k)
    off, rt, rd = orc.permute(ids, cfg.E)
    xp = orc.gather(d["x"], rt)
    h = orc.grouped_gateup(xp, off, d["wg"], d["wu"])
    y = orc.grouped_down(h, off, d["wd"])
    out = orc.combine(y, rd, w)
    assert (out == full["out"]).all() and (h == full["h"]).all() and (y == full["y"]).all()


def test_intermediate_size_matches_page_figure():
    """The Triton MoE page (setupai.cc), key points, says fusing gate+up removes
    a 470 MB intermediate buffer. One [T*k, F] bf16 tensor of the
    Mixtral-shaped layer at T=8192, top-2 is 16384*14336*2 B = 469.8 MB, which
    rounds to that figure (a consistency check of this project's reading)."""
    cfg = synth.CONFIGS["mixtral_large"]
    T = 8192
    nbytes = T * cfg.k * cfg.F * 2
    assert nbytes == 469_762_048 and round(nbytes / 1e6) == 470

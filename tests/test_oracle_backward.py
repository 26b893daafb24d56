"""Pins of the oracle's training backward (oracle.backward, route_backward):
central finite differences of an independent numpy float64 dense forward
(every expert on every token, masked by the routing) for every gradient
output; exact linearity in dout; dout = 0 and W_down = 0 special cases; and
the softmax-over-top-k backward against finite differences, with its rows
summing to zero. CPU only."""
import numpy as np
import pytest
import torch


def bf16(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def f64(u: np.ndarray) -> np.ndarray:
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dense_forward(x, ids, w, wg, wu, wd):
    """out[t] = sum_j w[t,j] * (silu(x_t Wg[e]) * (x_t Wu[e])) Wd[e], float64,
    every expert on every token, masked by the routing."""
    T, k = ids.shape
    E = wg.shape[0]
    out = np.zeros((T, wd.shape[2]))
    for e in range(E):
        g = x @ wg[e]
        u = x @ wu[e]
        y = (g / (1 + np.exp(-g)) * u) @ wd[e]
        mask = np.zeros(T)
        for j in range(k):
            mask += np.where(ids[:, j] == e, w[:, j], 0.0)
        out += mask[:, None] * y
    return out


def make_case(seed, T=7, H=12, F=10, E=4, k=2):
    rng = np.random.default_rng(seed)
    x = bf16(rng.standard_normal((T, H)))
    wg = bf16(rng.standard_normal((E, H, F)) * 0.3)
    wu = bf16(rng.standard_normal((E, H, F)) * 0.3)
    wd = bf16(rng.standard_normal((E, F, H)) * 0.3)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.1, 0.9, (T, k)).astype(np.float32)
    dout = bf16(rng.standard_normal((T, H)))
    return x, ids, w, wg, wu, wd, dout


@pytest.mark.parametrize("seed", [0, 1])
def test_backward_matches_finite_differences(orc, seed):
    x, ids, w, wg, wu, wd, dout = make_case(seed)
    g = orc.backward(x, ids, w, wg, wu, wd, dout)
    X, WG, WU, WD, R = f64(x), f64(wg), f64(wu), f64(wd), f64(dout)
    W = w.astype(np.float64)
    loss = lambda X, W, WG, WU, WD: float((dense_forward(X, ids, W, WG, WU, WD) * R).sum())
    rng = np.random.default_rng(100 + seed)
    args = [X, W, WG, WU, WD]
    for name, pos in (("dx", 0), ("dw", 1), ("dwg", 2), ("dwu", 3), ("dwd", 4)):
        a = args[pos]
        for _ in range(12):
            idx = tuple(rng.integers(0, s) for s in a.shape)
            eps = 1e-5 * max(1.0, abs(a[idx]))
            plus = [v.copy() for v in args]
            minus = [v.copy() for v in args]
            plus[pos][idx] += eps
            minus[pos][idx] -= eps
            fd = (loss(*plus) - loss(*minus)) / (2 * eps)
            assert abs(g[name][idx] - fd) <= 1e-6 * max(1.0, abs(fd)), (name, idx, g[name][idx], fd)


def test_backward_linear_in_dout_and_zero(orc):
    x, ids, w, wg, wu, wd, dout = make_case(3)
    g1 = orc.backward(x, ids, w, wg, wu, wd, dout)
    g2 = orc.backward(x, ids, w, wg, wu, wd, bf16(f64(dout) * 2))
    for n in g1:
        assert np.array_equal(g2[n], 2 * g1[n]), n
    g0 = orc.backward(x, ids, w, wg, wu, wd, np.zeros_like(dout))
    for n in g0:
        assert not g0[n].any(), n


def test_backward_zero_down_weights(orc):
    x, ids, w, wg, wu, wd, dout = make_case(4)
    g = orc.backward(x, ids, w, wg, wu, np.zeros_like(wd), dout)
    # y = 0 and dh = 0: no routing-weight, input or gate/up gradient
    for n in ("dw", "dx", "dwg", "dwu"):
        assert not g[n].any(), n
    assert g["dwd"].any()          # h^T dy does not vanish


def test_route_backward(orc):
    rng = np.random.default_rng(5)
    T, E, k = 6, 9, 3
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = orc.route(logits, k)
    w = w.astype(np.float32)
    dw = rng.standard_normal((T, k))
    dl = orc.route_backward(ids, w, dw, E)
    # finite differences of L = sum_j softmax(l_sel)_j dw_j in float64
    sel = np.take_along_axis(logits.astype(np.float64), ids.astype(np.int64), 1)

    def L(s):
        e = np.exp(s - s.max(axis=1, keepdims=True))
        return float(((e / e.sum(axis=1, keepdims=True)) * dw).sum())

    for t in range(T):
        for j in range(k):
            p, m = sel.copy(), sel.copy()
            p[t, j] += 1e-6
            m[t, j] -= 1e-6
            fd = (L(p) - L(m)) / 2e-6
            assert abs(dl[t, ids[t, j]] - fd) <= 1e-6
    # experts not selected get 0; each row sums to 0 (softmax invariance)
    mask = np.zeros((T, E), bool)
    np.put_along_axis(mask, ids.astype(np.int64), True, 1)
    assert not dl[~mask].any()
    # (exactly for exact weights; the fp32 weights sum to 1 within k * 2^-24,
    # which leaves sum_j w_j dw_j times that)
    s = np.abs((w.astype(np.float64) * dw).sum(axis=1))
    assert (np.abs(dl.sum(axis=1)) <= s * 2 * k * 2.0 ** -24 + 1e-15).all()
    # top-1: the weight is 1 whatever the logit, so the gradient is 0
    ids1, w1 = orc.route(logits, 1)
    w1 = w1.astype(np.float32)
    assert not orc.route_backward(ids1, w1, rng.standard_normal((T, 1)), E).any()


def test_sampled_backward_equals_full(orc):
    # the per-token and per-column forms repeat the full backward's
    # arithmetic in the same order: equal bit for bit, empty experts included
    x, ids, w, wg, wu, wd, dout = make_case(6, T=9, H=16, F=24, E=5, k=2)
    ids[:, :] = np.where(ids == 4, 3, ids)          # expert 4 gets no rows
    ids[:, 1] = np.where(ids[:, 1] == ids[:, 0], (ids[:, 0] + 1) % 4, ids[:, 1])
    g = orc.backward(x, ids, w, wg, wu, wd, dout)
    toks = [0, 3, 8, 3]
    dx, dw = orc.backward_tokens(x, ids, w, wg, wu, wd, dout, toks)
    assert np.array_equal(dx, g["dx"][toks]) and np.array_equal(dw, g["dw"][toks])
    ecol, fcol = [0, 1, 3, 4, 2], [0, 23, 7, 5, 11]
    cg, cu, cd = orc.backward_wcols(x, ids, w, wg, wu, wd, dout, ecol, fcol)
    for s, (e, f) in enumerate(zip(ecol, fcol)):
        assert np.array_equal(cg[s], g["dwg"][e, :, f])
        assert np.array_equal(cu[s], g["dwu"][e, :, f])
        assert np.array_equal(cd[s], g["dwd"][e, f, :])
    assert not cg[3].any() and not cd[3].any()      # expert 4: no rows


# ---- the shared expert's backward -------------------------------------------

def dense_shared(x, g, wsg, wsu, wsd):
    """s_t * (silu(x_t Wsg) * (x_t Wsu)) Wsd, float64; s_t = sigmoid(g_t), or 1
    when g is None."""
    a = x @ wsg
    y = (a / (1 + np.exp(-a)) * (x @ wsu)) @ wsd
    s = np.ones(x.shape[0]) if g is None else 1.0 / (1.0 + np.exp(-g))
    return s[:, None] * y


def make_shared(seed, T=6, H=12, Fs=14):
    rng = np.random.default_rng(seed)
    x = bf16(rng.standard_normal((T, H)))
    wsg = bf16(rng.standard_normal((H, Fs)) * 0.3)
    wsu = bf16(rng.standard_normal((H, Fs)) * 0.3)
    wsd = bf16(rng.standard_normal((Fs, H)) * 0.3)
    g = rng.standard_normal(T).astype(np.float32)
    dout = bf16(rng.standard_normal((T, H)))
    return x, wsg, wsu, wsd, g, dout


@pytest.mark.parametrize("gated", [False, True])
def test_shared_backward_matches_finite_differences(orc, gated):
    x, wsg, wsu, wsd, g, dout = make_shared(11)
    g = g if gated else None
    r = orc.shared_backward(x, wsg, wsu, wsd, g, dout)
    X, WG, WU, WD, R = f64(x), f64(wsg), f64(wsu), f64(wsd), f64(dout)
    G = None if g is None else g.astype(np.float64)
    loss = lambda X, G, WG, WU, WD: float((dense_shared(X, G, WG, WU, WD) * R).sum())
    args = [X, G, WG, WU, WD]
    rng = np.random.default_rng(7)
    for name, pos in (("dx", 0), ("dg", 1), ("dwsg", 2), ("dwsu", 3), ("dwsd", 4)):
        a = args[pos]
        if a is None:
            assert not r["dg"].any()
            continue
        for _ in range(10):
            idx = tuple(rng.integers(0, s) for s in a.shape)
            eps = 1e-5 * max(1.0, abs(a[idx]))
            plus = [None if v is None else v.copy() for v in args]
            minus = [None if v is None else v.copy() for v in args]
            plus[pos][idx] += eps
            minus[pos][idx] -= eps
            fd = (loss(*plus) - loss(*minus)) / (2 * eps)
            assert abs(r[name][idx] - fd) <= 1e-6 * max(1.0, abs(fd)), (name, idx, r[name][idx], fd)


def test_shared_backward_is_one_expert_layer(orc):
    """The shared term is a one-expert, top-1 layer with routing weight s_t:
    with s_t = 1 (no gate logits) and with s_t = 1/2 (gate logits 0, so s_t,
    1 - s_t and their product are exact) the shared backward equals the
    routed backward on those weights bit for bit, and the gate gradient is
    the routing-weight gradient times s (1 - s) = 1/4."""
    x, wsg, wsu, wsd, _, dout = make_shared(12)
    T = x.shape[0]
    ids = np.zeros((T, 1), np.int32)
    for g, w in ((None, 1.0), (np.zeros(T, np.float32), 0.5)):
        r = orc.shared_backward(x, wsg, wsu, wsd, g, dout)
        ref = orc.backward(x, ids, np.full((T, 1), w, np.float32), wsg[None], wsu[None],
                           wsd[None], dout)
        assert np.array_equal(r["dx"], ref["dx"])
        assert np.array_equal(r["dwsg"], ref["dwg"][0])
        assert np.array_equal(r["dwsu"], ref["dwu"][0])
        assert np.array_equal(r["dwsd"], ref["dwd"][0])
        if g is not None:
            assert np.array_equal(r["dg"], ref["dw"][:, 0] / 4)

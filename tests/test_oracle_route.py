"""Pins of the oracle's routing step (top-k with ties to the lower index,
softmax over the k chosen logits) against brute force, closed forms and
hand-worked fixtures. CPU only."""
import json
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_topk(logits, k):
    # full stable sort of each row by descending logit: numpy's stable sort
    # keeps equal keys (including -0.0 vs +0.0) in ascending index order
    return np.stack([np.argsort(-row.astype(np.float64), kind="stable")[:k]
                     for row in logits]).astype(np.int32)


def test_golden_route_cases(orc):
    with open(os.path.join(GOLDEN, "route_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        ids, w = orc.route(np.array([c["logits"]], np.float32), c["k"])
        assert ids[0].tolist() == c["ids"], c["why"]
        if c["w"] is not None:
            if c["w_exact"]:
                assert w[0].tolist() == c["w"], c["why"]
            else:
                np.testing.assert_allclose(w[0], c["w"], rtol=1e-6, err_msg=c["why"])


@pytest.mark.parametrize("kind", ["normal", "ties_int", "ties_bf16", "signed_zero", "equal"])
@pytest.mark.parametrize("E,k", [(8, 2), (60, 4), (256, 8), (5, 5), (33, 1)])
def test_route_ids_match_full_sort(orc, kind, E, k):
    from grouped_gemm_softmax_amd import synth
    cfg = synth.small_config(E=E, k=k)
    logits = synth.f32(synth.router_logits(cfg, 97, 3, "cpu", kind))
    ids, w = orc.route(logits, k)
    assert (ids == brute_topk(logits, k)).all()
    # weights: a probability vector, ratios fixed by the logit differences
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-14)
    chosen = np.take_along_axis(logits.astype(np.float64), ids, 1)
    ratio = w / w[:, :1]
    np.testing.assert_allclose(ratio, np.exp(chosen - chosen[:, :1]), rtol=1e-13)
    assert (np.diff(chosen, axis=1) <= 0).all()      # descending slot order


def test_route_k1_weight_is_one(orc):
    rng = np.random.default_rng(0)
    ids, w = orc.route(rng.standard_normal((50, 16)).astype(np.float32), 1)
    assert (w == 1.0).all()


@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_route_equal_logits_exact_uniform(orc, k):
    ids, w = orc.route(np.full((3, 16), 0.75, np.float32), k)
    assert (ids == np.arange(k)).all()
    assert (w == 1.0 / k).all()


def test_route_column_permutation_equivariance(orc):
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((40, 24)).astype(np.float32)   # no ties (a.s.)
    perm = rng.permutation(24)
    ids, w = orc.route(logits, 6)
    ids_p, w_p = orc.route(logits[:, perm], 6)
    assert (perm[ids_p] == ids).all()
    assert (w_p == w).all()


def test_route_rejects_nonfinite(orc):
    l = np.zeros((2, 4), np.float32)
    l[1, 2] = np.nan
    with pytest.raises(ValueError):
        orc.route(l, 2)
    l[1, 2] = np.inf
    with pytest.raises(ValueError):
        orc.route(l, 2)


def test_zipf_logits_top1_follows_zipf():
    """The Zipf(1.2)+Gumbel generator: top-1 is exactly Zipf distributed
    (Gumbel-max), so the hottest expert's share approaches p_1."""
    import torch
    from grouped_gemm_softmax_amd import synth
    cfg = synth.CONFIGS["dsv3"]
    logits = synth.router_logits(cfg, 20000, 0, "cpu")
    top1 = logits.argmax(1)
    share = torch.bincount(top1, minlength=cfg.E).double() / top1.numel()
    p = torch.tensor(sorted(synth.zipf_probs(cfg.E), reverse=True), dtype=torch.float64)
    got = share.sort(descending=True).values
    assert abs(got[0] - p[0]) < 0.01 and abs(got[1] - p[1]) < 0.01

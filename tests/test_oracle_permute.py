"""Pins of the oracle's permutation (stable counting sort by expert) against a
brute-force sort, exact invariants and hand-worked fixtures. CPU only."""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_permute_cases(orc):
    with open(os.path.join(GOLDEN, "permute_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        off, rt, rd = orc.permute(np.array(c["ids"], np.int32), c["E"])
        assert off.tolist() == c["offsets"]
        assert rt.tolist() == c["row_token"]
        assert rd.tolist() == c["row_dest"]


def brute_permute(ids, E):
    T, k = ids.shape
    flat = sorted(range(T * k), key=lambda i: (ids.flat[i], i))  # stable by (expert, t, j)
    row_token = np.array([i // k for i in flat], np.int32)
    row_dest = np.empty(T * k, np.int32)
    for p, i in enumerate(flat):
        row_dest[i] = p
    counts = np.bincount(ids.ravel(), minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return offsets, row_token, row_dest.reshape(T, k)


@pytest.mark.parametrize("T,E,k,kind", [(64, 8, 2, "normal"), (97, 60, 4, "normal"),
                                        (200, 256, 8, "zipf"), (31, 5, 5, "ties_int"),
                                        (1, 8, 2, "normal"), (0, 8, 2, "normal")])
def test_permute_matches_brute_force_and_invariants(orc, T, E, k, kind):
    from grouped_gemm_softmax_amd import synth
    cfg = synth.small_config(E=E, k=k)
    logits = synth.f32(synth.router_logits(cfg, T, 1, "cpu", kind))
    ids, _ = orc.route(logits, k)
    off, rt, rd = orc.permute(ids, E)
    b_off, b_rt, b_rd = brute_permute(ids, E)
    assert (off == b_off).all() and (rt == b_rt).all() and (rd == b_rd).all()
    A = T * k
    assert off[0] == 0 and off[E] == A and (np.diff(off) >= 0).all()
    assert sorted(rd.ravel().tolist()) == list(range(A))          # bijection
    assert (rt[rd] == np.arange(T)[:, None]).all()                # inverse maps
    seg = np.searchsorted(off, rd, side="right") - 1              # segment of each row
    assert (seg == ids).all()
    for e in range(E):                                            # ascending tokens
        assert (np.diff(rt[off[e]:off[e + 1]]) > 0).all()


def test_gather_is_bit_copy(orc):
    rng = np.random.default_rng(2)
    x = rng.integers(0, 65536, (10, 24), dtype=np.uint16)
    ids = rng.integers(0, 4, (10, 3)).astype(np.int32)
    # make each token's experts distinct
    ids = np.stack([rng.permutation(4)[:3] for _ in range(10)]).astype(np.int32)
    off, rt, rd = orc.permute(ids, 4)
    xp = orc.gather(x, rt)
    assert (xp == x[rt]).all()


def test_permute_rejects_bad_ids(orc):
    with pytest.raises(ValueError):
        orc.permute(np.array([[0, 4]], np.int32), 4)

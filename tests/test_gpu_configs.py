"""GPU parity at the full sizes of every configured layer (Mixtral-8x7B-,
DeepSeek-V3- and Qwen2-MoE-shaped, every batch size), in the launch
configuration bench.py times (moe_forward and moe_forward_packed), for the
seeds 0, 1 and 2 of the per-batch inputs (tokens x, router logits, shared-
expert gate logits; the weights are the seed-0 ones, which bounds host
memory). Routing and the permutation are compared with the oracle in full
and bit for bit.

Layer outputs are compared on a stratified sample of tokens that the oracle
computes one token at a time (each token's output depends on that token
alone): for every expert, every 16-row block of its row segment holds at
least one sampled assignment, so every row tile of every tile class the
grouped GEMMs can run (their tiles are whole multiples of 16 rows starting
at the expert's first row) is checked, including each expert's last partial
tile; random tokens then fill the sample to at least 1024 tokens (all of
them when T <= 1024). Every output column of a sampled token is compared."""
import numpy as np
import pytest
import torch

from grouped_gemm_softmax_amd import binding as B
from grouped_gemm_softmax_amd import synth
from helpers import (BLOCK, MIN_SAMPLE, assert_close, check_block_coverage, gpu_bf16_f64,
                     rel_l2, route_weight_bound, say, stratified_tokens)

SEEDS = (0, 1, 2)
CASES = [(name, T, seed) for name in ("mixtral", "mixtral_large", "dsv3", "qwen2")
         for T in synth.CONFIGS[name].Ts for seed in SEEDS]


def test_stratified_sample_covers_every_block():
    """The sampler on a skewed routing (host only): all blocks covered, at
    least min(T, 1024) tokens, no duplicates."""
    rng = np.random.default_rng(5)
    T, E, k = 3000, 40, 4
    p = np.arange(1, E + 1, dtype=np.float64) ** -1.2
    p /= p.sum()
    ids = np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    flat = ids.reshape(-1)
    order = np.lexsort((np.arange(flat.size), flat))
    row_token = (order // k).astype(np.int32)
    row_dest = np.empty(flat.size, np.int64)
    row_dest[order] = np.arange(flat.size)
    offsets = np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))])
    toks, nb = stratified_tokens(offsets, row_token, T, rng)
    assert len(toks) >= 1024 and len(np.unique(toks)) == len(toks)
    check_block_coverage(toks, offsets, row_dest.reshape(T, k))
    assert nb >= T * k // BLOCK


@pytest.fixture(scope="module")
def weights_cache():
    cache = {}
    yield cache
    cache.clear()


def _weights(cache, name):
    """Device weights and their host copies, drawn once per config."""
    if name not in cache:
        cache.clear()
        torch.cuda.empty_cache()
        layer = synth.make_layer(name, 1, seed=0, device="cuda")
        host = dict(wg=synth.u16(layer.w_gate), wu=synth.u16(layer.w_up),
                    wd=synth.u16(layer.w_down))
        if layer.shared is not None:
            host["shared"] = {k: synth.u16(v) for k, v in layer.shared.items()
                              if k != "gate_logits"}
        cache[name] = (layer, host)
    return cache[name]


def _packed(cache, name):
    """Packed copies of the cached device weights (made once per config)."""
    key = name + ":packed"
    if key not in cache:
        layer, _ = cache[name]
        pk = dict(wg=B.moe_pack_weights(layer.w_gate), wu=B.moe_pack_weights(layer.w_up),
                  wd=B.moe_pack_weights(layer.w_down))
        if layer.shared is not None:
            pk["shared"] = {n: B.moe_pack_weights(layer.shared[n])
                            for n in ("w_gate", "w_up", "w_down")}
        cache[key] = pk
    return cache[key]


@pytest.mark.gpu
@pytest.mark.parametrize("name,T,seed", CASES, ids=[f"{n}-T{t}-s{s}" for n, t, s in CASES])
def test_full_size_forward(name, T, seed, weights_cache, orc):
    cfg = synth.CONFIGS[name]
    wl, host = _weights(weights_cache, name)
    layer = synth.make_layer(name, T, seed=seed, device="cuda", with_shared=False,
                             with_weights=False)
    layer.w_gate, layer.w_up, layer.w_down = wl.w_gate, wl.w_up, wl.w_down
    shared = None
    sh_host = None
    if cfg.Fs:
        g = synth.shared_gate_logits(cfg, T, seed, "cuda")
        shared = dict(wl.shared, gate_logits=g)
        sh_host = dict(host["shared"], gate_logits=None if g is None else synth.f32(g))
    k = cfg.k
    say("moe_forward full size", name, T, seed, (cfg.H, cfg.F, cfg.E, k, cfg.Fs))
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    out = B.moe_forward(layer.x, layer.logits, k, layer.w_gate, layer.w_up, layer.w_down,
                        shared=shared, topk_ids=ids, topk_w=w)
    say("moe_permute full size", name, T, seed)
    off, rt, rd, xp = B.moe_permute(layer.x, ids, cfg.E)
    # the packed-weight layer (what bench.py times)
    pk = _packed(weights_cache, name)
    say("moe_forward_packed full size", name, T, seed)
    outp = B.moe_forward(layer.x, layer.logits, k, pk["wg"], pk["wu"], pk["wd"],
                         shared=None if shared is None else dict(pk["shared"],
                                                                 gate_logits=shared["gate_logits"]))
    torch.cuda.synchronize()

    # routing and permutation: in full, bit for bit
    x = synth.u16(layer.x)
    logits = synth.f32(layer.logits)
    ids_ref, w_ref = orc.route(logits, k)
    assert (ids.cpu().numpy() == ids_ref).all()
    bound = route_weight_bound(logits, ids_ref, w_ref)
    assert (np.abs(w.cpu().numpy().astype(np.float64) - w_ref) <= bound).all()
    off_ref, rt_ref, rd_ref = orc.permute(ids_ref, cfg.E)
    assert (off.cpu().numpy() == off_ref).all()
    assert (rt.cpu().numpy() == rt_ref).all()
    assert (rd.cpu().numpy() == rd_ref).all()
    assert (synth.u16(xp) == x[rt_ref]).all()

    # outputs: the stratified sample
    rng = np.random.default_rng([T, seed])
    toks, nblocks = stratified_tokens(off_ref, rt_ref, T, rng)
    check_block_coverage(toks, off_ref, rd_ref)
    assert len(toks) >= min(T, MIN_SAMPLE)
    say("oracle tokens", name, T, seed, len(toks), "tokens over", nblocks, "row blocks")
    ref, ids_s, _ = orc.forward_tokens(x, logits, k, host["wg"], host["wu"], host["wd"], toks,
                                       shared=sh_host)
    assert (ids_s == ids_ref[toks]).all()
    got = gpu_bf16_f64(out)[toks]
    assert_close(got, ref, f"out[{name}, T={T}, seed={seed}]")
    assert rel_l2(got, ref) < 1e-2

    # packed weights: bit-identical to the row-major layer
    assert torch.equal(outp.view(torch.int16), out.view(torch.int16))

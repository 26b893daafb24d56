"""Shared helpers of the GPU parity tests: input staging and the tolerance
checks. The expected values always come from the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

from grouped_gemm_softmax_amd import synth

# Output tolerance, for every bf16 result of the layer (h, y_perm, out)
# against the fp64 oracle: max |gpu - ref| <= 2e-2 * max(1, |ref|), with
# |ref| the max-norm of the row (a token's output, an assignment's h or y
# row). The error of each output of a row is set by the size of the terms
# summed into it (that row's expert outputs, with their bf16-rounded h), not
# by how far those terms happen to cancel in one column, so the row's scale
# is the right one; the elementwise form would demand more of a cancelling
# column than its summands' roundings allow.
TOL = 2e-2
U = 2.0 ** -24   # fp32 unit roundoff

# Full-size parity samples: at least this many tokens (all when T is
# smaller), and every BLOCK-row block of every expert's rows covered.
MIN_SAMPLE = 1024
BLOCK = 16


def say(*a):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print("[case]", *a, file=sys.stderr, flush=True)


def bf16_to_f64(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gpu_bf16_f64(t: torch.Tensor) -> np.ndarray:
    return bf16_to_f64(synth.u16(t))


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str, tol: float = TOL):
    """max |gpu - ref| <= tol * max(1, |ref|) per row (the last axis is the
    row; |ref| the row's max-norm). Also reports how many elements exceed the
    stricter elementwise form tol * max(1, |ref_i|)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    if ref.size == 0:
        return
    assert np.isfinite(gpu).all(), what
    err = np.abs(gpu - ref)
    scale = np.abs(ref).max(axis=-1, keepdims=True) if ref.ndim else np.abs(ref)
    bound = tol * np.maximum(1.0, scale)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {err.size} elements out of tolerance; worst at {i}: "
            f"gpu={gpu[i]!r} ref={ref[i]!r} err={err[i]:.3e} bound={np.broadcast_to(bound, err.shape)[i]:.3e}")
    elem = int((err > tol * np.maximum(1.0, np.abs(ref))).sum())
    if elem:
        say(f"{what}: {elem} of {err.size} elements beyond the elementwise form "
            f"(max err/row bound {float((err / bound).max()):.3f})")


def rel_l2(gpu, ref) -> float:
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(np.asarray(gpu) - ref) / (n if n else 1.0))


def route_weight_bound(logits: np.ndarray, ids: np.ndarray, w_ref: np.ndarray) -> np.ndarray:
    """Per-element bound on |w_gpu - w_ref| for the fp32 softmax over the k
    chosen logits against the fp64 oracle: the fp32 difference l_j - m is off
    by at most |d| u, exp of it then by |d| u relative; expf adds <= 2 ulp, the
    k-term sum k u and the division u; the sum's own error carries over from
    the largest |d| term. Bound: (2 max|d| + k + 5) u relative, per token."""
    chosen = np.take_along_axis(logits.astype(np.float64), ids.astype(np.int64), 1)
    d = np.abs(chosen - chosen[:, :1])
    k = ids.shape[1]
    rel = (2.0 * d.max(axis=1, keepdims=True) + k + 5.0) * U
    return rel * np.abs(w_ref) + 1e-30


def host_layer(layer):
    """numpy (host) copies of a synth.Layer for the oracle."""
    d = dict(x=synth.u16(layer.x), logits=synth.f32(layer.logits),
             wg=synth.u16(layer.w_gate), wu=synth.u16(layer.w_up),
             wd=synth.u16(layer.w_down))
    sh = None
    if layer.shared is not None:
        g = layer.shared["gate_logits"]
        sh = dict(w_gate=synth.u16(layer.shared["w_gate"]),
                  w_up=synth.u16(layer.shared["w_up"]),
                  w_down=synth.u16(layer.shared["w_down"]),
                  gate_logits=None if g is None else synth.f32(g))
    return d, sh


def to_dev(a: np.ndarray, dtype=None, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:           # bf16 bit patterns
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    if dtype is not None and t.dtype != dtype:
        t = t.to(dtype)
    return t.to(device)


def stratified_tokens(offsets, row_token, T, rng, block=BLOCK, fill=MIN_SAMPLE):
    """Tokens such that every `block`-row block of every expert's segment
    [offsets[e], offsets[e+1]) holds a row of a chosen token; then random
    other tokens up to min(T, fill). Returns the sorted tokens and the
    number of blocks."""
    covered = np.zeros(row_token.shape[0], bool)
    chosen = set()
    nblocks = 0
    tok_rows = {}
    for p, t in enumerate(row_token):
        tok_rows.setdefault(int(t), []).append(p)
    for e in range(len(offsets) - 1):
        for b0 in range(int(offsets[e]), int(offsets[e + 1]), block):
            b1 = min(b0 + block, int(offsets[e + 1]))
            nblocks += 1
            if covered[b0:b1].any():
                continue
            t = int(row_token[rng.integers(b0, b1)])
            chosen.add(t)
            covered[tok_rows[t]] = True
    want = min(T, fill)
    if len(chosen) < want:
        rest = np.setdiff1d(np.arange(T), np.fromiter(chosen, np.int64, len(chosen)))
        chosen.update(int(t) for t in rng.choice(rest, want - len(chosen), replace=False))
    return np.array(sorted(chosen), np.int64), nblocks


def check_block_coverage(toks, offsets, row_dest, block=BLOCK):
    """Every block of every expert holds a row of a sampled token."""
    rows = np.sort(row_dest[toks].reshape(-1))
    for e in range(len(offsets) - 1):
        for b0 in range(int(offsets[e]), int(offsets[e + 1]), block):
            b1 = min(b0 + block, int(offsets[e + 1]))
            i = np.searchsorted(rows, b0)
            assert i < rows.size and rows[i] < b1, ("uncovered block", e, b0, b1)

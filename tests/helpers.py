"""Shared helpers of the GPU parity tests: input staging and the tolerance
checks. The expected values always come from the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

from grouped_gemm_softmax_amd import synth

# Output tolerance: |gpu - ref| <= 2e-2 * max(1, |ref|) per element, for every
# bf16 result of the layer (h, y_perm, out) against the fp64 oracle.
TOL = 2e-2
U = 2.0 ** -24   # fp32 unit roundoff


def say(*a):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print("[case]", *a, file=sys.stderr, flush=True)


def bf16_to_f64(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gpu_bf16_f64(t: torch.Tensor) -> np.ndarray:
    return bf16_to_f64(synth.u16(t))


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str, tol: float = TOL):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    if ref.size == 0:
        return
    err = np.abs(gpu - ref)
    bound = tol * np.maximum(1.0, np.abs(ref))
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {err.size} elements out of tolerance; worst at {i}: "
            f"gpu={gpu[i]!r} ref={ref[i]!r} err={err[i]:.3e} bound={bound[i]:.3e}")
    assert np.isfinite(gpu).all(), what


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

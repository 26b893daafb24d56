"""CPU oracle for the fused MoE expert layer (ctypes wrapper over liboracle.so).

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this module. The product
package never imports it, and the oracle shares no code with the HIP path.

All arrays are numpy: bf16 tensors as uint16 bit patterns, router logits as
float32, every arithmetic result as float64. The C source (moe_oracle.c)
states the definition it follows and the readings taken where the pages are
silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# gcc flags: plain IEEE arithmetic (no FMA contraction, no fast-math) so that
# every operation rounds as written; OpenMP only distributes independent rows.
GCC_FLAGS = ["-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fno-fast-math",
             "-fopenmp", "-shared", "-fPIC", "-std=c11", "-Wall"]
# the same arithmetic under AddressSanitizer and UndefinedBehaviorSanitizer
# (any report aborts); such a build is loaded with gcc's libasan preloaded
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=undefined"]


def build(force: bool = True) -> str:
    """Compile moe_oracle.c into liboracle.so with gcc; return the path."""
    if force or not os.path.exists(_LIB) or (
            os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(path: str) -> str:
    """Compile moe_oracle.c with the sanitizers into `path`."""
    flags = [f for f in GCC_FLAGS if f != "-O3"] + SANITIZE_FLAGS
    subprocess.run(["gcc", *flags, "-o", path, _SRC, "-lm"], check=True)
    return path


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int


def lib():
    global _lib
    if _lib is None:
        # MOE_ORACLE_LIBRARY: another build of the same source (the sanitized one)
        path = os.environ.get("MOE_ORACLE_LIBRARY") or build(force=False)
        L = ctypes.CDLL(path)
        L.oracle_num_threads.restype = _I
        L.oracle_set_num_threads.argtypes = [_I]
        L.oracle_set_num_threads.restype = None
        L.oracle_router_logits.argtypes = [_P, _I64, _I, _I, _P, _P]
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_quantize_e4m3.argtypes = [_P, _I64, _I, _I, _P, _P]
        L.oracle_dequant_e4m3.argtypes = [_P, _P, _I64, _I, _I, _P]
        L.oracle_dequant_e4m3.restype = None
        L.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
        L.oracle_e2m1_value.restype = ctypes.c_double
        L.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
        L.oracle_e8m0_value.restype = ctypes.c_double
        L.oracle_quantize_mxfp4.argtypes = [_P, _I64, _I, _I, _P, _P]
        L.oracle_dequant_mxfp4.argtypes = [_P, _P, _I64, _I, _I, _P]
        L.oracle_dequant_mxfp4.restype = None
        L.oracle_quantize_mxfp8.argtypes = [_P, _I64, _I, _I, _P, _P]
        L.oracle_dequant_mxfp8.argtypes = [_P, _P, _I64, _I, _I, _P]
        L.oracle_dequant_mxfp8.restype = None
        L.oracle_route.argtypes = [_P, _I64, _I, _I, _P, _P]
        L.oracle_permute.argtypes = [_P, _I64, _I, _I, _P, _P, _P]
        L.oracle_gather.argtypes = [_P, _P, _I64, _I, _P]
        L.oracle_gather.restype = None
        L.oracle_gateup_rows.argtypes = [_P, _I64, _I, _I, _P, _P, _P]
        L.oracle_down_rows.argtypes = [_P, _I64, _I, _I, _P, _P]
        L.oracle_grouped_gateup.argtypes = [_P, _P, _I, _I, _I, _P, _P, _P]
        L.oracle_grouped_down.argtypes = [_P, _P, _I, _I, _I, _P, _P]
        L.oracle_combine.argtypes = [_P, _P, _P, _I64, _I, _I, _P, _P, _P]
        L.oracle_combine.restype = None
        L.oracle_shared_gate.argtypes = [_P, _I64, _P]
        L.oracle_shared_gate.restype = None
        L.oracle_forward.argtypes = ([_P, _P, _I64, _I, _I, _I, _I, _P, _P, _P,
                                      _I, _P, _P, _P, _P] + [_P] * 8)
        L.oracle_forward_tokens.argtypes = ([_P, _P, _I64, _I, _I, _I, _I, _P,
                                             _P, _P, _I, _P, _P, _P, _P, _P,
                                             _I64, _P, _P, _P])
        L.oracle_backward.argtypes = [_P, _P, _P, _I64, _I, _I, _I, _I, _P, _P, _P, _P,
                                      _P, _P, _P, _P, _P]
        L.oracle_shared_backward.argtypes = [_P, _I64, _I, _I, _P, _P, _P, _P, _P, _P, _P,
                                             _P, _P, _P]
        L.oracle_backward_tokens.argtypes = [_P, _P, _P, _I64, _I, _I, _I, _I, _P, _P, _P,
                                             _P, _P, _I64, _P, _P]
        L.oracle_backward_wcols.argtypes = [_P, _P, _P, _I64, _I, _I, _I, _I, _P, _P, _P,
                                            _P, _P, _P, _I64, _P, _P, _P]
        L.oracle_route_backward.argtypes = [_P, _P, _P, _I64, _I, _I, _P]
        L.oracle_route_backward.restype = None
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of later oracle calls (results do not depend on it)."""
    lib().oracle_set_num_threads(int(n))


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def router_logits(x: np.ndarray, wr: np.ndarray) -> np.ndarray:
    """Router projection logits[t,e] = sum_h x[t,h] wr[e,h] in fp64.
    x [T,H] u16, wr [E,H] u16 -> float64 [T,E]."""
    x, wr = _c(x, np.uint16), _c(wr, np.uint16)
    T, H = x.shape
    E = wr.shape[0]
    assert wr.shape == (E, H)
    out = np.empty((T, E), np.float64)
    _check(lib().oracle_router_logits(_p(x), T, H, E, _p(wr), _p(out)),
           "router_logits")
    return out


def e4m3_values() -> np.ndarray:
    """Values of the 256 E4M3 codes (float64; NaN for the NaN codes)."""
    return np.array([lib().oracle_e4m3_value(c) for c in range(256)], np.float64)


def quantize_e4m3(w: np.ndarray):
    """bf16 weights [G,K,N] (or [K,N]: G = 1) -> (codes uint8 same shape,
    per-column power-of-two scales float64 [G,N])."""
    w = _c(w, np.uint16)
    squeeze = w.ndim == 2
    if squeeze:
        w = w[None]
    G, K, N = w.shape
    codes = np.empty((G, K, N), np.uint8)
    scales = np.empty((G, N), np.float64)
    _check(lib().oracle_quantize_e4m3(_p(w), G, K, N, _p(codes), _p(scales)), "quantize_e4m3")
    return (codes[0], scales[0]) if squeeze else (codes, scales)


def dequant_e4m3(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """value(code) * scale per column -> float64, same shape as codes."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.float64)
    squeeze = codes.ndim == 2
    if squeeze:
        codes, scales = codes[None], scales[None]
    G, K, N = codes.shape
    out = np.empty((G, K, N), np.float64)
    lib().oracle_dequant_e4m3(_p(codes), _p(scales), G, K, N, _p(out))
    return out[0] if squeeze else out


def e2m1_values() -> np.ndarray:
    """Values of the 16 E2M1 codes (float64)."""
    return np.array([lib().oracle_e2m1_value(c) for c in range(16)], np.float64)


def e8m0_value(s: int) -> float:
    return lib().oracle_e8m0_value(s)


def quantize_mxfp4(w: np.ndarray):
    """bf16 weights [G,K,N] (or [K,N]: G = 1) -> (codes uint8 0..15 same
    shape, scale bytes uint8 [G, ceil(K/32), N]; scale = 2^(byte - 127))."""
    w = _c(w, np.uint16)
    squeeze = w.ndim == 2
    if squeeze:
        w = w[None]
    G, K, N = w.shape
    codes = np.empty((G, K, N), np.uint8)
    sb = np.empty((G, -(-K // 32), N), np.uint8)
    _check(lib().oracle_quantize_mxfp4(_p(w), G, K, N, _p(codes), _p(sb)), "quantize_mxfp4")
    return (codes[0], sb[0]) if squeeze else (codes, sb)


def dequant_mxfp4(codes: np.ndarray, scale_bytes: np.ndarray) -> np.ndarray:
    """value(code) * 2^(scale byte - 127) of its 32-row block -> float64."""
    codes = _c(codes, np.uint8)
    scale_bytes = _c(scale_bytes, np.uint8)
    squeeze = codes.ndim == 2
    if squeeze:
        codes, scale_bytes = codes[None], scale_bytes[None]
    G, K, N = codes.shape
    out = np.empty((G, K, N), np.float64)
    lib().oracle_dequant_mxfp4(_p(codes), _p(scale_bytes), G, K, N, _p(out))
    return out[0] if squeeze else out


def quantize_mxfp8(w: np.ndarray):
    """bf16 weights [G,K,N] (or [K,N]: G = 1) -> (E4M3 codes uint8 same
    shape, scale bytes uint8 [G, ceil(K/32), N]; scale = 2^(byte - 127))."""
    w = _c(w, np.uint16)
    squeeze = w.ndim == 2
    if squeeze:
        w = w[None]
    G, K, N = w.shape
    codes = np.empty((G, K, N), np.uint8)
    sb = np.empty((G, -(-K // 32), N), np.uint8)
    _check(lib().oracle_quantize_mxfp8(_p(w), G, K, N, _p(codes), _p(sb)), "quantize_mxfp8")
    return (codes[0], sb[0]) if squeeze else (codes, sb)


def dequant_mxfp8(codes: np.ndarray, scale_bytes: np.ndarray) -> np.ndarray:
    """value(code) * 2^(scale byte - 127) of its 32-row block -> float64."""
    codes = _c(codes, np.uint8)
    scale_bytes = _c(scale_bytes, np.uint8)
    squeeze = codes.ndim == 2
    if squeeze:
        codes, scale_bytes = codes[None], scale_bytes[None]
    G, K, N = codes.shape
    out = np.empty((G, K, N), np.float64)
    lib().oracle_dequant_mxfp8(_p(codes), _p(scale_bytes), G, K, N, _p(out))
    return out[0] if squeeze else out


def backward(x, ids, w, wg, wu, wd, dout):
    """Backward of the routed layer for a fixed routing (ids int32 [T,k], w
    fp32 [T,k]); x, weights, dout bf16. Returns dict(dx [T,H], dw [T,k],
    dwg [E,H,F], dwu [E,H,F], dwd [E,F,H]), float64."""
    x = _c(x, np.uint16)
    ids, w = _c(ids, np.int32), _c(w, np.float32)
    wg, wu, wd = _c(wg, np.uint16), _c(wu, np.uint16), _c(wd, np.uint16)
    dout = _c(dout, np.uint16)
    T, H = x.shape
    k = ids.shape[1]
    E, _, F = wg.shape
    r = dict(dx=np.empty((T, H)), dw=np.empty((T, k)), dwg=np.empty((E, H, F)),
             dwu=np.empty((E, H, F)), dwd=np.empty((E, F, H)))
    _check(lib().oracle_backward(_p(x), _p(ids), _p(w), T, H, F, E, k, _p(wg), _p(wu), _p(wd),
                                 _p(dout), _p(r["dx"]), _p(r["dw"]), _p(r["dwg"]), _p(r["dwu"]),
                                 _p(r["dwd"])), "backward")
    return r


def shared_backward(x, wsg, wsu, wsd, gate_logits, dout):
    """Backward of the shared expert's term s_t * y_sh[t] (s_t = 1 without
    gate logits, else the sigmoid of gate_logits [T] fp32); x, weights
    (W_sg, W_su [H,Fs], W_sd [Fs,H]) and dout bf16. Returns dict(dx [T,H]
    (the shared expert's part of the input gradient), dg [T] (the gate-logit
    gradient, zeros without gate logits), dwsg, dwsu [H,Fs], dwsd [Fs,H]),
    float64."""
    x, dout = _c(x, np.uint16), _c(dout, np.uint16)
    wsg, wsu, wsd = _c(wsg, np.uint16), _c(wsu, np.uint16), _c(wsd, np.uint16)
    T, H = x.shape
    Fs = wsg.shape[1]
    g = None if gate_logits is None else _c(gate_logits, np.float32)
    r = dict(dx=np.empty((T, H)), dg=np.zeros(T), dwsg=np.empty((H, Fs)),
             dwsu=np.empty((H, Fs)), dwsd=np.empty((Fs, H)))
    _check(lib().oracle_shared_backward(_p(x), T, H, Fs, _p(wsg), _p(wsu), _p(wsd),
                                        None if g is None else _p(g), _p(dout), _p(r["dx"]),
                                        _p(r["dg"]), _p(r["dwsg"]), _p(r["dwsu"]),
                                        _p(r["dwsd"])), "shared_backward")
    return r


def backward_tokens(x, ids, w, wg, wu, wd, dout, tokens):
    """dx [n,H] and the routing-weight gradient [n,k] of the listed tokens
    only (equal to those rows of backward()), float64."""
    x, dout = _c(x, np.uint16), _c(dout, np.uint16)
    ids, w = _c(ids, np.int32), _c(w, np.float32)
    wg, wu, wd = _c(wg, np.uint16), _c(wu, np.uint16), _c(wd, np.uint16)
    tokens = _c(np.asarray(tokens, dtype=np.int64), np.int64)
    T, H = x.shape
    k = ids.shape[1]
    E, _, F = wg.shape
    n = tokens.shape[0]
    dx, dw = np.empty((n, H)), np.empty((n, k))
    _check(lib().oracle_backward_tokens(_p(x), _p(ids), _p(w), T, H, F, E, k, _p(wg), _p(wu),
                                        _p(wd), _p(dout), _p(tokens), n, _p(dx), _p(dw)),
           "backward_tokens")
    return dx, dw


def backward_wcols(x, ids, w, wg, wu, wd, dout, ecol, fcol):
    """For each pair (e, f): column f of dW_gate[e] and dW_up[e] and row f
    of dW_down[e], each [n,H] float64 (equal to those elements of
    backward())."""
    x, dout = _c(x, np.uint16), _c(dout, np.uint16)
    ids, w = _c(ids, np.int32), _c(w, np.float32)
    wg, wu, wd = _c(wg, np.uint16), _c(wu, np.uint16), _c(wd, np.uint16)
    ecol = _c(np.asarray(ecol, dtype=np.int32), np.int32)
    fcol = _c(np.asarray(fcol, dtype=np.int32), np.int32)
    T, H = x.shape
    k = ids.shape[1]
    E, _, F = wg.shape
    n = ecol.shape[0]
    g, u, d = np.empty((n, H)), np.empty((n, H)), np.empty((n, H))
    _check(lib().oracle_backward_wcols(_p(x), _p(ids), _p(w), T, H, F, E, k, _p(wg), _p(wu),
                                       _p(wd), _p(dout), _p(ecol), _p(fcol), n, _p(g), _p(u),
                                       _p(d)), "backward_wcols")
    return g, u, d


def route_backward(ids, w, dw, E: int) -> np.ndarray:
    """d logits [T,E] of the softmax over the k selected logits."""
    ids, w, dw = _c(ids, np.int32), _c(w, np.float32), _c(dw, np.float64)
    T, k = ids.shape
    dl = np.empty((T, E))
    lib().oracle_route_backward(_p(ids), _p(w), _p(dw), T, E, k, _p(dl))
    return dl


def route(logits: np.ndarray, k: int):
    """Top-k (ties -> lower index) + softmax over the k logits.
    Returns ids int32 [T,k], w float64 [T,k]."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    _check(lib().oracle_route(_p(logits), T, E, k, _p(ids), _p(w)), "route")
    return ids, w


def permute(ids: np.ndarray, E: int):
    """Stable counting sort by expert. Returns offsets [E+1], row_token [A],
    row_dest [T,k] (all int32)."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    offsets = np.empty(E + 1, np.int32)
    row_token = np.empty(T * k, np.int32)
    row_dest = np.empty((T, k), np.int32)
    _check(lib().oracle_permute(_p(ids), T, E, k, _p(offsets), _p(row_token),
                                _p(row_dest)), "permute")
    return offsets, row_token, row_dest


def gather(x: np.ndarray, row_token: np.ndarray) -> np.ndarray:
    x = _c(x, np.uint16)
    row_token = _c(row_token, np.int32)
    T, H = x.shape
    A = row_token.shape[0]
    if A and (row_token.min() < 0 or row_token.max() >= T):
        raise ValueError("row_token out of range")
    out = np.empty((A, H), np.uint16)
    lib().oracle_gather(_p(x), _p(row_token), A, H, _p(out))
    return out


def gateup_rows(x: np.ndarray, wg: np.ndarray, wu: np.ndarray) -> np.ndarray:
    """One expert: h = silu(x Wg) * (x Wu). x [M,H] u16, wg/wu [H,F] u16."""
    x, wg, wu = _c(x, np.uint16), _c(wg, np.uint16), _c(wu, np.uint16)
    M, H = x.shape
    F = wg.shape[1]
    assert wg.shape == (H, F) and wu.shape == (H, F)
    h = np.empty((M, F), np.float64)
    _check(lib().oracle_gateup_rows(_p(x), M, H, F, _p(wg), _p(wu), _p(h)),
           "gateup_rows")
    return h


def down_rows(h: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """One expert: y = h Wd. h [M,F] f64, wd [F,H] u16."""
    h, wd = _c(h, np.float64), _c(wd, np.uint16)
    M, F = h.shape
    H = wd.shape[1]
    assert wd.shape == (F, H)
    y = np.empty((M, H), np.float64)
    _check(lib().oracle_down_rows(_p(h), M, F, H, _p(wd), _p(y)), "down_rows")
    return y


def grouped_gateup(x_perm, offsets, wg, wu) -> np.ndarray:
    x_perm, offsets = _c(x_perm, np.uint16), _c(offsets, np.int32)
    wg, wu = _c(wg, np.uint16), _c(wu, np.uint16)
    E, H, F = wg.shape
    A = int(offsets[E])
    assert x_perm.shape == (A, H) and wu.shape == (E, H, F)
    h = np.empty((A, F), np.float64)
    _check(lib().oracle_grouped_gateup(_p(x_perm), _p(offsets), E, H, F,
                                       _p(wg), _p(wu), _p(h)), "grouped_gateup")
    return h


def grouped_down(h, offsets, wd) -> np.ndarray:
    h, offsets, wd = _c(h, np.float64), _c(offsets, np.int32), _c(wd, np.uint16)
    E, F, H = wd.shape
    A = int(offsets[E])
    assert h.shape == (A, F)
    y = np.empty((A, H), np.float64)
    _check(lib().oracle_grouped_down(_p(h), _p(offsets), E, F, H, _p(wd),
                                     _p(y)), "grouped_down")
    return y


def shared_gate(gate_logits: Optional[np.ndarray], T: int) -> np.ndarray:
    s = np.empty(T, np.float64)
    g = None if gate_logits is None else _c(gate_logits, np.float32)
    lib().oracle_shared_gate(_p(g), T, _p(s))
    return s


def combine(y, row_dest, w, y_sh=None, s=None) -> np.ndarray:
    """out[t] = sum_j w[t,j] y[row_dest[t,j]] (+ s[t] y_sh[t])."""
    y, row_dest, w = _c(y, np.float64), _c(row_dest, np.int32), _c(w, np.float64)
    T, k = row_dest.shape
    H = y.shape[1]
    if row_dest.size and (row_dest.min() < 0 or row_dest.max() >= y.shape[0]):
        raise ValueError("row_dest out of range")
    if y_sh is not None:
        y_sh, s = _c(y_sh, np.float64), _c(s, np.float64)
    out = np.empty((T, H), np.float64)
    lib().oracle_combine(_p(y), _p(row_dest), _p(w), T, H, k, _p(y_sh), _p(s),
                         _p(out))
    return out


def _shared_args(shared):
    if shared is None:
        return 0, None, None, None, None
    wsg = _c(shared["w_gate"], np.uint16)
    wsu = _c(shared["w_up"], np.uint16)
    wsd = _c(shared["w_down"], np.uint16)
    g = shared.get("gate_logits")
    g = None if g is None else _c(g, np.float32)
    return wsg.shape[1], wsg, wsu, wsd, g


def forward(x, logits, k, wg, wu, wd, shared=None, keep_intermediates=True):
    """Whole layer. shared: None or dict(w_gate [H,Fs], w_up [H,Fs],
    w_down [Fs,H], gate_logits [T] or None). Returns a dict."""
    x, logits = _c(x, np.uint16), _c(logits, np.float32)
    wg, wu, wd = _c(wg, np.uint16), _c(wu, np.uint16), _c(wd, np.uint16)
    T, H = x.shape
    E, _, F = wg.shape
    A = T * k
    Fs, wsg, wsu, wsd, g = _shared_args(shared)
    r = dict(out=np.empty((T, H), np.float64), ids=np.empty((T, k), np.int32),
             w=np.empty((T, k), np.float64), offsets=np.empty(E + 1, np.int32),
             row_token=np.empty(A, np.int32), row_dest=np.empty((T, k), np.int32))
    if keep_intermediates:
        r["h"] = np.empty((A, F), np.float64)
        r["y"] = np.empty((A, H), np.float64)
    _check(lib().oracle_forward(
        _p(x), _p(logits), T, H, F, E, k, _p(wg), _p(wu), _p(wd), Fs, _p(wsg),
        _p(wsu), _p(wsd), _p(g), _p(r["out"]), _p(r["ids"]), _p(r["w"]),
        _p(r["offsets"]), _p(r["row_token"]), _p(r["row_dest"]),
        _p(r.get("h")), _p(r.get("y"))), "forward")
    return r


def forward_tokens(x, logits, k, wg, wu, wd, tokens, shared=None):
    """Output rows for the listed tokens only. Returns (out [n,H], ids, w)."""
    x, logits = _c(x, np.uint16), _c(logits, np.float32)
    wg, wu, wd = _c(wg, np.uint16), _c(wu, np.uint16), _c(wd, np.uint16)
    tokens = _c(np.asarray(tokens, dtype=np.int64), np.int64)
    T, H = x.shape
    E, _, F = wg.shape
    n = tokens.shape[0]
    Fs, wsg, wsu, wsd, g = _shared_args(shared)
    out = np.empty((n, H), np.float64)
    ids = np.empty((n, k), np.int32)
    w = np.empty((n, k), np.float64)
    _check(lib().oracle_forward_tokens(
        _p(x), _p(logits), T, H, F, E, k, _p(wg), _p(wu), _p(wd), Fs, _p(wsg),
        _p(wsu), _p(wsd), _p(g), _p(tokens), n, _p(out), _p(ids), _p(w)),
        "forward_tokens")
    return out, ids, w


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float64/float32 values to bf16 (round-to-nearest-even) and return
    the uint16 bit patterns. Used to turn oracle results into the GPU's
    storage type for reporting."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

"""Python binding of libmoe.so (ctypes). Argument marshalling only: every step
of the layer runs in the library's HIP kernels. torch supplies device memory
and the current HIP stream.

The function names match the C ABI in include/moe.h. Outputs that are not
passed in are allocated with torch on the inputs' device. A non-zero status
raises MoeError with the library's status text.
"""
from __future__ import annotations

import ctypes
import functools
import inspect
import os
import re
from typing import Optional

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_LIBRARY points the binding at another build of the same library (used
# to compare kernel variants); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("MOE_LIBRARY") or os.path.join(PKG, "libmoe.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "moe.h")


# moe_status values the binding tests for (include/moe.h)
MOE_ERR_BAD_IDS = -6


class MoeError(RuntimeError):
    def __init__(self, status: int, text: str, call: str):
        super().__init__(f"{call}: {text} (status {status})")
        self.status = status


class SharedExpert(ctypes.Structure):
    _fields_ = [("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("Fs", ctypes.c_int32),
                ("gate_logits", ctypes.c_void_p)]


class SharedExpertGrads(ctypes.Structure):
    _fields_ = [("dw_gate", ctypes.c_void_p), ("dw_up", ctypes.c_void_p),
                ("dw_down", ctypes.c_void_p), ("d_gate_logits", ctypes.c_void_p)]


class SharedExpertFp8(ctypes.Structure):
    _fields_ = [("w_gate", ctypes.c_void_p), ("s_gate", ctypes.c_void_p),
                ("w_up", ctypes.c_void_p), ("s_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("s_down", ctypes.c_void_p),
                ("Fs", ctypes.c_int32), ("gate_logits", ctypes.c_void_p)]


class SharedExpertMxfp4(ctypes.Structure):
    _fields_ = [("w_gate", ctypes.c_void_p), ("s_gate", ctypes.c_void_p),
                ("w_up", ctypes.c_void_p), ("s_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("s_down", ctypes.c_void_p),
                ("Fs", ctypes.c_int32), ("gate_logits", ctypes.c_void_p)]


class SharedExpertMxfp8(ctypes.Structure):
    _fields_ = [("w_gate", ctypes.c_void_p), ("s_gate", ctypes.c_void_p),
                ("w_up", ctypes.c_void_p), ("s_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("s_down", ctypes.c_void_p),
                ("Fs", ctypes.c_int32), ("gate_logits", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [_I]),
    "moe_route": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "moe_router_workspace_bytes": (_SZ, [_I, _I, _I, _I]),
    "moe_router_route": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "moe_permute_workspace_bytes": (_SZ, [_I, _I, _I]),
    "moe_permute": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_gateup_swiglu": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P, _P]),
    "moe_down": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P]),
    "moe_grouped_ffn_workspace_bytes": (_SZ, [_I, _I]),
    "moe_grouped_ffn": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_combine": (_I, [_P, _P, _P, _I, _I, _I, _P, _P]),
    "moe_forward_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "moe_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "moe_forward_routed": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P,
                                _SZ, _P]),
    "moe_forward": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P,
                         ctypes.POINTER(SharedExpert), _P, _P, _P, _P, _SZ, _P]),
    "moe_pack_weights_bytes": (_SZ, [_I, _I, _I]),
    "moe_pack_weights": (_I, [_P, _I, _I, _I, _P, _SZ, _P]),
    "moe_gateup_swiglu_packed": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P, _P]),
    "moe_down_packed": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P]),
    "moe_forward_packed": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P,
                                ctypes.POINTER(SharedExpert), _P, _P, _P, _P, _SZ, _P]),
    "moe_forward_packed_noalloc": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P,
                                        ctypes.POINTER(SharedExpert), _P, _P, _P, _P]),
    "moe_fp8_weights_bytes": (_SZ, [_I, _I, _I]),
    "moe_quantize_fp8": (_I, [_P, _I, _I, _I, _P, _SZ, _P, _P]),
    "moe_gateup_swiglu_fp8": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
    "moe_down_fp8": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P, _P]),
    "moe_forward_fp8": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P,
                             ctypes.POINTER(SharedExpertFp8), _P, _P, _P, _P, _SZ, _P]),
    "moe_mxfp4_weights_bytes": (_SZ, [_I, _I, _I]),
    "moe_mxfp4_scales_bytes": (_SZ, [_I, _I, _I]),
    "moe_quantize_mxfp4": (_I, [_P, _I, _I, _I, _P, _SZ, _P, _SZ, _P]),
    "moe_gateup_swiglu_mxfp4": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
    "moe_down_mxfp4": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P, _P]),
    "moe_forward_mxfp4": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P,
                               ctypes.POINTER(SharedExpertMxfp4), _P, _P, _P, _P, _SZ, _P]),
    "moe_mxfp8_weights_bytes": (_SZ, [_I, _I, _I]),
    "moe_mxfp8_scales_bytes": (_SZ, [_I, _I, _I]),
    "moe_quantize_mxfp8": (_I, [_P, _I, _I, _I, _P, _SZ, _P, _SZ, _P]),
    "moe_gateup_swiglu_mxfp8": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
    "moe_down_mxfp8": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P, _P]),
    "moe_forward_mxfp8": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P,
                               ctypes.POINTER(SharedExpertMxfp8), _P, _P, _P, _P, _SZ, _P]),
    "moe_backward_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "moe_backward": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P,
                          _P, _P, _SZ, _P]),
    "moe_route_backward": (_I, [_P, _P, _P, _I, _I, _I, _P, _P]),
    "moe_backward_shared_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "moe_backward_shared": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P,
                                 ctypes.POINTER(SharedExpert), _P, _P, _P, _P, _P, _P,
                                 ctypes.POINTER(SharedExpertGrads), _P, _SZ, _P]),
    "moe_set_dispatch_override": (_I, [_I, _I]),
    "moe_set_combine_override": (_I, [_I]),
    "moe_set_diagnostics": (_I, [_I, _I]),
    "moe_check_topk_ids": (_I, [_P, _I, _I, _I, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so. Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m grouped_gemm_softmax_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def header_symbols(path: str = HEADER):
    """Function names declared in include/moe.h."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on_stream(fn):
    """Run a wrapper with `stream` (when one is given) as torch's current
    stream, so that the tensors it allocates (outputs it creates, workspace it
    frees on return) belong to the stream the library enqueues on: the caching
    allocator then reuses a freed workspace block only for later work of that
    stream, never while its kernels may still read or write it."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        bound = sig.bind(*args, **kwargs)
        stream = bound.arguments.get("stream")
        if stream is None:
            return fn(*args, **kwargs)
        with torch.cuda.stream(stream):
            return fn(*args, **kwargs)

    return wrapper


def _check(status: int, call: str):
    if status != 0:
        raise MoeError(status, lib().moe_status_string(status).decode(), call)


def _need(t: torch.Tensor, dtype, name: str):
    if t.dtype != dtype or not t.is_contiguous():
        raise TypeError(f"{name}: expected contiguous {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name}: expected a device tensor")


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


@_on_stream
def moe_route(logits: torch.Tensor, k: int, topk_ids=None, topk_w=None, stream=None):
    _need(logits, torch.float32, "logits")
    T, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(lib().moe_route(_ptr(logits), T, E, k, _ptr(topk_ids), _ptr(topk_w),
                           _stream(stream)), "moe_route")
    return topk_ids, topk_w


def moe_router_workspace_bytes(T: int, H: int, E: int, k: int) -> int:
    return int(lib().moe_router_workspace_bytes(T, H, E, k))


@_on_stream
def moe_router_route(x: torch.Tensor, w_router: torch.Tensor, k: int, logits=False,
                     ws=None, out=None, stream=None):
    """x bf16 [T,H], w_router bf16 [E,H] -> (topk_ids [T,k], topk_w [T,k]), plus
    the fp32 logits [T,E] as a third element when `logits` is True."""
    _need(x, torch.bfloat16, "x")
    _need(w_router, torch.bfloat16, "w_router")
    T, H = x.shape
    E = w_router.shape[0]
    if w_router.shape[1] != H:
        raise ValueError(f"w_router: expected [E,{H}], got {tuple(w_router.shape)}")
    dev = x.device
    if out is None:
        out = (torch.empty((T, k), dtype=torch.int32, device=dev),
               torch.empty((T, k), dtype=torch.float32, device=dev),
               torch.empty((T, E), dtype=torch.float32, device=dev) if logits else None)
    topk_ids, topk_w, lg = out
    if ws is None:
        ws = torch.empty(max(moe_router_workspace_bytes(T, H, E, k), 16), dtype=torch.uint8,
                         device=dev)
    _check(lib().moe_router_route(_ptr(x), _ptr(w_router), T, H, E, k, _ptr(lg),
                                  _ptr(topk_ids), _ptr(topk_w), _ptr(ws), ws.numel(),
                                  _stream(stream)), "moe_router_route")
    return (topk_ids, topk_w, lg) if lg is not None else (topk_ids, topk_w)


def moe_permute_workspace_bytes(T: int, E: int, k: int) -> int:
    return int(lib().moe_permute_workspace_bytes(T, E, k))


@_on_stream
def moe_permute(x: torch.Tensor, topk_ids: torch.Tensor, E: int, ws=None, out=None,
                stream=None):
    """Returns (expert_offsets [E+1], row_token [T*k], row_dest [T,k], x_perm [T*k,H])."""
    _need(x, torch.bfloat16, "x")
    _need(topk_ids, torch.int32, "topk_ids")
    T, H = x.shape
    k = topk_ids.shape[1]
    dev = x.device
    if out is None:
        out = (torch.empty(E + 1, dtype=torch.int32, device=dev),
               torch.empty(T * k, dtype=torch.int32, device=dev),
               torch.empty((T, k), dtype=torch.int32, device=dev),
               torch.empty((T * k, H), dtype=torch.bfloat16, device=dev))
    offsets, row_token, row_dest, x_perm = out
    if ws is None:
        ws = torch.empty(max(moe_permute_workspace_bytes(T, E, k), 16),
                         dtype=torch.uint8, device=dev)
    _check(lib().moe_permute(_ptr(x), _ptr(topk_ids), T, H, E, k, _ptr(offsets),
                             _ptr(row_token), _ptr(row_dest), _ptr(x_perm), _ptr(ws),
                             ws.numel(), _stream(stream)), "moe_permute")
    return offsets, row_token, row_dest, x_perm


class PackedWeight:
    """A [G,K,N] weight tensor in the library's packed block layout (from
    moe_pack_weights). `data` is the packed device buffer (uint8)."""

    def __init__(self, data: torch.Tensor, G: int, K: int, N: int):
        self.data, self.G, self.K, self.N = data, G, K, N
        self.shape = (G, K, N)

    def data_ptr(self) -> int:
        return self.data.data_ptr()


def moe_pack_weights_bytes(G: int, K: int, N: int) -> int:
    return int(lib().moe_pack_weights_bytes(G, K, N))


@_on_stream
def moe_pack_weights(w: torch.Tensor, stream=None) -> PackedWeight:
    """w bf16 [G,K,N] (or [K,N], taken as G = 1) -> PackedWeight."""
    _need(w, torch.bfloat16, "w")
    G, K, N = (1, *w.shape) if w.dim() == 2 else w.shape
    nbytes = moe_pack_weights_bytes(G, K, N)
    data = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=w.device)
    _check(lib().moe_pack_weights(_ptr(w), G, K, N, _ptr(data), data.numel(),
                                  _stream(stream)), "moe_pack_weights")
    return PackedWeight(data, G, K, N)


def _weight(w, name: str, packed: bool):
    if packed:
        if not isinstance(w, PackedWeight):
            raise TypeError(f"{name}: expected a PackedWeight (moe_pack_weights)")
    else:
        _need(w, torch.bfloat16, name)
    return w


class Fp8Weight:
    """A [G,K,N] weight tensor as E4M3 codes in the library's block layout
    (`codes`, uint8) with per-column fp32 power-of-two scales (`scales`,
    [G,N]), from moe_quantize_fp8."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor, G: int, K: int, N: int):
        self.codes, self.scales, self.G, self.K, self.N = codes, scales, G, K, N
        self.shape = (G, K, N)


def moe_fp8_weights_bytes(G: int, K: int, N: int) -> int:
    return int(lib().moe_fp8_weights_bytes(G, K, N))


@_on_stream
def moe_quantize_fp8(w: torch.Tensor, stream=None) -> Fp8Weight:
    """w bf16 [G,K,N] (or [K,N], taken as G = 1) -> Fp8Weight."""
    _need(w, torch.bfloat16, "w")
    G, K, N = (1, *w.shape) if w.dim() == 2 else w.shape
    nbytes = moe_fp8_weights_bytes(G, K, N)
    codes = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=w.device)
    scales = torch.empty((G, N), dtype=torch.float32, device=w.device)
    _check(lib().moe_quantize_fp8(_ptr(w), G, K, N, _ptr(codes), codes.numel(), _ptr(scales),
                                  _stream(stream)), "moe_quantize_fp8")
    return Fp8Weight(codes, scales, G, K, N)


def _fp8(w, name):
    if not isinstance(w, Fp8Weight):
        raise TypeError(f"{name}: expected an Fp8Weight (moe_quantize_fp8)")
    return w


class Mxfp4Weight:
    """A [G,K,N] weight tensor in MXFP4: E2M1 codes in the library's block
    layout (`codes`, uint8, two per byte) and E8M0 scale bytes, one per 32
    K-values of a column (`scales`, uint8), from moe_quantize_mxfp4."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor, G: int, K: int, N: int):
        self.codes, self.scales, self.G, self.K, self.N = codes, scales, G, K, N
        self.shape = (G, K, N)


def moe_mxfp4_weights_bytes(G: int, K: int, N: int) -> int:
    return int(lib().moe_mxfp4_weights_bytes(G, K, N))


def moe_mxfp4_scales_bytes(G: int, K: int, N: int) -> int:
    return int(lib().moe_mxfp4_scales_bytes(G, K, N))


@_on_stream
def moe_quantize_mxfp4(w: torch.Tensor, stream=None) -> Mxfp4Weight:
    """w bf16 [G,K,N] (or [K,N], taken as G = 1) -> Mxfp4Weight."""
    _need(w, torch.bfloat16, "w")
    G, K, N = (1, *w.shape) if w.dim() == 2 else w.shape
    nc, ns = moe_mxfp4_weights_bytes(G, K, N), moe_mxfp4_scales_bytes(G, K, N)
    codes = torch.empty(max(nc, 16), dtype=torch.uint8, device=w.device)
    scales = torch.empty(max(ns, 16), dtype=torch.uint8, device=w.device)
    _check(lib().moe_quantize_mxfp4(_ptr(w), G, K, N, _ptr(codes), codes.numel(), _ptr(scales),
                                    scales.numel(), _stream(stream)), "moe_quantize_mxfp4")
    return Mxfp4Weight(codes, scales, G, K, N)


class Mxfp8Weight:
    """A [G,K,N] weight tensor in MXFP8: E4M3 codes in the fp8 block layout
    (`codes`, uint8) and E8M0 scale bytes, one per 32 K-values of a column
    (`scales`, uint8, the mxfp4 layout), from moe_quantize_mxfp8."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor, G: int, K: int, N: int):
        self.codes, self.scales, self.G, self.K, self.N = codes, scales, G, K, N
        self.shape = (G, K, N)


def moe_mxfp8_weights_bytes(G: int, K: int, N: int) -> int:
    return int(lib().moe_mxfp8_weights_bytes(G, K, N))


def moe_mxfp8_scales_bytes(G: int, K: int, N: int) -> int:
    return int(lib().moe_mxfp8_scales_bytes(G, K, N))


@_on_stream
def moe_quantize_mxfp8(w: torch.Tensor, stream=None) -> Mxfp8Weight:
    """w bf16 [G,K,N] (or [K,N], taken as G = 1) -> Mxfp8Weight."""
    _need(w, torch.bfloat16, "w")
    G, K, N = (1, *w.shape) if w.dim() == 2 else w.shape
    nc, ns = moe_mxfp8_weights_bytes(G, K, N), moe_mxfp8_scales_bytes(G, K, N)
    codes = torch.empty(max(nc, 16), dtype=torch.uint8, device=w.device)
    scales = torch.empty(max(ns, 16), dtype=torch.uint8, device=w.device)
    _check(lib().moe_quantize_mxfp8(_ptr(w), G, K, N, _ptr(codes), codes.numel(), _ptr(scales),
                                    scales.numel(), _stream(stream)), "moe_quantize_mxfp8")
    return Mxfp8Weight(codes, scales, G, K, N)


_QUANT = {Fp8Weight: "fp8", Mxfp4Weight: "mxfp4", Mxfp8Weight: "mxfp8"}


def _quant_kind(w):
    """'fp8' / 'mxfp4' / 'mxfp8' for quantized weights, None otherwise."""
    return _QUANT.get(type(w))


def _same_kind(kind, w, name):
    if _quant_kind(w) != kind:
        raise TypeError(f"{name}: expected {kind} weights like the others")
    return w


@_on_stream
def moe_gateup_swiglu(x_perm, expert_offsets, w_gate, w_up, h=None, stream=None):
    """w_gate, w_up: bf16 [E,H,F] tensors, PackedWeight (packed call) or
    Fp8Weight (fp8 call)."""
    kind = _quant_kind(w_gate)
    if kind:
        _need(x_perm, torch.bfloat16, "x_perm")
        _need(expert_offsets, torch.int32, "expert_offsets")
        _same_kind(kind, w_up, "w_up")
        M, H = x_perm.shape
        E, _, F = w_gate.shape
        if h is None:
            h = torch.empty((M, F), dtype=torch.bfloat16, device=x_perm.device)
        name = "moe_gateup_swiglu_" + kind
        _check(getattr(lib(), name)(
            _ptr(x_perm), _ptr(expert_offsets), M, H, F, E, _ptr(w_gate.codes),
            _ptr(w_gate.scales), _ptr(w_up.codes), _ptr(w_up.scales), _ptr(h),
            _stream(stream)), name)
        return h
    packed = isinstance(w_gate, PackedWeight)
    _need(x_perm, torch.bfloat16, "x_perm")
    _need(expert_offsets, torch.int32, "expert_offsets")
    _weight(w_gate, "w_gate", packed)
    _weight(w_up, "w_up", packed)
    M, H = x_perm.shape
    E, _, F = w_gate.shape
    if h is None:
        h = torch.empty((M, F), dtype=torch.bfloat16, device=x_perm.device)
    fn = lib().moe_gateup_swiglu_packed if packed else lib().moe_gateup_swiglu
    _check(fn(_ptr(x_perm), _ptr(expert_offsets), M, H, F, E, _ptr(w_gate), _ptr(w_up),
              _ptr(h), _stream(stream)),
           "moe_gateup_swiglu_packed" if packed else "moe_gateup_swiglu")
    return h


@_on_stream
def moe_down(h, expert_offsets, w_down, y_perm=None, stream=None):
    """w_down: bf16 [E,F,H] tensor, PackedWeight (packed call) or Fp8Weight."""
    kind = _quant_kind(w_down)
    if kind:
        _need(h, torch.bfloat16, "h")
        _need(expert_offsets, torch.int32, "expert_offsets")
        M, F = h.shape
        E, _, H = w_down.shape
        if y_perm is None:
            y_perm = torch.empty((M, H), dtype=torch.bfloat16, device=h.device)
        name = "moe_down_" + kind
        _check(getattr(lib(), name)(_ptr(h), _ptr(expert_offsets), M, F, H, E,
                                    _ptr(w_down.codes), _ptr(w_down.scales), _ptr(y_perm),
                                    _stream(stream)), name)
        return y_perm
    packed = isinstance(w_down, PackedWeight)
    _need(h, torch.bfloat16, "h")
    _need(expert_offsets, torch.int32, "expert_offsets")
    _weight(w_down, "w_down", packed)
    M, F = h.shape
    E, _, H = w_down.shape
    if y_perm is None:
        y_perm = torch.empty((M, H), dtype=torch.bfloat16, device=h.device)
    fn = lib().moe_down_packed if packed else lib().moe_down
    _check(fn(_ptr(h), _ptr(expert_offsets), M, F, H, E, _ptr(w_down), _ptr(y_perm),
              _stream(stream)), "moe_down_packed" if packed else "moe_down")
    return y_perm


def moe_grouped_ffn_workspace_bytes(M: int, F: int) -> int:
    return int(lib().moe_grouped_ffn_workspace_bytes(M, F))


@_on_stream
def moe_grouped_ffn(x_perm, expert_offsets, w_gate, w_up, w_down, y_perm=None, ws=None,
                    stream=None):
    """Steps 3+4 with h in the workspace. Returns (h, y_perm): h [M,F] bf16 is
    a view of the start of ws, where the library leaves it."""
    _need(x_perm, torch.bfloat16, "x_perm")
    _need(expert_offsets, torch.int32, "expert_offsets")
    for n, t in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _need(t, torch.bfloat16, n)
    M, H = x_perm.shape
    E, _, F = w_gate.shape
    if y_perm is None:
        y_perm = torch.empty((M, H), dtype=torch.bfloat16, device=x_perm.device)
    if ws is None:
        ws = torch.empty(max(moe_grouped_ffn_workspace_bytes(M, F), 16), dtype=torch.uint8,
                         device=x_perm.device)
    _check(lib().moe_grouped_ffn(_ptr(x_perm), _ptr(expert_offsets), M, H, F, E,
                                 _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(y_perm),
                                 _ptr(ws), ws.numel(), _stream(stream)), "moe_grouped_ffn")
    h = ws[:M * F * 2].view(torch.bfloat16).view(M, F)
    return h, y_perm


@_on_stream
def moe_combine(y_perm, row_dest, topk_w, out=None, stream=None):
    _need(y_perm, torch.bfloat16, "y_perm")
    _need(row_dest, torch.int32, "row_dest")
    _need(topk_w, torch.float32, "topk_w")
    T, k = row_dest.shape
    H = y_perm.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y_perm.device)
    _check(lib().moe_combine(_ptr(y_perm), _ptr(row_dest), _ptr(topk_w), T, H, k,
                             _ptr(out), _stream(stream)), "moe_combine")
    return out


def moe_forward_workspace_bytes(T, H, F, E, k, Fs=0) -> int:
    return int(lib().moe_forward_workspace_bytes(T, H, F, E, k, Fs))


def moe_workspace_bytes(T, H, F, E, k, Fs=0) -> int:
    return int(lib().moe_workspace_bytes(T, H, F, E, k, Fs))


def moe_set_dispatch_override(decode_path: int = -1, tile_class: int = -1):
    """Testing hook: force the decode-size gate/up path (0 LDS ring, 1
    register streaming) and the tile class (0 small, 1 mid, 2 128-row,
    3 256-row) of later calls in this process; -1 is the automatic choice."""
    _check(lib().moe_set_dispatch_override(decode_path, tile_class),
           "moe_set_dispatch_override")


def moe_set_combine_override(mode: int = -1):
    """Testing hook: 1 lets decode-size down projections of the fused layer
    combine in their epilogue; 0 or -1 (automatic) keeps the combine in a
    launch of its own."""
    _check(lib().moe_set_combine_override(mode), "moe_set_combine_override")


def moe_set_diagnostics(trace: int = -1, check_ids: int = -1):
    """Launch trace to stderr (trace=1, as MOE_TRACE=1) and the id check of
    the calls that take caller expert ids (check_ids=1, as MOE_DEBUG=1); 0
    turns either off, -1 restores the environment's setting."""
    _check(lib().moe_set_diagnostics(trace, check_ids), "moe_set_diagnostics")


@_on_stream
def moe_check_topk_ids(topk_ids: torch.Tensor, E: int, stream=None) -> bool:
    """True when every id of topk_ids [T, k] lies in [0, E) (checked on the
    GPU; waits for the result)."""
    _need(topk_ids, torch.int32, "topk_ids")
    T, k = topk_ids.shape
    st = lib().moe_check_topk_ids(_ptr(topk_ids), T, k, E, _stream(stream))
    if st == MOE_ERR_BAD_IDS:
        return False
    _check(st, "moe_check_topk_ids")
    return True


def _shared_struct(shared, packed):
    if shared is None:
        return None, 0
    for n in ("w_gate", "w_up", "w_down"):
        _weight(shared[n], "shared " + n, packed)
    Fs = shared["w_gate"].shape[-1]
    g = shared.get("gate_logits")
    return SharedExpert(shared["w_gate"].data_ptr(), shared["w_up"].data_ptr(),
                        shared["w_down"].data_ptr(), Fs,
                        None if g is None else g.data_ptr()), Fs


@_on_stream
def moe_forward_routed(x, topk_ids, topk_w, w_gate, w_up, w_down,
                       shared: Optional[dict] = None, out=None, ws=None, stream=None):
    """Layer steps 2-5 from a given routing (topk_ids int32 [T,k], topk_w
    fp32 [T,k]); weights row-major or all PackedWeight. Returns out."""
    packed = isinstance(w_gate, PackedWeight)
    _need(x, torch.bfloat16, "x")
    _need(topk_ids, torch.int32, "topk_ids")
    _need(topk_w, torch.float32, "topk_w")
    for n, t in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _weight(t, n, packed)
    T, H = x.shape
    E, _, F = w_gate.shape
    k = topk_ids.shape[1]
    sh, Fs = _shared_struct(shared, packed)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = torch.empty(max(moe_forward_workspace_bytes(T, H, F, E, k, Fs), 16),
                         dtype=torch.uint8, device=x.device)
    _check(lib().moe_forward_routed(_ptr(x), _ptr(topk_ids), _ptr(topk_w), T, H, F, E, k,
                                    _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                    ctypes.byref(sh) if sh is not None else None,
                                    1 if packed else 0, _ptr(out), _ptr(ws), ws.numel(),
                                    _stream(stream)), "moe_forward_routed")
    return out


@_on_stream
def moe_forward(x, logits, k, w_gate, w_up, w_down, shared: Optional[dict] = None,
                out=None, topk_ids=None, topk_w=None, ws=None, stream=None):
    """Whole layer. shared: None or dict(w_gate [H,Fs], w_up [H,Fs],
    w_down [Fs,H], gate_logits [T] fp32 or None). Returns out [T,H] bf16.
    With PackedWeight weights (all of them, shared expert included: packed
    from [1,H,Fs] / [1,Fs,H]) this calls moe_forward_packed."""
    if _quant_kind(w_gate):
        return _forward_quant(x, logits, k, w_gate, w_up, w_down, shared, out, topk_ids,
                              topk_w, ws, stream)
    packed = isinstance(w_gate, PackedWeight)
    _need(x, torch.bfloat16, "x")
    _need(logits, torch.float32, "logits")
    for n, t in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _weight(t, n, packed)
    T, H = x.shape
    E, _, F = w_gate.shape
    sh, Fs = _shared_struct(shared, packed)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = torch.empty(max(moe_forward_workspace_bytes(T, H, F, E, k, Fs), 16),
                         dtype=torch.uint8, device=x.device)
    fn = lib().moe_forward_packed if packed else lib().moe_forward
    _check(fn(_ptr(x), _ptr(logits), T, H, F, E, k, _ptr(w_gate), _ptr(w_up), _ptr(w_down),
              ctypes.byref(sh) if sh is not None else None, _ptr(out), _ptr(topk_ids),
              _ptr(topk_w), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_forward_packed" if packed else "moe_forward")
    return out


@_on_stream
def moe_forward_packed_noalloc(x, logits, k, w_gate, w_up, w_down,
                               shared: Optional[dict] = None, out=None, topk_ids=None,
                               topk_w=None, stream=None):
    """moe_forward_packed with the library's fixed device workspace (no
    workspace is allocated; `out` and the optional routing outputs are
    allocated here only when not given). All weights PackedWeight."""
    _need(x, torch.bfloat16, "x")
    _need(logits, torch.float32, "logits")
    for n, t in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _weight(t, n, True)
    T, H = x.shape
    E, _, F = w_gate.shape
    sh, _ = _shared_struct(shared, True)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _check(lib().moe_forward_packed_noalloc(
        _ptr(x), _ptr(logits), T, H, F, E, k, _ptr(w_gate), _ptr(w_up), _ptr(w_down),
        ctypes.byref(sh) if sh is not None else None, _ptr(out), _ptr(topk_ids), _ptr(topk_w),
        _stream(stream)), "moe_forward_packed_noalloc")
    return out


@_on_stream
def _forward_quant(x, logits, k, w_gate, w_up, w_down, shared, out, topk_ids, topk_w, ws,
                   stream):
    """moe_forward_fp8, moe_forward_mxfp4 or moe_forward_mxfp8, by the weights' kind."""
    kind = _quant_kind(w_gate)
    _need(x, torch.bfloat16, "x")
    _need(logits, torch.float32, "logits")
    for n, t in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _same_kind(kind, t, n)
    T, H = x.shape
    E, _, F = w_gate.shape
    sh, Fs = None, 0
    if shared is not None:
        for n in ("w_gate", "w_up", "w_down"):
            _same_kind(kind, shared[n], "shared " + n)
        Fs = shared["w_gate"].shape[-1]
        g = shared.get("gate_logits")
        cls = {"fp8": SharedExpertFp8, "mxfp4": SharedExpertMxfp4,
               "mxfp8": SharedExpertMxfp8}[kind]
        sh = cls(shared["w_gate"].codes.data_ptr(), shared["w_gate"].scales.data_ptr(),
                 shared["w_up"].codes.data_ptr(), shared["w_up"].scales.data_ptr(),
                 shared["w_down"].codes.data_ptr(), shared["w_down"].scales.data_ptr(), Fs,
                 None if g is None else g.data_ptr())
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = torch.empty(max(moe_forward_workspace_bytes(T, H, F, E, k, Fs), 16),
                         dtype=torch.uint8, device=x.device)
    name = "moe_forward_" + kind
    _check(getattr(lib(), name)(
        _ptr(x), _ptr(logits), T, H, F, E, k, _ptr(w_gate.codes), _ptr(w_gate.scales),
        _ptr(w_up.codes), _ptr(w_up.scales), _ptr(w_down.codes), _ptr(w_down.scales),
        ctypes.byref(sh) if sh is not None else None, _ptr(out), _ptr(topk_ids), _ptr(topk_w),
        _ptr(ws), ws.numel(), _stream(stream)), name)
    return out


def moe_backward_workspace_bytes(T, H, F, E, k) -> int:
    return int(lib().moe_backward_workspace_bytes(T, H, F, E, k))


@_on_stream
def moe_backward_shared_workspace_bytes(T, H, F, E, k, Fs) -> int:
    return lib().moe_backward_shared_workspace_bytes(T, H, F, E, k, Fs)


def moe_backward(x, topk_ids, topk_w, w_gate, w_up, w_down, dout, shared: Optional[dict] = None,
                 ws=None, stream=None):
    """Gradients of the layer (row-major bf16 weights) for the routing
    (topk_ids int32 [T,k], topk_w fp32 [T,k]) and the output gradient dout
    [T,H] bf16. Returns dict(dx [T,H] bf16, d_topk_w [T,k] fp32, dw_gate,
    dw_up [E,H,F] fp32, dw_down [E,F,H] fp32). With `shared` (dict(w_gate,
    w_up [H,Fs], w_down [Fs,H] bf16, gate_logits [T] fp32 or None), as for
    moe_forward) dx includes the shared expert's part and the dict adds
    dw_gate_sh, dw_up_sh [H,Fs], dw_down_sh [Fs,H] and d_gate_logits [T]
    (None without gate logits), all fp32."""
    for n, t, dt in (("x", x, torch.bfloat16), ("topk_ids", topk_ids, torch.int32),
                     ("topk_w", topk_w, torch.float32), ("w_gate", w_gate, torch.bfloat16),
                     ("w_up", w_up, torch.bfloat16), ("w_down", w_down, torch.bfloat16),
                     ("dout", dout, torch.bfloat16)):
        _need(t, dt, n)
    T, H = x.shape
    E, _, F = w_gate.shape
    k = topk_ids.shape[1]
    dev = x.device
    g = dict(dx=torch.empty((T, H), dtype=torch.bfloat16, device=dev),
             d_topk_w=torch.empty((T, k), dtype=torch.float32, device=dev),
             dw_gate=torch.empty((E, H, F), dtype=torch.float32, device=dev),
             dw_up=torch.empty((E, H, F), dtype=torch.float32, device=dev),
             dw_down=torch.empty((E, F, H), dtype=torch.float32, device=dev))
    if shared is None:
        if ws is None:
            ws = torch.empty(max(moe_backward_workspace_bytes(T, H, F, E, k), 16),
                             dtype=torch.uint8, device=dev)
        _check(lib().moe_backward(_ptr(x), _ptr(topk_ids), _ptr(topk_w), T, H, F, E, k,
                                  _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(dout),
                                  _ptr(g["dx"]), _ptr(g["d_topk_w"]), _ptr(g["dw_gate"]),
                                  _ptr(g["dw_up"]), _ptr(g["dw_down"]), _ptr(ws), ws.numel(),
                                  _stream(stream)), "moe_backward")
        return g
    sw = {n: shared[n] for n in ("w_gate", "w_up", "w_down")}
    for n, t in sw.items():
        _need(t, torch.bfloat16, "shared " + n)
    gl = shared.get("gate_logits")
    if gl is not None:
        _need(gl, torch.float32, "shared gate_logits")
    Fs = sw["w_gate"].shape[1]
    g.update(dw_gate_sh=torch.empty((H, Fs), dtype=torch.float32, device=dev),
             dw_up_sh=torch.empty((H, Fs), dtype=torch.float32, device=dev),
             dw_down_sh=torch.empty((Fs, H), dtype=torch.float32, device=dev),
             d_gate_logits=None if gl is None else torch.empty(T, dtype=torch.float32,
                                                               device=dev))
    st = SharedExpert(_ptr(sw["w_gate"]), _ptr(sw["w_up"]), _ptr(sw["w_down"]), Fs, _ptr(gl))
    sg = SharedExpertGrads(_ptr(g["dw_gate_sh"]), _ptr(g["dw_up_sh"]), _ptr(g["dw_down_sh"]),
                           _ptr(g["d_gate_logits"]))
    if ws is None:
        ws = torch.empty(max(moe_backward_shared_workspace_bytes(T, H, F, E, k, Fs), 16),
                         dtype=torch.uint8, device=dev)
    _check(lib().moe_backward_shared(_ptr(x), _ptr(topk_ids), _ptr(topk_w), T, H, F, E, k,
                                     _ptr(w_gate), _ptr(w_up), _ptr(w_down), ctypes.byref(st),
                                     _ptr(dout), _ptr(g["dx"]), _ptr(g["d_topk_w"]),
                                     _ptr(g["dw_gate"]), _ptr(g["dw_up"]), _ptr(g["dw_down"]),
                                     ctypes.byref(sg), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_backward_shared")
    return g


@_on_stream
def moe_route_backward(topk_ids, topk_w, d_topk_w, E, d_logits=None, stream=None):
    """Router-logit gradient [T,E] fp32 through the softmax over the k
    selected logits."""
    _need(topk_ids, torch.int32, "topk_ids")
    _need(topk_w, torch.float32, "topk_w")
    _need(d_topk_w, torch.float32, "d_topk_w")
    T, k = topk_ids.shape
    if d_logits is None:
        d_logits = torch.empty((T, E), dtype=torch.float32, device=topk_ids.device)
    _check(lib().moe_route_backward(_ptr(topk_ids), _ptr(topk_w), _ptr(d_topk_w), T, E, k,
                                    _ptr(d_logits), _stream(stream)), "moe_route_backward")
    return d_logits

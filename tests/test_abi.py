"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/moe.h declares, reports workspace sizes, and rejects
bad arguments with the documented status before enqueuing anything.

Every call here fails validation (or has T == 0), so no kernel is launched;
the fake pointer values are never dereferenced."""
import ctypes

import pytest

from grouped_gemm_softmax_amd import binding as B

OK, INVALID, SHAPE, MISALIGNED, WS_SMALL, HIP, BAD_IDS = 0, -1, -2, -3, -4, -5, -6
P = ctypes.c_void_p(0x10000)        # 16-byte aligned fake address (never read)
Q = ctypes.c_void_p(0x10008)        # 8 mod 16: misaligned for bf16 tensors
NULL = None


@pytest.fixture(scope="module")
def L():
    return B.lib()


def test_library_exports_every_header_symbol(L):
    names = B.header_symbols()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(B._SIGNATURES)


def test_workspace_bytes_alias():
    for args in [(32, 4096, 14336, 8, 2, 0), (4096, 7168, 2048, 256, 8, 2048), (0, 64, 96, 8, 2, 0)]:
        assert B.moe_workspace_bytes(*args) == B.moe_forward_workspace_bytes(*args)


def test_dispatch_override_hook(L):
    assert L.moe_set_dispatch_override(2, -1) == INVALID
    assert L.moe_set_dispatch_override(-1, 4) == INVALID
    assert L.moe_set_dispatch_override(-2, -1) == INVALID
    assert L.moe_set_dispatch_override(1, 3) == OK
    assert L.moe_set_dispatch_override(-1, -1) == OK


def test_combine_override_hook(L):
    assert L.moe_set_combine_override(2) == INVALID
    assert L.moe_set_combine_override(-2) == INVALID
    assert L.moe_set_combine_override(1) == OK
    assert L.moe_set_combine_override(0) == OK
    assert L.moe_set_combine_override(-1) == OK


def test_diagnostics_hook(L):
    assert L.moe_set_diagnostics(2, 0) == INVALID
    assert L.moe_set_diagnostics(0, -2) == INVALID
    assert L.moe_set_diagnostics(0, 1) == OK
    # with the id check on, argument validation still comes first: these
    # calls fail before anything (the check included) reaches the GPU
    ws = B.moe_permute_workspace_bytes(100, 8, 2)
    assert L.moe_permute(P, P, 100, 64, 8, 2, P, P, P, P, P, ws - 1, NULL) == WS_SMALL
    assert L.moe_route_backward(P, P, P, 4, 8, 9, P, NULL) == SHAPE
    assert L.moe_check_topk_ids(P, 4, 9, 8, NULL) == SHAPE
    assert L.moe_set_diagnostics(-1, -1) == OK


def test_check_topk_ids_validation(L):
    assert L.moe_check_topk_ids(P, -1, 2, 8, NULL) == INVALID       # T < 0
    assert L.moe_check_topk_ids(P, 4, 0, 8, NULL) == INVALID        # k < 1
    assert L.moe_check_topk_ids(P, 4, 2, 2000, NULL) == SHAPE       # E > 1024
    assert L.moe_check_topk_ids(NULL, 4, 2, 8, NULL) == INVALID     # null ids
    assert L.moe_check_topk_ids(ctypes.c_void_p(0x10002), 4, 2, 8, NULL) == MISALIGNED
    assert L.moe_check_topk_ids(NULL, 0, 2, 8, NULL) == OK          # T = 0: no-op


def test_status_strings(L):
    for s in (OK, INVALID, SHAPE, MISALIGNED, WS_SMALL, HIP, BAD_IDS):
        txt = B.moe_status_string(s)
        assert txt and txt != "unknown moe status"
    assert B.moe_status_string(7) == "unknown moe status"


def test_route_validation(L):
    assert L.moe_route(P, 4, 8, 0, P, P, NULL) == INVALID          # k < 1
    assert L.moe_route(P, 4, 8, 9, P, P, NULL) == SHAPE            # k > E
    assert L.moe_route(P, 4, 2000, 2, P, P, NULL) == SHAPE         # E > 1024
    assert L.moe_route(P, 4, 32, 17, P, P, NULL) == SHAPE          # k > 16
    assert L.moe_route(P, -1, 8, 2, P, P, NULL) == INVALID         # T < 0
    assert L.moe_route(NULL, 4, 8, 2, P, P, NULL) == INVALID       # null logits
    assert L.moe_route(P, 4, 8, 2, ctypes.c_void_p(0x10002), P, NULL) == MISALIGNED
    assert L.moe_route(NULL, 0, 8, 2, NULL, NULL, NULL) == OK      # T = 0: no-op


def _router_ws_model(T, H, E, k, cus=256):
    """Router plan as documented: tiles of 16*nt tokens x 16*nb experts; H cut
    into slices of whole 64-wide chunks, at least 4 chunks each, until the
    blocks reach 3 per compute unit (one slice when all experts fit a block
    and the tiles give a block per compute unit); one slice with all experts
    in the block ranks in the GEMM kernel (no workspace), else
    nslices*T*E fp32 partials."""
    if T == 0 or k > E:
        return 0
    nb = 1 if E <= 16 else 2 if E <= 32 else 4
    nt = 1 if T <= 16 else 2 if T <= 32 else 4
    tiles = -(-T // (16 * nt)) * -(-E // (16 * nb))
    chunks = -(-H // 64)
    S = -(-3 * cus // tiles)
    if E <= 16 * nb and tiles >= cus:
        S = 1
    S = min(max(1, S), -(-chunks // 4))
    per = -(-chunks // S)
    nslices = -(-chunks // per)
    if nslices == 1 and E <= 16 * nb:
        return 0
    return -(-nslices * T * E * 4 // 256) * 256


@pytest.mark.parametrize("T,H,E,k", [(1, 4096, 8, 2), (32, 4096, 8, 2), (16, 2048, 60, 4),
                                     (128, 7168, 256, 8), (4096, 7168, 256, 8),
                                     (16384, 2048, 60, 4), (40000, 2048, 60, 4),
                                     (20, 256, 1024, 16), (70, 200, 33, 3), (5, 64, 1, 1),
                                     (64, 256, 16, 4), (0, 256, 8, 2), (16, 128, 8, 9)])
def test_router_workspace_bytes(T, H, E, k):
    assert B.moe_router_workspace_bytes(T, H, E, k) == _router_ws_model(T, H, E, k)


def test_router_workspace_fused_cases():
    # all experts in one block and one K-slice: no workspace
    assert B.moe_router_workspace_bytes(64, 256, 16, 4) == 0      # H = 4 chunks
    assert B.moe_router_workspace_bytes(16384, 2048, 60, 4) == 0  # >= 256 tiles
    assert B.moe_router_workspace_bytes(16, 60, 8, 2) == 0        # invalid H


def test_router_route_validation(L):
    ws = B.moe_router_workspace_bytes(16, 2048, 60, 4)
    assert ws > 0
    args = lambda x=P, w=P, T=16, H=2048, E=60, k=4, lg=NULL, ids=P, ws_p=P, ws_bytes=ws: (
        x, w, T, H, E, k, lg, ids, P, ws_p, ws_bytes, NULL)
    assert L.moe_router_route(*args(x=NULL)) == INVALID
    assert L.moe_router_route(*args(w=NULL)) == INVALID
    assert L.moe_router_route(*args(ids=NULL)) == INVALID
    assert L.moe_router_route(*args(x=Q)) == MISALIGNED
    assert L.moe_router_route(*args(w=Q)) == MISALIGNED
    assert L.moe_router_route(*args(lg=ctypes.c_void_p(0x10002))) == MISALIGNED
    assert L.moe_router_route(*args(ws_p=Q)) == MISALIGNED
    assert L.moe_router_route(*args(H=60)) == SHAPE                  # H % 8 != 0
    assert L.moe_router_route(*args(k=61)) == SHAPE                  # k > E
    assert L.moe_router_route(*args(E=2000)) == SHAPE                # E > 1024
    assert L.moe_router_route(*args(k=0)) == INVALID
    assert L.moe_router_route(*args(ws_bytes=ws - 1)) == WS_SMALL
    assert L.moe_router_route(*args(ws_p=NULL)) == INVALID
    assert L.moe_router_route(NULL, NULL, 0, 64, 8, 2, NULL, NULL, NULL, NULL, 0, NULL) == OK


def test_permute_validation(L):
    ws = B.moe_permute_workspace_bytes(100, 8, 2)
    assert ws > 0 and ws % 256 == 0
    assert B.moe_permute_workspace_bytes(100, 8, 9) == 0
    args = lambda x=P, xp=P, ws_bytes=ws, H=64: (x, P, 100, H, 8, 2, P, P, P, xp, P, ws_bytes, NULL)
    assert L.moe_permute(*args(x=NULL)) == INVALID
    assert L.moe_permute(*args(x=Q)) == MISALIGNED
    assert L.moe_permute(*args(xp=Q)) == MISALIGNED
    assert L.moe_permute(*args(H=60)) == SHAPE                     # H % 8 != 0
    assert L.moe_permute(*args(ws_bytes=ws - 1)) == WS_SMALL
    assert L.moe_permute(NULL, NULL, 0, 64, 8, 2, NULL, NULL, NULL, NULL, NULL, 0, NULL) == OK


def test_ffn_validation(L):
    assert L.moe_gateup_swiglu(P, P, 128, 64, 100, 8, P, P, P, NULL) == SHAPE    # F % 8
    assert L.moe_gateup_swiglu(P, P, 128, 64, 96, 0, P, P, P, NULL) == INVALID   # E = 0
    assert L.moe_gateup_swiglu(P, P, 128, 64, 96, 8, P, NULL, P, NULL) == INVALID
    assert L.moe_gateup_swiglu(P, P, 128, 64, 96, 8, Q, P, P, NULL) == MISALIGNED
    assert L.moe_down(P, P, 128, 96, 64, 8, P, Q, NULL) == MISALIGNED
    assert L.moe_down(P, NULL, 128, 96, 64, 8, P, P, NULL) == INVALID
    assert L.moe_down(P, P, 1 << 20, 4096, 4096, 8, P, P, NULL) == SHAPE        # > 2^31 elements
    ws = B.moe_grouped_ffn_workspace_bytes(128, 96)
    assert ws == 128 * 96 * 2
    assert B.moe_grouped_ffn_workspace_bytes(3, 8) == 256                       # 256-byte units
    assert B.moe_grouped_ffn_workspace_bytes(3, 12) == 0                        # F % 8
    assert L.moe_grouped_ffn(P, P, 128, 64, 96, 8, P, P, NULL, P, P, ws, NULL) == INVALID
    assert L.moe_grouped_ffn(P, P, 128, 64, 96, 8, P, P, P, P, NULL, ws, NULL) == INVALID
    assert L.moe_grouped_ffn(P, P, 128, 64, 96, 8, P, P, P, P, Q, ws, NULL) == MISALIGNED
    assert L.moe_grouped_ffn(P, P, 128, 64, 96, 8, P, P, P, P, P, ws - 1, NULL) == WS_SMALL
    assert L.moe_grouped_ffn(NULL, NULL, 0, 64, 96, 8, NULL, NULL, NULL, NULL, NULL, 0,
                             NULL) == OK


def test_combine_validation(L):
    assert L.moe_combine(P, P, P, 10, 64, 0, P, NULL) == INVALID
    assert L.moe_combine(P, P, P, 10, 64, 17, P, NULL) == SHAPE
    assert L.moe_combine(P, P, P, 10, 63, 2, P, NULL) == SHAPE
    assert L.moe_combine(P, P, P, 10, 64, 2, Q, NULL) == MISALIGNED
    assert L.moe_combine(NULL, NULL, NULL, 0, 64, 2, NULL, NULL) == OK


def _fwd(L, T=32, H=64, F=96, E=8, k=2, x=P, ws=P, ws_bytes=None, shared=None, out=P):
    if ws_bytes is None:
        ws_bytes = B.moe_forward_workspace_bytes(T, H, F, E, k, shared.Fs if shared else 0)
    return L.moe_forward(x, P, T, H, F, E, k, P, P, P,
                         ctypes.byref(shared) if shared else None, out, NULL, NULL,
                         ws, ws_bytes, NULL)


def test_forward_validation(L):
    assert _fwd(L, x=NULL) == INVALID
    assert _fwd(L, out=Q) == MISALIGNED
    assert _fwd(L, k=9) == SHAPE
    assert _fwd(L, ws_bytes=16) == WS_SMALL
    bad_shared = B.SharedExpert(0x10000, 0x10000, 0x10000, 20, None)   # Fs % 8 != 0
    assert _fwd(L, shared=bad_shared, ws_bytes=1 << 40) == SHAPE
    null_shared = B.SharedExpert(0x10000, None, 0x10000, 32, None)
    assert _fwd(L, shared=null_shared, ws_bytes=1 << 40) == INVALID
    assert L.moe_forward(NULL, NULL, 0, 64, 96, 8, 2, NULL, NULL, NULL, None, NULL,
                         NULL, NULL, NULL, 0, NULL) == OK


def test_fp8_weights_bytes():
    assert B.moe_fp8_weights_bytes(2, 200, 328) == 2 * 6 * 4 * 4096   # ceil(N/64) x ceil(K/64)
    assert B.moe_fp8_weights_bytes(1, 64, 64) == 4096
    assert B.moe_fp8_weights_bytes(0, 64, 64) == 0
    assert B.moe_fp8_weights_bytes(1, 60, 64) == 0                   # K % 8 != 0


def test_fp8_calls_validation(L):
    nb = B.moe_fp8_weights_bytes(2, 64, 96)
    q = lambda w=P, G=2, K=64, N=96, c=P, nbytes=nb, s=P: L.moe_quantize_fp8(w, G, K, N, c, nbytes, s, NULL)
    assert q(w=NULL) == INVALID
    assert q(s=NULL) == INVALID
    assert q(G=0) == INVALID
    assert q(K=60) == SHAPE
    assert q(c=Q) == MISALIGNED
    assert q(s=Q) == MISALIGNED
    assert q(nbytes=nb - 1) == WS_SMALL
    g = lambda sg=P, su=P, wg=P: L.moe_gateup_swiglu_fp8(P, P, 16, 64, 96, 2, wg, sg, P, su, P, NULL)
    assert g(sg=NULL) == INVALID
    assert g(su=Q) == MISALIGNED
    assert g(wg=Q) == MISALIGNED
    assert L.moe_down_fp8(P, P, 16, 96, 64, 2, P, NULL, P, NULL) == INVALID
    assert L.moe_down_fp8(P, P, 0, 96, 64, 2, NULL, NULL, NULL, NULL) == OK     # M = 0
    ws = B.moe_forward_workspace_bytes(10, 64, 96, 8, 2, 0)
    f = lambda sd=P, ws_bytes=ws: L.moe_forward_fp8(P, P, 10, 64, 96, 8, 2, P, P, P, P, P, sd,
                                                     None, P, NULL, NULL, P, ws_bytes, NULL)
    assert f(sd=NULL) == INVALID
    assert f(ws_bytes=ws - 1) == WS_SMALL
    bad = B.SharedExpertFp8(0x10000, 0x10000, 0x10000, 0x10000, 0x10000, None, 32, None)
    assert L.moe_forward_fp8(P, P, 10, 64, 96, 8, 2, P, P, P, P, P, P, ctypes.byref(bad), P,
                             NULL, NULL, P, 1 << 40, NULL) == INVALID          # null shared scale
    assert L.moe_forward_fp8(NULL, NULL, 0, 64, 96, 8, 2, NULL, NULL, NULL, NULL, NULL, NULL,
                             None, NULL, NULL, NULL, NULL, 0, NULL) == OK      # T = 0


def test_mxfp4_bytes():
    # codes: ceil(N/64) x ceil(K/64) blocks of 2 KB; scales: ceil(N/64) x
    # 4*ceil(K/128) x 64 bytes
    assert B.moe_mxfp4_weights_bytes(2, 200, 328) == 2 * 6 * 4 * 2048
    assert B.moe_mxfp4_scales_bytes(2, 200, 328) == 2 * 6 * 8 * 64
    assert B.moe_mxfp4_weights_bytes(1, 64, 64) == 2048
    assert B.moe_mxfp4_scales_bytes(1, 64, 64) == 4 * 64
    assert B.moe_mxfp4_weights_bytes(0, 64, 64) == 0
    assert B.moe_mxfp4_scales_bytes(1, 60, 64) == 0                   # K % 8 != 0


def test_mxfp4_calls_validation(L):
    nc, ns = B.moe_mxfp4_weights_bytes(2, 64, 96), B.moe_mxfp4_scales_bytes(2, 64, 96)
    q = lambda w=P, G=2, K=64, N=96, c=P, ncb=nc, s=P, nsb=ns: L.moe_quantize_mxfp4(
        w, G, K, N, c, ncb, s, nsb, NULL)
    assert q(w=NULL) == INVALID
    assert q(s=NULL) == INVALID
    assert q(G=0) == INVALID
    assert q(N=100) == SHAPE
    assert q(c=Q) == MISALIGNED
    assert q(s=Q) == MISALIGNED
    assert q(ncb=nc - 1) == WS_SMALL
    assert q(nsb=ns - 1) == WS_SMALL
    g = lambda sg=P, su=P, wg=P: L.moe_gateup_swiglu_mxfp4(P, P, 16, 64, 96, 2, wg, sg, P, su, P,
                                                           NULL)
    assert g(sg=NULL) == INVALID
    assert g(su=Q) == MISALIGNED
    assert g(wg=Q) == MISALIGNED
    assert L.moe_down_mxfp4(P, P, 16, 96, 64, 2, P, NULL, P, NULL) == INVALID
    assert L.moe_down_mxfp4(P, P, 0, 96, 64, 2, NULL, NULL, NULL, NULL) == OK   # M = 0
    ws = B.moe_forward_workspace_bytes(10, 64, 96, 8, 2, 0)
    f = lambda sd=P, ws_bytes=ws: L.moe_forward_mxfp4(P, P, 10, 64, 96, 8, 2, P, P, P, P, P, sd,
                                                       None, P, NULL, NULL, P, ws_bytes, NULL)
    assert f(sd=NULL) == INVALID
    assert f(ws_bytes=ws - 1) == WS_SMALL
    bad = B.SharedExpertMxfp4(0x10000, 0x10000, 0x10000, None, 0x10000, 0x10000, 32, None)
    assert L.moe_forward_mxfp4(P, P, 10, 64, 96, 8, 2, P, P, P, P, P, P, ctypes.byref(bad), P,
                               NULL, NULL, P, 1 << 40, NULL) == INVALID        # null shared scale
    assert L.moe_forward_mxfp4(NULL, NULL, 0, 64, 96, 8, 2, NULL, NULL, NULL, NULL, NULL, NULL,
                               None, NULL, NULL, NULL, NULL, 0, NULL) == OK    # T = 0


def test_mxfp8_bytes():
    # codes: the fp8 layout, ceil(N/64) x ceil(K/64) blocks of 4 KB; scales:
    # the mxfp4 layout, ceil(N/64) x 4*ceil(K/128) x 64 bytes
    assert B.moe_mxfp8_weights_bytes(2, 200, 328) == 2 * 6 * 4 * 4096
    assert B.moe_mxfp8_scales_bytes(2, 200, 328) == 2 * 6 * 8 * 64
    assert B.moe_mxfp8_weights_bytes(1, 64, 64) == 4096
    assert B.moe_mxfp8_scales_bytes(1, 64, 64) == 4 * 64
    assert B.moe_mxfp8_weights_bytes(0, 64, 64) == 0
    assert B.moe_mxfp8_scales_bytes(1, 60, 64) == 0                   # K % 8 != 0


def test_mxfp8_calls_validation(L):
    nc, ns = B.moe_mxfp8_weights_bytes(2, 64, 96), B.moe_mxfp8_scales_bytes(2, 64, 96)
    q = lambda w=P, G=2, K=64, N=96, c=P, ncb=nc, s=P, nsb=ns: L.moe_quantize_mxfp8(
        w, G, K, N, c, ncb, s, nsb, NULL)
    assert q(w=NULL) == INVALID
    assert q(s=NULL) == INVALID
    assert q(G=0) == INVALID
    assert q(N=100) == SHAPE
    assert q(c=Q) == MISALIGNED
    assert q(s=Q) == MISALIGNED
    assert q(ncb=nc - 1) == WS_SMALL
    assert q(nsb=ns - 1) == WS_SMALL
    g = lambda sg=P, su=P, wg=P: L.moe_gateup_swiglu_mxfp8(P, P, 16, 64, 96, 2, wg, sg, P, su, P,
                                                           NULL)
    assert g(sg=NULL) == INVALID
    assert g(su=Q) == MISALIGNED
    assert g(wg=Q) == MISALIGNED
    assert L.moe_down_mxfp8(P, P, 16, 96, 64, 2, P, NULL, P, NULL) == INVALID
    assert L.moe_down_mxfp8(P, P, 0, 96, 64, 2, NULL, NULL, NULL, NULL) == OK   # M = 0
    ws = B.moe_forward_workspace_bytes(10, 64, 96, 8, 2, 0)
    f = lambda sd=P, ws_bytes=ws: L.moe_forward_mxfp8(P, P, 10, 64, 96, 8, 2, P, P, P, P, P, sd,
                                                       None, P, NULL, NULL, P, ws_bytes, NULL)
    assert f(sd=NULL) == INVALID
    assert f(ws_bytes=ws - 1) == WS_SMALL
    bad = B.SharedExpertMxfp8(0x10000, 0x10000, 0x10000, None, 0x10000, 0x10000, 32, None)
    assert L.moe_forward_mxfp8(P, P, 10, 64, 96, 8, 2, P, P, P, P, P, P, ctypes.byref(bad), P,
                               NULL, NULL, P, 1 << 40, NULL) == INVALID        # null shared scale
    assert L.moe_forward_mxfp8(NULL, NULL, 0, 64, 96, 8, 2, NULL, NULL, NULL, NULL, NULL, NULL,
                               None, NULL, NULL, NULL, NULL, 0, NULL) == OK    # T = 0


def test_forward_routed_validation(L):
    ws = B.moe_forward_workspace_bytes(10, 64, 96, 8, 2, 0)
    args = lambda x=P, ids=P, w=P, k=2, packed=0, ws_bytes=ws: (
        x, ids, w, 10, 64, 96, 8, k, P, P, P, None, packed, P, P, ws_bytes, NULL)
    assert L.moe_forward_routed(*args(x=NULL)) == INVALID
    assert L.moe_forward_routed(*args(ids=NULL)) == INVALID
    assert L.moe_forward_routed(*args(w=NULL)) == INVALID
    assert L.moe_forward_routed(*args(ids=ctypes.c_void_p(0x10002))) == MISALIGNED
    assert L.moe_forward_routed(*args(packed=2)) == INVALID
    assert L.moe_forward_routed(*args(k=9)) == SHAPE
    assert L.moe_forward_routed(*args(ws_bytes=ws - 1)) == WS_SMALL
    assert L.moe_forward_routed(NULL, NULL, NULL, 0, 64, 96, 8, 2, NULL, NULL, NULL, None, 0,
                                NULL, NULL, 0, NULL) == OK


def _down_ksplit(T, H, F, E, k, Fs, cus=256):
    """Re-statement of the host heuristic for K-slices of the fused layer's
    down projection, as (routed, shared). Tile: large (256 rows x 256
    columns, 32-deep stages) at >= 192 rows per expert, large128 (128 x 256,
    64-deep) at 64..191 when its expected items reach 2 x CUs, else large;
    small (32 x 64, 64-deep) below 64. Expected items: one partial row tile per touched expert plus
    the full ones, times the column tiles (plus the shared expert's). The
    split doubles while twice the items still fit in 2 x CUs and each slice
    keeps >= 256 and >= 4 stages of K. The shared expert's items are split
    further, to about the routed items' K-steps, while they are fewer than
    2 x CUs and keep >= 4 K-steps each."""
    A = T * k
    rows = A // E
    BT, BF, BK = (256, 256, 32) if rows >= 192 else (128, 256, 64) if rows >= 64 else (32, 64, 64)
    if BT == 128:
        items128 = (min(A, E) + A // 128) * -(-H // 256)
        if Fs:
            items128 += (1 + T // 128) * -(-H // 256)
        if items128 < 2 * cus:
            BT = 256
    ntile = -(-H // BF)
    items = (min(A, E) + A // BT) * ntile
    min_k = F
    if Fs:
        items += (1 + T // BT) * ntile
        min_k = min(F, Fs)
    split = 1
    while (split < 8 and items * split * 2 <= 2 * cus and min_k // (split * 2) >= 256
           and min_k // (split * 2) >= 4 * BK):
        split *= 2
    shared = split
    if Fs:
        steps0 = -(-(-(-F // BK)) // split)
        nk1 = -(-Fs // BK)
        items1 = -(-T // BT) * ntile
        r = min(8, max(1, (nk1 + steps0 // 2) // steps0))
        if r > split and items1 < 2 * cus and nk1 // r >= 4:
            shared = r
    return split, shared


def _layout_model(T, H, F, E, k, Fs):
    """Independent re-statement of the documented forward workspace layout."""
    al = lambda v: (v + 255) // 256 * 256
    A = T * k
    # routing chunk (tokens per histogram row): about T/128, within 4 .. min(32, 256/k)
    chunk = min(max(4, -(-T // 128)), min(32, 256 // k))
    nch = (T + chunk - 1) // chunk
    S, S_sh = _down_ksplit(T, H, F, E, k, Fs)
    parts = [nch * E * 4, A * 4, A * 4, (E + 1) * 4, A * 4, A * 4, A * H * 2,
             A * F * 2, T * Fs * 2, S * A * H * 4, S_sh * T * (H if Fs else 0) * 4,
             T * ((H + 63) // 64) * 4]   # arrival counters of the epilogue combine
    return sum(al(p) for p in parts)


@pytest.mark.parametrize("T,H,F,E,k,Fs", [(64, 256, 512, 8, 2, 0), (4096, 7168, 2048, 256, 8, 2048),
                                          (16384, 2048, 1408, 60, 4, 5632), (1, 4096, 14336, 8, 2, 0),
                                          (32, 4096, 14336, 8, 2, 0), (16, 2048, 1408, 60, 4, 5632),
                                          (128, 7168, 2048, 256, 8, 2048),
                                          (1024, 2048, 1408, 60, 4, 5632),
                                          (40, 128, 256, 16, 2, 768), (200, 128, 256, 4, 2, 1024)])
def test_forward_workspace_bytes(T, H, F, E, k, Fs):
    got = B.moe_forward_workspace_bytes(T, H, F, E, k, Fs)
    assert got == _layout_model(T, H, F, E, k, Fs)
    if (T, H) == (1, 4096):
        assert _down_ksplit(T, H, F, E, k, Fs) == (4, 4)   # two experts: 128 items -> split 4
    if (T, Fs) in ((16, 5632), (1024, 5632)):
        assert _down_ksplit(T, H, F, E, k, Fs)[1] == 4   # shared K = 4 x routed K
    if (T, H, F, Fs) == (40, 128, 256, 768):
        assert _down_ksplit(T, H, F, E, k, Fs) == (1, 3)   # the GPU test's shared split
    if (T, H, F, Fs) == (200, 128, 256, 1024):
        assert _down_ksplit(T, H, F, E, k, Fs) == (1, 4)
    assert B.moe_forward_workspace_bytes(T, H, F, E, k, 3) == 0      # Fs % 8


def test_pack_weights_validation(L):
    # documented size: G * ceil(N/64) * ceil(K/64) blocks of 64 x 64 bf16
    assert B.moe_pack_weights_bytes(8, 4096, 14336) == 8 * 224 * 64 * 8192
    assert B.moe_pack_weights_bytes(3, 200, 328) == 3 * 6 * 4 * 8192
    assert B.moe_pack_weights_bytes(1, 8, 8) == 8192
    assert B.moe_pack_weights_bytes(0, 64, 64) == 0
    assert B.moe_pack_weights_bytes(2, 60, 64) == 0                    # K % 8
    nbytes = B.moe_pack_weights_bytes(2, 64, 128)
    assert L.moe_pack_weights(P, 0, 64, 128, P, nbytes, NULL) == INVALID
    assert L.moe_pack_weights(P, 2, 64, 100, P, nbytes, NULL) == SHAPE
    assert L.moe_pack_weights(NULL, 2, 64, 128, P, nbytes, NULL) == INVALID
    assert L.moe_pack_weights(P, 2, 64, 128, Q, nbytes, NULL) == MISALIGNED
    assert L.moe_pack_weights(P, 2, 64, 128, P, nbytes - 1, NULL) == WS_SMALL


def test_packed_calls_validation(L):
    assert L.moe_gateup_swiglu_packed(P, P, 128, 64, 100, 8, P, P, P, NULL) == SHAPE
    assert L.moe_gateup_swiglu_packed(P, P, 128, 64, 96, 8, P, NULL, P, NULL) == INVALID
    assert L.moe_down_packed(P, P, 128, 96, 64, 8, Q, P, NULL) == MISALIGNED
    assert L.moe_forward_packed(NULL, P, 32, 64, 96, 8, 2, P, P, P, None, P, NULL, NULL,
                                P, 1 << 30, NULL) == INVALID
    assert L.moe_forward_packed(P, P, 32, 64, 96, 8, 9, P, P, P, None, P, NULL, NULL,
                                P, 1 << 30, NULL) == SHAPE
    assert L.moe_forward_packed(NULL, NULL, 0, 64, 96, 8, 2, NULL, NULL, NULL, None, NULL,
                                NULL, NULL, NULL, 0, NULL) == OK


def test_backward_workspace_bytes():
    for args in [(64, 128, 96, 8, 2), (4096, 7168, 2048, 256, 8), (1, 64, 48, 3, 1)]:
        base = B.moe_backward_workspace_bytes(*args)
        assert base > 0 and base % 256 == 0
        assert B.moe_backward_shared_workspace_bytes(*args, 0) == base
        assert B.moe_backward_shared_workspace_bytes(*args, 256) > base
    assert B.moe_backward_shared_workspace_bytes(64, 128, 96, 8, 2, 60) == 0   # Fs % 8 != 0
    assert B.moe_backward_shared_workspace_bytes(64, 128, 96, 8, 2, -8) == 0


def test_backward_shared_validation(L):
    ws = B.moe_backward_shared_workspace_bytes(10, 64, 48, 4, 2, 32)
    sh = B.SharedExpert(0x10000, 0x10000, 0x10000, 32, None)
    sg = B.SharedExpertGrads(0x10000, 0x10000, 0x10000, None)
    args = lambda shared, grads, T=10, ws_bytes=ws: (
        P, P, P, T, 64, 48, 4, 2, P, P, P, shared, P, P, P, P, P, P, grads, P, ws_bytes, NULL)
    assert L.moe_backward_shared(*args(ctypes.byref(sh), None)) == INVALID        # no grads
    assert L.moe_backward_shared(*args(ctypes.byref(sh), ctypes.byref(sg), ws_bytes=ws - 1)) == WS_SMALL
    bad = B.SharedExpert(0x10000, 0x10000, 0x10000, 36, None)                        # Fs % 8
    assert L.moe_backward_shared(*args(ctypes.byref(bad), ctypes.byref(sg))) == SHAPE
    mis = B.SharedExpertGrads(0x10002, 0x10000, 0x10000, None)                       # dw_gate
    assert L.moe_backward_shared(*args(ctypes.byref(sh), ctypes.byref(mis))) == MISALIGNED
    gated = B.SharedExpert(0x10000, 0x10000, 0x10000, 32, 0x10000)                   # needs d_gate
    assert L.moe_backward_shared(*args(ctypes.byref(gated), ctypes.byref(sg))) == INVALID
    # without the shared expert it validates as moe_backward
    assert L.moe_backward_shared(*args(None, None, ws_bytes=B.moe_backward_workspace_bytes(
        10, 64, 48, 4, 2) - 1)) == WS_SMALL

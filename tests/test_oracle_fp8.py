"""Pins of the oracle's FP8 (OCP E4M3) weight format: the code table and the
quantizer against torch's float8_e4m3fn conversions (a library routine), the
spec's named values, the per-column scale rule, ties to even, and exact
dequantization into bf16. CPU only."""
import numpy as np
import pytest
import torch

from grouped_gemm_softmax_amd import synth


def bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def test_e4m3_table_matches_torch(orc):
    v = orc.e4m3_values()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(v), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert (v[ok] == ref[ok]).all()
    assert (np.signbit(v[ok]) == np.signbit(ref[ok])).all()


def test_e4m3_named_values(orc):
    v = orc.e4m3_values()
    # largest finite, smallest normal, smallest subnormal, one, minus two
    assert v[0x7E] == 448.0 and v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9
    assert v[0x07] == 7 * 2.0 ** -9 and v[0x38] == 1.0 and v[0xC0] == -2.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and v[0x80] == 0.0
    # the 127 non-negative finite codes increase strictly
    assert (np.diff(v[:127]) > 0).all()


def _weights(G, K, N, seed):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((G, K, N)) * 0.02
    w[:, :, 0] = 0.0                                   # an all-zero column
    w[:, :, 1] *= 1e6                                  # a wide column
    w[:, :, 2] *= 1e-30                                # a tiny column
    return bf16_bits(w.astype(np.float32))


@pytest.mark.parametrize("G,K,N,seed", [(1, 64, 16, 0), (3, 200, 40, 1), (2, 1024, 8, 2)])
def test_quantize_matches_torch_cast(orc, G, K, N, seed):
    w = _weights(G, K, N, seed)
    codes, scales = orc.quantize_e4m3(w)
    wf = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    # scale rule: the smallest power of two with max|w| <= 448 * scale
    amax = np.abs(wf).max(axis=1)
    assert (np.log2(scales) == np.round(np.log2(scales))).all()
    assert (amax <= 448 * scales).all()
    assert ((amax == 0) | (amax > 224 * scales)).all()
    assert (scales[amax == 0] == 1.0).all()
    # codes: torch's round-to-nearest-even cast of w / scale
    ref = torch.from_numpy(wf / scales[:, None, :]).float().to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()
    assert (codes == ref).all()


def test_quantize_ties_to_even(orc):
    # scale 1 (max 448): 1.0625 lies halfway between codes 0x38 and 0x39,
    # 1.1875 between 0x39 and 0x3A, 2^-10 between 0 and the least subnormal,
    # 3 * 2^-10 between the subnormal codes 0x01 and 0x02
    col = np.array([448.0, 1.0625, 1.1875, 2.0 ** -10, -1.0625, 3 * 2.0 ** -10], np.float32)
    codes, scales = orc.quantize_e4m3(bf16_bits(col)[:, None])
    assert scales[0] == 1.0
    assert codes[:, 0].tolist() == [0x7E, 0x38, 0x3A, 0x00, 0xB8, 0x02]


def test_dequant_is_exact_in_bf16(orc):
    w = _weights(2, 300, 24, 3)
    codes, scales = orc.quantize_e4m3(w)
    d = orc.dequant_e4m3(codes, scales)
    # every dequantized weight is a bf16 value: the bf16 round trip is exact
    back = (bf16_bits(d.astype(np.float32)).astype(np.uint32) << 16).view(np.float32)
    assert (back.astype(np.float64) == d).all()
    # and the quantization error is within half a code step: 2^-4 relative
    # for normal codes (3 mantissa bits), 2^-10 * scale absolute below them
    wf = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    err = np.abs(d - wf)
    bound = np.maximum(np.abs(wf) * 2.0 ** -4, 2.0 ** -10 * scales[:, None, :])
    assert (err <= bound).all()

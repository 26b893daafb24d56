"""Pins of the oracle's MXFP8 weight format (E4M3 codes, one E8M0 scale per
32 K-values of a column; OCP Microscaling Formats specification v1.0, FP8
E4M3 elements): the element rounding against torch's float8_e4m3fn casts (a
library routine) of the clamped, scaled weights; a hand-worked block (ties to
even on the code grid, saturation at 448, subnormal codes, the scale rule);
the raised minimum exponent and all-zero blocks; exact invariances (sign,
powers of two); the error bound; exact dequantization into bf16. CPU only."""
import numpy as np
import pytest
import torch

E4M3_MAX = 448.0


def bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def as_f64(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def torch_e4m3(v: np.ndarray) -> np.ndarray:
    """Codes of v (clamped to the finite range: the MX rule saturates) by
    torch's float32 -> float8_e4m3fn conversion."""
    t = torch.from_numpy(np.clip(v, -E4M3_MAX, E4M3_MAX).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# A hand-worked block (one column, 9 rows): the largest |w| is 500, floor(log2
# 500) = 8, so X = 0 (scale byte 127) and the codes are the E4M3 roundings of
# w itself: 448 = 1.75 * 2^8 is the largest code (0x7E); 480 and 500 saturate
# to it; 1 = 2^0 is exponent field 7 (0x38); -3 = -1.5 * 2^1 is 0xC4; 2^-9 is
# the smallest subnormal (0x01); 1.5 * 2^-9 lies halfway between codes 1 and
# 2 and goes to the even one; 17 = 1.0625 * 2^4 lies halfway between 16
# (0x58) and 18 (0x59) and goes to 16.
HAND_W = [448.0, 480.0, 500.0, 1.0, 0.0, -3.0, 2.0 ** -9, 1.5 * 2.0 ** -9, 17.0]
HAND_CODES = [0x7E, 0x7E, 0x7E, 0x38, 0x00, 0xC4, 0x01, 0x02, 0x58]


@pytest.mark.parametrize("shift", [0, -10, 20, -100])
def test_hand_worked_block(orc, shift):
    w = bf16_bits(np.array(HAND_W, np.float32) * np.float32(2.0 ** shift))[:, None]
    codes, sb = orc.quantize_mxfp8(w)
    assert codes[:, 0].tolist() == HAND_CODES
    assert sb.shape == (1, 1) and int(sb[0, 0]) == 127 + shift


def test_elements_match_torch_casts_and_scale_rule(orc):
    rng = np.random.default_rng(11)
    G, K, N = 2, 200, 40                       # 7 K-blocks, the last one 8 rows
    w = rng.standard_normal((G, K, N)) * 0.02
    w[0, :, 7] *= 3000.0                       # a wide column
    w[1, 40:70, 9] = rng.standard_normal(30) * 1e-3
    u = bf16_bits(w.astype(np.float32))
    wf = as_f64(u)
    codes, sb = orc.quantize_mxfp8(u)
    assert sb.shape == (G, 7, N)
    X = sb.astype(np.int64) - 127
    for b in range(7):
        blk = wf[:, 32 * b:32 * b + 32, :]
        amax = np.abs(blk).max(axis=1)                      # [G, N]
        x = X[:, b, :]
        # the MX scale rule: the block's largest magnitude lands in [256, 512)
        r = amax / np.exp2(x)
        assert ((r >= 256) & (r < 512)).all()
        v = blk / np.exp2(x)[:, None, :]
        assert (codes[:, 32 * b:32 * b + 32, :] == torch_e4m3(v)).all()


def test_zero_and_tiny_blocks(orc):
    w = np.zeros((64, 3), np.float32)
    w[:32, 1] = -0.0
    w[:, 2] = 2.0 ** -112                      # below 2^-109: X raised to -117
    w[5, 2] = 3 * 2.0 ** -113
    codes, sb = orc.quantize_mxfp8(bf16_bits(w))
    assert (sb[:, 0] == 127).all() and (sb[:, 1] == 127).all()
    assert (codes[:, 0] == 0).all() and (codes[:32, 1] == 0x80).all()
    assert (sb[:, 2] == 127 - 117).all()
    # 2^-112 / 2^-117 = 32 = 2^5 (exponent field 12); 3 * 2^-113 / 2^-117 = 48
    assert codes[0, 2] == 12 << 3 and codes[5, 2] == (12 << 3) | 4


def test_sign_and_power_of_two_invariance(orc):
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((2, 96, 24)) * 0.05).astype(np.float32)
    c0, s0 = orc.quantize_mxfp8(bf16_bits(w))
    c1, s1 = orc.quantize_mxfp8(bf16_bits(-w))
    assert (c1 == (c0 ^ 0x80)).all() and (s1 == s0).all()
    c2, s2 = orc.quantize_mxfp8(bf16_bits(w * np.float32(2.0 ** 9)))
    assert (c2 == c0).all() and (s2.astype(int) == s0.astype(int) + 9).all()


def test_dequantized_weights_are_bf16_and_close(orc):
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((3, 136, 72)) * 0.02).astype(np.float32)
    u = bf16_bits(w)
    wf = as_f64(u)
    codes, sb = orc.quantize_mxfp8(u)
    d = orc.dequant_mxfp8(codes, sb)
    # every dequantized weight is exactly a bf16 value
    assert (as_f64(bf16_bits(d.astype(np.float32))) == d).all()
    # within half a code step (E4M3 steps are 2^(e-3) in the value's binade,
    # 2^-9 below 2^-6), times the block scale; scaled magnitudes above 448
    # (at most 512 by the scale rule) saturate to 448
    X = np.repeat(sb.astype(np.int64) - 127, 32, axis=1)[:, :136, :]
    v = np.abs(wf) / np.exp2(X)
    step = np.where(v < 2.0 ** -6, 2.0 ** -9, np.exp2(np.floor(np.log2(np.maximum(v, 1e-300))) - 3))
    bound = np.where(v > E4M3_MAX, v - E4M3_MAX, 0.5 * step) * np.exp2(X)
    assert (np.abs(d - wf) <= bound + 1e-300).all()
    sat = v > E4M3_MAX
    assert sat.any() and (np.abs(d[sat]) == E4M3_MAX * np.exp2(X[sat])).all()

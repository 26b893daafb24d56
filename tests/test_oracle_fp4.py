"""Pins of the oracle's MXFP4 weight format (E2M1 codes, one E8M0 scale per
32 K-values of a column; OCP Microscaling Formats specification v1.0): the
code table against the spec's listed values, a hand-worked block (ties to
even, saturation at 6, the scale rule), exact invariances (sign, powers of
two), the error bound, and exact dequantization into bf16. CPU only."""
import numpy as np
import pytest
import torch


def bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def as_f64(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_e2m1_table_is_the_specs(orc):
    # the spec's FP4 (E2M1) table: codes 0..7 positive, 8..15 their negatives
    listed = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    v = orc.e2m1_values()
    assert v[:8].tolist() == listed
    assert (v[8:] == -np.array(listed)).all() and np.signbit(v[8]) and not np.signbit(v[0])


def test_e8m0_values(orc):
    assert orc.e8m0_value(127) == 1.0 and orc.e8m0_value(0) == 2.0 ** -127
    assert orc.e8m0_value(254) == 2.0 ** 127 and np.isnan(orc.e8m0_value(255))


# A hand-worked block (one column, 12 rows): largest |w| = 7, floor(log2 7)
# = 2, so X = 0 (scale byte 127) and the codes are the E2M1 roundings of w
# itself. 1.75 is halfway between 1.5 (mantissa 1) and 2 (mantissa 0) -> 2;
# 0.25 between 0 and 0.5 -> 0; 0.75 -> 1; 1.25 -> 1; 2.5 -> 2; 3.5 -> 4;
# 5 -> 4; 7 saturates to 6; -4 keeps its sign.
HAND_W = [6.0, 3.0, 1.75, 0.25, 0.75, 1.25, 2.5, 3.5, 5.0, 7.0, -4.0, 0.0]
HAND_CODES = [0x7, 0x5, 0x4, 0x0, 0x2, 0x2, 0x4, 0x6, 0x6, 0x7, 0xE, 0x0]


@pytest.mark.parametrize("shift", [0, -10, 20, -120])
def test_hand_worked_block(orc, shift):
    w = bf16_bits(np.array(HAND_W, np.float32) * np.float32(2.0 ** shift))[:, None]
    codes, sb = orc.quantize_mxfp4(w)
    assert codes[:, 0].tolist() == HAND_CODES
    assert sb.shape == (1, 1) and int(sb[0, 0]) == 127 + shift


def test_scale_rule_and_blocks(orc):
    rng = np.random.default_rng(7)
    G, K, N = 2, 200, 24                       # 7 K-blocks, the last one 8 rows
    w = rng.standard_normal((G, K, N)) * 0.02
    w[:, 32:64, 3] = 0.0                       # an all-zero block
    w[1, :, 5] *= 1e-37                        # blocks below 2^-123: X raised to -125
    u = bf16_bits(w.astype(np.float32))
    wf = as_f64(u)
    codes, sb = orc.quantize_mxfp4(u)
    assert sb.shape == (G, 7, N)
    X = sb.astype(np.int64) - 127
    amax = np.stack([np.abs(wf[:, 32 * b:32 * b + 32, :]).max(axis=1) for b in range(7)], 1)
    zero = amax == 0
    low = (~zero) & (amax < 2.0 ** -123)
    norm = ~(zero | low)
    r = amax[norm] / 2.0 ** X[norm]
    assert ((r >= 4) & (r < 8)).all()          # X = floor(log2 amax) - 2
    assert (X[zero] == 0).all() and (X[low] == -125).all() and low.any()
    assert (codes[:, 32:64, 3] & 7 == 0).all()


def test_sign_and_power_of_two_invariance(orc):
    rng = np.random.default_rng(8)
    u = bf16_bits((rng.standard_normal((3, 96, 16)) * 0.05).astype(np.float32))
    codes, sb = orc.quantize_mxfp4(u)
    neg_codes, neg_sb = orc.quantize_mxfp4(u ^ np.uint16(0x8000))
    assert (neg_codes == codes ^ 8).all() and (neg_sb == sb).all()
    up_codes, up_sb = orc.quantize_mxfp4(bf16_bits(as_f64(u).astype(np.float32) * 2.0 ** 9))
    assert (up_codes == codes).all() and (up_sb.astype(int) == sb.astype(int) + 9).all()


def test_error_bound_and_exact_bf16(orc):
    rng = np.random.default_rng(9)
    u = bf16_bits((rng.standard_normal((2, 300, 40)) * 0.02).astype(np.float32))
    codes, sb = orc.quantize_mxfp4(u)
    d = orc.dequant_mxfp4(codes, sb)
    wf = as_f64(u)
    scale = np.repeat(2.0 ** (sb.astype(np.int64) - 127), 32, axis=1)[:, :300, :]
    err = np.abs(d - wf)
    # half a code step: 0.25 * scale below 2 * scale, else at most one step
    # (2 * scale, the gap between 4 and 6 and the saturation above 6)
    assert (err <= 2 * scale).all()
    small = np.abs(wf) < 2 * scale
    assert (err[small] <= 0.25 * scale[small]).all()
    # every dequantized weight is a bf16 value
    assert (as_f64(bf16_bits(d.astype(np.float32))) == d).all()

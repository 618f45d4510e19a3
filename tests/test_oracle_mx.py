"""Pins of the oracle's MXFP4 mode (OCP Microscaling Formats v1.0: FP4 E2M1
elements with one shared E8M0 power-of-two scale per 32 consecutive channels):
closed forms of the shared-exponent rule, a brute-force nearest-value search
that shares no code with the oracle's rounding, zero and tiny blocks, the
power-of-two shift invariance, and the block indexing of the dequantized
values."""
import math

import numpy as np
import pytest

import oracle
from workloads import TAU, WORKLOADS, draw

E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])   # code & 7 -> magnitude


def _q(x):
    """MXFP4-quantize fp32 rows [N, 128] through the oracle; returns the
    dequantized values (float64) and the scale bytes [N, 4]."""
    x = np.asarray(x, np.float32).reshape(1, 1, -1, 128)
    packed, byte = oracle.quantize_mxfp4_blocks(x)
    codes = oracle.unpack_fp4(packed)[0, 0]
    vals = oracle.decode(codes, oracle.E2M1)
    X = np.ldexp(1.0, byte[0, 0].astype(np.int64) - 127)
    return vals * np.repeat(X, 32, axis=1), byte[0, 0], codes


@pytest.mark.parametrize("m,want", [(1.0, 4.0), (1.25, 4.0), (1.375, 6.0), (1.5, 6.0), (1.75, 6.0), (1.999, 6.0)])
@pytest.mark.parametrize("k", [-20, -1, 0, 3, 40])
def test_shared_exponent_and_block_max_code(m, k, want):
    """A block whose largest magnitude is m * 2**k (1 <= m < 2) gets the scale
    2**(k - 2), byte k - 2 + 127; that element becomes 4 m rounded to E2M1 with
    ties to even (5 -> 4) and saturation (7 -> 6): closed forms."""
    x = np.zeros((1, 128), np.float32)
    x[0, :32] = np.float32(0.5 * 2.0 ** k)
    x[0, 7] = np.float32(-m * 2.0 ** k)
    vals, byte, _ = _q(x)
    assert byte[0, 0] == k - 2 + 127
    assert vals[0, 7] == -want * 2.0 ** (k - 2)
    assert vals[0, 0] == 2.0 ** (k - 1)        # 0.5 * 2**k / 2**(k-2) = 2: exact
    assert np.all(byte[0, 1:] == 0) and np.all(vals[0, 32:] == 0)


def test_codes_are_nearest_by_search():
    """Every element is the nearest of sign * {0, .5, 1, 1.5, 2, 3, 4, 6} * X to
    its value clamped at 6 X, ties to the even code (mantissa bit 0): a direct
    search over the value table, independent of the oracle's rounding."""
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((64, 128)) * np.exp(rng.uniform(-8, 8, (64, 1)))).astype(np.float32)
    # exact ties: multiples of X / 4 in the blocks of some rows
    x[:8] = (rng.integers(-24, 25, (8, 128)) * 0.25).astype(np.float32)
    vals, byte, codes = _q(x)
    X = np.repeat(np.ldexp(1.0, byte.astype(np.int64) - 127), 32, axis=1)
    y = np.clip(x.astype(np.float64) / X, -6.0, 6.0)
    cand = np.sign(y)[..., None] * E2M1_MAGS                          # [..., 8]
    dist = np.abs(cand - y[..., None])
    best = dist.min(axis=-1, keepdims=True)
    tie_ok = np.isclose(dist, best, rtol=0, atol=0)
    # among the nearest candidates prefer the even code (indices 0, 2, 4, 6 of the table)
    even = (np.arange(8) % 2 == 0)
    choice = np.where(tie_ok & even, 1, 0) + np.where(tie_ok, 1, 0)
    want = np.take_along_axis(cand, choice.argmax(axis=-1)[..., None], axis=-1)[..., 0] * X
    assert np.array_equal(np.abs(vals), np.abs(want))
    assert np.all((vals == 0) | (np.sign(vals) == np.sign(x)))


def test_zero_and_tiny_blocks():
    x = np.zeros((3, 128), np.float32)
    x[1, :32] = np.float32(2.0 ** -130)      # fp32 subnormal: the byte clamps at 0, X = 2**-127
    x[1, 32:64] = np.float32(2.0 ** -120)    # byte = -120 - 2 + 127 = 5, value / X = 4
    x[2, 64:96] = -np.float32(3.0 * 2 ** 60)  # byte = 61 - 2 + 127, value / X = -6
    vals, byte, codes = _q(x)
    assert np.all(byte[0] == 0) and np.all(codes[0] == 0)
    assert byte[1, 0] == 0 and np.all(vals[1, :32] == 0)     # 2**-130 / 2**-127 = 0.125 -> 0
    assert byte[1, 1] == 5 and np.all(vals[1, 32:64] == 2.0 ** -120)
    assert byte[2, 2] == 61 - 2 + 127 and np.all(vals[2, 64:96] == -3.0 * 2 ** 60)


def test_power_of_two_shift_moves_only_the_scale():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 128)).astype(np.float32)
    v1, b1, c1 = _q(x)
    for j in (-9, 5):
        v2, b2, c2 = _q(x * np.float32(2.0 ** j))
        assert np.array_equal(c1, c2) and np.array_equal(b2.astype(int), b1.astype(int) + j)
        assert np.array_equal(v2, v1 * 2.0 ** j)


def test_dequantized_blocks_by_loops():
    """dequantize_qk of the MXFP4 codes equals code * 2**(byte - 127) with the
    block index d // 32, written out element by element."""
    qb, kb, vb = draw(WORKLOADS["tiny"], seq_len=40, seed=9)
    z = oracle.quantize(qb, kb, vb, fmt="mxfp4")
    got = oracle.dequantize_qk(z.k_codes, z.k_scales, "mxfp4", 0, 0, 1)
    codes = oracle.unpack_fp4(z.k_codes[0, 1])
    for n in range(40):
        for d in range(128):
            c = int(codes[n, d])
            mag = E2M1_MAGS[c & 7]
            want = (-mag if c & 8 else mag) * 2.0 ** (int(z.k_scales[0, 1, n, d // 32]) - 127)
            assert got[n, d] == want


def test_forward_close_to_exact_attention():
    """The MXFP4 forward of the tiny workload stays near exact fp64 attention
    (the same order of error as the 16-channel FP4 mode)."""
    qb, kb, vb = draw(WORKLOADS["tiny"])
    z = oracle.quantize(qb, kb, vb, fmt="mxfp4")
    for h in range(2):
        o = oracle.attend(z, TAU, 0, h)
        ex = oracle.exact_attention(oracle.bf16_bits_to_f64(qb[0, h]), oracle.bf16_bits_to_f64(kb[0, h]),
                                    oracle.bf16_bits_to_f64(vb[0, h]), TAU)
        err = np.abs(o - ex)
        assert err.max() < 0.25 and err.mean() < 0.02, (err.max(), err.mean())

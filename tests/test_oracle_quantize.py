"""Pins of the oracle's statistics and quantize steps: inputs built so the
right answer is known by construction, error bounds of round-to-nearest, and
cross-checks against library routines."""
import numpy as np
import pytest

import oracle
from oracle import E2M1, E4M3, decode
from workloads import WORKLOADS, draw, to_bf16_bits


def _bits(x):
    return to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_channel_mean_by_construction():
    """K = c_d + a zero-mean +-r pattern: the mean is c_d exactly."""
    B, H, N, D = 1, 2, 96, 128
    c = (np.arange(D, dtype=np.float32) / 8 - 5)[None, None, None, :]
    r = np.where(np.arange(N) % 2 == 0, 1.5, -1.5).astype(np.float32)[None, None, :, None]
    k = oracle.bf16_bits_to_f64(_bits(c + r * np.ones((B, H, N, D), np.float32)))
    mu, vmax = oracle.channel_stats(k, -2.0 * k)
    assert np.array_equal(mu, np.broadcast_to(c[:, :, 0, :], mu.shape))
    assert np.array_equal(vmax, np.abs(2.0 * k).max(axis=2).astype(np.float32))


def test_channel_mean_agrees_with_numpy_mean():
    w = WORKLOADS["tiny"]
    _, kb, vb = draw(w)
    k = oracle.bf16_bits_to_f64(kb)
    mu, _ = oracle.channel_stats(k, k)
    ref = k.mean(axis=2).astype(np.float32)
    ulp = np.spacing(np.abs(ref))
    assert np.all(np.abs(mu - ref) <= ulp)


def test_fp8_block_scales_by_construction():
    """Block t holds max |x| = 2^t at one element: scale 2^t/448, code +-448."""
    B, H, N, D, blk = 1, 1, 100, 128, 32         # 4 blocks, the last one short (4 tokens)
    rng = np.random.default_rng(3)
    x = (rng.uniform(-0.9, 0.9, (B, H, N, D))).astype(np.float32)
    for t in range(4):
        n0 = t * blk
        x[0, 0, n0:n0 + blk] *= np.float32(2.0 ** t)
        x[0, 0, n0 + 1, 7 + t] = np.float32((-1) ** t * 2.0 ** t)
    codes, scales = oracle.quantize_fp8_blocks(x, blk)
    assert scales.shape == (1, 1, 4)
    for t in range(4):
        assert scales[0, 0, t] == np.float32(np.float32(2.0 ** t) / np.float32(448))
        assert codes[0, 0, t * blk + 1, 7 + t] == (0x7E if t % 2 == 0 else 0xFE)
    vals = decode(codes, E4M3) * np.repeat(scales[0, 0].astype(np.float64), blk)[None, None, :N, None]
    err = np.abs(vals - x)
    s_tok = np.repeat(scales[0, 0].astype(np.float64), blk)[:N][None, None, :, None]
    normal = np.abs(x) >= s_tok * 2.0 ** -6
    assert np.all(err[normal] <= (2.0 ** -4 + 1e-6) * np.abs(x[normal]))
    assert np.all(err[~normal] <= (2.0 ** -10 + 1e-7) * np.broadcast_to(s_tok, x.shape)[~normal])


def test_q_and_k_take_their_own_block_sizes():
    """block_q = 128, block_k = 64 on a K whose mean is 0 (each channel
    alternates +-a): Q has one scale per 128 tokens, K one per 64 tokens, and
    K's two halves (a = 1, then a = 4) get scales 1/448 and 4/448."""
    N, D = 128, 128
    sign = np.where(np.arange(N) % 2 == 0, 1.0, -1.0)[:, None]
    a = np.where(np.arange(N) < 64, 1.0, 4.0)[:, None]
    k = (sign * a * np.ones((N, D)))[None, None].astype(np.float32)
    q = np.ones((1, 1, N, D), np.float32)
    z = oracle.quantize(_bits(q), _bits(k), _bits(q), block_q=128, block_k=64)
    assert np.all(z.k_mean == 0)
    assert z.q_scales.shape == (1, 1, 1) and z.q_scales[0, 0, 0] == np.float32(1.0 / 448)
    assert z.k_scales.shape == (1, 1, 2)
    assert z.k_scales[0, 0, 0] == np.float32(1.0 / 448) and z.k_scales[0, 0, 1] == np.float32(4.0 / 448)
    assert np.all(np.abs(decode(z.k_codes, E4M3)) == 448)


def test_zero_block_gives_zero_scale_and_codes():
    x = np.zeros((1, 1, 130, 128), np.float32)
    x[0, 0, 64:] = 1.0
    codes, scales = oracle.quantize_fp8_blocks(x, 64)
    assert scales[0, 0, 0] == 0 and np.all(codes[0, 0, :64] == 0)
    assert scales[0, 0, 1] == np.float32(1.0 / 448) and np.all(codes[0, 0, 64:] == 0x7E)


def test_blocks_without_an_fp32_inverse_scale_are_zero_blocks():
    """F / amax overflows fp32 when amax < F / FLT_MAX (about 1.3e-36 for
    F = 448 and 1.8e-38 for F = 6).  Such a block has no fp32 inverse scale:
    scale 0 and zero codes, with no NaN from 0 * inf.  A block just above the
    limit keeps full-range codes (+-448, +-6) and its subnormal fp32 scale."""
    flt_max = float(np.finfo(np.float32).max)
    assert 1e-37 < 448 / flt_max < 2e-36 and 1.5e-38 < 6 / flt_max < 2e-38
    pattern = np.where(np.arange(128) % 3 == 0, 0.0, np.where(np.arange(128) % 2 == 0, 1.0, -0.5))
    pattern[1] = -1.0
    x = np.zeros((1, 1, 192, 128), np.float32)
    x[0, 0, :64] = np.float32(1e-37) * pattern
    x[0, 0, 64:128] = np.float32(2e-36) * pattern
    x[0, 0, 128:] = pattern
    codes, scales = oracle.quantize_fp8_blocks(x, 64)
    assert scales[0, 0, 0] == 0 and np.all(codes[0, 0, :64] == 0)
    assert scales[0, 0, 1] == np.float32(np.float32(2e-36) / np.float32(448)) and scales[0, 0, 1] < 2.0 ** -126
    vals = decode(codes[0, 0, 64:128], E4M3)
    assert np.max(vals) == 448 and np.min(vals) == -448 and np.all(vals[:, pattern == 0] == 0)
    assert scales[0, 0, 2] == np.float32(1 / 448)
    g = np.zeros((1, 1, 1, 128), np.float32)
    g[0, 0, 0, :16] = np.float32(1.5e-38) * pattern[:16]
    g[0, 0, 0, 16:32] = np.float32(2e-38) * pattern[:16]
    packed, fscales = oracle.quantize_fp4_groups(g)
    assert fscales[0, 0, 0, 0] == 0 and np.all(packed[0, 0, 0, :8] == 0)
    assert fscales[0, 0, 0, 1] > 0 and np.max(np.abs(decode(oracle.unpack_fp4(packed)[0, 0, 0, 16:32], E2M1))) == 6
    v = np.zeros((1, 1, 4, 128))
    v[0, 0, :, 0], v[0, 0, :, 1] = 1e-37, 2e-36
    vcodes, vscales = oracle.quantize_v(v, np.abs(v).max(axis=2).astype(np.float32))
    assert vscales[0, 0, 0] == 0 and np.all(vcodes[0, 0, :, 0] == 0)
    assert vscales[0, 0, 1] > 0 and np.all(decode(vcodes[0, 0, :, 1], E4M3) == 448)


def test_fp4_groups_and_nibble_order():
    """One token whose first group spans the full E2M1 range (scale 1), so
    the codes are read off the format table; the even channel is the low nibble."""
    x = np.zeros((1, 1, 1, 128), np.float32)
    x[0, 0, 0, :8] = [6.0, -6.0, 3.0, 0.5, 1.5, -4.0, 0.75, 2.5]
    x[0, 0, 0, 16:32] = 12.0                     # second group: scale 2, all codes 6.0 -> 0x7
    packed, scales = oracle.quantize_fp4_groups(x)
    assert packed.shape == (1, 1, 1, 64) and scales.shape == (1, 1, 1, 8)
    assert scales[0, 0, 0, 0] == 1.0 and scales[0, 0, 0, 1] == 2.0 and scales[0, 0, 0, 2] == 0.0
    # codes: 6->7, -6->F, 3->5, 0.5->1, 1.5->3, -4->E, 0.75->2 (ties to 1.0), 2.5->4 (ties to 2.0)
    assert list(packed[0, 0, 0, :4]) == [0xF7, 0x15, 0xE3, 0x42]
    assert np.all(packed[0, 0, 0, 8:16] == 0x77)
    assert np.all(packed[0, 0, 0, 16:] == 0)
    assert np.array_equal(oracle.unpack_fp4(packed)[0, 0, 0, :8], [7, 15, 5, 1, 3, 14, 2, 4])


def test_fp4_error_bound():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, 2, 50, 128)).astype(np.float32)
    packed, scales = oracle.quantize_fp4_groups(x)
    vals = decode(oracle.unpack_fp4(packed), E2M1).reshape(1, 2, 50, 8, 16)
    s = scales.astype(np.float64)[..., None]
    xg = x.reshape(1, 2, 50, 8, 16).astype(np.float64)
    err = np.abs(vals * s - xg)
    y = np.abs(xg) / s
    bound = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0)) * s + 1e-6 * np.abs(xg)
    assert np.all(err <= bound)
    assert np.all(np.abs(vals).max(axis=-1) == 6.0)


def test_v_channel_max_maps_to_448():
    w = WORKLOADS["tiny"]
    _, _, vb = draw(w)
    v = oracle.bf16_bits_to_f64(vb)
    vmax = np.abs(v).max(axis=2).astype(np.float32)
    codes, scales = oracle.quantize_v(v, vmax)
    vals = decode(codes, E4M3)
    assert np.all(np.abs(vals).max(axis=2) == 448.0)
    assert np.all(scales == (vmax / np.float32(448)).astype(np.float32))


def test_k_smoothing_removes_constant_key_offset_exactly():
    """Adding a constant vector to every key moves the mean by exactly that
    vector (values chosen so every step is exact), so the K codes and scales
    are bit-identical."""
    rng = np.random.default_rng(5)
    B, H, N, D = 1, 1, 256, 128
    k = (np.round(rng.uniform(-7, 7, (B, H, N, D)) * 16) / 16).astype(np.float32)
    c = rng.integers(-8, 9, D).astype(np.float32)
    q = rng.standard_normal((B, H, N, D)).astype(np.float32)
    v = rng.standard_normal((B, H, N, D)).astype(np.float32)
    z1 = oracle.quantize(_bits(q), _bits(k), _bits(v), block_q=64, block_k=64)
    z2 = oracle.quantize(_bits(q), _bits(k + c), _bits(v), block_q=64, block_k=64)
    assert np.array_equal(z2.k_mean, z1.k_mean + c)
    assert np.array_equal(z1.k_codes, z2.k_codes) and np.array_equal(z1.k_scales, z2.k_scales)
    for fmt in ("fp4", "mxfp4"):
        a = oracle.quantize(_bits(q), _bits(k), _bits(v), fmt=fmt)
        b = oracle.quantize(_bits(q), _bits(k + c), _bits(v), fmt=fmt)
        assert np.array_equal(a.k_codes, b.k_codes) and np.array_equal(a.k_scales, b.k_scales)


@pytest.mark.parametrize("name", ["tiny", "dev1024", "kontext1024"])
def test_fp64_key_sum_is_exact_in_any_order(name):
    """For the synthetic inputs every partial sum of K over tokens is exactly
    representable in fp64: per (b, h, channel), with e_hi and e_lo the
    exponent fields of the largest and the smallest nonzero |K| (e_lo at
    least 1), e_hi - e_lo + ceil(log2 N) <= 45, so all values are multiples
    of 2^(e_lo - 134) and every partial sum is below 2^53 of them.  Any
    summation order then gives the exact sum, and the statistics pass never
    needs its exact re-summation on these workloads."""
    w = WORKLOADS[name]
    _, kb, _ = draw(w, heads=min(w.heads, 4))
    mag = (kb & 0x7FFF).astype(np.int32)
    e_hi = (mag.max(axis=2) >> 7)
    e_lo = np.maximum(np.where(mag > 0, mag, 0x7FFF).min(axis=2) >> 7, 1)
    n = kb.shape[2]
    assert np.all(e_hi - e_lo + int(np.ceil(np.log2(n))) <= 45)
    # the criterion is sufficient: the exact sum fits 53 bits of the smallest unit
    k = oracle.bf16_bits_to_f64(kb)
    unit = np.ldexp(1.0, e_lo - 134)
    assert np.all(np.abs(k).sum(axis=2) / unit < 2.0 ** 53)

"""Pins of the oracle's format codecs against independent definitions:
torch's float8_e4m3fn and bfloat16 casts, and brute-force nearest search over
each format's value table."""
import numpy as np
import pytest
import torch

from oracle import BF16, E2M1, E4M3, decode, encode, f64_to_bf16_bits, round_to


def _e4m3_table():
    """All 256 E4M3 codes decoded by torch (an independent implementation)."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).float().double().numpy()


def test_e4m3_decode_matches_torch_for_every_code():
    ours = decode(np.arange(256), E4M3)
    theirs = _e4m3_table()
    nan_ours = np.isnan(ours)
    assert np.array_equal(nan_ours, np.isnan(theirs))
    assert nan_ours.sum() == 2                        # 0x7F and 0xFF
    assert np.array_equal(ours[~nan_ours], theirs[~nan_ours])
    assert np.array_equal(np.signbit(ours[~nan_ours]), np.signbit(theirs[~nan_ours]))
    finite = ours[~nan_ours]
    assert len(finite) == 254 and finite.max() == 448.0
    assert np.min(np.abs(finite[finite != 0])) == 2.0 ** -9


def test_e4m3_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    assert np.array_equal(encode(decode(codes, E4M3), E4M3), codes)


def _nearest_even_bruteforce(x, table, codes_of_table):
    """Nearest value of a finite value table; ties to the even (mantissa lsb 0) code."""
    d = np.abs(x[:, None] - table[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    lsb_even = (codes_of_table & 1) == 0
    pick = np.where(cand & lsb_even[None, :], 1, 0)
    only = cand.sum(axis=1) == 1
    idx = np.where(only, cand.argmax(axis=1), pick.argmax(axis=1))
    return table[idx]


def _midpoint_probes(table):
    pos = np.unique(table[table >= 0])
    mids = (pos[1:] + pos[:-1]) / 2
    probes = [mids]
    for m in mids:
        m32 = np.float32(m)
        probes.append(np.array([np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9))],
                               dtype=np.float64))
    p = np.concatenate(probes + [pos])
    return np.concatenate([p, -p])


def test_e4m3_rounding_matches_torch_and_bruteforce():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.uniform(-500, 500, 200000), rng.standard_normal(200000) * 4,
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 50000), _midpoint_probes(decode(np.arange(127), E4M3)),
    ]).astype(np.float32).astype(np.float64)
    ours = round_to(x, E4M3)
    clamped = np.clip(x, -448.0, 448.0)
    theirs = torch.from_numpy(clamped.astype(np.float32)).to(torch.float8_e4m3fn).float().double().numpy()
    assert np.array_equal(ours, theirs)
    assert np.array_equal(np.signbit(ours), np.signbit(theirs))
    table = decode(np.arange(127), E4M3)
    brute = _nearest_even_bruteforce(np.abs(clamped), table, np.arange(127))
    assert np.array_equal(np.abs(ours), brute)
    tc = torch.from_numpy(clamped.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(encode(ours, E4M3), tc)


def test_e4m3_saturates_and_keeps_sign():
    x = np.array([448.0, 463.9, 464.0, 470.0, 1e6, -1e6, -1e-30, 2.0 ** -10, 3 * 2.0 ** -11])
    r = round_to(x, E4M3)
    assert list(r[:6]) == [448, 448, 448, 448, 448, -448]
    assert r[6] == 0 and np.signbit(r[6])
    assert r[7] == 0                      # 2^-10 is the tie between 0 and 2^-9: even -> 0
    assert r[8] == 2.0 ** -9              # 1.5 * 2^-10 rounds up to the smallest subnormal


E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def test_e2m1_value_table():
    vals = decode(np.arange(16), E2M1)
    assert np.array_equal(vals[:8], E2M1_VALUES)
    assert np.array_equal(vals[8:], -E2M1_VALUES)
    assert np.array_equal(encode(vals, E2M1), np.arange(16))


@pytest.mark.parametrize("x,want", [(0.25, 0.0), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0), (2.5, 2.0),
                                    (3.5, 4.0), (5.0, 4.0), (7.0, 6.0), (100.0, 6.0), (0.2, 0.0),
                                    (0.26, 0.5), (4.99, 4.0), (5.01, 6.0)])
def test_e2m1_ties_and_saturation(x, want):
    assert round_to(np.array([x]), E2M1)[0] == want
    assert round_to(np.array([-x]), E2M1)[0] == -want


def test_e2m1_rounding_matches_bruteforce():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-7, 7, 100000), _midpoint_probes(E2M1_VALUES)])
    x = x.astype(np.float32).astype(np.float64)
    ours = round_to(x, E2M1)
    brute = _nearest_even_bruteforce(np.abs(np.clip(x, -6, 6)), E2M1_VALUES, np.arange(8))
    assert np.array_equal(np.abs(ours), brute)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(2)
    x32 = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                          # exact ties: low 16 bits 0x8000
                          (rng.integers(0x3F000000, 0x41000000, 1000, dtype=np.uint32) & 0xFFFF0000
                           | 0x8000).view(np.float32)])
    ours = f64_to_bf16_bits(x32.astype(np.float64))
    theirs = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    assert BF16.mant_bits == 7

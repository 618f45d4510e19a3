"""Pins of the oracle's selective correction (the VC-Attention-style FP8 mode):
the count k = ceil(rho N), the top-k selection with ties to the lower index
(against brute force), the per-token error on hand-built tokens whose codes
are known, and the corrected forward against exact attention and the plain
FP8 forward."""
import itertools
import math

import numpy as np
import pytest

import oracle
from workloads import TAU, WORKLOADS, draw, to_bf16_bits


@pytest.mark.parametrize("n,rho,want", [(8704, 0.005, 44), (16896, 0.005, 85), (4608, 0.005, 24), (320, 0.005, 2),
                                        (200, 0.005, 1), (1, 0.005, 1), (7, 1.0, 7), (10, 0.3, 3), (9, 1e-6, 1)])
def test_count_is_ceil_rho_n(n, rho, want):
    assert oracle.vc_count(n, rho) == want


def test_selection_matches_brute_force_with_ties():
    """Among all k-subsets, the selection is the one with the largest errors,
    and among equal errors the lower indices: the lexicographically smallest
    index tuple of the subsets whose sorted errors are largest."""
    rng = np.random.default_rng(4)
    for trial in range(30):
        n = int(rng.integers(1, 9))
        err = rng.integers(0, 4, n).astype(float)      # many ties
        k = int(rng.integers(1, n + 1))
        best = None
        for sub in itertools.combinations(range(n), k):
            key = (sorted((-err[i] for i in sub)), sub)
            if best is None or key < best:
                best = key
        assert list(oracle.vc_select(err, k)) == list(best[1]), (err, k)


def test_token_error_on_known_codes():
    """A Q block whose largest magnitude is 448 has scale 1, so a value's code
    is the value itself when E4M3 holds it: 16 and 448 are exact (error 0),
    17 lies between 16 and 18 and rounds to even 16 (error 1), 100 rounds to
    96 (error 16), 0.3 to 0.3125 (error 0.0125^2)."""
    N, D = 128, 128
    q = np.zeros((1, 1, N, D), np.float32)
    q[0, 0, 0, 0] = 448.0
    q[0, 0, 1, :4] = [16.0, 17.0, 17.0, 100.0]
    q[0, 0, 2, 5] = 0.3
    qb = to_bf16_bits(q)
    kb = to_bf16_bits(np.ones((1, 1, N, D), np.float32))
    z = oracle.quantize(qb, kb, kb, fmt="fp8", block_q=128)
    assert z.q_scales[0, 0, 0] == 1.0
    e = oracle.vc_token_error(z, qb, 0, 0)
    x03 = float(oracle.bf16_bits_to_f64(to_bf16_bits(np.array([0.3], np.float32)))[0])   # the bf16 input
    assert e[0] == 0 and e[1] == 1 + 1 + 16 and np.all(e[3:] == 0)
    assert e[2] == (x03 - 0.3125) ** 2


def test_all_tokens_corrected_is_exact_attention():
    """rho = 1 corrects every token: O is exact softmax attention of the bf16
    inputs, rounded to bf16, in every row."""
    qb, kb, vb = draw(WORKLOADS["tiny"], seq_len=100, seed=5)
    o, sel = oracle.vc_forward(qb, kb, vb, rho=1.0, block_q=64)
    assert sel.shape == (1, 2, 100)
    for h in range(2):
        q, k, v = (oracle.bf16_bits_to_f64(x[0, h]) for x in (qb, kb, vb))
        want = oracle.f64_to_bf16_bits(oracle.exact_attention(q, k, v, TAU))
        assert np.array_equal(o[0, h], want)


def test_uncorrected_rows_are_the_fp8_rows():
    """Rows not selected are the plain FP8 forward's rows bit for bit; the
    selected rows are the exact ones, and they are the rows with the largest
    quantization error."""
    qb, kb, vb = draw(WORKLOADS["tiny"])
    o, sel = oracle.vc_forward(qb, kb, vb, block_q=64)
    plain = oracle.forward(qb, kb, vb, block_q=64)
    z = oracle.quantize(qb, kb, vb, fmt="fp8", block_q=64)
    for h in range(2):
        rest = np.setdiff1d(np.arange(320), sel[0, h])
        assert np.array_equal(o[0, h, rest], plain[0, h, rest])
        e = oracle.vc_token_error(z, qb, 0, h)
        assert e[sel[0, h]].min() >= e[rest].max()
        q, k, v = (oracle.bf16_bits_to_f64(x[0, h]) for x in (qb, kb, vb))
        want = oracle.f64_to_bf16_bits(oracle.exact_attention(q, k, v, TAU, sel[0, h]))
        assert np.array_equal(o[0, h, sel[0, h]], want)


def test_correction_lowers_the_error_of_its_rows():
    """On the tiny workload the corrected rows are closer to exact attention
    than their FP8 rows were (they are exact up to the bf16 rounding)."""
    qb, kb, vb = draw(WORKLOADS["tiny"])
    o, sel = oracle.vc_forward(qb, kb, vb, rho=0.05, block_q=64)
    plain = oracle.forward(qb, kb, vb, block_q=64)
    for h in range(2):
        q, k, v = (oracle.bf16_bits_to_f64(x[0, h]) for x in (qb, kb, vb))
        ex = oracle.exact_attention(q, k, v, TAU, sel[0, h])
        e_vc = np.abs(oracle.bf16_bits_to_f64(o[0, h, sel[0, h]]) - ex).max()
        e_fp8 = np.abs(oracle.bf16_bits_to_f64(plain[0, h, sel[0, h]]) - ex).max()
        assert e_vc <= 2.0 ** -8 * np.abs(ex).max() and e_fp8 > 4 * e_vc   # half a bf16 step

"""CPU checks of the rounding bound in kernel_error: the CPU emulation of the
FP8 kernel's arithmetic reproduces the raw differences seen on the GPU, for
the causes recorded with the GPU tests, and stays within the bound."""
import numpy as np
import pytest

import kernel_error
import oracle
from workloads import TAU, WORKLOADS, draw


def _scaled(bits, e):
    x = ((bits.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** e)).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _case(seq_len, seed, batch, heads, b, h, block_q, shift=0):
    qb, kb, vb = draw(WORKLOADS["tiny"], batch=batch, heads=heads, seq_len=seq_len, seed=seed)
    if shift:
        qb = _scaled(qb, shift)
    return oracle.quantize(qb[b:b + 1, h:h + 1], kb[b:b + 1, h:h + 1], vb[b:b + 1, h:h + 1], fmt="fp8",
                           block_q=block_q, block_k=64)


def test_emulated_kernel_reproduces_the_ragged_midpoint_flip():
    """N = 129, block_q = 64, batch 1 of the ragged GPU test (seed 629): the
    GPU's raw max-abs there is 1.221e-2.  The emulation gives the same value
    at query 65, channel 96, where the first step's weight of key 3 is
    448 p = 304.000731, 2.4e-6 above the E4M3 midpoint 304: the oracle codes
    it 320, and the truncated score takes it below."""
    z = _case(129, 500 + 129, 2, 1, 1, 0, 64)
    want, allowed, diag = kernel_error.output_allowance(z, TAU, 0, 0)
    got = kernel_error.emulate_fp8_attention(z, TAU, 0, 0)
    raw = np.abs(got - want)
    i, d = np.unravel_index(raw.argmax(), raw.shape)
    assert (i, d) == (65, 96) and abs(raw.max() - 1.221e-2) < 1e-5
    st = diag["trace"]["steps"][0]
    v = oracle.P_SCALE * st["p"][65, 3]
    assert abs(v - 304.000731) < 1e-6 and st["w"][65, 3] == 320.0
    assert raw[i, d] <= allowed[i, d]


def test_peaked_one_hot_rows_round_bf16_ties_the_other_way():
    """Q times 2^8 (the peaked GPU test, seed 45): in one-hot rows (l = 1)
    the oracle's output before rounding is exactly a bf16 tie above 2, where
    one bf16 step is 2^-6 = 0.0156; the emulated fp32 epilogue lands a last
    bit off the tie and rounds to the other neighbour, one step away."""
    z = _case(300, 45, 1, 2, 0, 1, 128, shift=8)
    want, allowed, diag = kernel_error.output_allowance(z, TAU, 0, 0)
    tr = diag["trace"]
    got = kernel_error.emulate_fp8_attention(z, TAU, 0, 0)
    raw = np.abs(got - want)
    big = np.argwhere(raw > 1e-2)
    assert len(big) > 0
    for i, d in big:
        assert raw[i, d] == 2.0 ** -6 and 2 <= abs(want[i, d]) < 4
    ties = [(i, d) for i, d in big if tr["l"][i] == 1.0]
    assert ties
    for i, d in ties:
        x = tr["out"][i, d]
        assert oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(np.array([x + 2.0 ** -8])))[0] != \
            oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(np.array([x - 2.0 ** -8])))[0]   # a tie: +-2^-8 split
        sp = 2.0 ** (np.floor(np.log2(abs(x))) - 7)                    # the bf16 step at x
        assert abs(x) / sp - np.floor(abs(x) / sp) == 0.5
    assert np.all(raw <= allowed)


@pytest.mark.parametrize("seq_len,seed,batch,heads,b,h,block_q,shift", [
    (65, 565, 2, 1, 0, 0, 64, 0),
    (129, 629, 2, 1, 1, 0, 64, 0),
    (129, 629, 2, 1, 0, 0, 128, 0),
    (320, 1001, 1, 2, 0, 0, 64, 0),
    (300, 45, 1, 2, 0, 0, 128, 4),
    (300, 45, 1, 2, 0, 1, 128, 4),
    (300, 45, 1, 2, 0, 0, 128, 8),
])
def test_bound_covers_emulated_kernel(seq_len, seed, batch, heads, b, h, block_q, shift):
    z = _case(seq_len, seed, batch, heads, b, h, block_q, shift)
    want, allowed, _ = kernel_error.output_allowance(z, TAU, 0, 0)
    got = kernel_error.emulate_fp8_attention(z, TAU, 0, 0)
    assert np.all(np.abs(got - want) <= allowed)


def test_bound_is_zero_for_exact_products():
    """Sums whose products are all multiples of their truncation step
    (2^-14 of the largest product's binade) have a zero truncation bound; a
    smaller product is lost, and its whole size is the bound."""
    A = np.array([[448.0, 2.0, -0.5], [1.0, 1.0, 1.0]])
    B = np.array([[1.0, 1.0, 1.0], [448.0, -448.0, 16.0]])
    assert np.all(kernel_error.mfma_sum_error(A, B, k=3) == 0)
    # a product below 2^-14 of the largest one's binade is lost: |err| <= its size
    A2 = np.array([[448.0, 0.015625]])
    B2 = np.array([[448.0, 256.0]])
    assert kernel_error.mfma_sum_error(A2, B2, k=2)[0, 0] == 4.0

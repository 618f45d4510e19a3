"""Pins of the oracle's attention step: brute force on tiny inputs, the
exact fp64 softmax when the quantizers are removed, closed forms and
hand-worked examples of the online softmax."""
import math

import numpy as np
import pytest

import oracle
from oracle import E4M3, decode
from workloads import TAU, WORKLOADS, draw, to_bf16_bits


def _bits(x):
    return to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_exact_attention_matches_bruteforce_loops():
    rng = np.random.default_rng(10)
    N, D = 11, 5
    q, k, v = (rng.standard_normal((N, D)) for _ in range(3))
    tau = 0.37
    want = np.zeros((N, D))
    for i in range(N):
        s = [tau * sum(q[i, d] * k[j, d] for d in range(D)) for j in range(N)]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        z = sum(e)
        for d in range(D):
            want[i, d] = sum(e[j] * v[j, d] for j in range(N)) / z
    assert np.allclose(oracle.exact_attention(q, k, v, tau), want, rtol=0, atol=1e-14)


@pytest.mark.parametrize("step", [1, 7, 64, 300])
def test_online_softmax_without_quantizers_is_exact_softmax(step):
    rng = np.random.default_rng(11)
    R, N, D = 9, 300, 16
    S = rng.standard_normal((R, N)) * 3
    V = rng.standard_normal((N, D))
    acc, l = oracle.online_softmax_av(S, V, step=step, quantize_p=False)
    got = acc / (oracle.P_SCALE * l)[:, None]
    w = np.exp(S - S.max(axis=1, keepdims=True))
    want = (w / w.sum(axis=1, keepdims=True)) @ V
    assert np.max(np.abs(got - want)) <= 1e-12
    # the weights p/l sum to one
    acc1, l1 = oracle.online_softmax_av(S, np.ones((N, 1)), step=step, quantize_p=False)
    assert np.max(np.abs(acc1[:, 0] / (oracle.P_SCALE * l1) - 1)) <= 1e-14


def test_smoothing_leaves_exact_attention_unchanged():
    rng = np.random.default_rng(12)
    q, k, v = (rng.standard_normal((64, 128)) for _ in range(3))
    k = k + rng.standard_normal(128) * 3
    a = oracle.exact_attention(q, k, v, TAU)
    b = oracle.exact_attention(q, k - k.mean(axis=0), v, TAU)
    assert np.max(np.abs(a - b)) <= 1e-12


def test_worked_example_one_step():
    """p = [1, 0.3]: P codes 448 and E4M3(134.4) = 128; l sums the
    unquantized p (1.3); O = (448*1 + 128*2) / (448 * 1.3)."""
    S = np.array([[0.0, math.log(0.3)]])
    V = np.array([[1.0], [2.0]])
    acc, l = oracle.online_softmax_av(S, V, step=64)
    assert acc[0, 0] == 448 + 128 * 2
    assert abs(l[0] - 1.3) < 1e-15
    assert abs(acc[0, 0] / (448 * l[0]) - 704 / (448 * 1.3)) < 1e-15


def test_worked_example_step_size_changes_codes():
    """S = [0, 2]: one-key steps code both weights as 448 (each relative to
    its own running max) and give the exact softmax; one two-key step codes
    exp(-2)*448 = 60.63 as 60."""
    S = np.array([[0.0, 2.0]])
    V = np.array([[1.0], [3.0]])
    e2 = math.exp(-2.0)
    acc1, l1 = oracle.online_softmax_av(S, V, step=1)
    assert abs(acc1[0, 0] - (e2 * 448 + 448 * 3)) < 1e-12 and abs(l1[0] - (1 + e2)) < 1e-15
    acc2, l2 = oracle.online_softmax_av(S, V, step=2)
    assert acc2[0, 0] == 60 + 448 * 3 and abs(l2[0] - (1 + e2)) < 1e-15


def test_worked_example_running_max_is_kept():
    """S = [2, 0] in one-key steps: the second step's own maximum (0) is below
    the running one (2), so its weight is coded relative to 2: E4M3(448 e^-2)
    = 60, not 448; l = 1 + e^-2."""
    S = np.array([[2.0, 0.0]])
    V = np.array([[1.0], [3.0]])
    e2 = math.exp(-2.0)
    acc, l = oracle.online_softmax_av(S, V, step=1)
    assert acc[0, 0] == 448 + 60 * 3 and abs(l[0] - (1 + e2)) < 1e-15


def _tiny_inputs(N, seed=13, H=1):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, H, N, 128)).astype(np.float32)
    k = (rng.standard_normal((1, H, N, 128)) + rng.standard_normal(128) * 3).astype(np.float32)
    v = rng.standard_normal((1, H, N, 128)).astype(np.float32)
    return _bits(q), _bits(k), _bits(v)


def test_single_token_closed_form():
    qb, kb, vb = _tiny_inputs(1)
    qz = oracle.quantize(qb, kb, vb, block_q=64, block_k=64)
    o = oracle.attend(qz, TAU, 0, 0)
    want = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(
        decode(qz.v_codes[0, 0, 0], E4M3) * qz.v_scales[0, 0].astype(np.float64)))
    assert np.array_equal(o[0], want)
    assert np.array_equal(o[0], oracle.bf16_bits_to_f64(vb)[0, 0, 0])   # V round-trips at its own max


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
def test_zero_queries_closed_form(fmt):
    """Q = 0: every score is 0, every P code is 448, l = N, so O is the mean of
    the dequantized V codes."""
    N = 200
    qb, kb, vb = _tiny_inputs(N)
    qb = np.zeros_like(qb)
    qz = oracle.quantize(qb, kb, vb, fmt=fmt, block_q=64, block_k=64)
    o = oracle.attend(qz, TAU, 0, 0)
    vd = decode(qz.v_codes[0, 0], E4M3).mean(axis=0) * qz.v_scales[0, 0].astype(np.float64)
    want = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(vd))
    assert np.array_equal(o, np.broadcast_to(want, o.shape))


def test_constant_values_row_sum_bound():
    """V = c per channel: every V code is 448, so O/c = sum(P)/(448 l),
    within the E4M3 rounding bound of the weights."""
    N = 320
    qb, kb, _ = _tiny_inputs(N)
    c = np.linspace(0.5, 3.0, 128).astype(np.float32)
    vb = _bits(np.broadcast_to(c, (1, 1, N, 128)))
    cv = oracle.bf16_bits_to_f64(vb)[0, 0, 0]
    qz = oracle.quantize(qb, kb, vb, block_q=64, block_k=64)
    o = oracle.attend(qz, TAU, 0, 0)
    rel = np.abs(o / cv - 1)
    assert np.all(rel <= 2.0 ** -4 + N * 2.0 ** -10 / 448 + 2.0 ** -8)


def test_value_power_of_two_scaling_is_exact():
    qb, kb, vb = _tiny_inputs(150)
    v2 = _bits(oracle.bf16_bits_to_f64(vb) * 4)
    o1 = oracle.attend(oracle.quantize(qb, kb, vb, block_q=64, block_k=64), TAU, 0, 0)
    o2 = oracle.attend(oracle.quantize(qb, kb, v2, block_q=64, block_k=64), TAU, 0, 0)
    assert np.array_equal(o2, 4 * o1)


def test_query_rows_depend_only_on_their_own_block():
    """Changing queries of another Q block leaves a row's output unchanged;
    changing a query in the same block changes its scale and may change it."""
    qb, kb, vb = _tiny_inputs(256)
    q2 = qb.copy()
    q2[0, 0, 128:] = _bits(oracle.bf16_bits_to_f64(qb[0, 0, 128:]) * 3)
    o1 = oracle.attend(oracle.quantize(qb, kb, vb, block_q=128), TAU, 0, 0)
    o2 = oracle.attend(oracle.quantize(q2, kb, vb, block_q=128), TAU, 0, 0)
    assert np.array_equal(o1[:128], o2[:128])
    assert not np.array_equal(o1[128:], o2[128:])


def test_row_subset_equals_full():
    qb, kb, vb = _tiny_inputs(200, H=2)
    qz = oracle.quantize(qb, kb, vb, block_q=64, block_k=64)
    full = oracle.attend(qz, TAU, 0, 1)
    rows = [0, 5, 63, 64, 199]
    assert np.array_equal(oracle.attend(qz, TAU, 0, 1, rows=rows), full[rows])


def test_forward_close_to_exact_attention_tiny():
    """Magnitude sanity: the quantized path stays near unquantized attention
    (reported bound, loose)."""
    w = WORKLOADS["tiny"]
    qb, kb, vb = draw(w)
    o = oracle.bf16_bits_to_f64(oracle.forward(qb, kb, vb, block_q=64, block_k=64))
    q, k, v = (oracle.bf16_bits_to_f64(x) for x in (qb, kb, vb))
    ex = np.stack([oracle.exact_attention(q[0, h], k[0, h], v[0, h], TAU) for h in range(2)])[None]
    err = np.abs(o - ex)
    assert err.max() < 0.1 and err.mean() < 0.01

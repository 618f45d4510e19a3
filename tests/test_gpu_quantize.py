"""GPU parity of the quantize step: codes, scales and statistics are compared
bit for bit with the oracle, at the full sizes of every workload (the oracle
evaluates sampled (b, h) pairs: every (b, h) is quantized independently)."""
import numpy as np
import pytest

import oracle
import precision_attention_qsdpa_amd as qs
from gpu_helpers import read_workspace, run_quantize, tiny_magnitude_inputs
from workloads import WORKLOADS, draw

pytestmark = pytest.mark.gpu


def sample_heads(w):
    if w.batch * w.heads <= 4:
        return [(b, h) for b in range(w.batch) for h in range(w.heads)]
    return sorted({(0, 0), (w.batch - 1, w.heads - 1), (w.batch // 2, w.heads // 2)})


def check_quantize(qb, kb, vb, fmt, block_q, heads, label):
    B, H, N, _ = qb.shape
    params = qs.make_params(B, H, N, fmt=fmt, block_q=block_q)
    print(f"[quantize] {label} B={B} H={H} N={N} fmt={fmt} bq={block_q}", flush=True)
    ws = run_quantize(qb, kb, vb, params)
    got = read_workspace(ws, params, N)
    for b, h in heads:
        z = oracle.quantize(qb[b:b + 1, h:h + 1], kb[b:b + 1, h:h + 1], vb[b:b + 1, h:h + 1],
                            fmt=fmt, block_q=block_q, block_k=64)
        for name, want in (("q_codes", z.q_codes), ("k_codes", z.k_codes), ("v_codes", z.v_codes),
                           ("q_scales", z.q_scales), ("k_scales", z.k_scales), ("k_mean", z.k_mean),
                           ("v_scales", z.v_scales), ("v_amax", z.v_amax)):
            g = got[name][b:b + 1, h:h + 1]
            assert g.shape == want.shape, (name, g.shape, want.shape)
            if g.dtype == np.float32:
                ok = np.array_equal(g.view(np.uint32), want.astype(np.float32).view(np.uint32))
            else:
                ok = np.array_equal(g, want)
            if not ok:
                bad = np.argwhere(g.reshape(want.shape) != want)
                pytest.fail(f"{label} {name} (b={b},h={h}): {len(bad)} mismatches, first at {bad[:3].tolist()}")
        if fmt == "fp4":
            # the operands the FP4 score MFMAs take: x = fp32 of the oracle's exact
            # code * scale, times 2^-E of its 64-key tile (E = biased exponent of the
            # tile's largest scale - 138, as documented in include/qsdpa.h), then
            # hi = f16(x), lo8 = E4M3(fp32(x - hi) * 2^5), hi8 = E4M3(hi * 2^-6)
            x = oracle.dequantize_qk(z.k_codes, z.k_scales, fmt, 16, 0, 0).astype(np.float32)
            sk = np.zeros((got["k_exp"].shape[2] * 64, 8), np.float32)
            sk[:N] = z.k_scales[0, 0]
            smax = sk.reshape(-1, 64 * 8).max(axis=1)
            E = ((smax.view(np.uint32) >> 23) & 0xFF).astype(np.int32) - 138
            if not np.array_equal(got["k_exp"][b, h], E):
                pytest.fail(f"{label} k_exp (b={b},h={h}): {got['k_exp'][b, h][:8]} != {E[:8]}")
            x = np.ldexp(x, -np.repeat(E, 64)[:N, None]).astype(np.float32)
            hi = x.astype(np.float16)
            lo = (x - hi.astype(np.float32)).astype(np.float32)
            lo8 = oracle.encode(oracle.round_to(np.ldexp(lo.astype(np.float64), 5), oracle.E4M3), oracle.E4M3)
            hi8 = oracle.encode(oracle.round_to(np.ldexp(hi.astype(np.float64), -6), oracle.E4M3), oracle.E4M3)
            for name, want in (("k_hi", hi.view(np.uint16)), ("k_lo8", lo8), ("k_hi8", hi8)):
                g = got[name][b, h]
                if not np.array_equal(g, want):
                    bad = np.argwhere(g != want)
                    pytest.fail(f"{label} {name} (b={b},h={h}): {len(bad)} mismatches, first at {bad[:3].tolist()}")
    for name in ("q_codes_pad", "k_codes_pad", "v_codes_pad", "q_scales_pad", "k_scales_pad", "k_hilo_pad"):
        if name in got:
            assert not np.any(got[name]), f"{label}: {name} not zero"


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_quantize_bit_exact_full_size(gpu_lib, name):
    w = WORKLOADS[name]
    qb, kb, vb = draw(w)
    check_quantize(qb, kb, vb, w.fmt, w.block_q, sample_heads(w), name)


@pytest.mark.parametrize("N", [1, 63, 65, 100, 129, 1000])
@pytest.mark.parametrize("fmt,bq", [("fp8", 64), ("fp8", 128), ("fp4", 128), ("mxfp4", 128)])
def test_quantize_ragged_lengths(gpu_lib, N, fmt, bq):
    qb, kb, vb = draw(WORKLOADS["tiny"], batch=2, heads=2, seq_len=N, seed=77 + N)
    check_quantize(qb, kb, vb, fmt, bq, [(b, h) for b in range(2) for h in range(2)], f"N={N}")


def test_quantize_zero_blocks(gpu_lib):
    """All-zero Q blocks and a zero V channel: zero scales and codes."""
    qb, kb, vb = draw(WORKLOADS["tiny"], seq_len=300, seed=5)
    qb = qb.copy(); vb = vb.copy()
    qb[:, :, 64:128] = 0
    vb[:, :, :, 5] = 0
    for fmt in ("fp8", "fp4", "mxfp4"):
        check_quantize(qb, kb, vb, fmt, 64, [(0, 0), (0, 1)], f"zero-{fmt}")


@pytest.mark.parametrize("fmt,bq", [("fp8", 64), ("fp8", 128), ("fp4", 128), ("mxfp4", 128)])
def test_quantize_tiny_magnitudes(gpu_lib, fmt, bq):
    """Blocks and V channels below the fp32 overflow limit of their inverse
    scale get zero scales and codes (no 0 * inf), blocks just above it keep
    full-range codes with subnormal scales, and bf16 subnormals are coded as
    the oracle codes them."""
    qb, kb, vb = tiny_magnitude_inputs()
    z = oracle.quantize(qb[:, :1], kb[:, :1], vb[:, :1], fmt=fmt, block_q=bq, block_k=64)
    assert np.all(z.k_mean == 0) and z.v_scales[0, 0, 3] == 0 and z.v_scales[0, 0, 4] > 0
    if fmt == "fp8" and bq == 64:
        assert z.q_scales[0, 0, 1] == 0 and z.k_scales[0, 0, 1] == 0 and 0 < z.q_scales[0, 0, 2] < 2.0 ** -126
    check_quantize(qb, kb, vb, fmt, bq, [(0, 0), (0, 1)], f"tiny-{fmt}-bq{bq}")


def e2m1_tie_rows(rng, n_rows):
    """Rows of 128 bf16-exact values in which every 16-channel group holds
    magnitude 6 once, so that both FP4 scalings are exactly 1 (fp32 scale
    6/6, MXFP4 exponent byte 127), and whose other values sit on the E2M1
    rounding ties, one bf16 step either side of them, on the code values and
    on signed zeros."""
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    pool = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0] + ties
    for t in ties:
        ulp = 2.0 ** (np.floor(np.log2(t)) - 7)          # bf16 spacing at t
        pool += [t - ulp, t + ulp]
    pool = np.array(pool, dtype=np.float32)
    rows = np.empty((n_rows, 128), dtype=np.float32)
    for i in range(n_rows):
        for grp in range(8):
            vals = rng.choice(pool, 16) * rng.choice(np.array([-1.0, 1.0], np.float32), 16)
            vals[rng.integers(16)] = rng.choice(np.array([-6.0, 6.0], np.float32))
            rows[i, 16 * grp:16 * grp + 16] = vals
    bits = rows.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "values must be exact in bf16"
    return (bits >> 16).astype(np.uint16)


@pytest.mark.parametrize("fmt", ["fp4", "mxfp4"])
def test_quantize_e2m1_ties(gpu_lib, fmt):
    """E2M1 encoding at its rounding ties: Q and K values whose scaled value
    is exactly a tie, a neighbour of one, a code value or a signed zero.  K's
    token n + 64 is -K's token n, so its channel means are exactly 0 and the
    smoothing leaves it unchanged."""
    rng = np.random.default_rng(2024)
    N = 128
    qb = e2m1_tie_rows(rng, N).reshape(1, 1, N, 128)
    kh = e2m1_tie_rows(rng, N // 2)
    kb = np.concatenate([kh, kh ^ np.uint16(0x8000)]).reshape(1, 1, N, 128)
    _, _, vb = draw(WORKLOADS["tiny"], heads=1, seq_len=N, seed=9)
    check_quantize(qb, kb, vb, fmt, 128, [(0, 0)], f"ties-{fmt}")


@pytest.mark.parametrize("bq", [64, 128])
def test_quantize_e4m3_every_bf16_value(gpu_lib, bq):
    """The device E4M3 encoder against the oracle's on every finite bf16 value
    of magnitude up to 448 (34754 values: zeros, subnormals, every E4M3 code,
    tie and midpoint neighbour a bf16 value can be), at unit scale: every Q
    and K scale block and every V channel also holds 448, so each inverse scale
    is 448 / 448 = 1 and each code is E4M3 of the input itself.  K's second
    half is its first half negated, so its channel means are exactly 0 and the
    smoothing leaves it unchanged."""
    top = 0x43E0                                  # bf16 bits of 448
    pos = np.arange(top + 1, dtype=np.uint16)      # +0 .. 448
    vals = np.concatenate([pos, pos | np.uint16(0x8000)])
    N = 320

    def filled(src, n_tok, rows, cols):
        """n_tok x 128 bf16 patterns: 448 at (rows, cols), src (repeated) elsewhere"""
        x = np.zeros((n_tok, 128), np.uint16)
        mark = np.zeros((n_tok, 128), bool)
        mark[rows, cols] = True
        x[mark] = top
        x[~mark] = np.resize(src, int((~mark).sum()))
        return x

    q = filled(vals, N, np.arange(0, N, 64), 0)                # a 448 in every 64-token block
    v = filled(vals[::-1], N, 0, np.arange(128))               # a 448 in every channel
    kh = filled(pos, N // 2, [0, 64, 128], 1)                  # with the negated half: 448 in every block
    k = np.concatenate([kh, kh ^ np.uint16(0x8000)])
    shaped = lambda x: x.reshape(1, 1, N, 128)
    assert np.isin(vals, q).all() and np.isin(vals, k).all() and np.isin(vals, v).all()
    check_quantize(shaped(q), shaped(k), shaped(v), "fp8", bq, [(0, 0)], f"every-bf16-bq{bq}")


@pytest.mark.parametrize("fmt", ["fp4", "mxfp4"])
def test_quantize_e2m1_every_bf16_value(gpu_lib, fmt):
    """The device E2M1 encoder against the oracle's on every finite bf16 value
    of magnitude up to 6 (33154 values), at unit scale: every 16-channel group
    of every Q and K token holds a 6, so the FP4 scale is 6 / 6 = 1 and the
    MXFP4 shared exponent is floor(log2 6) - 2 = 0, and each code is E2M1 of
    the input itself.  K's second half is its first half negated (channel
    means exactly 0); V holds the same values."""
    top = 0x40C0                                  # bf16 bits of 6
    pos = np.arange(top + 1, dtype=np.uint16)      # +0 .. 6
    vals = np.concatenate([pos, pos | np.uint16(0x8000)])
    N = 320

    def filled(src, n_tok):
        """n_tok x 128 bf16 patterns: 6 at channel 16 j of every token, src (repeated) elsewhere"""
        x = np.zeros((n_tok, 128), np.uint16)
        mark = np.zeros((n_tok, 128), bool)
        mark[:, ::16] = True
        x[mark] = top
        x[~mark] = np.resize(src, int((~mark).sum()))
        return x

    q = filled(vals, N)
    v = filled(vals[::-1], N)
    kh = filled(pos, N // 2)
    k = np.concatenate([kh, kh ^ np.uint16(0x8000)])
    shaped = lambda x: x.reshape(1, 1, N, 128)
    assert np.isin(vals, q).all() and np.isin(vals, k).all()
    check_quantize(shaped(q), shaped(k), shaped(v), fmt, 128, [(0, 0)], f"every-bf16-{fmt}")


@pytest.mark.parametrize("fmt,bq", [("fp8", 64), ("fp4", 128), ("mxfp4", 128)])
def test_quantize_k_mean_exact_beyond_fp64_range(gpu_lib, fmt, bq):
    """K channels whose values span more binades than fp64 partial sums hold
    (so a blocked fp64 sum drops low bits or cancels the wrong way): the
    channel mean is still fp32(fp64(exact sum) / N), bit for bit."""
    import math
    from gpu_helpers import fixed_order_fp64_sum, wide_span_inputs
    qb, kb, vb = wide_span_inputs()
    N = qb.shape[2]
    for h in range(2):
        exact = math.fsum(oracle.bf16_bits_to_f64(kb[0, h, :, 0]))
        # a blocked fp64 sum of channel 0 loses the small values beside +-2^60
        assert fixed_order_fp64_sum(kb[0, h, :, 0]) != exact
        assert np.float32(fixed_order_fp64_sum(kb[0, h, :, 0]) / N) != np.float32(exact / N)
    check_quantize(qb, kb, vb, fmt, bq, [(0, 0), (0, 1)], f"wide-span-{fmt}")

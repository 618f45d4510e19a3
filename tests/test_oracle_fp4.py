"""Pins of the oracle's FP4 score path (E2M1 codes with an fp32 scale per 16
consecutive channels of one token): the dequantized values written out
element by element, the same values against the E2M1 error bound of the
inputs (with group maxima taken here, not by the oracle), and the FP4
forward against exact attention.

The FP8 and FP4 schemes differ only in the precision of the query/key side
(NVIDIA RTX AI optimiert FLUX.1 fuer Bilddaten mit niedriger Genauigkeit,
hyper.ai/de, the paragraph on the SageAttention paper series), so every FP4
score comes from these dequantized values."""
import numpy as np

import oracle
from workloads import TAU, WORKLOADS, draw

E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])   # code & 7 -> magnitude


def _fp4(seq_len=40, seed=9):
    qb, kb, vb = draw(WORKLOADS["tiny"], seq_len=seq_len, seed=seed)
    return (qb, kb, vb), oracle.quantize(qb, kb, vb, fmt="fp4")


def test_fp4_dequantized_groups_by_loops():
    """dequantize_qk of FP4 Q and K codes equals sign * magnitude(code) *
    scale[n, d // 16] for every token n and channel d, with the codes read
    from their nibbles (the even channel in the low nibble)."""
    _, z = _fp4()
    for codes, scales in ((z.q_codes, z.q_scales), (z.k_codes, z.k_scales)):
        for h in range(2):
            got = oracle.dequantize_qk(codes, scales, "fp4", 0, 0, h)
            assert got.shape == (40, 128)
            for n in range(40):
                for d in range(128):
                    byte = int(codes[0, h, n, d // 2])
                    c = byte & 0xF if d % 2 == 0 else byte >> 4
                    mag = E2M1_MAGS[c & 7]
                    want = (-mag if c & 8 else mag) * float(scales[0, h, n, d // 16])
                    assert got[n, d] == want, (h, n, d)


def test_fp4_dequantized_values_within_e2m1_bound_of_inputs():
    """Every dequantized FP4 value is within the E2M1 rounding bound of the
    value it codes (Q, and K minus its channel mean), with the bound built
    from each 16-channel group's largest magnitude computed here: a step of
    s/2 (|x|/s < 2), s (2..4) or 2 s (4..6), s = amax/6, so at most half a
    step away (plus fp32 rounding of the scaled value)."""
    (qb, kb, _), z = _fp4()
    q = oracle.bf16_bits_to_f64(qb)[0].astype(np.float32)
    ks = oracle.bf16_bits_to_f64(kb)[0].astype(np.float32) - z.k_mean[0][:, None, :]
    for x, codes, scales in ((q, z.q_codes, z.q_scales), (ks, z.k_codes, z.k_scales)):
        for h in range(2):
            got = oracle.dequantize_qk(codes, scales, "fp4", 0, 0, h)
            xg = x[h].astype(np.float64)
            amax = np.abs(xg.reshape(40, 8, 16)).max(axis=2)           # [40, 8]
            s = np.repeat(amax / 6.0, 16, axis=1)                      # [40, 128]
            y = np.abs(xg) / s
            half_step = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0)) * s
            assert np.all(np.abs(got - xg) <= half_step * (1 + 1e-6) + 1e-6 * np.abs(xg)), h
            # the group maximum itself is coded exactly as +-6 s
            top = np.abs(xg) == np.repeat(amax, 16, axis=1)
            assert np.allclose(np.abs(got[top]), 6.0 * s[top], rtol=1e-6, atol=0)


def test_fp4_forward_close_to_exact_attention():
    """The FP4 forward of the tiny workload against exact fp64 attention of
    the unquantized inputs: max-abs 0.11 / 0.14 and mean-abs 0.010 on its two
    heads, whose outputs have an RMS of about 0.095 (MXFP4: 0.12 / 0.012;
    FP8: 0.054 / 0.0037).  A group scale taken from the wrong group moves
    the mean error to about 0.037, and scores without the scales to 0.6."""
    qb, kb, vb = draw(WORKLOADS["tiny"])
    z = oracle.quantize(qb, kb, vb, fmt="fp4")
    for h in range(2):
        o = oracle.attend(z, TAU, 0, h)
        ex = oracle.exact_attention(oracle.bf16_bits_to_f64(qb[0, h]), oracle.bf16_bits_to_f64(kb[0, h]),
                                    oracle.bf16_bits_to_f64(vb[0, h]), TAU)
        err = np.abs(o - ex)
        assert err.max() < 0.25 and err.mean() < 0.02, (err.max(), err.mean())

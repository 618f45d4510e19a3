"""Plain CPU oracle of quantized scaled-dot-product attention (test
infrastructure: see ``oracle/__init__.py``).

What the pages fix
------------------
* Attention (SDPA) of the FLUX transformer is the operation that is
  quantized, and its quantization is the core of the work (NVIDIA RTX AI,
  저정밀 양자화로 FLUX.1 Kontext 최적화, hyper.ai/kr, the paragraph on
  quantization strategy).
* The FP8 and FP4 schemes are alike and differ only in the precision given
  to the query/key/value side; attention itself is kept mainly in FP8 for
  numerical stability, which is why FP4 gains less than FP8 (NVIDIA RTX AI
  optimiert FLUX.1 fuer Bilddaten mit niedriger Genauigkeit, hyper.ai/de,
  the paragraph on the SageAttention paper series and on "Tabelle 1").
* Kontext concatenates the input-image tokens to the output-image tokens, so
  one joint attention runs over [text | output image | context image]
  (same articles; NVIDIA RTX AI accélère FLUX.1 Kontext, hyper.ai/fr,
  "Explications Techniques").  There is no mask: every query sees every key.

What the pages leave open, and the reading taken here
------------------------------------------------------
The pages print no formula.  The oracle computes, per (batch, head), with
head dimension D = 128, queries i and keys j:

1. Channel statistics.  mu[d] = fp32( fp64(sum_n K[n, d]) / N ), where the
   sum is the exact sum rounded once to fp64 (``math.fsum``) and the divide is
   one fp64 division; vmax[d] = max_n |V[n, d]|.
2. K smoothing.  Ks = fp32(K - mu): one correctly rounded fp32 subtraction.
   Softmax is unchanged by subtracting one vector from every key, so the
   smoothing only moves K's per-channel offset out of the quantized range.
3. Q and K codes.  FP8 mode: one scale per block of ``block`` consecutive
   tokens (all 128 channels; the last block may be short).  FP4 mode: one
   scale per 16 consecutive channels of one token.  For a block with
   a = max |x|: if a == 0 the scale and all codes are 0; otherwise
   inv = fp32(F / a), s = fp32(a / F), code = E(fp32(x * inv)) with F = 448,
   E = E4M3 (FP8) or F = 6, E = E2M1 (FP4).  The value of a code is code * s.
   A block whose fp32 inverse F / a overflows (0 < a < F / FLT_MAX, values
   below about 1.3e-36 for FP8 and 1.8e-38 for FP4) has no fp32 inverse scale
   and is coded as an all-zero block too.
4. V codes (FP8 in both modes, since attention stays FP8).  Per channel d:
   inv = fp32(448 / vmax[d]), sV[d] = fp32(vmax[d] / 448),
   code = E4M3(fp32(V * inv)); zero rule as in 3.
5. Scores in fp64 from the dequantized codes: S = tau * Qdq . Kdq^T.
6. Online softmax over steps of 64 consecutive keys in ascending order (a
   short last step is allowed): m_t = max(m_{t-1}, max_j S_ij);
   alpha = exp(m_{t-1} - m_t); p = exp(S_ij - m_t);
   P = E4M3(fp32(448 p)) (the decision taken in fp32);
   l = alpha l + sum_j p (the unquantized p);
   acc = alpha acc + sum_j P_ij Vcode_jd.
7. O[i, d] = bf16( acc[d] * sV[d] / (448 l) ), rounded to nearest even.

The step of 64 keys matters: P's codes are taken relative to the running
maximum, so a different step gives different codes.

Selective correction (VC-Attention-style)
-----------------------------------------
The VisualGen article (FLUX 3 Image Klein Base, devotd.net, "왜 이런 차이가
나나") names VC-Attention FP8 with rho = 0.005 as FP8 attention that corrects
only the tokens with a large error, and says no more.  The reading taken
here: the tokens are the query tokens (rows of O); a token's error is its own
FP8 quantization error, e_i = sum_d (q_id - code_id s_i)^2; per (b, h) the
k = ceil(rho N) tokens with the largest e_i (ties to the lower index) get the
unquantized softmax attention of the bf16 inputs in place of their quantized
row.

MXFP4 mode (beyond the pages)
-----------------------------
The pages' FP4 scheme has an fp32 scale per 16 channels.  The MXFP4 mode
instead follows the OCP Microscaling Formats (MX) specification v1.0 (the
FP4 E2M1 element type with a shared E8M0 scale per block of 32 elements),
the block format that the scaled MFMA of the target GPU applies in hardware.
Step 3 becomes, for each token and each block of 32 consecutive channels
with a = max |x|: if a == 0 the scale byte and all codes are 0; otherwise
the shared exponent is floor(log2 a) minus 2 (the exponent of E2M1's largest
normal value 6 = 1.5 * 2**2), stored biased by 127 and clamped to [0, 254];
X = 2**(byte - 127) and code = E2M1(x / X), nearest even, saturating at 6
(so magnitudes in (6 X, 8 X) become 6 X).  Steps 1, 2 and 4-7 are unchanged.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from .formats import E2M1, E4M3, bf16_bits_to_f64, decode, encode, f32, f64_to_bf16_bits, round_to

FP8 = "fp8"
FP4 = "fp4"
MXFP4 = "mxfp4"
MX_BLOCK = 32          # channels per E8M0 scale in MXFP4 mode
E8M0_BIAS = 127
P_SCALE = 448.0        # P codes are E4M3(448 p): p <= 1 fills the FP8 range
SOFTMAX_STEP = 64      # keys per online-softmax step
FP4_GROUP = 16         # channels per FP4 scale


# --------------------------------------------------------------------------
# 1-4: statistics and quantization
# --------------------------------------------------------------------------
def channel_stats(k: np.ndarray, v: np.ndarray):
    """mu[b,h,d] (fp32 mean of K over tokens) and vmax[b,h,d] (fp32 max |V|).

    ``k`` and ``v`` are float64 [B, H, N, D] holding bf16 values."""
    B, H, N, D = k.shape
    mu = np.empty((B, H, D), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            cols = k[b, h].T            # [D, N]
            for d in range(D):
                total = math.fsum(cols[d].tolist())
                mu[b, h, d] = np.float32(total / N)
    vmax = np.abs(v).max(axis=2).astype(np.float32)
    return mu, vmax


def smooth_k(k: np.ndarray, mu: np.ndarray) -> np.ndarray:
    """fp32(K - mu) for float64 K holding bf16 values and fp32 mu [B,H,D]."""
    return k.astype(np.float32) - mu[:, :, None, :]


def _live(amax: np.ndarray, fmax: float) -> np.ndarray:
    """Blocks that get codes: those whose inverse scale fp32(F / amax) is
    finite.  That excludes amax = 0, and also 0 < amax < F / FLT_MAX (about
    1.3e-36 for F = 448, 1.8e-38 for F = 6), where the fp32 inverse overflows:
    such a block is coded like an all-zero block (scale 0, codes 0)."""
    with np.errstate(divide="ignore", over="ignore"):
        inv = np.float32(fmax) / np.asarray(amax, dtype=np.float32)
    return np.isfinite(inv) & (np.asarray(amax) > 0)


def _codes_from(x32: np.ndarray, amax: np.ndarray, fmax: float, fmt):
    """Codes of fp32 values ``x32`` given each element's block maximum
    ``amax`` (broadcast to x32's shape)."""
    fmax32 = np.float32(fmax)
    live = _live(amax, fmax)
    safe = np.where(live, amax, np.float32(1.0)).astype(np.float32)
    inv = (fmax32 / safe).astype(np.float32)
    scaled = (x32 * inv).astype(np.float32)
    vals = round_to(scaled.astype(np.float64), fmt)
    vals = np.where(live, vals, 0.0)
    return encode(vals, fmt)


def quantize_fp8_blocks(x32: np.ndarray, block: int):
    """Per-token-block FP8 codes.  x32 float32 [B,H,N,D] ->
    (codes uint8 [B,H,N,D], scales fp32 [B,H,ceil(N/block)])."""
    B, H, N, D = x32.shape
    nblk = -(-N // block)
    amax_blk = np.zeros((B, H, nblk), dtype=np.float32)
    for t in range(nblk):
        amax_blk[:, :, t] = np.abs(x32[:, :, t * block:(t + 1) * block, :]).max(axis=(2, 3))
    scales = np.where(_live(amax_blk, 448.0), amax_blk / np.float32(448.0), np.float32(0.0)).astype(np.float32)
    amax_tok = np.repeat(amax_blk, block, axis=2)[:, :, :N, None]
    codes = _codes_from(x32, np.broadcast_to(amax_tok, x32.shape), 448.0, E4M3)
    return codes, scales


def quantize_fp4_groups(x32: np.ndarray, group: int = FP4_GROUP):
    """Per-(token, 16-channel group) FP4 codes.  x32 float32 [B,H,N,D] ->
    (packed uint8 [B,H,N,D/2], scales fp32 [B,H,N,D/group]).  Two codes per
    byte, the even channel in the low nibble."""
    B, H, N, D = x32.shape
    g = x32.reshape(B, H, N, D // group, group)
    amax = np.abs(g).max(axis=4)
    scales = np.where(_live(amax, 6.0), amax / np.float32(6.0), np.float32(0.0)).astype(np.float32)
    codes = _codes_from(g, np.broadcast_to(amax[..., None], g.shape), 6.0, E2M1).reshape(B, H, N, D)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, scales


def quantize_mxfp4_blocks(x32: np.ndarray, block: int = MX_BLOCK):
    """MXFP4 codes: per (token, 32-channel block) a shared power-of-two scale.
    x32 float32 [B,H,N,D] -> (packed uint8 [B,H,N,D/2], scale bytes uint8
    [B,H,N,D/32]).  The scale byte is the biased exponent e of X = 2**(e-127);
    codes as in FP4 mode (two per byte, the even channel in the low nibble)."""
    B, H, N, D = x32.shape
    g = x32.astype(np.float64).reshape(B, H, N, D // block, block)
    amax = np.abs(g).max(axis=4)
    _, e = np.frexp(amax)                      # amax = f * 2**e, f in [0.5, 1)
    shared = (e - 1) - 2                       # floor(log2 amax) - emax(E2M1)
    byte = np.clip(shared + E8M0_BIAS, 0, 254)
    byte = np.where(amax > 0, byte, 0).astype(np.uint8)
    X = np.ldexp(1.0, byte.astype(np.int64) - E8M0_BIAS)
    vals = round_to(g / X[..., None], E2M1)    # x / X is exact: X is a power of two
    vals = np.where(amax[..., None] > 0, vals, 0.0)
    codes = encode(vals, E2M1).reshape(B, H, N, D)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, byte


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    """Inverse of the nibble packing: uint8 [..., D/2] -> codes [..., D]."""
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def quantize_v(v: np.ndarray, vmax: np.ndarray):
    """Per-channel FP8 codes of V.  v float64 [B,H,N,D] holding bf16 values,
    vmax fp32 [B,H,D] -> (codes uint8 [B,H,N,D], scales fp32 [B,H,D])."""
    v32 = v.astype(np.float32)
    scales = np.where(_live(vmax, 448.0), vmax / np.float32(448.0), np.float32(0.0)).astype(np.float32)
    amax = np.broadcast_to(vmax[:, :, None, :], v32.shape)
    return _codes_from(v32, amax, 448.0, E4M3), scales


@dataclass
class Quantized:
    """Output of the quantize step, in natural (token-major) layouts."""
    fmt: str
    block_q: int
    block_k: int
    q_codes: np.ndarray   # fp8: uint8 [B,H,N,D]; fp4, mxfp4: packed uint8 [B,H,N,D/2]
    q_scales: np.ndarray  # fp8: fp32 [B,H,nQ];   fp4: fp32 [B,H,N,D/16]; mxfp4: E8M0 bytes [B,H,N,D/32]
    k_codes: np.ndarray
    k_scales: np.ndarray
    k_mean: np.ndarray    # fp32 [B,H,D]
    v_codes: np.ndarray   # uint8 [B,H,N,D]
    v_scales: np.ndarray  # fp32 [B,H,D]
    v_amax: np.ndarray    # fp32 [B,H,D]


def quantize(q_bits, k_bits, v_bits, *, fmt: str = FP8, block_q: int = 128, block_k: int = 64) -> Quantized:
    """Steps 1-4 for bf16 bit patterns (uint16 [B,H,N,D])."""
    if fmt not in (FP8, FP4, MXFP4):
        raise ValueError(fmt)
    q = bf16_bits_to_f64(q_bits)
    k = bf16_bits_to_f64(k_bits)
    v = bf16_bits_to_f64(v_bits)
    mu, vmax = channel_stats(k, v)
    ks = smooth_k(k, mu)
    q32 = q.astype(np.float32)
    if fmt == FP8:
        qc, qs = quantize_fp8_blocks(q32, block_q)
        kc, kscl = quantize_fp8_blocks(ks, block_k)
    elif fmt == FP4:
        qc, qs = quantize_fp4_groups(q32)
        kc, kscl = quantize_fp4_groups(ks)
    else:
        qc, qs = quantize_mxfp4_blocks(q32)
        kc, kscl = quantize_mxfp4_blocks(ks)
    vc, vs = quantize_v(v, vmax)
    return Quantized(fmt, block_q, block_k, qc, qs, kc, kscl, mu, vc, vs, vmax)


def dequantize_qk(codes, scales, fmt: str, block: int, b: int, h: int) -> np.ndarray:
    """fp64 values code * scale of one (b, h), [N, D]; exact in fp64."""
    if fmt == FP8:
        vals = decode(codes[b, h], E4M3)
        N = vals.shape[0]
        s = np.repeat(scales[b, h].astype(np.float64), block)[:N]
        return vals * s[:, None]
    vals = decode(unpack_fp4(codes[b, h]), E2M1)
    N, D = vals.shape
    if fmt == MXFP4:
        s = np.ldexp(1.0, scales[b, h].astype(np.int64) - E8M0_BIAS)   # [N, D/32]
        return (vals.reshape(N, D // MX_BLOCK, MX_BLOCK) * s[:, :, None]).reshape(N, D)
    s = scales[b, h].astype(np.float64)                     # [N, D/16]
    return (vals.reshape(N, D // FP4_GROUP, FP4_GROUP) * s[:, :, None]).reshape(N, D)


# --------------------------------------------------------------------------
# 5-7: attention
# --------------------------------------------------------------------------
def online_softmax_av(S: np.ndarray, V: np.ndarray, *, step: int = SOFTMAX_STEP, quantize_p: bool = True,
                      trace: list | None = None):
    """Step 6 for fp64 scores S [R, N] and values V [N, D].

    Returns (acc [R, D], l [R]).  With ``quantize_p`` the weights fed to the
    value product are E4M3(fp32(448 p)); without it they are 448 p exactly, so
    acc / (448 l) is then plain softmax(S) V.

    ``trace``, if a list, receives one record per step (for the tests that
    bound how far a correct fp32 implementation may land from this result):
    the first key j0, the running maxima before and after the step, alpha,
    the unquantized p and the weights w."""
    R, N = S.shape
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    acc = np.zeros((R, V.shape[1]))
    for j0 in range(0, N, step):
        Sb = S[:, j0:j0 + step]
        m_new = np.maximum(m, Sb.max(axis=1))
        alpha = np.exp(m - m_new)
        p = np.exp(Sb - m_new[:, None])
        if quantize_p:
            v = P_SCALE * p
            w = round_to(f32(v).astype(np.float64), E4M3)
        else:
            w = P_SCALE * p
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + w @ V[j0:j0 + step]
        if trace is not None:
            trace.append({"j0": j0, "m_prev": m, "m": m_new, "alpha": alpha, "p": p, "w": w})
        m = m_new
    return acc, l


def attend(qz: Quantized, tau: float, b: int, h: int, rows=None, *, trace: dict | None = None):
    """Steps 5-7 for one (b, h).  Returns O as float64 bf16 values [R, D]
    for the query rows ``rows`` (all rows if None).

    ``trace``, if a dict, receives the intermediates (for the tests): the
    dequantized Q rows and K ("Qd", "Kd"), the scores "S", the V codes "Vc",
    the V scales "sv", "acc", "l", the output before its bf16 rounding
    "out", and the per-step records of ``online_softmax_av`` ("steps")."""
    Qd = dequantize_qk(qz.q_codes, qz.q_scales, qz.fmt, qz.block_q, b, h)
    Kd = dequantize_qk(qz.k_codes, qz.k_scales, qz.fmt, qz.block_k, b, h)
    if rows is not None:
        Qd = Qd[np.asarray(rows)]
    S = float(tau) * (Qd @ Kd.T)
    Vc = decode(qz.v_codes[b, h], E4M3)
    steps = [] if trace is not None else None
    acc, l = online_softmax_av(S, Vc, trace=steps)
    sv = qz.v_scales[b, h].astype(np.float64)[None, :]
    out = acc * sv / (P_SCALE * l)[:, None]
    if trace is not None:
        trace.update(Qd=Qd, Kd=Kd, S=S, Vc=Vc, sv=sv[0], acc=acc, l=l, out=out, steps=steps)
    return bf16_bits_to_f64(f64_to_bf16_bits(out))


def forward(q_bits, k_bits, v_bits, *, fmt: str = FP8, block_q: int = 128, block_k: int = 64,
            tau: float = float(np.float32(1.0 / math.sqrt(128.0)))) -> np.ndarray:
    """Whole path: bf16 bits [B,H,N,D] in, bf16 bits [B,H,N,D] out."""
    qz = quantize(q_bits, k_bits, v_bits, fmt=fmt, block_q=block_q, block_k=block_k)
    B, H, N, D = q_bits.shape
    out = np.empty((B, H, N, D), dtype=np.uint16)
    for b in range(B):
        for h in range(H):
            out[b, h] = f64_to_bf16_bits(attend(qz, tau, b, h))
    return out


# --------------------------------------------------------------------------
# Selective correction of the high-error tokens (VC-Attention-style)
# --------------------------------------------------------------------------
VC_RHO = 0.005   # fraction of tokens corrected


def vc_count(n_tokens: int, rho: float) -> int:
    """Tokens corrected per (b, h): k = ceil(rho N), at least 1 and at most N."""
    return min(n_tokens, max(1, math.ceil(rho * n_tokens - 1e-9)))


def vc_token_error(qz: Quantized, q_bits, b: int, h: int) -> np.ndarray:
    """Per query token i of (b, h): e_i = sum_d (q_id - code_id * s_i)^2, the
    squared L2 norm of the token's own FP8 quantization error (q the bf16
    input, code * s its dequantized value), summed exactly (math.fsum)."""
    if qz.fmt != FP8:
        raise ValueError("the selective correction is defined for the FP8 mode")
    q = bf16_bits_to_f64(q_bits[b, h])
    dq = q - dequantize_qk(qz.q_codes, qz.q_scales, FP8, qz.block_q, b, h)   # exact in fp64
    return np.array([math.fsum((row * row).tolist()) for row in dq])


def vc_select(err: np.ndarray, k: int) -> np.ndarray:
    """The k tokens with the largest error, ties to the lower index; returned
    in ascending index order."""
    order = sorted(range(len(err)), key=lambda i: (-err[i], i))
    return np.array(sorted(order[:k]), dtype=np.int64)


def vc_forward(q_bits, k_bits, v_bits, *, rho: float = VC_RHO, block_q: int = 128, block_k: int = 64,
               tau: float = float(np.float32(1.0 / math.sqrt(128.0)))):
    """FP8 quantized attention with the high-error tokens corrected: per
    (b, h), the k = ceil(rho N) query tokens whose own quantization error
    (vc_token_error) is largest get the unquantized softmax attention of the
    bf16 inputs (fp64, rounded to bf16) in place of their quantized row.
    Returns (O bf16 bits [B,H,N,D], selected rows [B,H,k])."""
    qz = quantize(q_bits, k_bits, v_bits, fmt=FP8, block_q=block_q, block_k=block_k)
    B, H, N, D = q_bits.shape
    kk = vc_count(N, rho)
    out = np.empty((B, H, N, D), dtype=np.uint16)
    sel = np.empty((B, H, kk), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            o = attend(qz, tau, b, h)
            sel[b, h] = vc_select(vc_token_error(qz, q_bits, b, h), kk)
            q, k, v = (bf16_bits_to_f64(x[b, h]) for x in (q_bits, k_bits, v_bits))
            o[sel[b, h]] = bf16_bits_to_f64(f64_to_bf16_bits(exact_attention(q, k, v, tau, sel[b, h])))
            out[b, h] = f64_to_bf16_bits(o)
    return out, sel


def exact_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, tau: float, rows=None) -> np.ndarray:
    """Unquantized softmax(tau Q K^T) V in fp64 for one (b, h): q, k, v
    float64 [N, D]; returns [R, D] for the query rows ``rows``."""
    if rows is not None:
        q = q[np.asarray(rows)]
    S = float(tau) * (q @ k.T)
    S = S - S.max(axis=1, keepdims=True)
    w = np.exp(S)
    w /= w.sum(axis=1, keepdims=True)
    return w @ v

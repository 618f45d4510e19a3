"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
library through its binding, and read the workspace back in the oracle's
natural layouts.  (No arithmetic of the method lives here.)"""
from __future__ import annotations

import numpy as np
import torch

import precision_attention_qsdpa_amd as qs


def to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).cuda()


def from_dev(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def vtile_key_order() -> np.ndarray:
    """key held by byte p of a V tile row (documented in include/qsdpa.h)."""
    p = np.arange(64)
    g, kb, r = p >> 5, (p >> 4) & 1, p & 15
    return 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3)


def read_workspace(ws: torch.Tensor, params, N: int) -> dict:
    """Workspace sections as numpy arrays in natural layouts, tokens < N."""
    L = qs.qsdpa_workspace_layout(params)
    BH = params.batch * params.heads
    B, H = params.batch, params.heads
    raw = ws.cpu().numpy()

    def sec(off, count, dtype):
        return raw[off:off + count * np.dtype(dtype).itemsize].view(dtype)

    crb = L.code_row_bytes
    out = {}
    out["q_codes"] = sec(L.q_codes, BH * L.n_pad * crb, np.uint8).reshape(B, H, L.n_pad, crb)[:, :, :N]
    out["k_codes"] = sec(L.k_codes, BH * L.n_pad * crb, np.uint8).reshape(B, H, L.n_pad, crb)[:, :, :N]
    if params.qk_format == qs.QSDPA_QK_FP8_E4M3:
        nq = -(-N // params.block_q)
        nk = -(-N // params.block_k)
        out["q_scales"] = sec(L.q_scales, BH * L.q_scale_count, np.float32).reshape(B, H, -1)[:, :, :nq]
        out["k_scales"] = sec(L.k_scales, BH * L.k_scale_count, np.float32).reshape(B, H, -1)[:, :, :nk]
        out["q_scales_pad"] = sec(L.q_scales, BH * L.q_scale_count, np.float32).reshape(B, H, -1)[:, :, nq:]
        out["k_scales_pad"] = sec(L.k_scales, BH * L.k_scale_count, np.float32).reshape(B, H, -1)[:, :, nk:]
    elif params.qk_format == qs.QSDPA_QK_FP4_E2M1:
        out["q_scales"] = sec(L.q_scales, BH * L.q_scale_count, np.float32).reshape(B, H, L.n_pad, 8)[:, :, :N]
        out["k_scales"] = sec(L.k_scales, BH * L.k_scale_count, np.float32).reshape(B, H, L.n_pad, 8)[:, :, :N]
    else:
        # MXFP4: Q scale bytes token-major; K scale bytes in the score MFMA's lane
        # order: tile t, entry 32g + r, byte 2kb + h -> key 64t + 32kb + r, block 2h + g
        qsb = sec(L.q_scales, BH * L.q_scale_count, np.uint8).reshape(B, H, L.n_pad, 4)
        ksl = sec(L.k_scales, BH * L.k_scale_count, np.uint8).reshape(B, H, L.n_pad // 64, 2, 32, 2, 2)  # t,g,r,kb,h
        ksn = ksl.transpose(0, 1, 2, 5, 4, 6, 3).reshape(B, H, L.n_pad, 4)                          # t,kb,r,h,g
        out["q_scales"], out["k_scales"] = qsb[:, :, :N], ksn[:, :, :N]
        out["q_scales_pad"], out["k_scales_pad"] = qsb[:, :, N:], ksn[:, :, N:]
    out["k_mean"] = sec(L.k_mean, BH * 128, np.float32).reshape(B, H, 128)
    out["v_scales"] = sec(L.v_scales, BH * 128, np.float32).reshape(B, H, 128)
    out["v_amax"] = sec(L.v_amax, BH * 128, np.float32).reshape(B, H, 128)
    vt = sec(L.v_codes, BH * L.n_pad * 128, np.uint8).reshape(B, H, L.n_pad // 64, 128, 64)
    nat = np.empty((B, H, L.n_pad // 64, 64, 128), np.uint8)
    nat[:, :, :, vtile_key_order(), :] = vt.transpose(0, 1, 2, 4, 3)
    nat = nat.reshape(B, H, L.n_pad, 128)
    out["v_codes"] = nat[:, :, :N]
    out["v_codes_pad"] = nat[:, :, N:]
    out["q_codes_pad"] = sec(L.q_codes, BH * L.n_pad * crb, np.uint8).reshape(B, H, L.n_pad, crb)[:, :, N:]
    out["k_codes_pad"] = sec(L.k_codes, BH * L.n_pad * crb, np.uint8).reshape(B, H, L.n_pad, crb)[:, :, N:]
    if params.qk_format == qs.QSDPA_QK_FP4_E2M1:
        # expanded K, per 64-key tile: the f16 hi tile (16 KB, 8-channel chunk c of
        # key row r at chunk position c ^ (r & 15)), then the correction tile (16 KB,
        # 16-byte chunk 2c + i of key row r at position (2c + i) ^ (r & 15): E4M3
        # lo8 (i = 0) or hi8 (i = 1) of channels 16c .. 16c + 15)
        tiles = L.n_pad // 64
        raw_t = sec(L.k_expanded, BH * tiles * 32768, np.uint8).reshape(B, H, tiles, 2, 64, 16, 16)
        r = np.arange(64)[:, None]
        pos = np.arange(16)[None, :] ^ (r & 15)                  # [64 rows, 16 chunks] -> stored position
        nat = np.take_along_axis(raw_t, pos[None, None, None, None, :, :, None], axis=5)   # chunks in order
        hi = np.ascontiguousarray(nat[:, :, :, 0]).view(np.uint16).reshape(B, H, tiles, 64, 128)
        cor = nat[:, :, :, 1].reshape(B, H, tiles, 64, 8, 2, 16)                          # [.., c, i, byte]
        lo8 = cor[..., 0, :].reshape(B, H, tiles, 64, 128)
        hi8 = cor[..., 1, :].reshape(B, H, tiles, 64, 128)
        flat = lambda a: a.reshape(B, H, L.n_pad, 128)
        out["k_hi"], out["k_lo8"], out["k_hi8"] = flat(hi)[:, :, :N], flat(lo8)[:, :, :N], flat(hi8)[:, :, :N]
        out["k_hilo_pad"] = np.concatenate([flat(hi)[:, :, N:].view(np.uint8).reshape(B, H, -1),
                                            flat(lo8)[:, :, N:].reshape(B, H, -1),
                                            flat(hi8)[:, :, N:].reshape(B, H, -1)], axis=2)
        # then the power-of-two exponent E of each tile (int32 [B, H, n_pad/64])
        out["k_exp"] = sec(L.k_expanded + BH * tiles * 32768, BH * tiles, np.int32).reshape(
            B, H, L.n_pad // 64)
    return out


def run_quantize(q_bits, k_bits, v_bits, params):
    q, k, v = to_dev(q_bits), to_dev(k_bits), to_dev(v_bits)
    ws = qs.empty_workspace(params)
    ws.fill_(0xA5)   # poison: every byte the layout promises must be written
    qs.qsdpa_quantize(q, k, v, ws, params)
    torch.cuda.synchronize()
    return ws


def run_forward(q_bits, k_bits, v_bits, params):
    q, k, v = to_dev(q_bits), to_dev(k_bits), to_dev(v_bits)
    out = qs.qsdpa_forward(q, k, v, params=params)
    torch.cuda.synchronize()
    return from_dev(out)


def tiny_magnitude_inputs(N: int = 300, seed: int = 31):
    """bf16 bit patterns of Q, K, V [1, 2, N, 128] (N even, N >= 216) with
    token bands and V channels whose magnitudes sit around the limit below
    which an inverse scale F / amax overflows fp32 (F / FLT_MAX is about
    1.3e-36 for F = 448 and 1.8e-38 for F = 6): tokens 64..127 near 1e-37,
    128..191 near 7e-37, 192..207 bf16 subnormals near 4e-39, 208..215 deep
    subnormals that are mostly 0; every 7th value of those bands exactly 0;
    V channels 3, 4, 5 near 1e-37, 7e-37 and 4e-39, channel 6 all 0; the rest
    N(0, 1).  K is made of pairs of opposite tokens, so its channel mean is
    exactly 0 and smoothing leaves it unchanged."""
    from workloads import to_bf16_bits

    rng = np.random.default_rng(seed)
    band = np.ones(N, np.float32)
    band[64:128], band[128:192], band[192:208], band[208:216] = 1e-37, 2e-36 / 3, 4e-39, 1e-41
    holes = np.ones(128, np.float32)
    holes[::7] = 0

    def shaped(x):
        x = x * band[None, None, :, None]
        x[:, :, 64:216] *= holes
        return x

    q = shaped(rng.standard_normal((1, 2, N, 128)).astype(np.float32))
    half = rng.standard_normal((1, 2, N // 2, 128)).astype(np.float32)
    k = np.empty((1, 2, N, 128), np.float32)
    k[:, :, 0::2], k[:, :, 1::2] = half, -half
    k = shaped(k)
    v = rng.standard_normal((1, 2, N, 128)).astype(np.float32)
    v[..., 3] *= np.float32(1e-37)
    v[..., 4] *= np.float32(2e-36 / 3)
    v[..., 5] *= np.float32(4e-39)
    v[..., 6] = 0
    return to_bf16_bits(q), to_bf16_bits(k), to_bf16_bits(v)


def wide_span_inputs(N: int = 1000, seed: int = 11):
    """bf16 bit patterns of Q, K, V [1, 2, N, 128] (N >= 800) whose K channels
    0..4 span far more binades than an fp64 sum can hold exactly: channel 0
    has +-2^60 at two tokens that cancel (head 0: tokens 5 and 250, one range
    of 256 tokens; head 1: tokens 3 and 700, two ranges), channel 1 one token
    of 2^100, channel 2 bf16 subnormals on every other token, channel 3
    opposite pairs +-x with x from 2^-100 to 2^100, channel 4 +-2^40 on every
    16th token; the other channels and Q, V are N(0, 1)."""
    from workloads import WORKLOADS, draw
    qb, kb, vb = draw(WORKLOADS["tiny"], seq_len=N, seed=seed)
    kb = kb.copy()
    rng = np.random.default_rng(seed)
    big = lambda e: np.uint16(0x3F80 + (e << 7))          # bf16 bits of 2^e
    for h, (i, j) in enumerate([(5, 250), (3, 700)]):
        kb[0, h, i, 0] = big(60)
        kb[0, h, j, 0] = big(60) | np.uint16(0x8000)
        kb[0, h, 17 + h, 1] = big(100)
        kb[0, h, ::2, 2] = rng.integers(1, 128, len(kb[0, h, ::2, 2])).astype(np.uint16)
        half = N // 2
        e = rng.integers(-100, 101, half)
        x = (big(0) + (e << 7).astype(np.int32) + rng.integers(0, 128, half)).astype(np.uint16)
        kb[0, h, :half, 3] = x
        kb[0, h, half:2 * half, 3] = x ^ np.uint16(0x8000)
        kb[0, h, ::16, 4] = big(40) | (rng.integers(0, 2, len(kb[0, h, ::16, 4])) << 15).astype(np.uint16)
    return qb, kb, vb


def fixed_order_fp64_sum(col: np.ndarray) -> float:
    """fp64 sum of one K channel (bf16 bits, N tokens) in a fixed blocked
    order: within each range of 256 tokens, 16 running sums over the tokens
    r, r + 16, ... (r = 0..15), added in r order; then the ranges in order."""
    x = (col.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    total = 0.0
    for s in range(0, len(x), 256):
        part = 0.0
        for r in range(16):
            acc = 0.0
            for v in x[s + r:s + 256:16]:
                acc += v
            part += acc
        total += part
    return total

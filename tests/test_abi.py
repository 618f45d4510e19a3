"""Host-side checks of the C ABI (no GPU call is made): the library loads,
exports every function that include/qsdpa.h declares, validates arguments and
lays out the workspace as documented.  Every forward/quantize call here is
rejected by validation before any launch."""
import ctypes
import os
import re

import numpy as np

import pytest

import precision_attention_qsdpa_amd as qs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "qsdpa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qsdpa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = qs.load()
    names = _header_functions()
    assert set(names) == set(qs.EXPORTS)
    for n in names:
        assert getattr(lib, n) is not None


def test_abi_version_and_status_strings():
    assert qs.load().qsdpa_abi_version() == qs.ABI_VERSION == 7
    for st in range(-7, 1):
        assert qs.status_string(st) not in ("", "unknown status")
    assert qs.status_string(-99) == "unknown status"


@pytest.mark.parametrize("change,status", [
    (dict(batch=0), qs.QSDPA_ERR_INVALID_ARG), (dict(heads=-1), qs.QSDPA_ERR_INVALID_ARG),
    (dict(seq_len=0), qs.QSDPA_ERR_INVALID_ARG), (dict(head_dim=64), qs.QSDPA_ERR_UNSUPPORTED),
    (dict(block_q=96), qs.QSDPA_ERR_UNSUPPORTED), (dict(block_k=128), qs.QSDPA_ERR_UNSUPPORTED),
    (dict(qk_format=7), qs.QSDPA_ERR_UNSUPPORTED), (dict(softmax_scale=0.0), qs.QSDPA_ERR_INVALID_ARG),
    (dict(softmax_scale=float("inf")), qs.QSDPA_ERR_INVALID_ARG),
    (dict(softmax_scale=float("nan")), qs.QSDPA_ERR_INVALID_ARG),
    (dict(batch=70000), qs.QSDPA_ERR_UNSUPPORTED),
    (dict(batch=4096, heads=16, seq_len=1 << 22), qs.QSDPA_ERR_UNSUPPORTED),
    (dict(batch=256, heads=128, seq_len=1 << 21), qs.QSDPA_ERR_INVALID_ARG),
])
def test_invalid_params(change, status):
    p = qs.make_params(1, 2, 320)
    for k, v in change.items():
        setattr(p, k, v)
    assert qs.qsdpa_validate_params(p) == status
    assert qs.qsdpa_workspace_bytes(p) == 0
    lib = qs.load()
    assert lib.qsdpa_forward(ctypes.byref(p), 256, 256, 256, 1 << 40, 1 << 41, 1 << 30, None) == status


@pytest.mark.parametrize("fmt", ["fp8", "fp4", "mxfp4"])
def test_size_limits_are_exact(fmt):
    """The largest accepted N and B*H pass, one more is refused."""
    ok = qs.make_params(1, 1, qs.MAX_SEQ_LEN, fmt=fmt)
    assert qs.qsdpa_validate_params(ok) == qs.QSDPA_OK
    assert qs.qsdpa_workspace_bytes(ok) > 0
    assert qs.qsdpa_validate_params(qs.make_params(1, 1, qs.MAX_SEQ_LEN + 1, fmt=fmt)) == qs.QSDPA_ERR_UNSUPPORTED
    assert qs.qsdpa_validate_params(qs.make_params(5, qs.MAX_BH // 5, 64, fmt=fmt)) == qs.QSDPA_OK
    assert qs.qsdpa_validate_params(qs.make_params(2, (qs.MAX_BH + 1) // 2, 64, fmt=fmt)) == qs.QSDPA_ERR_UNSUPPORTED
    # B*H*n_pad*128 at the element limit, then one 128-token tile more
    assert qs.qsdpa_validate_params(qs.make_params(4096, 1, 1 << 17, fmt=fmt)) == qs.QSDPA_OK
    assert qs.qsdpa_validate_params(qs.make_params(4096, 1, (1 << 17) + 1, fmt=fmt)) == qs.QSDPA_ERR_INVALID_ARG


def test_header_limits_match_binding():
    import os
    hdr = open(os.path.join(os.path.dirname(qs.PKG), "include", "qsdpa.h")).read()
    assert "#define QSDPA_MAX_SEQ_LEN (1 << 22)" in hdr and qs.MAX_SEQ_LEN == 1 << 22
    assert "#define QSDPA_MAX_BH 65535" in hdr and qs.MAX_BH == 65535
    assert "#define QSDPA_MAX_ELEMS (1LL << 36)" in hdr and qs.MAX_ELEMS == 1 << 36


def test_fp4_group_checked_only_in_fp4_mode():
    p = qs.make_params(1, 1, 64, fmt="fp4", fp4_group=32)
    assert qs.qsdpa_validate_params(p) == qs.QSDPA_ERR_UNSUPPORTED
    p = qs.make_params(1, 1, 64, fmt="fp8", fp4_group=32)
    assert qs.qsdpa_validate_params(p) == qs.QSDPA_OK
    p = qs.make_params(1, 1, 64, fmt="fp4", block_q=96)      # block sizes unused in FP4 mode
    assert qs.qsdpa_validate_params(p) == qs.QSDPA_OK
    # MXFP4: fixed 32-channel blocks; block sizes and the FP4 group are not used
    p = qs.make_params(1, 1, 64, fmt="mxfp4", block_q=96, block_k=32, fp4_group=7)
    assert qs.qsdpa_validate_params(p) == qs.QSDPA_OK
    p = qs.make_params(1, 1, 64, fmt="fp8")
    p.qk_format = 3
    assert qs.qsdpa_validate_params(p) == qs.QSDPA_ERR_UNSUPPORTED


def _round(x, a):
    return (x + a - 1) // a * a


@pytest.mark.parametrize("B,H,N,fmt,bq", [(1, 2, 320, "fp8", 64), (1, 24, 8704, "fp8", 128),
                                          (2, 24, 16896, "fp4", 128), (3, 5, 1, "fp8", 128),
                                          (1, 1, 1000, "fp4", 64), (2, 24, 16896, "mxfp4", 128),
                                          (1, 3, 77, "mxfp4", 64)])
def test_workspace_closed_form(B, H, N, fmt, bq):
    """One byte per Q/K code in FP8 mode (half a byte in the FP4 modes), one byte
    per V code, fp32 scales (one E8M0 byte per 32 channels in MXFP4 mode),
    padded to 128 tokens, 256-byte aligned sections; in FP4 mode also the
    expansion of K (f16 hi plus the E4M3 lo8 and hi8: 4 bytes per element) and
    an int32 exponent per 64-key tile."""
    p = qs.make_params(B, H, N, fmt=fmt, block_q=bq)
    L = qs.qsdpa_workspace_layout(p)
    BH, npad = B * H, _round(N, 128)
    splits = -(-N // 256)
    crb = 128 if fmt == "fp8" else 64
    qsc = {"fp8": npad // bq, "fp4": npad * 8, "mxfp4": npad * 4}[fmt]
    ksc = {"fp8": npad // 64, "fp4": npad * 8, "mxfp4": npad * 4}[fmt]
    sb = 1 if fmt == "mxfp4" else 4
    sizes = [BH * npad * crb, BH * npad * crb, BH * npad * 128, BH * qsc * sb, BH * ksc * sb,
             BH * 512, BH * 512, BH * 512, BH * splits * 128 * 16,
             BH * npad * 128 * 4 + BH * (npad // 64) * 4 if fmt == "fp4" else 0]
    assert (L.n_pad, L.code_row_bytes, L.q_scale_count, L.k_scale_count, L.stats_splits) == (npad, crb, qsc, ksc, splits)
    assert L.total == sum(_round(s, 256) for s in sizes)
    assert qs.qsdpa_workspace_bytes(p) == L.total
    offs = [L.q_codes, L.k_codes, L.v_codes, L.q_scales, L.k_scales, L.k_mean, L.v_scales, L.v_amax, L.stats,
            L.k_expanded]
    for (o, s), o2 in zip(zip(offs, sizes), offs[1:] + [L.total]):
        assert o % 256 == 0 and o + s <= o2
    # FP8 halves the bf16 bytes of Q, K and V; FP4 Q/K codes (V stays FP8) cut them 3x
    qkv_bf16 = 3 * BH * N * 128 * 2
    codes = sizes[0] + sizes[1] + sizes[2]
    assert (L.k_expanded == L.total) == (fmt != "fp4")
    if N % 128 == 0:
        assert codes * (2 if fmt == "fp8" else 3) == qkv_bf16


def test_buffer_checks_before_any_launch():
    lib = qs.load()
    p = qs.make_params(1, 2, 320)
    need = qs.qsdpa_workspace_bytes(p)
    t = 2 * 320 * 128 * 2
    ok = dict(q=0x10000000, k=0x20000000, v=0x30000000, o=0x40000000, ws=0x50000000, n=need)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.qsdpa_forward(ctypes.byref(p), a["q"], a["k"], a["v"], a["o"], a["ws"], a["n"], None)

    assert call(q=None) == qs.QSDPA_ERR_INVALID_ARG
    assert call(ws=None) == qs.QSDPA_ERR_INVALID_ARG
    assert call(q=0x10000008) == qs.QSDPA_ERR_ALIGNMENT
    assert call(o=0x40000004) == qs.QSDPA_ERR_ALIGNMENT
    assert call(ws=0x50000010) == qs.QSDPA_ERR_ALIGNMENT
    assert call(n=need - 1) == qs.QSDPA_ERR_WORKSPACE_TOO_SMALL
    assert call(o=0x10000000 + t - 16) == qs.QSDPA_ERR_ALIAS
    assert call(o=0x50000000 + need - 256) == qs.QSDPA_ERR_ALIAS
    assert call(v=0x50000000 - t + 16) == qs.QSDPA_ERR_ALIAS
    assert lib.qsdpa_attention(ctypes.byref(p), 0x50000000, need - 1, 0x40000000, None) == \
        qs.QSDPA_ERR_WORKSPACE_TOO_SMALL
    assert lib.qsdpa_quantize(ctypes.byref(p), 0x10000000, None, 0x30000000, 0x50000000, need, None) == \
        qs.QSDPA_ERR_INVALID_ARG
    assert lib.qsdpa_workspace_layout(ctypes.byref(p), None) == qs.QSDPA_ERR_INVALID_ARG


def test_binding_rejects_host_tensors_before_the_library():
    """q, k, v, out and the workspace must be CUDA tensors on one device: the
    binding raises before any pointer reaches the library."""
    import torch
    q = torch.zeros(1, 1, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="contiguous CUDA bfloat16"):
        qs.qsdpa_forward(q, q, q)
    with pytest.raises(ValueError, match="workspace must be a contiguous CUDA tensor"):
        qs._check_workspace(torch.empty(64, dtype=torch.uint8), torch.device("cuda", 0))


def test_noalloc_rejects_problems_beyond_the_scratch_array():
    """qsdpa_forward_noalloc returns before any GPU call when the workspace
    would exceed the static scratch array (or the parameters are invalid)."""
    lib = qs.load()
    fits = qs.make_params(1, 24, 8704, fmt="fp8")
    assert qs.qsdpa_workspace_bytes(fits) <= qs.QSDPA_SCRATCH_BYTES
    big = qs.make_params(2, 24, 16896, fmt="fp8")
    assert qs.qsdpa_workspace_bytes(big) > qs.QSDPA_SCRATCH_BYTES
    assert lib.qsdpa_forward_noalloc(ctypes.byref(big), 256, 512, 768, 1 << 40, None) == \
        qs.QSDPA_ERR_SCRATCH_TOO_SMALL
    bad = qs.make_params(1, 2, 320, block_q=96)
    assert lib.qsdpa_forward_noalloc(ctypes.byref(bad), 256, 512, 768, 1 << 40, None) == qs.QSDPA_ERR_UNSUPPORTED
    assert "static scratch" in qs.status_string(qs.QSDPA_ERR_SCRATCH_TOO_SMALL)


def test_vc_layout_and_validation():
    """The selective correction's plan: k = ceil(rho N) rows per (b,h) (the
    oracle's count), padded to 32, key ranges that cover N, sections after
    qsdpa_forward's workspace; FP8 only, rho in (0, 1]."""
    import oracle
    for (B, H, N, rho) in [(1, 24, 8704, 0.005), (1, 2, 320, 0.005), (2, 1, 1, 0.005), (1, 3, 1000, 1.0),
                           (2, 24, 16896, 0.005), (1, 1, 129, 0.3)]:
        p = qs.make_params(B, H, N, fmt="fp8")
        L = qs.qsdpa_vc_workspace_layout(p, rho)
        assert L.count == oracle.vc_count(N, float(np.float32(rho)))
        assert L.count_pad % 32 == 0 and L.count <= L.count_pad < L.count + 32
        assert L.chunk_keys % 32 == 0 and (L.chunks - 1) * L.chunk_keys < N <= L.chunks * L.chunk_keys
        assert L.token_error >= qs.qsdpa_workspace_bytes(p) and L.token_error % 256 == 0
        assert L.total == qs.load().qsdpa_vc_workspace_bytes(ctypes.byref(p), ctypes.c_float(rho))
    p = qs.make_params(1, 2, 320, fmt="fp8")
    for bad in (0.0, -0.1, 1.5, float("nan")):
        with pytest.raises(qs.QsdpaError):
            qs.qsdpa_vc_workspace_layout(p, bad)
    with pytest.raises(qs.QsdpaError) as e:
        qs.qsdpa_vc_workspace_layout(qs.make_params(1, 2, 320, fmt="mxfp4"), 0.005)
    assert e.value.status == qs.QSDPA_ERR_UNSUPPORTED

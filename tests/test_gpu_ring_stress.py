"""The race-detection build of the library (libqsdpa_stress.so, the same
sources built with QSDPA_RING_STRESS: every wave sleeps pseudo-random times
at the points where the attention kernels' tile ring hands LDS stages between
waves) gives outputs bit-identical to the normal build, in every mode, on
the forward and on quantize + attention, repeatedly.  A missing wait or
barrier in the ring would let a wave read a stage before it landed or after
another wave refilled it, and the perturbed timing would change the result."""
import ctypes
import os

import numpy as np
import pytest
import torch

import precision_attention_qsdpa_amd as qs
from gpu_helpers import from_dev, to_dev
from workloads import WORKLOADS, draw

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def stress_lib(gpu_lib):
    path = os.path.join(os.path.dirname(qs.LIB_PATH), "libqsdpa_stress.so")
    if not os.path.exists(path):
        pytest.fail(f"{path} is missing: build it with `python -m precision_attention_qsdpa_amd.build`")
    lib = ctypes.CDLL(path)
    P, vp, sz = ctypes.POINTER(qs.QsdpaParams), ctypes.c_void_p, ctypes.c_size_t
    lib.qsdpa_abi_version.restype = ctypes.c_int
    lib.qsdpa_forward.restype = ctypes.c_int
    lib.qsdpa_forward.argtypes = [P, vp, vp, vp, vp, vp, sz, vp]
    lib.qsdpa_quantize.restype = ctypes.c_int
    lib.qsdpa_quantize.argtypes = [P, vp, vp, vp, vp, sz, vp]
    lib.qsdpa_attention.restype = ctypes.c_int
    lib.qsdpa_attention.argtypes = [P, vp, sz, vp, vp]
    assert lib.qsdpa_abi_version() == qs.ABI_VERSION
    return lib


CASES = [("fp8", 1, 2, 65, 64), ("fp8", 2, 1, 129, 64), ("fp8", 1, 3, 777, 128), ("fp8", 1, 24, 8704, 128),
         ("mxfp4", 1, 2, 129, 128), ("mxfp4", 1, 6, 3000, 128), ("fp4", 1, 2, 300, 128), ("fp4", 1, 4, 2100, 128)]


@pytest.mark.parametrize("fmt,B,H,N,bq", CASES)
def test_stress_build_is_bit_identical(stress_lib, fmt, B, H, N, bq):
    qb, kb, vb = draw(WORKLOADS["tiny"], batch=B, heads=H, seq_len=N, seed=600 + N)
    params = qs.make_params(B, H, N, fmt=fmt, block_q=bq)
    print(f"[stress] fmt={fmt} B={B} H={H} N={N} bq={bq}", flush=True)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    ref = from_dev(qs.qsdpa_forward(q, k, v, params=params))
    ws = qs.empty_workspace(params)
    nbytes = ws.numel()
    stream = torch.cuda.current_stream().cuda_stream
    for rep in range(3):
        o = torch.full_like(q, float("nan"))
        st = stress_lib.qsdpa_forward(ctypes.byref(params), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                      ws.data_ptr(), nbytes, stream)
        assert st == qs.QSDPA_OK
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(o), ref), f"forward, repeat {rep}"
    o = torch.full_like(q, float("nan"))
    assert stress_lib.qsdpa_quantize(ctypes.byref(params), q.data_ptr(), k.data_ptr(), v.data_ptr(), ws.data_ptr(),
                                     nbytes, stream) == qs.QSDPA_OK
    assert stress_lib.qsdpa_attention(ctypes.byref(params), ws.data_ptr(), nbytes, o.data_ptr(), stream) == qs.QSDPA_OK
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(o), ref), "quantize + attention"

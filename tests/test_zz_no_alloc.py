"""qsdpa_forward_noalloc, whose workspace is the library's static scratch
array, against qsdpa_forward through the C ABI, bit for bit: calls in a row,
each smaller than the first (the Kontext workload in FP8 fills 81.5 MB of the
96 MiB array), in the three modes.  The array keeps the previous call's
contents; no call depends on them."""
import numpy as np
import pytest
import torch

import precision_attention_qsdpa_amd as qs
from gpu_helpers import from_dev, to_dev
from workloads import WORKLOADS, draw

pytestmark = pytest.mark.gpu


def _run(bits, params):
    q, k, v = (to_dev(x) for x in bits)
    ref = qs.qsdpa_forward(q, k, v, params=params)
    out = torch.full_like(q, float("nan"))
    qs.qsdpa_forward_noalloc(q, k, v, out, params)
    torch.cuda.synchronize()
    return from_dev(out), from_dev(ref)


def test_noalloc_matches_forward(gpu_lib):
    w = WORKLOADS["kontext1024"]
    calls = [("kontext1024 fp8", draw(w), qs.make_params(w.batch, w.heads, w.seq_len, fmt="fp8", block_q=128)),
             ("mxfp4 [1,3,1500]", draw(WORKLOADS["tiny"], heads=3, seq_len=1500, seed=81),
              qs.make_params(1, 3, 1500, fmt="mxfp4")),
             ("fp4 [1,2,777]", draw(WORKLOADS["tiny"], heads=2, seq_len=777, seed=82),
              qs.make_params(1, 2, 777, fmt="fp4")),
             ("fp8 bq64 [2,1,129]", draw(WORKLOADS["tiny"], batch=2, heads=1, seq_len=129, seed=83),
              qs.make_params(2, 1, 129, fmt="fp8", block_q=64))]
    sizes = [qs.qsdpa_workspace_bytes(p) for _, _, p in calls]
    assert sizes[0] <= qs.QSDPA_SCRATCH_BYTES and all(s < sizes[0] for s in sizes[1:])
    for label, bits, params in calls:
        print(f"[noalloc] {label}: workspace {qs.qsdpa_workspace_bytes(params)} bytes", flush=True)
        got, ref = _run(bits, params)
        assert np.array_equal(got, ref), label


def test_noalloc_rejects_oversize_before_launch(gpu_lib):
    w = WORKLOADS["gen2048_fp8"]
    params = qs.make_params(w.batch, w.heads, 128, fmt="fp8")
    params.seq_len = w.seq_len      # sizes checked by the library, not by torch: tiny tensors suffice
    q = torch.zeros((1, 1, 128, 128), dtype=torch.bfloat16, device="cuda")
    lib = qs.load()
    import ctypes
    st = lib.qsdpa_forward_noalloc(ctypes.byref(params), q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(),
                                   None)
    assert st == qs.QSDPA_ERR_SCRATCH_TOO_SMALL

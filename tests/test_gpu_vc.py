"""GPU parity of the selective correction (qsdpa_forward_vc) against the
oracle: each token's quantization error (fp64) against the oracle's exact
sum, the corrected rows as a valid top-k of those errors (equal to the
oracle's selection unless two errors tie within the fp64 rounding), the
corrected rows against exact attention, and every other row equal to
qsdpa_forward bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import precision_attention_qsdpa_amd as qs
from gpu_helpers import from_dev, run_forward, to_dev
from workloads import TAU, WORKLOADS, draw

pytestmark = pytest.mark.gpu

MAX_ABS = 1e-2
MEAN_ABS = 1e-3


def run_vc(qb, kb, vb, params, rho):
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    out, ws = qs.qsdpa_forward_vc(q, k, v, rho=rho, params=params)
    torch.cuda.synchronize()
    L = qs.qsdpa_vc_workspace_layout(params, rho)
    Lb = qs.qsdpa_workspace_layout(params)
    raw = ws.cpu().numpy()
    BH, npad = params.batch * params.heads, Lb.n_pad
    err = raw[L.token_error:L.token_error + BH * npad * 8].view(np.float64).reshape(params.batch, params.heads, npad)
    sel = raw[L.selected:L.selected + BH * L.count_pad * 4].view(np.int32).reshape(params.batch, params.heads,
                                                                                   L.count_pad)
    return from_dev(out), err[..., :params.seq_len], sel[..., :L.count], L.count


def check(qb, kb, vb, fmt_bq, rho, heads, label, rows_of=None):
    B, H, N = qb.shape[0], qb.shape[1], qb.shape[2]
    bq = fmt_bq
    params = qs.make_params(B, H, N, fmt="fp8", block_q=bq)
    print(f"[vc] {label}: B={B} H={H} N={N} bq={bq} rho={rho}", flush=True)
    got, err, sel, k = run_vc(qb, kb, vb, params, rho)
    plain = run_forward(qb, kb, vb, params)
    assert k == oracle.vc_count(N, float(np.float32(rho)))
    raw_errs = []
    for b, h in heads:
        z = oracle.quantize(qb[b:b + 1, h:h + 1], kb[b:b + 1, h:h + 1], vb[b:b + 1, h:h + 1], fmt="fp8",
                            block_q=bq, block_k=64)
        e = oracle.vc_token_error(z, qb[b:b + 1, h:h + 1], 0, 0)
        # the errors: fp64 sums of exact squares' roundings vs the exact sum
        assert np.all(np.abs(err[b, h] - e) <= 1e-13 * e + 1e-300), label
        # the rows: a valid top-k of the oracle's errors, ascending; the
        # oracle's own selection unless errors tie within the fp64 rounding
        s = sel[b, h]
        assert np.all(np.diff(s) > 0) and s.min() >= 0 and s.max() < N
        want = oracle.vc_select(e, k)
        if not np.array_equal(s, want):
            rest = np.setdiff1d(np.arange(N), s)
            lo, hi = e[s].min(), (e[rest].max() if len(rest) else -1.0)
            assert hi <= lo * (1 + 1e-12), f"{label}: not a top-{k} selection"
            print(f"[vc] {label} (b={b}, h={h}): selection differs from the oracle's at an fp64 tie", flush=True)
        # corrected rows against exact attention of the bf16 inputs
        q, kk, v = (oracle.bf16_bits_to_f64(x[b, h]) for x in (qb, kb, vb))
        ex = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(oracle.exact_attention(q, kk, v, TAU, s)))
        d = np.abs(oracle.bf16_bits_to_f64(got[b, h, s]) - ex)
        raw_errs.append(d)
        # every other row is qsdpa_forward's
        rest = np.setdiff1d(np.arange(N), s)
        assert np.array_equal(got[b, h, rest], plain[b, h, rest]), label
    d = np.concatenate([x.ravel() for x in raw_errs])
    print(f"[vc] {label}: corrected rows vs exact attention max {d.max():.3e} mean {d.mean():.3e}", flush=True)
    assert d.max() <= MAX_ABS and d.mean() <= MEAN_ABS


def test_vc_kontext(gpu_lib):
    w = WORKLOADS["kontext1024"]
    qb, kb, vb = draw(w)
    check(qb, kb, vb, 128, qs.VC_RHO, [(0, 0), (0, 11), (0, 23)], "kontext1024")


def test_vc_gen2048(gpu_lib):
    """The 2048x2048 shape (B = 2, the classifier-free-guidance pair): 85
    corrected rows per head (three row groups of 32, so one recomputation
    workgroup has a wave without rows) over 16896 keys in 15 ranges."""
    w = WORKLOADS["gen2048_fp8"]
    qb, kb, vb = draw(w)
    check(qb, kb, vb, 128, qs.VC_RHO, [(0, 0), (1, 23)], "gen2048_fp8")


@pytest.mark.parametrize("N,bq,rho", [(1, 64, 0.005), (65, 64, 0.005), (129, 128, 0.1), (320, 64, 0.005),
                                      (1000, 128, 0.05), (300, 128, 1.0), (2100, 128, 0.02), (17000, 128, 0.005)])
def test_vc_ragged_and_rho(gpu_lib, N, bq, rho):
    qb, kb, vb = draw(WORKLOADS["tiny"], batch=2, heads=2, seq_len=N, seed=700 + N)
    check(qb, kb, vb, bq, rho, [(0, 0), (1, 1)], f"N={N} rho={rho}")


def test_vc_ties_go_to_the_lower_index(gpu_lib):
    """Every query token the same: every error is equal, so the first k
    tokens are corrected."""
    N = 1000
    qb, kb, vb = draw(WORKLOADS["tiny"], heads=2, seq_len=N, seed=77)
    qb = np.broadcast_to(qb[:, :, 3:4], qb.shape).copy()
    params = qs.make_params(1, 2, N, fmt="fp8", block_q=128)
    got, err, sel, k = run_vc(qb, kb, vb, params, 0.01)
    assert k == 10
    for h in range(2):
        assert np.all(err[0, h] == err[0, h, 0])
        assert np.array_equal(sel[0, h], np.arange(10))
    check(qb, kb, vb, 128, 0.01, [(0, 0), (0, 1)], "ties")


def test_vc_maximum_heads(gpu_lib):
    """B*H = 65535 (the largest accepted), 100 tokens each: one corrected row
    per head, 65535 selection workgroups and a recomputation grid of 65535
    workgroups; three heads spread over the batch are checked."""
    B, H, N = 5, 13107, 100
    assert B * H == qs.MAX_BH
    gen = torch.Generator(device="cuda")
    gen.manual_seed(65536)
    bits = [from_dev(torch.randn((B, H, N, 128), generator=gen, device="cuda", dtype=torch.bfloat16))
            for _ in range(3)]
    check(*bits, 128, qs.VC_RHO, [(0, 0), (2, H // 2), (B - 1, H - 1)], "max-heads")

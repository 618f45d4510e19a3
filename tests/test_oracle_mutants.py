"""Planted mistakes in the oracle, each of which its pins must catch.

Each case edits one line of the oracle's source: a dropped term, a wrong sign,
scale, block, index or axis.  It loads the edited module, swaps it in for the
real one for that test only, and runs the pins named for the mistake, which
must fail.  The oracle on disk is never changed.  A control loads the unedited
source the same way and checks that every pin used here still passes, so a
failure can come only from the planted mistake."""
import inspect
import types

import pytest

import oracle
import oracle.formats
import oracle.qsdpa
import test_oracle_attention as A
import test_oracle_fp4 as P4
import test_oracle_formats as F
import test_oracle_mx as M
import test_oracle_quantize as Q
import test_oracle_vc as VC

QS, FM = oracle.qsdpa, oracle.formats

# (name, module, source text, replacement, pins that must fail)
MUTANTS = [
    # online softmax (steps 6-7)
    ("row_sum_of_codes", QS, "l = alpha * l + p.sum(axis=1)", "l = alpha * l + w.sum(axis=1) / P_SCALE",
     [(A.test_worked_example_one_step, {})]),
    ("row_sum_not_rescaled", QS, "l = alpha * l + p.sum(axis=1)", "l = l + p.sum(axis=1)",
     [(A.test_online_softmax_without_quantizers_is_exact_softmax, {"step": 7})]),
    ("accumulator_not_rescaled", QS, "acc = alpha[:, None] * acc + w @ V[j0:j0 + step]",
     "acc = acc + w @ V[j0:j0 + step]",
     [(A.test_online_softmax_without_quantizers_is_exact_softmax, {"step": 7})]),
    ("max_not_carried", QS, "m_new = np.maximum(m, Sb.max(axis=1))", "m_new = Sb.max(axis=1)",
     [(A.test_worked_example_running_max_is_kept, {})]),
    ("p_scale_256", QS, "v = P_SCALE * p", "v = 256.0 * p", [(A.test_worked_example_one_step, {})]),
    ("p_not_quantized", QS, "w = round_to(f32(v).astype(np.float64), E4M3)", "w = v",
     [(A.test_worked_example_one_step, {}), (A.test_worked_example_step_size_changes_codes, {})]),
    ("epilogue_without_v_scale", QS, "out = acc * sv / (P_SCALE * l)[:, None]", "out = acc / (P_SCALE * l)[:, None]",
     [(A.test_single_token_closed_form, {}), (A.test_zero_queries_closed_form, {"fmt": "fp8"})]),
    ("epilogue_without_448", QS, "out = acc * sv / (P_SCALE * l)[:, None]", "out = acc * sv / l[:, None]",
     [(A.test_single_token_closed_form, {})]),
    # scores (step 5)
    ("scores_without_tau", QS, "S = float(tau) * (Qd @ Kd.T)", "S = Qd @ Kd.T",
     [(A.test_forward_close_to_exact_attention_tiny, {})]),
    ("softmax_over_queries", QS, "S = float(tau) * (Qd @ Kd.T)", "S = float(tau) * (Qd @ Kd.T).T",
     [(A.test_query_rows_depend_only_on_their_own_block, {}), (A.test_row_subset_equals_full, {})]),
    ("queries_smoothed_too", QS, "q32 = q.astype(np.float32)", "q32 = smooth_k(q, mu)",
     [(A.test_forward_close_to_exact_attention_tiny, {})]),
    # statistics and smoothing (steps 1-2)
    ("smoothing_adds_mean", QS, "return k.astype(np.float32) - mu[:, :, None, :]",
     "return k.astype(np.float32) + mu[:, :, None, :]",
     [(Q.test_k_smoothing_removes_constant_key_offset_exactly, {})]),
    ("mean_over_n_minus_1", QS, "mu[b, h, d] = np.float32(total / N)", "mu[b, h, d] = np.float32(total / (N - 1))",
     [(Q.test_channel_mean_by_construction, {}), (Q.test_channel_mean_agrees_with_numpy_mean, {})]),
    ("vmax_signed", QS, "vmax = np.abs(v).max(axis=2)", "vmax = v.max(axis=2)",
     [(Q.test_channel_mean_by_construction, {})]),
    # Q/K/V codes (steps 3-4)
    ("inverse_overflow_not_flushed", QS, "return np.isfinite(inv) & (np.asarray(amax) > 0)",
     "return np.asarray(amax) > 0", [(Q.test_blocks_without_an_fp32_inverse_scale_are_zero_blocks, {})]),
    ("k_blocks_of_block_q", QS, "kc, kscl = quantize_fp8_blocks(ks, block_k)",
     "kc, kscl = quantize_fp8_blocks(ks, block_q)", [(Q.test_q_and_k_take_their_own_block_sizes, {})]),
    ("block_max_reaches_next_token", QS, "np.abs(x32[:, :, t * block:(t + 1) * block, :])",
     "np.abs(x32[:, :, t * block:(t + 1) * block + 1, :])", [(Q.test_fp8_block_scales_by_construction, {})]),
    ("codes_divided_by_inverse", QS, "scaled = (x32 * inv).astype(np.float32)",
     "scaled = (x32 / inv).astype(np.float32)",
     [(Q.test_fp8_block_scales_by_construction, {}), (Q.test_zero_block_gives_zero_scale_and_codes, {})]),
    ("v_scale_per_token", QS, "amax = np.broadcast_to(vmax[:, :, None, :], v32.shape)",
     "amax = np.broadcast_to(np.abs(v32).max(axis=3, keepdims=True), v32.shape)",
     [(Q.test_v_channel_max_maps_to_448, {}), (A.test_single_token_closed_form, {})]),
    ("fp4_nibbles_swapped", QS,
     "codes = _codes_from(g, np.broadcast_to(amax[..., None], g.shape), 6.0, E2M1).reshape(B, H, N, D)\n"
     "    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)",
     "codes = _codes_from(g, np.broadcast_to(amax[..., None], g.shape), 6.0, E2M1).reshape(B, H, N, D)\n"
     "    packed = (codes[..., 1::2] | (codes[..., 0::2] << 4)).astype(np.uint8)",
     [(Q.test_fp4_groups_and_nibble_order, {})]),
    ("fp4_group_of_32", QS, "FP4_GROUP = 16 ", "FP4_GROUP = 32 ", [(Q.test_fp4_groups_and_nibble_order, {})]),
    ("fp4_max_code_4", QS, "scales = np.where(_live(amax, 6.0), amax / np.float32(6.0), np.float32(0.0))",
     "scales = np.where(_live(amax, 6.0), amax / np.float32(4.0), np.float32(0.0))",
     [(Q.test_fp4_groups_and_nibble_order, {}), (Q.test_fp4_error_bound, {})]),
    ("fp4_group_scales_reversed", QS,
     "return (vals.reshape(N, D // FP4_GROUP, FP4_GROUP) * s[:, :, None]).reshape(N, D)",
     "return (vals.reshape(N, D // FP4_GROUP, FP4_GROUP) * s[:, ::-1, None]).reshape(N, D)",
     [(P4.test_fp4_dequantized_groups_by_loops, {}), (P4.test_fp4_dequantized_values_within_e2m1_bound_of_inputs, {}),
      (P4.test_fp4_forward_close_to_exact_attention, {})]),
    ("fp4_group_scales_dropped", QS,
     "return (vals.reshape(N, D // FP4_GROUP, FP4_GROUP) * s[:, :, None]).reshape(N, D)",
     "return vals",
     [(P4.test_fp4_dequantized_groups_by_loops, {}), (P4.test_fp4_dequantized_values_within_e2m1_bound_of_inputs, {}),
      (P4.test_fp4_forward_close_to_exact_attention, {})]),
    ("mx_exponent_minus_1", QS, "shared = (e - 1) - 2", "shared = (e - 1) - 1",
     [(M.test_shared_exponent_and_block_max_code, {"m": 1.5, "k": 0, "want": 6.0})]),
    ("mx_scale_bias_126", QS, "X = np.ldexp(1.0, byte.astype(np.int64) - E8M0_BIAS)",
     "X = np.ldexp(1.0, byte.astype(np.int64) - 126)",
     [(M.test_shared_exponent_and_block_max_code, {"m": 1.5, "k": 0, "want": 6.0})]),
    # selective correction
    ("vc_selects_smallest", QS, "key=lambda i: (-err[i], i))", "key=lambda i: (err[i], i))",
     [(VC.test_selection_matches_brute_force_with_ties, {})]),
    ("vc_ties_to_higher_index", QS, "key=lambda i: (-err[i], i))", "key=lambda i: (-err[i], -i))",
     [(VC.test_selection_matches_brute_force_with_ties, {})]),
    ("vc_error_not_squared", QS, "math.fsum((row * row).tolist())", "math.fsum(np.abs(row).tolist())",
     [(VC.test_token_error_on_known_codes, {})]),
    ("vc_count_floor", QS, "max(1, math.ceil(rho * n_tokens - 1e-9))", "max(1, math.floor(rho * n_tokens))",
     [(VC.test_count_is_ceil_rho_n, {"n": 8704, "rho": 0.005, "want": 44})]),
    ("vc_rows_not_corrected", QS,
     "o[sel[b, h]] = bf16_bits_to_f64(f64_to_bf16_bits(exact_attention(q, k, v, tau, sel[b, h])))",
     "o[sel[b, h]] = o[sel[b, h]]",
     [(VC.test_all_tokens_corrected_is_exact_attention, {}), (VC.test_correction_lowers_the_error_of_its_rows, {})]),
    # format codecs
    ("round_half_away", FM, "r = np.rint(a / step) * step", "r = np.floor(a / step + 0.5) * step",
     [(F.test_e4m3_rounding_matches_torch_and_bruteforce, {}),
      (F.test_e2m1_ties_and_saturation, {"x": 2.5, "want": 2.0})]),
    ("no_saturation", FM, "a = np.minimum(a, fmt.max_finite)", "a = a",
     [(F.test_e4m3_saturates_and_keeps_sign, {})]),
    ("sign_dropped", FM, "return np.copysign(r, x)", "return r",
     [(F.test_e4m3_saturates_and_keeps_sign, {}), (F.test_e4m3_rounding_matches_torch_and_bruteforce, {})]),
    ("no_subnormal_floor", FM, "e = np.maximum(e - 1, fmt.emin)", "e = e - 1",
     [(F.test_e4m3_rounding_matches_torch_and_bruteforce, {})]),
    ("e4m3_bias_off_by_one", FM, "(exp_field + fmt.emin - 1).astype(np.int64)",
     "(exp_field + fmt.emin).astype(np.int64)", [(F.test_e4m3_decode_matches_torch_for_every_code, {})]),
    ("bf16_truncated", FM, "r = round_to(x, BF16, saturate=False).astype(np.float32)",
     "r = np.asarray(x, dtype=np.float32)", [(F.test_bf16_rounding_matches_torch, {})]),
    ("e2m1_max_4", FM, 'E2M1 = FloatFormat("e2m1", mant_bits=1, emin=0, max_finite=6.0, exp_bits=2)',
     'E2M1 = FloatFormat("e2m1", mant_bits=1, emin=0, max_finite=4.0, exp_bits=2)',
     [(F.test_e2m1_rounding_matches_bruteforce, {}), (F.test_e2m1_ties_and_saturation, {"x": 7.0, "want": 6.0})]),
]

TARGETS = (oracle, QS, FM, A, F, M, P4, Q, VC)


def _load(mod, old, new):
    """A fresh module built from ``mod``'s source with ``old`` replaced by ``new``."""
    src = inspect.getsource(mod)
    if old:
        assert src.count(old) == 1, f"mutation site not found once in {mod.__name__}: {old!r}"
        src = src.replace(old, new)
    m = types.ModuleType(mod.__name__)
    m.__package__ = "oracle"
    m.__file__ = mod.__file__
    exec(compile(src, f"<edited {mod.__name__}>", "exec"), m.__dict__)
    return m


def _install(monkeypatch, orig, edited):
    """Point every name that holds one of ``orig``'s objects (in the oracle
    package, its modules and the pin modules) at ``edited``'s object of the
    same name."""
    for name, new in vars(edited).items():
        if name.startswith("__"):
            continue
        old = getattr(orig, name, None)
        if old is None or old is new:
            continue
        for t in TARGETS:
            if getattr(t, name, None) is old:
                monkeypatch.setattr(t, name, new)


def _fails(fn, kw):
    try:
        fn(**kw)
    except Exception:   # an assertion, or the edited oracle crashing on the pin's input
        return True
    return False


@pytest.mark.filterwarnings("ignore::RuntimeWarning")   # an edited oracle may overflow or make NaN
@pytest.mark.parametrize("name,mod,old,new,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(monkeypatch, name, mod, old, new, pins):
    _install(monkeypatch, mod, _load(mod, old, new))
    missed = [fn.__name__ for fn, kw in pins if not _fails(fn, kw)]
    assert not missed, f"{name}: these pins pass with the planted mistake: {missed}"


@pytest.mark.parametrize("mod", [QS, FM], ids=["qsdpa", "formats"])
def test_control_unedited_source_passes_every_pin(monkeypatch, mod):
    _install(monkeypatch, mod, _load(mod, "", ""))
    pins = {(fn, tuple(sorted(kw.items()))) for *_, ps in MUTANTS for fn, kw in ps}
    failed = [fn.__name__ for fn, kw in pins if _fails(fn, dict(kw))]
    assert not failed, f"pins fail on the unedited oracle loaded as a copy: {failed}"

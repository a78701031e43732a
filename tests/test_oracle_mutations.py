"""Planted mistakes in the CPU oracle: every mutant below is a plausible slip in one
oracle function (a dropped term, a wrong sign or comparison, an off-by-one, a wrong
head mapping, a wrong rounding rule, a transposed operand), patched in for one test.
The pins in test_oracle_pins.py must catch each of them: at least one of the pins
listed with the mutant fails while it is in place.  CPU only; nothing here touches the
HIP library.
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle
import oracle.kvp_oracle as ko
import test_oracle_pins as pins

orig = {name: getattr(ko, name) for name in dir(ko) if callable(getattr(ko, name))}


# ---------------------------------------------------------------- mutants


def m_linear_no_bias(x, W, c=None, chunk=4096):
    return orig["score_linear"](x, W, None, chunk)


def m_linear_bias_subtracted(x, W, c=None, chunk=4096):
    s = orig["score_linear"](x, W, None, chunk)
    return s if c is None else s - np.asarray(c, dtype=np.float64)[None, :, None]


def m_linear_token_axis_swapped(x, W, c=None, chunk=4096):
    s = orig["score_linear"](x, W, c, chunk)
    return s[:, :, ::-1].copy()  # scores assigned to the wrong tokens


def m_gelu_tanh(a):
    return 0.5 * a * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (a + 0.044715 * a ** 3)))


def m_gelu_sign(a):
    return 0.5 * a * (1.0 - scipy.special.erf(a / math.sqrt(2.0)))


def m_mlp_no_b1(x, W1, b1, W2, b2, chunk=2048):
    return orig["score_mlp"](x, W1, None, W2, b2, chunk)


def m_mlp_no_b2(x, W1, b1, W2, b2, chunk=2048):
    return orig["score_mlp"](x, W1, b1, W2, None, chunk)


def m_mlp_relu(x, W1, b1, W2, b2, chunk=2048):
    a = np.matmul(x, W1.T) + (0 if b1 is None else b1)
    o = np.matmul(np.maximum(a, 0.0), W2.T) + (0 if b2 is None else b2)
    return o.transpose(0, 2, 1)


def m_quantile_wrong_tail(s, q):
    return orig["threshold_quantile"](s, 1.0 - q)


def m_quantile_nearest(s, q):
    return np.float32(np.quantile(np.asarray(s, dtype=np.float64).ravel(), q, method="nearest"))


def m_keep_window_off_by_one(s, tau, R):
    T = s.shape[-1]
    t = np.arange(T)
    return (np.asarray(s, dtype=np.float64) >= np.float64(tau)) | (t > T - R)


def m_keep_strict(s, tau, R):
    T = s.shape[-1]
    t = np.arange(T)
    return (np.asarray(s, dtype=np.float64) > np.float64(tau)) | (t >= T - R)


def m_keep_no_window(s, tau, R):
    return np.asarray(s, dtype=np.float64) >= np.float64(tau)


def m_partition_unstable(keep_row):
    kept, evicted = orig["partition_indices"](keep_row)
    return kept[::-1].copy(), evicted


def m_attend_no_scale(q, K, V, scale):
    return orig["attend_one"](q, K, V, 1.0)


def m_attend_max_normalised(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(q.shape[0])
    logits = (K @ q) * np.float64(scale)
    e = np.exp(logits - logits.max())
    return (e @ V) / e.max()


def m_attend_keys_as_values(q, K, V, scale):
    return orig["attend_one"](q, K, K, scale)


def m_gqa_interleaved(q, K, V, visible, scale):
    B, Hq, d = q.shape
    Hkv = K.shape[1]
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for j in range(Hq):
            h = j % Hkv
            idx = np.flatnonzero(visible[b, h])
            out[b, j] = orig["attend_one"](q[b, j], K[b, h, idx], V[b, h, idx], scale)
    return out


def m_sm_scale_inverse_d(d):
    return np.float32(1.0 / d)


def m_dms_delay_off_by_one(flags, p, w):
    t = np.arange(p + 1)
    return (~flags[..., :p + 1]) | (p - t <= w)


def m_dms_flag_on_zero(s):
    return ~(np.asarray(s, dtype=np.float64) > 0.0)


def m_prefill_no_self(keep, W):
    v = orig["prefill_visible"](keep, W)
    T = v.shape[-1]
    return v & ~np.eye(T, dtype=bool)


def m_prefill_window_off_by_one(keep, W):
    keep = np.asarray(keep, dtype=bool)
    T = keep.shape[-1]
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    return (j <= i) & (keep[..., None, :] | ((i - j) <= W))


def m_quant_qmax_plus_one(x, qmax):
    return orig["quantize_absmax"](x, qmax + 1)


def m_quant_half_away(x, qmax):
    xf = np.asarray(x, dtype=np.float32)
    a = np.float32(np.max(np.abs(xf))) if xf.size else np.float32(0)
    scale = np.float32(a / np.float32(qmax))
    if scale == 0:
        return np.zeros(xf.shape, dtype=np.int8), np.float32(0.0)
    y = xf / scale
    codes = np.clip(np.sign(y) * np.floor(np.abs(y) + 0.5), -qmax, qmax).astype(np.int8)
    return codes, scale


def m_quant_truncate(x, qmax):
    xf = np.asarray(x, dtype=np.float32)
    a = np.float32(np.max(np.abs(xf))) if xf.size else np.float32(0)
    scale = np.float32(a / np.float32(qmax))
    if scale == 0:
        return np.zeros(xf.shape, dtype=np.int8), np.float32(0.0)
    return np.clip(np.trunc(xf / scale), -qmax, qmax).astype(np.int8), scale


def m_beacon_v_left_exact(K, V, beacon, bits=8):
    Kh, Vh, codes = orig["beacon_kv"](K, V, beacon, bits)
    return Kh, np.array(V, dtype=np.float64, copy=True), codes


def m_beacon_v_with_k_scale(K, V, beacon, bits=8):
    Kh, Vh, (kc, ks, vc, vs) = orig["beacon_kv"](K, V, beacon, bits)
    Vh = np.array(V, dtype=np.float64, copy=True)
    dem = ~beacon
    Vh[dem] = vc[dem].astype(np.float64) * ks[dem][:, None].astype(np.float64)
    return Kh, Vh, (kc, ks, vc, vs)


def m_beacon_mask_inverted(K, V, beacon, bits=8):
    return orig["beacon_kv"](K, V, ~np.asarray(beacon, dtype=bool), bits)


def m_fp8_truncate(x):
    xf = np.asarray(x, dtype=np.float32)
    a = np.abs(xf).astype(np.float64)
    sign = np.where(np.signbit(xf), 0x80, 0).astype(np.int64)
    out = np.zeros(xf.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    out[sub] = np.floor(a[sub] * 2.0 ** 9).astype(np.int64)
    mant, ex = np.frexp(a[~sub])
    out[~sub] = ((ex - 1 + 7) << 3) + np.floor((mant * 2.0 - 1.0) * 8.0).astype(np.int64)
    out = np.where(a >= 448.0, 0x7E, np.minimum(out, 0x7E))
    return (sign | out).astype(np.uint8)


def m_fp8_subnormal_as_normal(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e, m = (c >> 3) & 0xF, (c & 0x7).astype(np.float64)
    val = sign * np.ldexp(1.0 + m / 8.0, (np.maximum(e, 1) - 7).astype(np.int64))
    return np.where((c & 0x7F) == 0x7F, np.nan, np.where((c & 0x7F) == 0, 0.0, val))


def m_fp8_scale_127(x):
    xf = np.asarray(x, dtype=np.float32)
    a = np.float32(np.max(np.abs(xf))) if xf.size else np.float32(0)
    scale = np.float32(a / np.float32(127.0))
    if scale == 0:
        return np.zeros(xf.shape, dtype=np.uint8), np.float32(0.0)
    return ko.fp8_e4m3_encode(xf / scale), scale


# (oracle function, mutant, pins that must catch it: (test function, kwargs))
P = pins
MUTANTS = [
    ("score_linear", m_linear_no_bias, [(P.test_score_linear_brute_force, {})]),
    ("score_linear", m_linear_bias_subtracted, [(P.test_score_linear_brute_force, {})]),
    ("score_linear", m_linear_token_axis_swapped, [(P.test_score_linear_brute_force, {})]),
    ("gelu_erf", m_gelu_tanh, [(P.test_gelu_erf_values, {}), (P.test_score_mlp_vs_torch_fp64, {})]),
    ("gelu_erf", m_gelu_sign, [(P.test_gelu_erf_values, {}), (P.test_score_mlp_vs_torch_fp64, {})]),
    ("score_mlp", m_mlp_no_b1, [(P.test_score_mlp_vs_torch_fp64, {})]),
    ("score_mlp", m_mlp_no_b2, [(P.test_score_mlp_vs_torch_fp64, {})]),
    ("score_mlp", m_mlp_relu, [(P.test_score_mlp_vs_torch_fp64, {})]),
    ("threshold_quantile", m_quantile_wrong_tail,
     [(P.test_threshold_keep_count, {"q": 0.75}), (P.test_threshold_is_the_linear_sample_quantile, {"n": 7, "q": 0.25})]),
    ("threshold_quantile", m_quantile_nearest,
     [(P.test_threshold_is_the_linear_sample_quantile, {"n": 7, "q": 0.25}),
      (P.test_threshold_is_the_linear_sample_quantile, {"n": 10, "q": 0.9})]),
    ("keep_mask", m_keep_window_off_by_one, [(P.test_keep_mask_brute_force_and_special_cases, {})]),
    ("keep_mask", m_keep_strict, [(P.test_keep_mask_brute_force_and_special_cases, {})]),
    ("keep_mask", m_keep_no_window, [(P.test_keep_mask_brute_force_and_special_cases, {})]),
    ("partition_indices", m_partition_unstable, [(P.test_partition_matches_boolean_indexing, {})]),
    ("attend_one", m_attend_no_scale, [(P.test_attention_brute_force_mpmath, {})]),
    ("attend_one", m_attend_max_normalised, [(P.test_attention_brute_force_mpmath, {})]),
    ("attend_one", m_attend_keys_as_values, [(P.test_attention_brute_force_mpmath, {})]),
    ("decode_attention", m_gqa_interleaved, [(P.test_gqa_head_mapping_is_contiguous, {})]),
    ("sm_scale", m_sm_scale_inverse_d, [(P.test_softmax_scale_is_the_sdpa_default, {})]),
    ("dms_visible", m_dms_delay_off_by_one, [(P.test_dms_hand_built_sequence, {})]),
    ("dms_evict_flags", m_dms_flag_on_zero, [(P.test_dms_hand_built_sequence, {})]),
    ("prefill_visible", m_prefill_no_self,
     [(P.test_prefill_visible_rows_match_the_decode_rules, {}),
      (P.test_prefill_attention_equals_masked_sdpa_and_special_cases, {})]),
    ("prefill_visible", m_prefill_window_off_by_one,
     [(P.test_prefill_visible_rows_match_the_decode_rules, {}),
      (P.test_prefill_attention_equals_masked_sdpa_and_special_cases, {})]),
    ("quantize_absmax", m_quant_qmax_plus_one,
     [(P.test_int8_roundtrip_bound_and_extremes, {}), (P.test_int4_roundtrip_bound_extremes_and_brute_force, {})]),
    ("quantize_absmax", m_quant_half_away,
     [(P.test_int8_on_grid_inputs_are_exact_and_round_half_even, {}),
      (P.test_int4_on_grid_inputs_are_exact_and_round_half_even, {})]),
    ("quantize_absmax", m_quant_truncate,
     [(P.test_int8_roundtrip_bound_and_extremes, {}), (P.test_int8_codes_match_brute_force, {})]),
    ("beacon_kv", m_beacon_v_left_exact,
     [(P.test_beacon_round_trip_of_k_and_v_halves, {"bits": 8}),
      (P.test_beacon_round_trip_of_k_and_v_halves, {"bits": 4})]),
    ("beacon_kv", m_beacon_v_with_k_scale, [(P.test_beacon_round_trip_of_k_and_v_halves, {"bits": 8})]),
    ("beacon_kv", m_beacon_mask_inverted,
     [(P.test_beacon_round_trip_of_k_and_v_halves, {"bits": 8}),
      (P.test_beacon_all_beacons_is_dense_and_demotion_changes_output, {})]),
    ("beacon_kv", m_beacon_v_left_exact, [(P.test_beacon_fp8_round_trip_of_k_and_v_halves, {})]),
    ("fp8_e4m3_encode", m_fp8_truncate,
     [(P.test_fp8_encode_rounds_to_nearest_even, {}), (P.test_fp8_encode_round_trips_every_code, {})]),
    ("fp8_e4m3_decode", m_fp8_subnormal_as_normal,
     [(P.test_fp8_decode_every_code_matches_library, {}), (P.test_fp8_encode_round_trips_every_code, {})]),
    ("quantize_absmax_fp8", m_fp8_scale_127,
     [(P.test_fp8_absmax_quantization_bound_and_extremes, {}),
      (P.test_beacon_fp8_round_trip_of_k_and_v_halves, {})]),
]


@pytest.mark.parametrize("name,mutant,catchers", MUTANTS,
                         ids=[f"{n}-{m.__name__}" for n, m, _ in MUTANTS])
def test_pins_catch_planted_mistake(monkeypatch, name, mutant, catchers):
    # the pins first pass on the oracle as it stands ...
    for pin, kw in catchers:
        pin(**kw)
    # ... and with the mistake planted (in the module and in the package namespace, so
    # calls between oracle functions see it too) at least one of them fails
    monkeypatch.setattr(ko, name, mutant)
    monkeypatch.setattr(oracle, name, mutant)
    caught = []
    for pin, kw in catchers:
        try:
            pin(**kw)
        except Exception as e:  # an assertion or a shape error both expose the mutant
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"no pin caught the planted mistake {mutant.__name__} in oracle.{name}"

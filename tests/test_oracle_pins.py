"""Pins of the CPU oracle against things other than itself: figures the pages print,
closed forms, brute force (explicit loops, 50-digit mpmath), library routines (torch
fp64 Linear/GELU/SDPA) and special cases that reduce to textbook attention.

Each test is chosen so that a plausible slip in the oracle (a dropped bias, a wrong
sign, an off-by-one in the recent window, a transposed operand, a wrong GQA head
mapping, a wrong rounding mode) fails at least one of them.
"""
import json
import math
import os

import mpmath
import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ------------------------------------------------------------------ page figures


def test_kv_footprint_matches_page_figure():
    g = golden()["llama1_65b_kv_cache_128k_tokens_GB"]
    a = g["assumption"]
    got = oracle.kv_cache_bytes(a["layers"], a["kv_heads"], a["head_dim"],
                                a["bytes_per_elem"], a["tokens"]) / 1e9
    assert abs(got - g["value"]) / g["value"] < g["rel_tol"]
    # linear in tokens (the DMS page's reading; the BeaconKV page's "exponential" is
    # a translation slip)
    assert oracle.kv_cache_bytes(80, 64, 128, 2, 2 * a["tokens"]) == 2 * oracle.kv_cache_bytes(
        80, 64, 128, 2, a["tokens"])


def _qwen3_8b_projection_macs(a):
    H, hd, ffn = a["hidden"], a.get("head_dim", 128), a.get("ffn", 12288)
    qh, kvh = a.get("q_heads", 32), a["kv_heads"]
    attn = H * qh * hd + 2 * H * kvh * hd + qh * hd * H
    mlp = 3 * H * ffn
    return attn + mlp


def test_scorer_overhead_matches_page_figures():
    g = golden()
    a = g["kvzap_mlp_overhead_percent_of_projection_flops"]["assumption"]
    proj = _qwen3_8b_projection_macs(a)
    mlp = 100.0 * oracle.scorer_macs("mlp", a["hidden"], a["mlp_inner"], a["kv_heads"]) / proj
    lin = 100.0 * oracle.scorer_macs("linear", a["hidden"], a["mlp_inner"], a["kv_heads"]) / proj
    gm = g["kvzap_mlp_overhead_percent_of_projection_flops"]
    gl = g["kvzap_linear_overhead_percent_of_projection_flops"]
    assert abs(mlp - gm["value"]) < gm["abs_tol"], mlp
    assert abs(lin - gl["value"]) < gl["abs_tol"], lin
    # the figures single out inner width 512 and one output per KV head
    assert abs(100.0 * oracle.scorer_macs("mlp", 4096, 1024, 8) / proj - 1.1) > 0.5
    assert abs(100.0 * oracle.scorer_macs("linear", 4096, 512, 32) / proj - 0.02) > 0.03


# ------------------------------------------------------------------ input bits


def test_bf16_decoding_exact():
    vals = torch.tensor([1.0, -2.5, 3.140625, 0.0, -0.0, 65280.0, 1e-3], dtype=torch.bfloat16)
    bits = vals.view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    assert np.array_equal(got, vals.float().double().numpy())
    assert oracle.as_f64(bits).dtype == np.float64


# ------------------------------------------------------------------ scoring


def test_score_linear_brute_force():
    rng = np.random.default_rng(1)
    B, T, H, Hkv = 2, 5, 7, 3
    x = rng.standard_normal((B, T, H))
    W = rng.standard_normal((Hkv, H))
    c = rng.standard_normal(Hkv)
    s = oracle.score_linear(x, W, c, chunk=2)
    for b in range(B):
        for h in range(Hkv):
            for t in range(T):
                acc = c[h]
                for i in range(H):
                    acc += x[b, t, i] * W[h, i]
                assert abs(s[b, h, t] - acc) < 1e-12
    assert s.shape == (B, Hkv, T)


def test_gelu_erf_values():
    # closed forms from the error function at 50 digits
    for a in (-3.0, -1.0, -0.25, 0.0, 0.5, 1.0, 2.0):
        ref = mpmath.mpf(0.5) * a * (1 + mpmath.erf(mpmath.mpf(a) / mpmath.sqrt(2)))
        assert abs(float(oracle.gelu_erf(np.array([a]))[0]) - float(ref)) < 1e-15
    # and it is not the tanh approximation
    a = 1.0
    tanh_form = 0.5 * a * (1 + math.tanh(math.sqrt(2 / math.pi) * (a + 0.044715 * a ** 3)))
    assert abs(float(oracle.gelu_erf(np.array([a]))[0]) - tanh_form) > 1e-5


def test_score_mlp_vs_torch_fp64():
    rng = np.random.default_rng(2)
    B, T, H, inner, Hkv = 2, 9, 16, 12, 3
    x = rng.standard_normal((B, T, H))
    W1 = rng.standard_normal((inner, H)) / 4
    b1 = rng.standard_normal(inner)
    W2 = rng.standard_normal((Hkv, inner)) / 3
    b2 = rng.standard_normal(Hkv)
    s = oracle.score_mlp(x, W1, b1, W2, b2, chunk=4)
    l1 = torch.nn.Linear(H, inner).double()
    l2 = torch.nn.Linear(inner, Hkv).double()
    with torch.no_grad():
        l1.weight.copy_(torch.from_numpy(W1)); l1.bias.copy_(torch.from_numpy(b1))
        l2.weight.copy_(torch.from_numpy(W2)); l2.bias.copy_(torch.from_numpy(b2))
        ref = l2(torch.nn.functional.gelu(l1(torch.from_numpy(x)), approximate="none"))
    assert np.allclose(s, ref.numpy().transpose(0, 2, 1), atol=1e-12, rtol=0)
    # biases are not dropped
    s0 = oracle.score_mlp(x, W1, None, W2, None)
    assert np.abs(s - s0).max() > 1e-3


# ------------------------------------------------------------------ threshold


@pytest.mark.parametrize("q", [0.5, 0.75, 0.9])
def test_threshold_keep_count(q):
    rng = np.random.default_rng(3)
    s = rng.standard_normal((2, 4, 1001))
    tau = oracle.threshold_quantile(s, q)
    n = s.size
    kept = int((s >= np.float64(tau)).sum())
    assert abs(kept - math.ceil((1 - q) * n)) <= 1
    assert tau.dtype == np.float32
    assert float(tau) == float(np.float32(np.quantile(s.ravel(), q)))


def _quantile_by_definition(values, q):
    """The 'linear' sample quantile written out: sort, v = (n - 1) q, interpolate
    between the order statistics at floor(v) and floor(v) + 1 (Hyndman & Fan's
    definition 7)."""
    a = sorted(float(x) for x in values)
    v = (len(a) - 1) * q
    i = math.floor(v)
    if i >= len(a) - 1:
        return a[-1]
    return a[i] + (a[i + 1] - a[i]) * (v - i)


@pytest.mark.parametrize("n,q", [(1, 0.3), (2, 0.5), (5, 0.0), (5, 1.0), (7, 0.25), (10, 0.9),
                                 (101, 0.75), (1000, 0.333)])
def test_threshold_is_the_linear_sample_quantile(n, q):
    rng = np.random.default_rng(n)
    s = np.round(rng.standard_normal(n) * 4) / 4  # ties included
    tau = oracle.threshold_quantile(s, q)
    want = _quantile_by_definition(s, q)
    assert abs(float(tau) - want) <= 1e-6 * max(1.0, abs(want))
    assert tau == np.float32(want) or abs(float(tau) - float(np.float32(want))) <= \
        np.spacing(np.float32(want))


# ------------------------------------------------------------------ mask


def _mask_loop(s, tau, R):
    T = s.shape[-1]
    out = np.zeros(s.shape, dtype=bool)
    for idx in np.ndindex(s.shape[:-1]):
        for t in range(T):
            recent = t > T - 1 - R
            out[idx + (t,)] = recent or (s[idx + (t,)] >= tau)
    return out


def test_keep_mask_brute_force_and_special_cases():
    rng = np.random.default_rng(4)
    s = rng.standard_normal((2, 3, 300))
    s[0, 0, 5] = np.nan
    s[1, 2, 290] = np.nan  # recent -> kept anyway
    tau = 0.3
    m = oracle.keep_mask(s, tau, 128)
    assert np.array_equal(m, _mask_loop(s, tau, 128))
    assert not m[0, 0, 5] and m[1, 2, 290]
    # tau = -inf: everything (except NaN outside the window) is kept
    s2 = rng.standard_normal((2, 3, 300))
    assert oracle.keep_mask(s2, -np.inf, 128).all()
    # tau = +inf: exactly the last R positions
    mi = oracle.keep_mask(s2, np.inf, 128)
    assert mi.sum(-1).tolist() == [[128] * 3] * 2
    assert mi[..., -128:].all() and not mi[..., :-128].any()
    # T <= R keeps all
    assert oracle.keep_mask(rng.standard_normal((1, 1, 100)), np.inf, 128).all()
    # an equal score is kept (s >= tau)
    s3 = np.array([[[0.5, 0.25, 1.0] + [0.0] * 200]])
    assert oracle.keep_mask(s3, 0.5, 128)[0, 0, 0]
    assert not oracle.keep_mask(s3, 0.5, 128)[0, 0, 1]


def test_partition_matches_boolean_indexing():
    rng = np.random.default_rng(5)
    keep = rng.random(257) < 0.3
    K = rng.standard_normal((257, 4))
    kept, ev = oracle.partition_indices(keep)
    assert np.array_equal(K[kept], K[keep])
    assert np.array_equal(K[ev], K[~keep])
    assert np.all(np.diff(kept) > 0) and np.all(np.diff(ev) > 0)
    assert len(kept) == int(keep.sum())  # count == popcount
    assert sorted(np.concatenate([kept, ev]).tolist()) == list(range(257))


# ------------------------------------------------------------------ attention


def _mp_attend(q, K, V, scale):
    mpmath.mp.dps = 50
    logits = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(a) * mpmath.mpf(b)
                                             for a, b in zip(k, q)) for k in K]
    m = max(logits)
    e = [mpmath.exp(x - m) for x in logits]
    z = mpmath.fsum(e)
    return [float(mpmath.fsum(e[i] * mpmath.mpf(V[i][c]) for i in range(len(e))) / z)
            for c in range(len(V[0]))]


def test_attention_brute_force_mpmath():
    rng = np.random.default_rng(6)
    q = rng.standard_normal(5)
    K = rng.standard_normal((7, 5)) * 3
    V = rng.standard_normal((7, 5))
    scale = float(oracle.sm_scale(5))
    got = oracle.attend_one(q, K, V, scale)
    ref = _mp_attend(q, K, V, scale)
    assert np.allclose(got, ref, atol=1e-13, rtol=0)
    # K and V are not interchangeable
    swapped = oracle.attend_one(q, V, K, scale)
    assert np.abs(swapped - got).max() > 1e-3


def _sdpa_gqa(q, K, V, mask, scale):
    # torch fp64 SDPA on the CPU with expanded KV heads (library routine)
    B, Hq, d = q.shape
    Hkv = K.shape[1]
    g = Hq // Hkv
    Kx = torch.from_numpy(K).repeat_interleave(g, dim=1)
    Vx = torch.from_numpy(V).repeat_interleave(g, dim=1)
    mx = torch.from_numpy(mask).repeat_interleave(g, dim=1)[:, :, None, :]
    qq = torch.from_numpy(q)[:, :, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(qq, Kx, Vx, attn_mask=mx,
                                                         scale=float(scale))
    return o[:, :, 0, :].numpy()


def test_softmax_scale_is_the_sdpa_default():
    # the library routine's own default scale (1/sqrt(d), scale=None) against the fp32
    # value the oracle hands to both paths: equal up to that value's rounding
    rng = np.random.default_rng(71)
    for d in (8, 64, 128):
        B, Hq, Hkv, T = 1, 4, 2, 50
        q = rng.standard_normal((B, Hq, d))
        K = rng.standard_normal((B, Hkv, T, d))
        V = rng.standard_normal((B, Hkv, T, d))
        got = oracle.decode_attention(q, K, V, np.ones((B, Hkv, T), bool), oracle.sm_scale(d))
        Kx = torch.from_numpy(K).repeat_interleave(Hq // Hkv, dim=1)
        Vx = torch.from_numpy(V).repeat_interleave(Hq // Hkv, dim=1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[:, :, None, :], Kx, Vx)[:, :, 0, :].numpy()
        assert np.allclose(got, ref, atol=1e-6, rtol=0), d


def test_dense_special_case_equals_sdpa():
    rng = np.random.default_rng(7)
    B, Hq, Hkv, T, d = 2, 8, 2, 300, 16
    q = rng.standard_normal((B, Hq, d))
    K = rng.standard_normal((B, Hkv, T, d))
    V = rng.standard_normal((B, Hkv, T, d))
    s = rng.standard_normal((B, Hkv, T))
    vis = oracle.keep_mask(s, -np.inf, 128)
    scale = oracle.sm_scale(d)
    got = oracle.decode_attention(q, K, V, vis, scale)
    ref = _sdpa_gqa(q, K, V, np.ones((B, Hkv, T), dtype=bool), scale)
    assert np.allclose(got, ref, atol=1e-12, rtol=0)


def test_sliding_window_special_case_equals_sdpa():
    rng = np.random.default_rng(8)
    B, Hq, Hkv, T, d = 1, 4, 2, 400, 8
    q = rng.standard_normal((B, Hq, d))
    K = rng.standard_normal((B, Hkv, T, d))
    V = rng.standard_normal((B, Hkv, T, d))
    s = rng.standard_normal((B, Hkv, T))
    vis = oracle.keep_mask(s, np.inf, 128)
    scale = oracle.sm_scale(d)
    got = oracle.decode_attention(q, K, V, vis, scale)
    window = np.zeros((B, Hkv, T), dtype=bool)
    window[..., T - 128:] = True  # the last 128 tokens, current one included
    ref = _sdpa_gqa(q, K, V, window, scale)
    assert np.allclose(got, ref, atol=1e-12, rtol=0)
    # and the same as dense attention on just the last 128
    ref2 = oracle.decode_attention(q, K[:, :, -128:], V[:, :, -128:],
                                   np.ones((B, Hkv, 128), bool), scale)
    assert np.allclose(got, ref2, atol=1e-12)


def test_gqa_head_mapping_is_contiguous():
    rng = np.random.default_rng(9)
    B, Hq, Hkv, T, d = 1, 6, 3, 20, 4
    q = rng.standard_normal((B, Hq, d))
    K = rng.standard_normal((B, Hkv, T, d))
    V = np.zeros((B, Hkv, T, d))
    for h in range(Hkv):
        V[0, h] = h + 1.0  # output value identifies the KV head that was read
    out = oracle.decode_attention(q, K, V, np.ones((B, Hkv, T), bool), 0.5)
    assert np.allclose(out[0, :, 0], [1, 1, 2, 2, 3, 3])


def test_attention_invariants():
    rng = np.random.default_rng(10)
    q = rng.standard_normal(8)
    K = rng.standard_normal((50, 8))
    V = rng.standard_normal((50, 8))
    o = oracle.attend_one(q, K, V, 0.3)
    perm = rng.permutation(50)
    assert np.allclose(o, oracle.attend_one(q, K[perm], V[perm], 0.3), atol=1e-14)
    assert np.all(o <= V.max(0) + 1e-12) and np.all(o >= V.min(0) - 1e-12)
    assert np.array_equal(oracle.attend_one(q, K[:0], V[:0], 0.3), np.zeros(8))
    # a single visible token returns its value row exactly
    assert np.allclose(oracle.attend_one(q, K[:1], V[:1], 0.3), V[0])
    # shift invariance of softmax in the logits: adding a constant to every k.q
    # (k -> k + c*q/|q|^2) leaves the output unchanged
    Kc = K + 2.0 * q / (q @ q)
    assert np.allclose(o, oracle.attend_one(q, Kc, V, 0.3), atol=1e-12)


# ------------------------------------------------------------------ DMS


def test_dms_hand_built_sequence():
    # scores: token 0 kept (s>=0), tokens 1,2 flagged, token 3 kept, token 4 flagged
    s = np.array([0.5, -1.0, -0.1, 0.0, -2.0, 1.0, 1.0, 1.0])
    flags = oracle.dms_evict_flags(s)
    assert flags.tolist() == [False, True, True, False, True, False, False, False]
    w = 3
    # token 1 (flagged) is seen by p = 1, 2, 3 and gone from p = 4 on
    assert [bool(oracle.dms_visible(flags, p, w)[1]) for p in range(1, 8)] == \
        [True, True, True, False, False, False, False]
    # token 4 (flagged) seen by p = 4, 5, 6, gone at p = 7
    assert [bool(oracle.dms_visible(flags, p, w)[4]) for p in range(4, 8)] == \
        [True, True, True, False]
    # unflagged tokens never leave
    for p in range(8):
        v = oracle.dms_visible(flags, p, w)
        assert v[0] and (p < 3 or v[3])
        assert len(v) == p + 1


def test_dms_limits_and_equivalence_with_kvzap_mask():
    rng = np.random.default_rng(11)
    s = rng.standard_normal((3, 500)) - 1.15
    flags = oracle.dms_evict_flags(s)
    p = 499
    # w = 0: immediate eviction (only unflagged)
    assert np.array_equal(oracle.dms_visible(flags, p, 0), ~flags)
    # w >= T: dense
    assert oracle.dms_visible(flags, p, 500).all()
    # same set as the KVzap rule with tau = 0 and recent window R = w
    for w in (1, 17, 256):
        for pp in (0, 10, 255, 256, 300, 499):
            assert np.array_equal(oracle.dms_visible(flags, pp, w),
                                  oracle.kvzap_visible_at_decode(s, 0.0, w, pp))


def test_dms_keep_fraction_statistics():
    rng = np.random.default_rng(12)
    T, w = 8192, 256
    s = rng.standard_normal(200 * T).reshape(200, T) + (-1.1503493803760079)
    vis = oracle.dms_visible(oracle.dms_evict_flags(s), T - 1, w)
    n = vis.sum(-1).mean()
    mean = 0.125 * (T - w) + w
    sd = math.sqrt(0.125 * 0.875 * (T - w) / 200)
    assert abs(n - mean) < 5 * sd


# ------------------------------------------------------------------ prefill under eviction


def _sdpa_prefill(q, K, V, mask, scale):
    # torch fp64 SDPA with a [B,Hkv,T,T] boolean mask, KV heads expanded (library routine)
    g = q.shape[1] // K.shape[1]
    Kx = torch.from_numpy(K).repeat_interleave(g, dim=1)
    Vx = torch.from_numpy(V).repeat_interleave(g, dim=1)
    mx = torch.from_numpy(mask).repeat_interleave(g, dim=1)
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), Kx, Vx, attn_mask=mx, scale=float(scale)).numpy()


def test_prefill_visible_rows_match_the_decode_rules():
    rng = np.random.default_rng(30)
    T = 300
    s = rng.standard_normal((2, T)) - 0.8
    tau, R = 0.1, 128
    vis = oracle.prefill_visible(s >= tau, R)
    flags = oracle.dms_evict_flags(s)
    dvis = oracle.prefill_visible(~flags, 17)
    for i in range(T):
        # query position i sees what the decode step at length i + 1 sees
        assert np.array_equal(vis[:, i, :i + 1], oracle.kvzap_visible_at_decode(s, tau, R, i))
        assert not vis[:, i, i + 1:].any()
        assert np.array_equal(dvis[:, i, :i + 1], oracle.dms_visible(flags, i, 17))
        assert not dvis[:, i, i + 1:].any()
    # brute force on a tiny case
    keep = np.array([True, False, False, True, False, False])
    W = 2
    bf = np.zeros((6, 6), bool)
    for i in range(6):
        for j in range(6):
            bf[i, j] = j <= i and (keep[j] or i - j < W)
    assert np.array_equal(oracle.prefill_visible(keep, W), bf)


def test_prefill_attention_equals_masked_sdpa_and_special_cases():
    rng = np.random.default_rng(31)
    B, Hq, Hkv, T, d, W = 2, 6, 2, 90, 8, 16
    q = rng.standard_normal((B, Hq, T, d))
    K = rng.standard_normal((B, Hkv, T, d)) * 2
    V = rng.standard_normal((B, Hkv, T, d))
    keep = rng.random((B, Hkv, T)) < 0.3
    scale = oracle.sm_scale(d)
    got = oracle.prefill_attention(q, K, V, keep, W, scale)
    # a mask built by explicit loops, attention by the library routine
    mask = np.zeros((B, Hkv, T, T), bool)
    for b in range(B):
        for h in range(Hkv):
            for i in range(T):
                for j in range(i + 1):
                    mask[b, h, i, j] = keep[b, h, j] or i - j < W
    assert np.allclose(got, _sdpa_prefill(q, K, V, mask, scale), atol=1e-12, rtol=0)
    # keep-all is causal attention
    allk = np.ones((B, Hkv, T), bool)
    causal = np.broadcast_to(np.tril(np.ones((T, T), bool)), (B, Hkv, T, T)).copy()
    assert np.allclose(oracle.prefill_attention(q, K, V, allk, W, scale),
                       _sdpa_prefill(q, K, V, causal, scale), atol=1e-12, rtol=0)
    # keep-none is a sliding window of W positions (current one included)
    band = causal & (np.arange(T)[:, None] - np.arange(T)[None, :] < W)
    assert np.allclose(oracle.prefill_attention(q, K, V, ~allk, W, scale),
                       _sdpa_prefill(q, K, V, band, scale), atol=1e-12, rtol=0)
    # row i equals one decode step at length i + 1 with its own query
    for i in (0, 1, W - 1, W, 57, T - 1):
        vis = oracle.prefill_visible(keep, W)[:, :, i, :i + 1]
        ref = oracle.decode_attention(q[:, :, i], K[:, :, :i + 1], V[:, :, :i + 1], vis, scale)
        assert np.allclose(got[:, :, i], ref, atol=1e-13, rtol=0)
    # W = 0 and nothing kept: no visible key, a zero row
    z = oracle.prefill_attention(q[:1, :3], K[:1, :1], V[:1, :1], ~allk[:1, :1], 0, scale)
    assert np.array_equal(z, np.zeros_like(z))


# ------------------------------------------------------------------ BeaconKV int8


def test_int8_roundtrip_bound_and_extremes():
    rng = np.random.default_rng(13)
    x = (rng.standard_normal(128) * 3).astype(np.float32)
    codes, scale = oracle.quantize_absmax_int8(x)
    assert scale.dtype == np.float32 and codes.dtype == np.int8
    xh = oracle.dequantize_int8(codes, scale)
    assert np.all(np.abs(x - xh) <= scale / 2 * (1 + 1e-6))
    i = np.argmax(np.abs(x))
    assert abs(int(codes[i])) == 127 and np.sign(codes[i]) == np.sign(x[i])
    assert np.abs(codes).max() == 127
    zc, zs = oracle.quantize_absmax_int8(np.zeros(16, np.float32))
    assert zs == 0 and not zc.any()


def test_int8_on_grid_inputs_are_exact_and_round_half_even():
    scale = np.float32(0.5)
    codes = np.array([127, -3, 0, 64, -127, 5], dtype=np.int8)
    x = (codes.astype(np.float32) * scale)
    c2, s2 = oracle.quantize_absmax_int8(x)
    assert s2 == scale and np.array_equal(c2, codes)
    assert np.array_equal(oracle.dequantize_int8(c2, s2), x.astype(np.float64))
    # ties go to even: a = 127 -> scale 1; 2.5 -> 2, 3.5 -> 4, -0.5 -> 0
    x = np.array([127.0, 2.5, 3.5, -0.5, -1.5], dtype=np.float32)
    c, s = oracle.quantize_absmax_int8(x)
    assert s == 1.0 and c.tolist() == [127, 2, 4, 0, -2]


def _nearest_code_brute(y: float, qmax: int) -> int:
    """The code nearest to y among -qmax..qmax, ties to the even code (brute force)."""
    best = None
    for c in range(-qmax, qmax + 1):
        key = (abs(y - c), c % 2)  # distance first, then prefer even
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_int4_roundtrip_bound_extremes_and_brute_force():
    rng = np.random.default_rng(15)
    for trial in range(20):
        x = (rng.standard_normal(64) * rng.uniform(0.01, 10)).astype(np.float32)
        codes, scale = oracle.quantize_absmax_int4(x)
        assert scale.dtype == np.float32 and scale == np.float32(np.abs(x).max() / np.float32(7))
        assert np.abs(codes).max() == 7 and codes.min() >= -7
        i = np.argmax(np.abs(x))
        assert abs(int(codes[i])) == 7 and np.sign(codes[i]) == np.sign(x[i])
        xh = oracle.dequantize_int8(codes, scale)
        assert np.all(np.abs(x - xh) <= scale / 2 * (1 + 1e-6))
        # every code is the nearest grid point of the fp32 quotient (brute force)
        y = x / scale
        assert [int(c) for c in codes] == [_nearest_code_brute(float(v), 7) for v in y]
    zc, zs = oracle.quantize_absmax_int4(np.zeros(8, np.float32))
    assert zs == 0 and not zc.any()


def test_int4_on_grid_inputs_are_exact_and_round_half_even():
    scale = np.float32(0.25)
    codes = np.array([7, -3, 0, 1, -7, 5, -6], dtype=np.int8)
    x = codes.astype(np.float32) * scale
    c2, s2 = oracle.quantize_absmax_int4(x)
    assert s2 == scale and np.array_equal(c2, codes)
    # a = 7 -> scale 1; ties go to even: 2.5 -> 2, 3.5 -> 4, -0.5 -> 0, 6.5 -> 6
    x = np.array([7.0, 2.5, 3.5, -0.5, 6.5, -4.5], dtype=np.float32)
    c, s = oracle.quantize_absmax_int4(x)
    assert s == 1.0 and c.tolist() == [7, 2, 4, 0, 6, -4]


def test_int8_codes_match_brute_force():
    rng = np.random.default_rng(16)
    x = (rng.standard_normal(128) * 2).astype(np.float32)
    codes, scale = oracle.quantize_absmax_int8(x)
    y = x / scale
    assert [int(c) for c in codes] == [_nearest_code_brute(float(v), 127) for v in y]


def test_beacon_int4_is_coarser_than_int8_and_all_beacons_is_dense():
    rng = np.random.default_rng(17)
    B, Hq, Hkv, T, d = 1, 4, 2, 64, 16
    q = rng.standard_normal((B, Hq, d))
    K = rng.standard_normal((B, Hkv, T, d)).astype(np.float32).astype(np.float64)
    V = rng.standard_normal((B, Hkv, T, d)).astype(np.float32).astype(np.float64)
    scale = oracle.sm_scale(d)
    allb = np.ones((B, Hkv, T), bool)
    dense = oracle.decode_attention(q, K, V, allb, scale)
    assert np.allclose(oracle.beacon_decode_attention(q, K, V, allb, scale, bits=4), dense, atol=1e-14)
    none = np.zeros((B, Hkv, T), bool)
    e8 = np.abs(oracle.beacon_decode_attention(q, K, V, none, scale, bits=8) - dense).max()
    e4 = np.abs(oracle.beacon_decode_attention(q, K, V, none, scale, bits=4) - dense).max()
    assert 1e-5 < e8 < e4 < 0.5
    # the demoted rows of an int4 round trip are on the row's 15-level grid
    Kh, Vh, (kc, ks, vc, vs) = oracle.beacon_kv(K, V, none, bits=4)
    assert np.abs(kc).max() == 7 and np.abs(vc).max() == 7
    assert np.array_equal(Kh, kc.astype(np.float64) * ks[..., None].astype(np.float64))


def test_beacon_all_beacons_is_dense_and_demotion_changes_output():
    rng = np.random.default_rng(14)
    B, Hq, Hkv, T, d = 1, 4, 2, 64, 16
    q = rng.standard_normal((B, Hq, d))
    K = rng.standard_normal((B, Hkv, T, d)).astype(np.float32).astype(np.float64)
    V = rng.standard_normal((B, Hkv, T, d)).astype(np.float32).astype(np.float64)
    scale = oracle.sm_scale(d)
    allb = np.ones((B, Hkv, T), bool)
    dense = oracle.decode_attention(q, K, V, allb, scale)
    assert np.allclose(oracle.beacon_decode_attention(q, K, V, allb, scale), dense, atol=1e-14)
    none = np.zeros((B, Hkv, T), bool)
    demoted = oracle.beacon_decode_attention(q, K, V, none, scale)
    diff = np.abs(demoted - dense).max()
    assert 1e-5 < diff < 0.1
    # rows on the int8 grid survive demotion exactly
    Kg = np.round(K * 10).clip(-127, 127) / 10.0
    Kg[..., 0] = 12.7  # absmax 12.7 -> scale fp32(0.1)
    Vg = Kg.copy()
    Kh, Vh, _ = oracle.beacon_kv(Kg.astype(np.float32).astype(np.float64),
                                 Vg.astype(np.float32).astype(np.float64), none)
    assert np.abs(Kh - Kg).max() < 1e-6


@pytest.mark.parametrize("bits", [8, 4])
def test_beacon_round_trip_of_k_and_v_halves(bits):
    """BeaconKV briefing, body: beacon entries stay at full precision, every other
    entry is stored at low precision.  Both halves of a demoted row, K and V, are
    replaced by their own codes times their own absmax scale; beacon rows keep their
    exact bits."""
    rng = np.random.default_rng(40 + bits)
    B, Hkv, T, d = 2, 2, 48, 16
    qmax = 127 if bits == 8 else 7
    K = (rng.standard_normal((B, Hkv, T, d)) * 2).astype(np.float32).astype(np.float64)
    V = (rng.standard_normal((B, Hkv, T, d)) * 0.5).astype(np.float32).astype(np.float64)
    beacon = rng.random((B, Hkv, T)) < 0.3
    beacon[0, 0, :5] = True
    beacon[1, 1, -5:] = False
    Kh, Vh, (kc, ks, vc, vs) = oracle.beacon_kv(K, V, beacon, bits=bits)
    # beacon rows: the exact input bits, no codes
    assert np.array_equal(Kh[beacon], K[beacon]) and np.array_equal(Vh[beacon], V[beacon])
    for X, Xh, c, s in ((K, Kh, kc, ks), (V, Vh, vc, vs)):
        dem = ~beacon
        # demoted rows: exactly code * scale of the row's own codes and scale
        assert np.array_equal(Xh[dem], c[dem].astype(np.float64) * s[dem][:, None].astype(np.float64))
        # the scale is the row's own absmax over qmax in fp32, and the absmax element maps to +-qmax
        a = np.abs(X[dem]).max(axis=1).astype(np.float32)
        assert np.array_equal(s[dem], (a / np.float32(qmax)).astype(np.float32))
        assert np.all(np.abs(c[dem]).max(axis=1) == qmax)
        # codes are the nearest grid points of x / scale (brute force over the grid)
        rows = np.flatnonzero(dem.ravel())[:6]
        Xr, cr, sr = X.reshape(-1, d), c.reshape(-1, d), s.ravel()
        for r in rows:
            y = Xr[r].astype(np.float32) / sr[r]
            assert [int(v) for v in cr[r]] == [_nearest_code_brute(float(v), qmax) for v in y]
        # a demoted row really moved, within half a grid step per element
        err = np.abs(Xh[dem] - X[dem])
        assert err.max() > 0
        assert np.all(err <= s[dem][:, None].astype(np.float64) / 2 * (1 + 1e-6))
    # the attention on a mixed mask differs from both the dense and the all-demoted one
    q = rng.standard_normal((B, 4, d))
    sc = oracle.sm_scale(d)
    allv = np.ones((B, Hkv, T), bool)
    mixed = oracle.beacon_decode_attention(q, K, V, beacon, sc, bits=bits)
    assert np.allclose(mixed, oracle.decode_attention(q, Kh, Vh, allv, sc), rtol=0, atol=1e-15)
    assert np.abs(mixed - oracle.decode_attention(q, K, V, allv, sc)).max() > 1e-6


# ---------------------------------------------------------------- fp8 E4M3 pool
# BeaconKV briefing, body: non-beacon entries are kept at low precision.  Reading (one
# of three formats): OCP FP8 E4M3 codes with one fp32 absmax scale per row.


def _torch_fp8_codes(x):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _nearest_fp8_brute(y: float) -> int:
    """Brute force over every finite code: the nearest value, ties to the even code."""
    vals = oracle.fp8_e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    a = abs(y)
    if a >= 448.0:
        k = 0x7E
    else:
        dist = np.abs(vals - a)
        best = np.flatnonzero(dist == dist.min())
        k = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
    return k | (0x80 if np.signbit(np.float32(y)) else 0)


def test_fp8_decode_every_code_matches_library():
    """The 256 E4M3 codes decode to the values of torch.float8_e4m3fn (an independent
    implementation of the OCP format): 0x7F and 0xFF are NaN, 0x7E is 448, 0x08 the
    smallest normal 2^-6, 0x01 the smallest subnormal 2^-9; positive codes ascend."""
    import torch
    c = np.arange(256, dtype=np.uint8)
    d = oracle.fp8_e4m3_decode(c)
    t = torch.from_numpy(c).view(torch.float8_e4m3fn).float().double().numpy()
    assert np.array_equal(np.isnan(d), np.isnan(t))
    assert np.array_equal(d[~np.isnan(d)], t[~np.isnan(t)])
    assert np.flatnonzero(np.isnan(d)).tolist() == [0x7F, 0xFF]
    assert d[0x7E] == 448.0 and d[0x08] == 2.0 ** -6 and d[0x01] == 2.0 ** -9
    assert d[0x80] == 0.0 and np.signbit(d[0x80]) and d[0xFE] == -448.0
    assert np.all(np.diff(d[:0x7F]) > 0)


def test_fp8_encode_round_trips_every_code():
    c = np.arange(256, dtype=np.uint8)
    d = oracle.fp8_e4m3_decode(c)
    ok = ~np.isnan(d)
    assert np.array_equal(oracle.fp8_e4m3_encode(d[ok].astype(np.float32)), c[ok])


def test_fp8_encode_rounds_to_nearest_even():
    """Midpoints between neighbouring codes go to the even code; one fp32 ulp either side
    of a midpoint goes to the nearer code; over random values in the finite range (and
    in the subnormal range) the codes equal torch's float32 -> float8_e4m3fn cast and a
    brute-force nearest-code search."""
    c = np.arange(0x7F, dtype=np.uint8)
    v = oracle.fp8_e4m3_decode(c)
    mid = ((v[:-1] + v[1:]) / 2).astype(np.float32)  # exact in fp32
    assert np.array_equal(oracle.fp8_e4m3_encode(mid), np.where(c[:-1] % 2 == 0, c[:-1], c[1:]))
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(0))
    assert np.array_equal(oracle.fp8_e4m3_encode(up), c[1:])
    assert np.array_equal(oracle.fp8_e4m3_encode(dn), c[:-1])
    rng = np.random.default_rng(7)
    xs = np.concatenate([mid, up, dn, rng.uniform(-447.9, 447.9, 20000).astype(np.float32),
                         rng.uniform(-2.0 ** -6, 2.0 ** -6, 5000).astype(np.float32)])
    xs = np.concatenate([xs, -xs]).astype(np.float32)
    assert np.array_equal(oracle.fp8_e4m3_encode(xs), _torch_fp8_codes(xs))
    for y in xs[::997]:
        assert int(oracle.fp8_e4m3_encode(np.array([y]))[0]) == _nearest_fp8_brute(float(y))


def test_fp8_saturation_reading():
    """Reading: magnitudes at or above 448 saturate to +-448 (the library cast turns
    those past the last midpoint into NaN); the absmax scaling never produces them."""
    x = np.array([448.0, np.nextafter(np.float32(448.0), np.float32(1e9)), 463.9, 464.0, 500.0,
                  1e30, -500.0, -1e30], dtype=np.float32)
    assert oracle.fp8_e4m3_encode(x).tolist() == [0x7E] * 6 + [0xFE] * 2


def test_fp8_absmax_quantization_bound_and_extremes():
    """scale = fp32(max |x| / 448); the largest element maps to +-448; every element is
    within half a code step of its value (2^-4 relative above 2^-6 scale, 2^-10 scale
    below); a zero row has scale 0 and zero codes."""
    rng = np.random.default_rng(17)
    for mag in (1e-3, 0.7, 3.0, 250.0, 3e4):
        x = (rng.standard_normal(128) * mag).astype(np.float32)
        x[5] = np.float32(0.0)
        c, s = oracle.quantize_absmax_fp8(x)
        a = np.float32(np.abs(x).max())
        assert s == np.float32(a / np.float32(448.0))
        assert int(c[np.argmax(np.abs(x))]) & 0x7F == 0x7E
        assert int(c[5]) & 0x7F == 0
        xh = oracle.dequantize_fp8(c, s)
        xd = x.astype(np.float64)
        tol = np.maximum(2.0 ** -4 * np.abs(xd), 2.0 ** -10 * float(s)) * (1 + 1e-6)
        assert np.all(np.abs(xh - xd) <= tol)
        assert np.array_equal(c, oracle.fp8_e4m3_encode(x / s))
    c, s = oracle.quantize_absmax_fp8(np.zeros(16, np.float32))
    assert s == 0 and not c.any()


def test_beacon_fp8_round_trip_of_k_and_v_halves():
    """BeaconKV with fp8 codes: beacon rows exact; a demoted K or V row is exactly the
    values of its own codes times its own scale, the codes are the brute-force nearest
    codes of x / scale, and the mixed-mask attention differs from the dense one."""
    rng = np.random.default_rng(44)
    B, Hkv, T, d = 2, 2, 40, 16
    K = (rng.standard_normal((B, Hkv, T, d)) * 2).astype(np.float32).astype(np.float64)
    V = (rng.standard_normal((B, Hkv, T, d)) * 0.5).astype(np.float32).astype(np.float64)
    beacon = rng.random((B, Hkv, T)) < 0.3
    Kh, Vh, (kc, ks, vc, vs) = oracle.beacon_kv(K, V, beacon, bits="fp8")
    assert np.array_equal(Kh[beacon], K[beacon]) and np.array_equal(Vh[beacon], V[beacon])
    dem = ~beacon
    for X, Xh, c, s in ((K, Kh, kc, ks), (V, Vh, vc, vs)):
        vals = oracle.fp8_e4m3_decode(c[dem])
        assert np.array_equal(Xh[dem], vals * s[dem][:, None].astype(np.float64))
        a = np.abs(X[dem]).max(axis=1).astype(np.float32)
        assert np.array_equal(s[dem], (a / np.float32(448.0)).astype(np.float32))
        Xr, cr, sr = X.reshape(-1, d), c.reshape(-1, d), s.ravel()
        for r in np.flatnonzero(dem.ravel())[:5]:
            y = Xr[r].astype(np.float32) / sr[r]
            assert [int(v) for v in cr[r]] == [_nearest_fp8_brute(float(v)) for v in y]
        assert np.abs(Xh[dem] - X[dem]).max() > 0
    q = rng.standard_normal((B, 4, d))
    sc = oracle.sm_scale(d)
    allv = np.ones((B, Hkv, T), bool)
    mixed = oracle.beacon_decode_attention(q, K, V, beacon, sc, bits="fp8")
    assert np.allclose(mixed, oracle.decode_attention(q, Kh, Vh, allv, sc), rtol=0, atol=1e-15)
    assert np.abs(mixed - oracle.decode_attention(q, K, V, allv, sc)).max() > 1e-6

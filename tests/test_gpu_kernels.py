"""Kernel-level parity of the HIP path (through the C ABI) against the CPU oracle.

Sizes span several tiles and ragged tails; pools are poison-filled (NaN / sentinel
ints) so unwritten or over-read elements show up.  Integer and byte results are
compared bit-exactly; scores within a stated absolute bound; attention outputs with
the parity tolerances (max-abs 2e-3 for bf16 KV, 1e-5 relative per output vector
for fp32 KV).
"""
import math

import numpy as np
import pytest
import torch

import kvp_workloads as W
import oracle
from kvp_testlib import (band_mask, check_attention, f64, np_bits, read_pool, read_pool8,
                         read_ring, unpack_bits, visible_positions)

pytestmark = pytest.mark.gpu
DEV = "cuda"

# fp32 score error bound: the band around tau is 1e-4, scores must agree well inside it
SCORE_ATOL = 2.5e-5


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_decode_attention_kvzap_amd as K
    K.load()
    return K


def seeded(shape, seed, dtype=torch.float32, scale=1.0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV) * scale).to(dtype)


def upload_selection(keep: np.ndarray):
    P, T = keep.shape
    idx = np.zeros((P, T), np.int32)
    cnt = np.zeros(P, np.int32)
    for p in range(P):
        k, e = oracle.partition_indices(keep[p])
        idx[p] = np.concatenate([k, e])
        cnt[p] = len(k)
    return torch.from_numpy(idx).to(DEV), torch.from_numpy(cnt).to(DEV)


def select_on_gpu(K, scores, T, tau, R):
    B, Hkv, _ = scores.shape
    P = B * Hkv
    bits = torch.full((P, (T + 31) // 32), -1, dtype=torch.int32, device=DEV)
    idx = torch.full((P, T), -5, dtype=torch.int32, device=DEV)
    cnt = torch.full((P,), -5, dtype=torch.int32, device=DEV)
    ws = torch.empty(max(1, K.kvp_select_workspace_size(B, Hkv, T) // 4), dtype=torch.int32,
                     device=DEV)
    K.kvp_select(scores, T, tau, R, bits, idx, cnt, ws)
    return bits, idx, cnt


def compact_ws(K, B, Hkv):
    return torch.empty(K.kvp_compact_workspace_size(B, Hkv) // 4, dtype=torch.int32, device=DEV)


# ---------------------------------------------------------------------------- score


def test_score_linear_f32_tiny_workload(K):
    wl = W.TINY
    x = W.hidden_states(wl, wl.T, DEV)
    sw = W.scorer_weights(wl, DEV)
    sc = K.Scorer(K.KVP_SCORER_LINEAR, sw.W1, sw.b1)
    s = torch.full((wl.B, wl.Hkv, wl.T), float("nan"), device=DEV)
    K.kvp_score(sc, x, s)
    ref = oracle.score_linear(f64(x), f64(sw.W1), f64(sw.b1))
    err = np.abs(s.cpu().double().numpy() - ref).max()
    assert err < SCORE_ATOL, err


@pytest.mark.parametrize("B,T,H,Hkv,ld", [(2, 300, 512, 8, 300), (3, 77, 256, 2, 80),
                                          (1, 1, 64, 1, 1), (2, 1000, 1024, 16, 1003),
                                          (16, 1, 4096, 8, 1), (4, 16, 8192, 8, 20),
                                          (64, 1, 4096, 8, 1)])
def test_score_linear_bf16(K, B, T, H, Hkv, ld):
    x = seeded((B, T, H), 1, torch.bfloat16)
    Wt = seeded((Hkv, H), 2, torch.bfloat16, 1 / math.sqrt(H))
    c = seeded((Hkv,), 3)
    sc = K.Scorer(K.KVP_SCORER_LINEAR, Wt, c)
    s = torch.full((B, Hkv, ld), float("nan"), device=DEV)
    n = K.kvp_score_workspace_size(sc, B, T)
    ws = torch.empty(max(1, n // 4), dtype=torch.float32, device=DEV) if n else None
    K.kvp_score(sc, x, s, ws)
    ref = oracle.score_linear(f64(x), f64(Wt), f64(c))
    got = s[..., :T].cpu().double().numpy()
    assert np.abs(got - ref).max() < SCORE_ATOL
    if ld > T:
        assert torch.isnan(s[..., T:]).all()  # padding untouched


@pytest.mark.parametrize("B,T,H,inner,Hkv,bias", [
    (2, 300, 256, 512, 8, True), (1, 513, 128, 256, 4, True), (3, 17, 64, 512, 16, True),
    (16, 1, 4096, 512, 8, True), (5, 3, 512, 256, 3, True), (64, 1, 1024, 1024, 16, True),
    (2, 77, 192, 768, 1, False),   # three K stages (the fewest with W2 / b1 staged in LDS), no bias
    (1, 300, 320, 256, 16, True),  # 16 heads: every W2 copy block holds a row
    (2, 200, 192, 256, 5, True)])
def test_score_mlp_bf16(K, B, T, H, inner, Hkv, bias):
    x = seeded((B, T, H), 11, torch.bfloat16)
    W1 = seeded((inner, H), 12, torch.bfloat16, 1 / math.sqrt(H))
    b1 = seeded((inner,), 13, scale=0.5) if bias else None
    W2 = seeded((Hkv, inner), 14, scale=1 / math.sqrt(inner))
    b2 = seeded((Hkv,), 15)
    sc = K.Scorer(K.KVP_SCORER_MLP, W1, b1, W2, b2)
    ws = torch.empty(K.kvp_score_workspace_size(sc, B, T) // 4, dtype=torch.float32, device=DEV)
    s = torch.full((B, Hkv, T), float("nan"), device=DEV)
    K.kvp_score(sc, x, s, ws)
    s2 = torch.full((B, Hkv, T), float("nan"), device=DEV)
    K.kvp_score(sc, x, s2, ws)
    assert torch.equal(s, s2)  # deterministic
    ref = oracle.score_mlp(f64(x), f64(W1), f64(b1) if bias else None, f64(W2), f64(b2))
    err = np.abs(s.cpu().double().numpy() - ref).max()
    assert err < SCORE_ATOL, err


# ---------------------------------------------------------------------------- select


@pytest.mark.parametrize("B,Hkv,T,ld,q,R", [(3, 5, 5000, 5003, 0.6, 128), (1, 1, 1, 1, 0.5, 128),
                                            (2, 2, 100, 100, 0.9, 128), (1, 4, 2048, 2048, 0.5, 0),
                                            (2, 3, 2049, 2050, 0.25, 256), (1, 2, 131, 131, 0.5, 3)])
def test_select_exact(K, B, Hkv, T, ld, q, R):
    s = seeded((B, Hkv, ld), 21)
    s[0, 0, T // 3] = float("nan")
    tau = float(oracle.threshold_quantile(f64(s)[..., :T], q))
    bits, idx, cnt = select_on_gpu(K, s, T, tau, R)
    keep = oracle.keep_mask(f64(s)[..., :T], np.float32(tau), R).reshape(B * Hkv, T)
    assert np.array_equal(unpack_bits(bits, T), keep)
    words = np_bits(bits).astype(np.uint32)
    if T % 32:
        assert (words[:, -1] >> np.uint32(T % 32) == 0).all()  # tail bits zero
    gi = np_bits(idx)
    gc = np_bits(cnt)
    for p in range(B * Hkv):
        k, e = oracle.partition_indices(keep[p])
        assert gc[p] == len(k)
        assert np.array_equal(gi[p], np.concatenate([k, e]))


@pytest.mark.parametrize("tau", [float("-inf"), float("inf")])
def test_select_limits(K, tau):
    B, Hkv, T = 2, 3, 700
    s = seeded((B, Hkv, T), 22)
    bits, idx, cnt = select_on_gpu(K, s, T, tau, 128)
    c = np_bits(cnt)
    if tau < 0:
        assert (c == T).all()
    else:
        assert (c == 128).all()
        assert (np_bits(idx)[:, :128] == np.arange(T - 128, T)).all()


# ---------------------------------------------------------------------------- compact


@pytest.mark.parametrize("dtype,d,ring_w", [(torch.bfloat16, 128, 0), (torch.bfloat16, 128, 128),
                                            (torch.float32, 64, 128), (torch.bfloat16, 64, 32),
                                            (torch.float32, 128, 0)])
def test_compact_exact(K, dtype, d, ring_w):
    B, Hkv, T = 2, 3, 700
    P = B * Hkv
    k = seeded((B, Hkv, T, d), 31, dtype)
    v = seeded((B, Hkv, T, d), 32, dtype)
    s = seeded((B, Hkv, T), 33)
    R = ring_w if ring_w else 128
    keep = oracle.keep_mask(f64(s), 0.3, R).reshape(P, T)
    idx, cnt = upload_selection(keep)
    kv = K.PagedKV.allocate(P, d, P * (T // 16 + 2), T // 16 + 2, dtype, DEV, poison=True)
    ring = K.Ring.allocate(P, ring_w, d, dtype, DEV, poison=True) if ring_w else None
    K.kvp_compact(k, v, idx, cnt, kv, compact_ws(K, B, Hkv), ring=ring, scores=s)
    assert K.kvp_check(kv) == 0
    kb = np_bits(k).reshape(P, T, d)
    vb = np_bits(v).reshape(P, T, d)
    sb = np_bits(s).reshape(P, T)
    for p in range(P):
        kept = np.flatnonzero(keep[p])
        pool_pos = kept[kept < T - ring_w] if ring_w else kept
        pos, Kp, Vp = read_pool(kv, p)
        assert np.array_equal(pos, pool_pos)
        assert np.array_equal(Kp, kb[p, pool_pos]) and np.array_equal(Vp, vb[p, pool_pos])
        if ring_w:
            rpos, Kr, Vr, Sr = read_ring(ring, p)
            want = kept[kept >= T - ring_w]
            assert np.array_equal(np.sort(rpos), want)
            assert ((rpos % ring_w) == np.flatnonzero(np_bits(ring.pos[p]) >= 0)).all()
            assert np.array_equal(Kr, kb[p, rpos]) and np.array_equal(Vr, vb[p, rpos])
            assert np.array_equal(Sr, sb[p, rpos])


def lp_quant(bits, x):
    """The oracle's codes and scale of one row in the pool's format (8, 4 or "fp8")."""
    if bits == "fp8":
        return oracle.quantize_absmax_fp8(x)
    return oracle.quantize_absmax(x, oracle.LP_QMAX[bits])


def lp_codes_equal(bits, gpu_codes, ref_codes):
    if bits == "fp8":  # E4M3 bytes: compare the bit patterns
        return np.array_equal(np.asarray(gpu_codes).view(np.uint8), np.asarray(ref_codes, np.uint8))
    return np.array_equal(gpu_codes, ref_codes)


@pytest.mark.parametrize("bits,d,dtype", [(8, 128, torch.bfloat16), (4, 128, torch.bfloat16),
                                          (4, 64, torch.bfloat16), (8, 64, torch.bfloat16),
                                          (4, 128, torch.float32), (8, 64, torch.float32),
                                          ("fp8", 128, torch.bfloat16), ("fp8", 64, torch.bfloat16),
                                          ("fp8", 128, torch.float32)])
def test_compact_demote_exact(K, bits, d, dtype):
    B, Hkv, T = 2, 2, 500
    P = B * Hkv
    k = seeded((B, Hkv, T, d), 41, dtype)
    v = seeded((B, Hkv, T, d), 42, dtype, 3.0)
    k[0, 0, 7] = 0  # all-zero row -> scale 0, codes 0
    qmax = 448 if bits == "fp8" else oracle.LP_QMAX[bits]
    # rows whose quotients x / scale sit on or next to rounding boundaries: ties (scale
    # exactly 1: row max = qmax, the rest halfway between neighbouring codes) and, with
    # an inexact scale, x = fp(scale * halfway point) and its neighbours
    if bits == "fp8":
        cv = oracle.fp8_e4m3_decode(np.arange(0x7F, dtype=np.uint8))
        mids = (cv[:-1] + cv[1:]) / 2
        half = np.resize(mids[::-1], d - 1) * np.where(np.arange(d - 1) % 2, -1.0, 1.0)
    else:
        half = (np.arange(d - 1) % (2 * qmax)) - qmax + 0.5
    ties = np.concatenate([[qmax], half]).astype(np.float32)
    sc = np.float32(np.float32(100.0) / np.float32(qmax))
    near = np.float32(sc) * half.astype(np.float32)
    near = near.astype(np.float32)
    near[1::3] = np.nextafter(near[1::3], np.float32(np.inf))
    near[2::3] = np.nextafter(near[2::3], np.float32(-np.inf))
    near = np.concatenate([[np.float32(100.0)], near]).astype(np.float32)
    for t, row in ((3, ties), (11, near)):
        k[0, 0, t] = torch.from_numpy(row).to(dtype)
        v[0, 0, t] = torch.from_numpy(-row).to(dtype)
    s = seeded((B, Hkv, T), 43)
    keep = oracle.keep_mask(f64(s), 0.8, 128).reshape(P, T)
    keep[0, [3, 7, 11]] = False  # the crafted rows are demoted
    idx, cnt = upload_selection(keep)
    kv = K.PagedKV.allocate(P, d, P * 40, 40, dtype, DEV, num_pages8=P * 40,
                            max_pages8_per_pair=40, poison=True, lp_bits=bits)
    ring = K.Ring.allocate(P, 128, d, dtype, DEV, poison=True)
    K.kvp_compact(k, v, idx, cnt, kv, compact_ws(K, B, Hkv), ring=ring, scores=s,
                  mode=K.KVP_COMPACT_DEMOTE_INT8)
    assert K.kvp_check(kv) == 0
    kf = f64(k).reshape(P, T, d)
    vf = f64(v).reshape(P, T, d)
    for p in range(P):
        ev = np.flatnonzero(~keep[p])
        pos, Kc, Vc, ks, vs = read_pool8(kv, p)
        assert np.array_equal(pos, ev)
        for i, t in enumerate(ev):
            c, sc = lp_quant(bits, kf[p, t])
            assert ks[i] == sc and lp_codes_equal(bits, Kc[i], c), (p, t)
            c, sc = lp_quant(bits, vf[p, t])
            assert vs[i] == sc and lp_codes_equal(bits, Vc[i], c), (p, t)
        # every position is held exactly once across bf16 pool, ring and int8 pool
        allpos = visible_positions(kv, ring, p)
        assert np.array_equal(allpos, np.arange(T))


# ---------------------------------------------------------------------------- attention


def build_cache(K, B, Hkv, T, d, dtype, keep, ring_w, seed, demote=False, poison=True, bits=8):
    P = B * Hkv
    k = seeded((B, Hkv, T, d), seed, dtype)
    v = seeded((B, Hkv, T, d), seed + 1, dtype)
    s = seeded((B, Hkv, T), seed + 2)
    idx, cnt = upload_selection(keep)
    maxpp = T // 16 + 2
    kw = dict(num_pages8=P * maxpp, max_pages8_per_pair=maxpp, lp_bits=bits) if demote else {}
    kv = K.PagedKV.allocate(P, d, P * maxpp, maxpp, dtype, DEV, poison=poison, **kw)
    ring = K.Ring.allocate(P, ring_w, d, dtype, DEV, poison=poison) if ring_w else None
    K.kvp_compact(k, v, idx, cnt, kv, compact_ws(K, B, Hkv), ring=ring, scores=s,
                  mode=K.KVP_COMPACT_DEMOTE_INT8 if demote else K.KVP_COMPACT_EVICT)
    return k, v, kv, ring


@pytest.mark.parametrize("B,Hq,Hkv,T,d,dtype,ring_w,keepfrac", [
    (2, 16, 4, 1000, 128, torch.bfloat16, 128, 0.3),
    (1, 8, 1, 3000, 128, torch.bfloat16, 0, 0.5),
    (3, 24, 3, 517, 64, torch.bfloat16, 64, 0.2),
    (1, 4, 2, 512, 64, torch.float32, 128, 0.5),
    (2, 8, 8, 300, 128, torch.float32, 0, 0.7),
    (1, 64, 8, 2000, 128, torch.bfloat16, 128, 0.25),
    (2, 4, 4, 40, 128, torch.bfloat16, 128, 0.5),
])
def test_decode_attn(K, B, Hq, Hkv, T, d, dtype, ring_w, keepfrac):
    P = B * Hkv
    g = torch.Generator().manual_seed(T + d)
    keep = (torch.rand((P, T), generator=g) < keepfrac).numpy()
    keep[:, T - (ring_w or 128):] = True
    k, v, kv, ring = build_cache(K, B, Hkv, T, d, dtype, keep, ring_w, seed=51)
    q = seeded((B, Hq, d), 54, dtype)
    out = torch.full((B, Hq, d), float("nan"), device=DEV)
    ws = K.decode_attn_workspace(B, Hq, kv)
    K.kvp_decode_attn(q, kv, ring, K.sm_scale(d), out, ws)
    ref = oracle.decode_attention(f64(q), f64(k), f64(v), keep.reshape(B, Hkv, T),
                                  oracle.sm_scale(d))
    check_attention(out, ref, dtype)
    # deterministic: a rerun (with a garbage-filled workspace) gives identical bits
    rerun_identical(K, q, kv, ring, d, out, ws)


def rerun_identical(K, q, kv, ring, d, out, ws):
    """A rerun on a garbage-filled workspace gives the same bits (the split does not
    depend on timing and every record is written before it is read)."""
    ws.fill_(-1)
    out2 = torch.full_like(out, float("nan"))
    K.kvp_decode_attn(q, kv, ring, K.sm_scale(d), out2, ws)
    assert torch.equal(out, out2)
    assert K.kvp_check(kv) == 0


def test_decode_attn_empty_pairs(K):
    B, Hq, Hkv, T, d = 2, 8, 2, 600, 128
    P = B * Hkv
    keep = np.zeros((P, T), bool)
    keep[1, ::3] = True
    keep[3, :] = True  # pair 0 and 2 have nothing visible -> zeros
    k, v, kv, ring = build_cache(K, B, Hkv, T, d, torch.bfloat16, keep, 0, seed=61)
    q = seeded((B, Hq, d), 64, torch.bfloat16)
    out = torch.full((B, Hq, d), float("nan"), device=DEV)
    ws = K.decode_attn_workspace(B, Hq, kv)
    K.kvp_decode_attn(q, kv, None, K.sm_scale(d), out, ws)
    ref = oracle.decode_attention(f64(q), f64(k), f64(v), keep.reshape(B, Hkv, T), oracle.sm_scale(d))
    check_attention(out, ref, torch.bfloat16)
    assert (out[0, :4] == 0).all() and (out[1, :4] == 0).all()


@pytest.mark.parametrize("bits,d,Hq,T", [(8, 128, 8, 900), (4, 128, 8, 900), (4, 64, 16, 777),
                                         ("fp8", 128, 8, 900), ("fp8", 64, 16, 777)])
def test_decode_attn_lowprec_pool(K, bits, d, Hq, T):
    B, Hkv = 2, 2
    P = B * Hkv
    s = seeded((B, Hkv, T), 71)
    keep = oracle.keep_mask(f64(s), 1.2, 128).reshape(P, T)
    k, v, kv, ring = build_cache(K, B, Hkv, T, d, torch.bfloat16, keep, 128, seed=72, demote=True,
                                 bits=bits)
    q = seeded((B, Hq, d), 75, torch.bfloat16)
    out = torch.full((B, Hq, d), float("nan"), device=DEV)
    ws = K.decode_attn_workspace(B, Hq, kv)
    K.kvp_decode_attn(q, kv, ring, K.sm_scale(d), out, ws)
    ref = oracle.beacon_decode_attention(f64(q), f64(k), f64(v), keep.reshape(B, Hkv, T),
                                         oracle.sm_scale(d), bits=bits)
    check_attention(out, ref, torch.bfloat16)
    if bits in (4, "fp8"):  # that pool really is read: int8 codes would give another result
        ref8 = oracle.beacon_decode_attention(f64(q), f64(k), f64(v), keep.reshape(B, Hkv, T),
                                              oracle.sm_scale(d), bits=8)
        assert np.abs(ref8 - ref).max() > (10 if bits == 4 else 1) * 2e-3


@pytest.mark.parametrize("bits,B,Hq,Hkv,T,d,ring_w,case", [
    (8, 2, 16, 2, 1500, 64, 128, "random"),   # int8 codes at d 64, g 8
    (4, 1, 32, 2, 2000, 128, 128, "random"),  # int4, g 16 (the largest group)
    (4, 8, 64, 8, 300, 128, 128, "random"),   # int4, 64 pairs of short contexts: many segments
    (8, 2, 8, 2, 700, 128, 0, "random"),      # int8 without a ring
    (4, 2, 8, 2, 900, 128, 128, "extremes"),  # one pair with no code region, one all codes
    (8, 2, 8, 2, 900, 128, 0, "extremes"),    # ... and one pair with no full-precision token
    ("fp8", 2, 16, 2, 1500, 64, 128, "random"),   # fp8 E4M3 codes at d 64, g 8
    ("fp8", 2, 8, 2, 900, 128, 0, "extremes"),    # fp8 pool with its edge pairs
])
def test_decode_attn_lowprec_edges(K, bits, B, Hq, Hkv, T, d, ring_w, case):
    """Attention over a full-precision pool (+ ring) and an int8 / int4 pool in one
    softmax, at the head-group, head-dim and pair-count limits and with regions of a
    pair empty; reruns on a garbage-filled workspace are bit-identical."""
    P = B * Hkv
    g = torch.Generator().manual_seed(T + d + (9 if bits == "fp8" else bits))
    keep = (torch.rand((P, T), generator=g) < 0.15).numpy()
    if case == "extremes":
        keep[0, :] = True   # nothing demoted
        keep[1, :] = False  # every token demoted (bar the ring, when there is one)
    if ring_w:
        keep[:, T - ring_w:] = True  # the ring's positions are never demoted
    k, v, kv, ring = build_cache(K, B, Hkv, T, d, torch.bfloat16, keep, ring_w, seed=81,
                                 demote=True, bits=bits)
    q = seeded((B, Hq, d), 84, torch.bfloat16)
    out = torch.full((B, Hq, d), float("nan"), device=DEV)
    ws = K.decode_attn_workspace(B, Hq, kv)
    K.kvp_decode_attn(q, kv, ring, K.sm_scale(d), out, ws)
    ref = oracle.beacon_decode_attention(f64(q), f64(k), f64(v), keep.reshape(B, Hkv, T),
                                         oracle.sm_scale(d), bits=bits)
    check_attention(out, ref, torch.bfloat16)
    rerun_identical(K, q, kv, ring, d, out, ws)


# ---------------------------------------------------------------------------- delayed step


@pytest.mark.parametrize("dtype,d,w,demote,bits", [(torch.bfloat16, 128, 64, False, 8),
                                                   (torch.float32, 64, 32, False, 8),
                                                   (torch.bfloat16, 128, 32, True, 8),
                                                   (torch.bfloat16, 128, 32, True, 4),
                                                   (torch.bfloat16, 64, 48, True, 4),
                                                   (torch.bfloat16, 128, 32, True, "fp8")])
def test_step_delayed_state_machine(K, dtype, d, w, demote, bits):
    """DMS: flagged tokens stay w steps; the visible set is re-derived from scratch by
    the oracle at every step and compared with the ring + pool content."""
    B, Hkv, Hq, T0, steps = 2, 3, 6, 200, 90
    P = B * Hkv
    total = T0 + steps
    s_all = seeded((B, Hkv, total), 81) - 1.15
    tau = 0.0
    flags = oracle.dms_evict_flags(f64(s_all).reshape(P, total))
    keep0 = oracle.dms_visible(flags[:, :T0], T0 - 1, w)
    k_all = seeded((B, Hkv, total, d), 82, dtype)
    v_all = seeded((B, Hkv, total, d), 83, dtype)
    idx, cnt = upload_selection(keep0)
    maxpp = total // 16 + 2
    kw = dict(num_pages8=P * maxpp, max_pages8_per_pair=maxpp, lp_bits=bits) if demote else {}
    kv = K.PagedKV.allocate(P, d, P * maxpp, maxpp, dtype, DEV, poison=True, **kw)
    ring = K.Ring.allocate(P, w, d, dtype, DEV, poison=True)
    scores0 = s_all[..., :T0].contiguous()
    K.kvp_compact(k_all[:, :, :T0].contiguous(), v_all[:, :, :T0].contiguous(), idx, cnt, kv,
                  compact_ws(K, B, Hkv), ring=ring, scores=scores0,
                  mode=K.KVP_COMPACT_DEMOTE_INT8 if demote else K.KVP_COMPACT_EVICT)
    ws = K.decode_attn_workspace(B, Hq, kv)
    kf, vf = f64(k_all), f64(v_all)
    for i in range(steps):
        p = T0 + i
        k_new = k_all[:, :, p].contiguous()
        v_new = v_all[:, :, p].contiguous()
        s_new = s_all[:, :, p].contiguous()
        K.kvp_step_delayed(kv, ring, k_new, v_new, s_new, tau, p)
        want = oracle.dms_visible(flags, p, w)
        for pr in range(P):
            got = np.sort(np.concatenate([read_pool(kv, pr)[0], read_ring(ring, pr)[0]]))
            assert np.array_equal(got, np.flatnonzero(want[pr])), (i, pr)
            if demote:
                assert np.array_equal(np.sort(np.concatenate([got, read_pool8(kv, pr)[0]])),
                                      np.arange(p + 1))
        if i in (0, 1, w - 1, w, w + 1, steps - 1):
            q = seeded((B, Hq, d), 900 + i, dtype)
            out = torch.full((B, Hq, d), float("nan"), device=DEV)
            K.kvp_decode_attn(q, kv, ring, K.sm_scale(d), out, ws)
            vis = want.reshape(B, Hkv, -1)
            if demote:
                ref = oracle.beacon_decode_attention(f64(q), kf[:, :, :p + 1], vf[:, :, :p + 1],
                                                     vis, oracle.sm_scale(d), bits=bits)
            else:
                ref = oracle.decode_attention(f64(q), kf[:, :, :p + 1], vf[:, :, :p + 1], vis,
                                              oracle.sm_scale(d))
            check_attention(out, ref, dtype)
    assert K.kvp_check(kv) == 0
    if demote:  # every demoted row (by compaction or by a step) holds the oracle's codes
        kr, vr = kf.reshape(P, total, d), vf.reshape(P, total, d)
        for pr in range(P):
            pos, Kc, Vc, ks, vs = read_pool8(kv, pr)
            assert len(pos) > w // 2
            for i, t in enumerate(pos):
                c, sc = lp_quant(bits, kr[pr, t])
                assert ks[i] == sc and lp_codes_equal(bits, Kc[i], c), (pr, t)
                c, sc = lp_quant(bits, vr[pr, t])
                assert vs[i] == sc and lp_codes_equal(bits, Vc[i], c), (pr, t)


def _same_cache(kvA, ringA, kvB, ringB):
    """Two caches hold the same logical content: rings and per-pair counters bit for
    bit, each pair's pool rows (positions, K, V; codes and scales of the low-precision
    pool) in block-table order.  Physical page ids may differ: pages come from an atomic
    bump allocator, so which pair gets which page depends on the waves' arrival order."""
    for n, t in ringA.tensors.items():
        iv = {1: torch.int8, 2: torch.int16, 4: torch.int32}[t.element_size()]
        assert torch.equal(t.view(iv), ringB.tensors[n].view(iv)), "ring " + n
    names = ["length", "page_top", "err"] + (["length8", "page8_top"] if kvA.c.num_pages8 else [])
    for n in names:
        assert torch.equal(kvA.tensors[n], kvB.tensors[n]), n
    for pr in range(kvA.c.num_pairs):
        for a, b in zip(read_pool(kvA, pr), read_pool(kvB, pr)):
            assert np.array_equal(a, b), ("pool", pr)
        if kvA.c.num_pages8:
            for a, b in zip(read_pool8(kvA, pr), read_pool8(kvB, pr)):
                assert np.array_equal(a, b), ("pool8", pr)


@pytest.mark.parametrize("kind,xdtype,H,inner,kvdtype,d,w,bias,demote", [
    ("linear", torch.bfloat16, 4096, 0, torch.bfloat16, 128, 64, True, False),
    ("linear", torch.float32, 256, 0, torch.float32, 64, 32, False, False),
    ("linear", torch.bfloat16, 1032, 0, torch.bfloat16, 128, 32, True, True),  # H % 512 != 0
    ("linear", torch.float32, 100, 0, torch.bfloat16, 64, 48, True, False),    # H % 256 != 0
    ("mlp", torch.bfloat16, 4096, 512, torch.bfloat16, 128, 64, True, False),   # 16 K slices
    ("mlp", torch.bfloat16, 8192, 512, torch.bfloat16, 128, 32, True, True),    # 32 K slices
    ("mlp", torch.bfloat16, 768, 256, torch.bfloat16, 64, 32, False, False),    # 3 slices, width 256
    ("mlp", torch.bfloat16, 512, 1024, torch.float32, 64, 48, True, False),     # width 1024
])
def test_score_step_delayed_fused(K, kind, xdtype, H, inner, kvdtype, d, w, bias, demote):
    """kvp_score_step_delayed: the new tokens' scores match the oracle's (and kvp_score's
    own small-batch scores), and the cache it leaves holds, bit for bit, what
    kvp_step_delayed_dev leaves when fed those scores -- two caches driven side by side
    for 80 steps (retentions, drops, demotions and page allocations included)."""
    B, Hkv, Hq, T0, steps = 3, 4, 8, 150, 80
    P = B * Hkv
    total = T0 + steps
    if kind == "linear":
        W1 = seeded((Hkv, H), 101, xdtype, scale=1.0 / math.sqrt(H))
        b1 = (seeded((Hkv,), 102) * 0.1 - 1.15) if bias else None
        sc = K.Scorer(K.KVP_SCORER_LINEAR, W1, b1)
    else:
        W1 = seeded((inner, H), 101, xdtype, scale=1.0 / math.sqrt(H))
        b1 = seeded((inner,), 102, scale=0.5) if bias else None
        W2 = seeded((Hkv, inner), 107, scale=1.0 / math.sqrt(inner))
        b2 = (seeded((Hkv,), 108) * 0.1 - 0.3) if bias else None
        sc = K.Scorer(K.KVP_SCORER_MLP, W1, b1, W2, b2)
    ws = torch.empty(max(1, K.kvp_score_workspace_size(sc, B, 1) // 4), dtype=torch.float32,
                     device=DEV)
    x_all = seeded((steps, B, 1, H), 103, xdtype)
    k_all = seeded((B, Hkv, total, d), 104, kvdtype)
    v_all = seeded((B, Hkv, total, d), 105, kvdtype)
    s0 = seeded((B, Hkv, T0), 106) - 1.15
    keep0 = oracle.dms_visible(oracle.dms_evict_flags(f64(s0).reshape(P, T0)), T0 - 1, w)
    idx, cnt = upload_selection(keep0)
    maxpp = total // 16 + 2
    kw = dict(num_pages8=P * maxpp, max_pages8_per_pair=maxpp, lp_bits=8) if demote else {}
    caches = []
    for _ in range(2):
        kv = K.PagedKV.allocate(P, d, P * maxpp, maxpp, kvdtype, DEV, poison=True, **kw)
        ring = K.Ring.allocate(P, w, d, kvdtype, DEV, poison=True)
        K.kvp_compact(k_all[:, :, :T0].contiguous(), v_all[:, :, :T0].contiguous(), idx, cnt, kv,
                      compact_ws(K, B, Hkv), ring=ring, scores=s0.contiguous(),
                      mode=K.KVP_COMPACT_DEMOTE_INT8 if demote else K.KVP_COMPACT_EVICT)
        tau = torch.zeros(1, dtype=torch.float32, device=DEV)
        pos = torch.tensor([T0, 0], dtype=torch.int32, device=DEV)
        caches.append((kv, ring, tau, pos))
    (kvA, ringA, tauA, posA), (kvB, ringB, tauB, posB) = caches
    s_new = torch.full((P,), float("nan"), dtype=torch.float32, device=DEV)
    s_sep = torch.full((B, Hkv, 1), float("nan"), dtype=torch.float32, device=DEV)
    ws_sep = torch.empty_like(ws)
    for i in range(steps):
        p = T0 + i
        k_new = k_all[:, :, p].contiguous()
        v_new = v_all[:, :, p].contiguous()
        K.kvp_score_step_delayed(sc, x_all[i], kvA, ringA, k_new, v_new, tauA, posA, s_new, ws)
        K.kvp_step_delayed(kvB, ringB, k_new, v_new, s_new, tauB, posB)
        if kind == "linear":
            ref = oracle.score_linear(f64(x_all[i]), f64(W1), f64(b1) if bias else None)
        else:
            ref = oracle.score_mlp(f64(x_all[i]), f64(W1), f64(b1) if bias else None, f64(W2),
                                   f64(b2) if bias else None)
        got = s_new.cpu().double().numpy()
        err = np.abs(got - ref.reshape(P)).max()
        assert err < 2.5e-5, (i, err)
        if i % 8 == 0:
            if not (kind == "linear" and xdtype == torch.bfloat16 and H % 32):  # kvp_score's shapes
                K.kvp_score(sc, x_all[i], s_sep, ws_sep)
                assert np.abs(got - s_sep.cpu().double().numpy().reshape(P)).max() < 1e-5
            _same_cache(kvA, ringA, kvB, ringB)
    _same_cache(kvA, ringA, kvB, ringB)
    assert int(posA[0]) == total and int(posA[1]) == 0
    assert K.kvp_check(kvA) == 0


# ---------------------------------------------------------------------------- errors


def test_capacity_overflow_reported(K):
    B, Hkv, T, d = 1, 2, 400, 128
    P = B * Hkv
    keep = np.ones((P, T), bool)
    idx, cnt = upload_selection(keep)
    k = seeded((B, Hkv, T, d), 91, torch.bfloat16)
    kv = K.PagedKV.allocate(P, d, 30, 30, torch.bfloat16, DEV)  # needs 2 * 25 pages
    K.kvp_compact(k, k, idx, cnt, kv, compact_ws(K, B, Hkv))
    assert K.kvp_check(kv) == 4  # KVP_E_CAPACITY
    assert int(kv.err[0]) & K.ERR_POOL_FULL
    assert int(kv.length.sum()) <= 30 * 16
    K.kvp_clear_error(kv)
    assert K.kvp_check(kv) == 0
    # table overflow
    kv2 = K.PagedKV.allocate(P, d, 100, 10, torch.bfloat16, DEV)
    K.kvp_compact(k, k, idx, cnt, kv2, compact_ws(K, B, Hkv))
    assert K.kvp_check(kv2) == 4 and int(kv2.err[0]) & K.ERR_TABLE_FULL
    # attention still runs on what fits
    q = seeded((B, 4, d), 92, torch.bfloat16)
    out = torch.zeros((B, 4, d), device=DEV)
    K.kvp_decode_attn(q, kv2, None, K.sm_scale(d), out, K.decode_attn_workspace(B, 4, kv2))
    assert torch.isfinite(out).all()


def test_argument_errors(K):
    B, Hkv, T, d = 1, 2, 64, 128
    kv = K.PagedKV.allocate(B * Hkv, d, 16, 8, torch.bfloat16, DEV)
    q = torch.zeros((B, 3, d), dtype=torch.bfloat16, device=DEV)  # 3 % 2 != 0
    out = torch.zeros((B, 3, d), device=DEV)
    with pytest.raises(K.KvpError) as e:
        K.kvp_decode_attn(q, kv, None, 0.1, out, K.decode_attn_workspace(B, 4, kv))
    assert e.value.status == 1
    q = torch.zeros((B, 4, d), dtype=torch.float32, device=DEV)  # dtype mismatch
    with pytest.raises(K.KvpError) as e:
        K.kvp_decode_attn(q, kv, None, 0.1, torch.zeros((B, 4, d), device=DEV),
                          K.decode_attn_workspace(B, 4, kv))
    assert e.value.status == 2
    q = torch.zeros((B, 4, d), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(K.KvpError) as e:  # undersized workspace
        K.kvp_decode_attn(q, kv, None, 0.1, torch.zeros((B, 4, d), device=DEV),
                          torch.zeros(4, dtype=torch.int32, device=DEV))
    assert e.value.status == 3
    s10 = torch.zeros((B, Hkv, 10), device=DEV)
    with pytest.raises(K.KvpError):  # ld_s < T
        K.kvp_select(s10, T, 0.0, 128, torch.zeros(4, dtype=torch.int32, device=DEV),
                     torch.zeros(4, dtype=torch.int32, device=DEV),
                     torch.zeros(4, dtype=torch.int32, device=DEV),
                     torch.zeros(16, dtype=torch.int32, device=DEV))
